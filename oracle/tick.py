"""CPU oracle of the Moshi/PersonaPlex lockstep tick (plain NumPy).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What one tick computes, per session slot, in the pages' order:

* PersonaPlex recipe (vLLM-Omni), "Architecture (Moshi RQ-Transformer, all
  native)": one frame per 80 ms tick; a per-frame token column [B, 17, 1]
  (row 0 inner-monologue text, rows 1-8 agent audio, rows 9-16 user audio)
  goes through the Helium temporal transformer (4096-d / 32 layers / 32
  heads) whose keys and values live in a ring KV cache with a 3000-frame
  sliding window and per-slot recycle; the depformer (1024-d / 6 layers / 16
  heads) then runs autoregressively over 16 codebooks and is reset each
  frame.
* vLLM-Omni PersonaPlex guide (mhpq.cn), "架构": RMSNorm with fp32 alpha,
  fused in-projection attention, interleaved RoPE at absolute positions,
  SiLU-gated MLP; "贪心解码与 Parity 约束": greedy decoding (temperature 0,
  top_k 1), one token per tick, relative-position causal mask.
* Same guide, "帧 token 布局": TEXT_INITIAL_TOKEN = text vocabulary size,
  AUDIO_INITIAL_TOKEN = codec cardinality (the tokens a fresh session's
  column starts from).

Readings taken where the pages are silent:
eps 1e-5 inside the square root; RoPE base 10000 on pairs (2i, 2i+1) with the
angle in fp64; window = the W most recent positions including the current
one; scale 1/sqrt(head_dim), no biases; fused rows laid out [q; k; v] and
[gate; up]; one output norm feeds the text head and all depformer input
projections; depformer step 0 is fed the chosen text token, step k the chosen
token of step k-1, its layers are shared across steps and carry no positional
encoding; depformer codebooks 0-7 are the agent rows, 8-15 predict the user
stream; argmax ties go to the lowest index; forced tokens replace the model's
choice but the model's own predictions are still returned.

Acoustic delay and embedding-form prefill (the recipe's interruption-latency
table: an 80 ms frame plus an 80 ms acoustic delay; its prompt injection:
voice embedding rows, silence frames and persona tokens are assembled into
prefill embeddings).  With a delay of D frames, codebooks 1-7 of both audio
streams run D ticks behind the text row and codebook 0: the column's user
rows 10-16 and the forced choices of agent rows 2-8 come from the frame D
ticks earlier (the initial audio token / no force before the first), and the
agent frame f is complete at tick f + D (codebook 0 chosen at tick f, 1-7 at
tick f + D).  An embedding-form prefill frame supplies the temporal input x
itself, in place of the 17-way gather-sum, with the same per-row forced
choices as a token frame.

Arithmetic: weights are the exact bf16 values upcast to `dtype` (fp32 by
default, fp64 for the shadow run); everything else is `dtype`, except the RoPE
angle, which is fp64 with cos/sin cast to `dtype`.  Slots are processed one
at a time.

Cache storage: the ring and the depformer's per-frame keys/values hold bf16
values (each stored key/value rounded to the nearest bf16, ties to even), as
the served model keeps its caches in the model's bf16 dtype (the guide singles
out only the RMSNorm alpha as fp32).  kv_store="exact" keeps them in `dtype`
instead (used by the fp64 shadow and closed-form checks).
"""
from __future__ import annotations

import numpy as np

from oracle import sampling

TEXT_ROW = 0
AGENT_ROWS = slice(1, 9)
USER_ROWS = slice(9, 17)


def upcast_bf16(bits: np.ndarray, dtype=np.float32) -> np.ndarray:
    """bf16 bit patterns -> values (exact in fp32 and fp64)."""
    b = np.asarray(bits, dtype=np.uint16)
    u = np.empty(b.shape, dtype=np.uint32)
    np.left_shift(b, 16, out=u, dtype=np.uint32)
    return u.view(np.float32).astype(dtype, copy=False)


def rmsnorm(x: np.ndarray, alpha: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with an fp32 scale ("架构": fp32 RMSNorm alpha):
    x * alpha / sqrt(mean(x^2) + eps)."""
    dt = x.dtype
    ms = np.mean(x * x, dtype=dt)
    return x * alpha.astype(dt) / np.sqrt(ms + dt.type(eps))


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU gate g / (1 + exp(-g)) ("架构": SiLU gating MLP)."""
    one = g.dtype.type(1)
    return g / (one + np.exp(-g))


def rope_interleaved(v: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Interleaved rotary embedding at absolute position `pos` ("架构":
    绝对位置处的交错 RoPE).  v is [H, Dh]; the pair (2i, 2i+1) of every head
    turns by pos * base^(-2i/Dh), the angle evaluated in fp64."""
    H, Dh = v.shape
    i = np.arange(Dh // 2, dtype=np.float64)
    theta = float(pos) * np.power(float(base), -2.0 * i / Dh)
    c = np.cos(theta).astype(v.dtype)
    s = np.sin(theta).astype(v.dtype)
    a = v[:, 0::2]
    b = v[:, 1::2]
    out = np.empty_like(v)
    out[:, 0::2] = a * c - b * s
    out[:, 1::2] = a * s + b * c
    return out


def softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Scaled dot-product attention of one query per head over n keys given in
    position order.  q [H, Dh]; keys, vals [n, H, Dh] -> [H, Dh]."""
    dt = q.dtype
    Dh = q.shape[1]
    scale = dt.type(1.0 / np.sqrt(Dh))
    s = np.einsum("hd,nhd->hn", q, keys) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", p, vals)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of each element (ties to even), returned as float32.
    fp64 input is first rounded to fp32."""
    u = np.array(x, dtype=np.float32).view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def greedy(logits: np.ndarray) -> int:
    """Greedy decoding ("贪心解码与 Parity 约束": temperature 0, top_k 1);
    the first maximum wins a tie.  NaN logits are an error."""
    if np.isnan(logits).any():
        raise FloatingPointError("NaN logits")
    return int(np.argmax(logits))


class _Slot:
    def __init__(self, dm, W, dt):
        self.K = np.zeros((dm.n_layers, W, dm.n_heads, dm.head_dim), dt)
        self.V = np.zeros_like(self.K)
        self.reset(dm)

    def reset(self, dm):
        self.pos = 0
        self.prev = np.array([dm.text_card] + [dm.audio_card] * 8, np.int64)
        self.queue = []        # prefill frames: dict(force=[9], user=[8] | None, x=[d] | None)
        self.ticks = 0         # ticks since the last reset
        self.user_hist = []    # frame-aligned user frames of past ticks (None: none given)
        self.force_hist = []   # frame-aligned forced agent rows of past ticks (-1: free)
        self.chosen_hist = []  # chosen agent rows of past ticks
        self.text_hist = []    # chosen text tokens of the last sampling.REP_WINDOW ticks
        self.live = False      # True after the first free-running tick
        self.ticked = False    # True after any tick since the last reset
        self.K[...] = 0
        self.V[...] = 0


class Oracle:
    """Batched lockstep engine state + tick, one slot at a time.

    weights: name -> array, bf16 bit patterns (uint16) for matrices and
    tables, fp32 for RMSNorm alphas, named as in the weight manifest of the
    input generator.  window: ring capacity W (frames)."""

    def __init__(self, dims, weights, B, window, dtype=np.float32, cache_weights=None, kv_store="bf16"):
        if kv_store not in ("bf16", "exact"):
            raise ValueError("kv_store must be 'bf16' or 'exact'")
        self.kv_store = kv_store
        self.dm = dims
        self.B = int(B)
        self.W = int(window)
        self.dt = np.dtype(dtype)
        self._raw = weights
        total = sum(a.size for a in weights.values())
        self._cache = {} if (cache_weights if cache_weights is not None else total < 50_000_000) else None
        self.slots = [_Slot(dims, self.W, self.dt) for _ in range(self.B)]
        self.taps = {}
        self.delay = 0
        self.sampling = None   # None: greedy; else dict(t_text, t_audio, top_k, top_p, rho)
        self.seeds = [0] * self.B

    def _store(self, v):
        """Value as kept in a key/value cache."""
        return round_bf16(v).astype(self.dt) if self.kv_store == "bf16" else v

    # ------------------------------------------------------------ weights
    def w(self, name):
        """Weight `name` as `dtype` values."""
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        a = self._raw[name]
        v = upcast_bf16(a, self.dt) if a.dtype == np.uint16 else a.astype(self.dt)
        if self._cache is not None:
            self._cache[name] = v
        return v

    def row(self, name, i):
        """Row i of table `name` as `dtype` values (an embedding lookup)."""
        if self._cache is not None and name in self._cache:
            return self._cache[name][i]
        a = self._raw[name]
        return upcast_bf16(a[i], self.dt) if a.dtype == np.uint16 else a[i].astype(self.dt)

    # ------------------------------------------------------------ session control
    def slot_reset(self, s):
        """Recycle slot s: position 0, column back to the initial tokens,
        forced queue cleared, ring emptied."""
        self.slots[s].reset(self.dm)

    def ring_fill(self, s, k_bits, v_bits):
        """Store keys/values for positions 0..n-1 (bf16 bits [L, n, H, Dh],
        the stored post-rotation values); the next tick runs at position n."""
        st = self.slots[s]
        n = k_bits.shape[1]
        if st.ticked or st.queue:
            raise RuntimeError("ring fill after a tick or a prefill")
        if n > self.W:
            raise ValueError("fill longer than the window")
        st.K[...] = 0
        st.V[...] = 0
        st.K[:, :n] = upcast_bf16(k_bits, self.dt)
        st.V[:, :n] = upcast_bf16(v_bits, self.dt)
        st.pos = n

    def prefill_forced(self, s, frames):
        """Queue forced frames [n, 17] for slot s (rows 0-8: token to choose
        or -1; rows 9-16: the user codes of that tick)."""
        st = self.slots[s]
        if st.live:
            raise RuntimeError("prefill on a live slot")
        for f in np.asarray(frames, np.int64).reshape(-1, 17):
            st.queue.append(dict(force=f[:9].copy(), user=f[9:].copy(), x=None))

    def prefill_embed(self, s, x, force=None):
        """Queue embedding-form prefill frames for slot s: x [n, d] is that
        tick's temporal input (replacing the gather-sum); force [n, 9] the
        tokens to choose for the text and agent rows or -1 (default all -1)."""
        st = self.slots[s]
        if st.live:
            raise RuntimeError("prefill on a live slot")
        x = np.asarray(x).reshape(-1, self.dm.d)
        force = np.full((len(x), 9), -1, np.int64) if force is None else np.asarray(force, np.int64).reshape(-1, 9)
        for xi, fi in zip(x, force):
            st.queue.append(dict(force=fi.copy(), user=None, x=xi.astype(self.dt)))

    def set_sampling(self, t_text, t_audio, top_k=0, top_p=1.0, rho=1.0):
        """Replace the greedy choice by sampling (the sampling module)."""
        self.sampling = dict(t_text=float(t_text), t_audio=float(t_audio), top_k=int(top_k), top_p=float(top_p),
                             rho=float(rho))

    def slot_seed(self, s, seed):
        self.seeds[s] = int(seed)

    def set_acoustic_delay(self, frames):
        """Delay of audio codebooks 1-7 behind the text row and codebook 0,
        in frames; only before any slot has ticked."""
        if any(st.ticked for st in self.slots):
            raise RuntimeError("delay change after a tick")
        if not 0 <= int(frames) <= 4:
            raise ValueError("delay outside 0..4")
        self.delay = int(frames)

    # ------------------------------------------------------------ the tick
    def step(self, user_codes):
        """One lockstep tick for all B slots.  user_codes int [B, 8].
        Returns tokens int [B, 9] = [pred_text, pred_agent_0..7]."""
        dm = self.dm
        user_codes = np.asarray(user_codes, np.int64).reshape(self.B, 8)
        hidden = np.zeros((dm.n_layers + 1, self.B, dm.d), self.dt)
        text_logits = np.zeros((self.B, dm.text_card), self.dt)
        dep_logits = np.zeros((self.B, dm.dep_q, dm.audio_card), self.dt)
        tokens = np.zeros((self.B, 9), np.int64)
        user_pred = np.zeros((self.B, dm.dep_q - 8), np.int64)
        chosen = np.zeros((self.B, 9), np.int64)
        agent_frame = np.zeros((self.B, 8), np.int64)
        agent_frame_valid = np.zeros(self.B, bool)
        for b in range(self.B):
            st = self.slots[b]
            frame = st.queue.pop(0) if st.queue else None
            if frame is None:
                st.live = True
            col, forced, x = self._column(st, user_codes[b], frame)
            r = self._tick_slot(st, col, forced, x, self.seeds[b])
            hidden[:, b] = r["hidden"]
            text_logits[b] = r["text_logits"]
            dep_logits[b] = r["dep_logits"]
            tokens[b] = r["tokens"]
            user_pred[b] = r["user_pred"]
            chosen[b] = r["chosen"]
            agent_frame[b], agent_frame_valid[b] = self._agent_frame(st, r["chosen"][1:])
        self.taps = dict(hidden=hidden, text_logits=text_logits, dep_logits=dep_logits,
                         user_pred=user_pred, chosen=chosen, agent_frame=agent_frame,
                         agent_frame_valid=agent_frame_valid)
        return tokens

    def _column(self, st, user, frame):
        """This tick's column, forced choices (-1 free) and given input x.

        The frame-aligned user frame and forced agent row of this tick enter
        the column for the text row and codebook 0 now, and for codebooks
        1-7 D ticks later."""
        A, D = self.dm.audio_card, self.delay
        if frame is None:
            u_now, f_now, x = np.array(user, np.int64), np.full(9, -1, np.int64), None
        else:
            u_now, f_now, x = frame["user"], frame["force"], frame["x"]
        u_old = st.user_hist[-D] if D and len(st.user_hist) >= D else (u_now if not D else None)
        f_old = st.force_hist[-D] if D and len(st.force_hist) >= D else (f_now[1:] if not D else None)
        user_rows = np.full(8, A, np.int64)
        if u_now is not None:
            user_rows[0] = u_now[0]
        if u_old is not None:
            user_rows[1:] = u_old[1:]
        forced = f_now.copy()
        forced[2:] = f_old[1:] if f_old is not None else -1
        st.user_hist = (st.user_hist + [u_now])[-max(D, 1):]
        st.force_hist = (st.force_hist + [f_now[1:].copy()])[-max(D, 1):]
        col = np.concatenate([st.prev, user_rows])
        return col, (forced if (forced >= 0).any() else None), x

    def _agent_frame(self, st, chosen_agent):
        """The agent frame completed by this tick: codebook 0 chosen D ticks
        ago, codebooks 1-7 chosen now; (frame, valid)."""
        D = self.delay
        st.chosen_hist = (st.chosen_hist + [np.asarray(chosen_agent, np.int64).copy()])[-(D + 1):]
        st.ticks += 1
        if st.ticks <= D:
            return np.zeros(8, np.int64), False
        return np.concatenate([st.chosen_hist[0][:1], st.chosen_hist[-1][1:]]), True

    def _choose(self, logits, seed, tick, row, history=()):
        """The model's own token for one row: greedy, or sampled."""
        if self.sampling is None:
            return greedy(logits)
        sp = self.sampling
        u = sampling.uniform(seed, tick, row)
        if row == 0:
            return sampling.sample(logits, u, sp["t_text"], sp["top_k"], sp["top_p"], sp["rho"], history)
        return sampling.sample(logits, u, sp["t_audio"], sp["top_k"], sp["top_p"])

    def _tick_slot(self, st, col, forced, x_given=None, seed=0):
        """One slot's tick.  col: the 17-row column (prev text+agent tokens,
        then the user rows); forced: 9 choices (-1 free) or None; x_given:
        an embedding-form frame's temporal input, or None."""
        dm, dt, W = self.dm, self.dt, self.W
        d, H, Dh, F = dm.d, dm.n_heads, dm.head_dim, dm.ffn
        eps = dm.norm_eps

        # 2. embedding: sum of the 17 row embeddings, in row order, unless
        #    the frame gives the input itself.
        if x_given is not None:
            x = np.array(x_given, dt)
        else:
            x = np.zeros(d, dt)
            x += self.row("emb.text", col[0])
            for r in range(1, 17):
                x += self.row(f"emb.audio.{r - 1}", col[r])
        hidden = [x.copy()]

        # 3. temporal transformer, one frame at absolute position pos.
        pos = st.pos
        lo = max(0, pos - W + 1)
        ring_idx = [p % W for p in range(lo, pos + 1)]
        for l in range(dm.n_layers):
            h = rmsnorm(x, self.w(f"layers.{l}.attn_norm"), eps)
            qkv = self.w(f"layers.{l}.wqkv") @ h
            q = qkv[0:d].reshape(H, Dh)
            k = qkv[d:2 * d].reshape(H, Dh)
            v = qkv[2 * d:3 * d].reshape(H, Dh)
            q = rope_interleaved(q, pos, dm.rope_base)
            k = rope_interleaved(k, pos, dm.rope_base)
            st.K[l, pos % W] = self._store(k)
            st.V[l, pos % W] = self._store(v)
            o = softmax_attend(q, st.K[l, ring_idx], st.V[l, ring_idx])
            x = x + self.w(f"layers.{l}.wo") @ o.reshape(d)
            h = rmsnorm(x, self.w(f"layers.{l}.mlp_norm"), eps)
            gu = self.w(f"layers.{l}.w_in") @ h
            m = silu(gu[:F]) * gu[F:]
            x = x + self.w(f"layers.{l}.w_out") @ m
            hidden.append(x.copy())

        # 4-5. output norm, text head, greedy text token.
        z = rmsnorm(x, self.w("out_norm"), eps)
        text_logits = self.w("text_head") @ z
        pred_text = self._choose(text_logits, seed, st.ticks, 0, st.text_hist)
        chosen_text = int(forced[0]) if forced is not None and forced[0] >= 0 else pred_text

        # 6. depformer over the 16 codebooks of this frame; its per-step
        #    keys/values start empty every tick.
        dd, dH, dDh, dF = dm.dep_d, dm.dep_heads, dm.dep_head_dim, dm.dep_ffn
        dK = np.zeros((dm.dep_layers, dm.dep_q, dH, dDh), dt)
        dV = np.zeros_like(dK)
        dep_logits = np.zeros((dm.dep_q, dm.audio_card), dt)
        preds, chosen_audio = [], []
        layers = [{k: self.w(f"dep.layers.{l}.{k}")
                   for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out")}
                  for l in range(dm.dep_layers)]
        tok = chosen_text
        for kq in range(dm.dep_q):
            table = "dep.emb.text" if kq == 0 else f"dep.emb.audio.{kq}"
            y = self.w(f"dep.in_proj.{kq}") @ z + self.row(table, tok)
            for l in range(dm.dep_layers):
                lw = layers[l]
                h = rmsnorm(y, lw["attn_norm"], eps)
                qkv = lw["wqkv"] @ h
                q = qkv[0:dd].reshape(dH, dDh)
                dK[l, kq] = self._store(qkv[dd:2 * dd].reshape(dH, dDh))
                dV[l, kq] = self._store(qkv[2 * dd:3 * dd].reshape(dH, dDh))
                o = softmax_attend(q, dK[l, :kq + 1], dV[l, :kq + 1])
                y = y + lw["wo"] @ o.reshape(dd)
                h = rmsnorm(y, lw["mlp_norm"], eps)
                gu = lw["w_in"] @ h
                y = y + lw["w_out"] @ (silu(gu[:dF]) * gu[dF:])
            yn = rmsnorm(y, self.w("dep.out_norm"), eps)
            lg = self.w(f"dep.head.{kq}") @ yn
            dep_logits[kq] = lg
            p = self._choose(lg, seed, st.ticks, 1 + kq)
            preds.append(p)
            c = p
            if kq < 8 and forced is not None and forced[1 + kq] >= 0:
                c = int(forced[1 + kq])
            chosen_audio.append(c)
            tok = c

        # 7. outputs and state.
        chosen = np.array([chosen_text] + chosen_audio[:8], np.int64)
        st.text_hist = (st.text_hist + [chosen_text])[-sampling.REP_WINDOW:]
        st.prev = chosen
        st.pos = pos + 1
        st.ticked = True
        return dict(hidden=np.stack(hidden), text_logits=text_logits, dep_logits=dep_logits,
                    tokens=np.array([pred_text] + preds[:8], np.int64),
                    user_pred=np.array(preds[8:], np.int64), chosen=chosen)
