"""CPU oracle of a streaming codec (Mimi-like): the decoder (code2wav) turns 8
codebook indices per 80 ms frame into 1920 audio samples at 24 kHz; the
encoder turns 1920 samples of user audio into 8 codebook indices.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What the pages fix (chenxutan.com PersonaPlex article, section 2.3 on Mimi;
PersonaPlex recipe, "Architecture"): a neural codec of the SoundStream /
EnCodec family that turns 12.5 Hz frames of 8 codebooks (2048 entries each,
1.1 kbps) back into 24 kHz audio, 1920 samples per frame; fully causal and
streaming; a transformer inside the decoder.  The pages give neither its
layers nor its weights, so the decoder here is one plain reading of that
family:

* residual-quantiser decoding: the frame's latent is the sum of the 8
  codebooks' rows, taken in codebook order;
* a causal transformer over frames with the temporal transformer's block
  (RMSNorm with fp32 alpha, fused QKV, interleaved RoPE at the frame's
  position, softmax attention over a sliding window of past frames whose
  keys and values are kept as bf16, SiLU-gated MLP), then an output RMSNorm;
* a convolutional decoder: a causal convolution, then one stage per stride
  (ELU, causal transposed convolution of kernel 2 x stride that upsamples by
  the stride, then a residual unit: ELU, causal convolution of kernel 3 to
  half the channels, ELU, 1 x 1 convolution back, added to the stage's
  upsampled signal), then ELU and a causal convolution to one channel.  The
  strides (2, 8, 6, 5, 4) multiply to 1920.
* the encoder mirrors it: a causal convolution from one channel, then per
  stage (the decoder's stages in reverse) a residual unit and ELU with a
  causal strided convolution of kernel 2 x stride that downsamples by the
  stride and doubles the channels, then ELU and a causal convolution to the
  latent width; the same transformer block with its own weights and output
  norm; then residual vector quantisation against the decoder's codebooks:
  code_q = the nearest row of codebook q to the residual (squared Euclidean
  distance, the lowest index on ties), residual -= that row, for q = 0..7.

Causal strided convolution with stride s (K = 2 s): output t reads inputs
t s - s + k, k = 0 .. K-1 (the previous block of s inputs and the current
one).

Causal convolution: y[o, t] = b[o] + sum_i sum_k w[o, i, k] x[i, t - (K-1-k)],
with x = 0 before the stream starts.  Causal transposed convolution with
stride s (PyTorch ConvTranspose1d form, weights here [C_out][C_in][K]): input
m adds w[o, i, k] x[i, m] to output m s + k; a call that receives inputs
M0..M1 emits outputs M0 s .. (M1+1) s - 1, whose contributions all come from
inputs up to M1 because K = 2 s (the overhang of input M1 is completed when
input M1 + 1 arrives).  Streaming state per slot: the frame position, the
transformer's key/value ring, and for each convolution the inputs it still
needs from earlier calls.

Arithmetic: weights are the exact bf16 values upcast to `dtype` (fp32 by
default, fp64 for a shadow run); everything else is `dtype`.
"""
from __future__ import annotations

import numpy as np

from oracle.tick import rmsnorm, rope_interleaved, round_bf16, silu, softmax_attend, upcast_bf16


def elu(x: np.ndarray) -> np.ndarray:
    """ELU with alpha 1: x for x > 0, exp(x) - 1 otherwise."""
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0)))


def causal_conv(x: np.ndarray, w: np.ndarray, b: np.ndarray, hist: np.ndarray) -> np.ndarray:
    """x [C_in][T], w [C_out][C_in][K], b [C_out], hist [C_in][K-1] (the
    K-1 inputs before x).  y [C_out][T], tap k multiplying x[t - (K-1-k)]."""
    K, T = w.shape[2], x.shape[1]
    xe = np.concatenate([hist, x], axis=1)
    y = np.repeat(b[:, None], T, axis=1)
    for k in range(K):
        y = y + w[:, :, k] @ xe[:, k:k + T]
    return y


def conv_transpose_causal(x: np.ndarray, w: np.ndarray, b: np.ndarray, prev: np.ndarray, s: int) -> np.ndarray:
    """x [C_in][T], w [C_out][C_in][K] with K = 2 s, prev [C_in][1] (the input
    before x).  Scatter form of the definition: every input m (prev is
    m = -1) adds w[:, :, k] x[:, m] to output m s + k; outputs 0 .. T s - 1
    are returned."""
    K, T = w.shape[2], x.shape[1]
    assert K == 2 * s
    xe = np.concatenate([prev, x], axis=1)
    y = np.repeat(b[:, None], T * s, axis=1)
    for j in range(T + 1):
        m = j - 1
        for k in range(K):
            n = m * s + k
            if 0 <= n < T * s:
                y[:, n] = y[:, n] + w[:, :, k] @ xe[:, j]
    return y


def strided_conv_causal(x: np.ndarray, w: np.ndarray, b: np.ndarray, hist: np.ndarray, s: int) -> np.ndarray:
    """x [C_in][T] with T a multiple of s, w [C_out][C_in][K] with K = 2 s,
    hist [C_in][K - s] (the inputs before x).  Output t [C_out][T / s] reads
    inputs t s - (K - s) + k at tap k."""
    K, T = w.shape[2], x.shape[1]
    assert K == 2 * s and T % s == 0
    To = T // s
    xe = np.concatenate([hist, x], axis=1)
    y = np.repeat(b[:, None], To, axis=1)
    for k in range(K):
        y = y + w[:, :, k] @ xe[:, k:k + To * s:s]
    return y


def nearest(r: np.ndarray, table: np.ndarray) -> tuple:
    """The row of table [n][d] nearest to r in squared Euclidean distance
    (the lowest index among equals), and every row's distance."""
    dist = np.sum((table - r[None, :]) ** 2, axis=1)
    return int(np.argmin(dist)), dist


class _State:
    def __init__(self, cd, W, dt):
        self.K = np.zeros((cd.n_layers, W, cd.n_heads, cd.head_dim), dt)
        self.V = np.zeros_like(self.K)
        self.hist = {}
        self.reset(cd, dt)

    def reset(self, cd, dt):
        self.pos = 0
        self.K[...] = 0
        self.V[...] = 0
        c = cd.channels
        self.hist = {"conv_in": np.zeros((cd.d, cd.conv_k - 1), dt),
                     "conv_out": np.zeros((c[-1], cd.conv_k - 1), dt)}
        for i in range(len(cd.strides)):
            self.hist[f"up.{i}"] = np.zeros((c[i], 1), dt)
            self.hist[f"res.{i}.a"] = np.zeros((c[i + 1], cd.res_k - 1), dt)


class _EncState:
    def __init__(self, cd, W, dt):
        self.K = np.zeros((cd.n_layers, W, cd.n_heads, cd.head_dim), dt)
        self.V = np.zeros_like(self.K)
        self.reset(cd, dt)

    def reset(self, cd, dt):
        self.pos = 0
        self.K[...] = 0
        self.V[...] = 0
        c, n = cd.channels, len(cd.strides)
        self.hist = {"enc.conv_in": np.zeros((1, cd.conv_k - 1), dt),
                     "enc.conv_out": np.zeros((c[0], cd.conv_k - 1), dt)}
        for j in range(n):
            self.hist[f"enc.res.{j}.a"] = np.zeros((c[n - j], cd.res_k - 1), dt)
            self.hist[f"enc.down.{j}"] = np.zeros((c[n - j], cd.strides[n - 1 - j]), dt)


class CodecOracle:
    """B independent streams; decode() takes one frame of 8 codes per slot."""

    def __init__(self, cd, weights, B, dtype=np.float32, kv_store="bf16"):
        self.cd, self.B, self.dt = cd, B, dtype
        self.W = cd.window
        self.kv_store = kv_store
        self.wts = {}
        for k, v in weights.items():
            self.wts[k] = upcast_bf16(v, dtype) if v.dtype == np.uint16 else np.asarray(v, dtype)
        self.slots = [_State(cd, self.W, dtype) for _ in range(B)]
        self.enc_slots = [_EncState(cd, self.W, dtype) for _ in range(B)]
        # Test hook for the bf16 rounding of stored keys and values, a decision
        # with two valid outcomes where the exact value lies at a rounding
        # midpoint within another implementation's rounding error:
        # store_hook(slot, layer, pos, k, v, k_stored, v_stored) -> the (k, v)
        # to store.  None: store this oracle's own rounding.
        self.store_hook = None
        self.enc_store_hook = None  # the same for the encoder's transformer
        # Test hook for the quantiser's argmin, an integer decision that a
        # near tie can send either way: code_hook(slot, q, residual, dist, code)
        # -> the code to take.  None: this oracle's own argmin.
        self.code_hook = None
        self._slot = 0

    def reset(self, s):
        self.slots[s].reset(self.cd, self.dt)
        self.enc_slots[s].reset(self.cd, self.dt)

    def _store(self, v):
        return round_bf16(v).astype(self.dt) if self.kv_store == "bf16" else v

    def decode(self, codes) -> np.ndarray:
        """codes int [B][8] -> pcm [B][samples]."""
        codes = np.asarray(codes).reshape(self.B, self.cd.n_q)
        out = []
        for b in range(self.B):
            self._slot = b
            out.append(self._frame(self.slots[b], codes[b]))
        return np.stack(out)

    # -- the pieces, in order

    def latent(self, codes) -> np.ndarray:
        """Residual-quantiser decoding: sum of the codebooks' rows in codebook order."""
        x = np.zeros(self.cd.d, self.dt)
        for q in range(self.cd.n_q):
            x = x + self.wts[f"codebook.{q}"][int(codes[q])]
        return x

    def transformer(self, st, x, prefix="") -> np.ndarray:
        """One frame through the causal transformer at position st.pos, then
        the output norm; stores this frame's keys and values.  prefix "enc."
        selects the encoder's weights."""
        return rmsnorm(self.blocks(st, x, prefix), self.wts[prefix + "out_norm"], self.cd.norm_eps)

    def blocks(self, st, x, prefix="") -> np.ndarray:
        """The transformer's layers for one frame at position st.pos."""
        cd, W = self.cd, self.W
        w = {k[len(prefix):]: v for k, v in self.wts.items() if k.startswith(prefix + "layers.")} if prefix else self.wts
        hook = self.enc_store_hook if prefix else self.store_hook
        d, H, Dh, F = cd.d, cd.n_heads, cd.head_dim, cd.ffn
        pos = st.pos
        ring_idx = [p % W for p in range(max(0, pos - W + 1), pos + 1)]
        for l in range(cd.n_layers):
            h = rmsnorm(x, w[f"layers.{l}.attn_norm"], cd.norm_eps)
            qkv = w[f"layers.{l}.wqkv"] @ h
            q = rope_interleaved(qkv[0:d].reshape(H, Dh), pos, cd.rope_base)
            k = rope_interleaved(qkv[d:2 * d].reshape(H, Dh), pos, cd.rope_base)
            v = qkv[2 * d:3 * d].reshape(H, Dh)
            ks, vs = self._store(k), self._store(v)
            if hook is not None:
                ks, vs = hook(self._slot, l, pos, k, v, ks, vs)
            st.K[l, pos % W] = ks
            st.V[l, pos % W] = vs
            o = softmax_attend(q, st.K[l, ring_idx], st.V[l, ring_idx])
            x = x + w[f"layers.{l}.wo"] @ o.reshape(d)
            h = rmsnorm(x, w[f"layers.{l}.mlp_norm"], cd.norm_eps)
            gu = w[f"layers.{l}.w_in"] @ h
            x = x + w[f"layers.{l}.w_out"] @ (silu(gu[:F]) * gu[F:])
        return x

    def _conv(self, st, name, x, key=None):
        """Causal convolution `name` of input x [C][T] with the stream's
        history under `key` (none for K = 1); the history is advanced."""
        w, b = self.wts[f"{name}.w"], self.wts[f"{name}.b"]
        K = w.shape[2]
        if K == 1:
            return causal_conv(x, w, b, np.zeros((x.shape[0], 0), self.dt))
        hist = st.hist[key]
        y = causal_conv(x, w, b, hist)
        st.hist[key] = np.concatenate([hist, x], axis=1)[:, -(K - 1):]
        return y

    def convs(self, st, z) -> np.ndarray:
        """The convolutional decoder for one frame: z [d] -> pcm [samples]."""
        cd, w = self.cd, self.wts
        h = self._conv(st, "conv_in", z[:, None], "conv_in")
        for i, s in enumerate(cd.strides):
            a = elu(h)
            u = conv_transpose_causal(a, w[f"up.{i}.w"], w[f"up.{i}.b"], st.hist[f"up.{i}"], s)
            st.hist[f"up.{i}"] = a[:, -1:]
            r = self._conv(st, f"res.{i}.a", elu(u), f"res.{i}.a")
            h = u + self._conv(st, f"res.{i}.b", elu(r))
        return self._conv(st, "conv_out", elu(h), "conv_out")[0]

    def _frame(self, st, codes) -> np.ndarray:
        z = self.transformer(st, self.latent(codes))
        st.last_z = z
        pcm = self.convs(st, z)
        st.pos += 1
        return pcm


    # -- the encoder

    def encode(self, pcm) -> np.ndarray:
        """pcm float [B][samples] -> codes int64 [B][n_q]."""
        pcm = np.asarray(pcm, self.dt).reshape(self.B, self.cd.samples)
        out = []
        for b in range(self.B):
            self._slot = b
            out.append(self._enc_frame(self.enc_slots[b], pcm[b]))
        return np.stack(out)

    def enc_convs(self, st, pcm) -> np.ndarray:
        """The encoder's convolutions for one frame: pcm [samples] -> y [d]."""
        cd, w = self.cd, self.wts
        n = len(cd.strides)
        h = self._conv(st, "enc.conv_in", pcm[None, :].astype(self.dt), "enc.conv_in")
        for j in range(n):
            s = cd.strides[n - 1 - j]
            r = self._conv(st, f"enc.res.{j}.a", elu(h), f"enc.res.{j}.a")
            h = h + self._conv(st, f"enc.res.{j}.b", elu(r))
            a = elu(h)
            key = f"enc.down.{j}"
            y = strided_conv_causal(a, w[f"{key}.w"], w[f"{key}.b"], st.hist[key], s)
            st.hist[key] = np.concatenate([st.hist[key], a], axis=1)[:, -s:]
            h = y
        return self._conv(st, "enc.conv_out", elu(h), "enc.conv_out")[:, 0]

    def quantise(self, z) -> np.ndarray:
        """Residual vector quantisation of z against the codebooks."""
        r = np.array(z, self.dt)
        codes = []
        for q in range(self.cd.n_q):
            table = self.wts[f"codebook.{q}"]
            c, dist = nearest(r, table)
            if self.code_hook is not None:
                c = self.code_hook(self._slot, q, r, dist, c)
            codes.append(c)
            r = r - table[c]
        return np.array(codes, np.int64)

    def _enc_frame(self, st, pcm) -> np.ndarray:
        st.last_y = self.enc_convs(st, pcm)
        z = self.transformer(st, st.last_y, "enc.")
        st.last_z = z
        st.pos += 1
        return self.quantise(z)


def encode_sequence(cd, weights, pcm, dtype=np.float64, kv_store="bf16") -> np.ndarray:
    """The whole-sequence definition of the encoder for one stream: pcm
    [T * samples] -> codes [T][n_q].  Every convolution runs once over the
    whole sequence with zeros before its start; the transformer and the
    quantiser then run frame by frame."""
    o = CodecOracle(cd, weights, 1, dtype, kv_store)
    st, w = o.enc_slots[0], o.wts
    n = len(cd.strides)

    def conv(name, x):
        K = w[f"{name}.w"].shape[2]
        return causal_conv(x, w[f"{name}.w"], w[f"{name}.b"], np.zeros((x.shape[0], K - 1), o.dt))

    h = conv("enc.conv_in", np.asarray(pcm, o.dt)[None, :])
    for j in range(n):
        s = cd.strides[n - 1 - j]
        r = conv(f"enc.res.{j}.a", elu(h))
        h = h + conv(f"enc.res.{j}.b", elu(r))
        h = strided_conv_causal(elu(h), w[f"enc.down.{j}.w"], w[f"enc.down.{j}.b"], np.zeros((h.shape[0], s), o.dt), s)
    y = conv("enc.conv_out", elu(h))  # [d][T]
    codes = []
    for t in range(y.shape[1]):
        z = o.transformer(st, y[:, t], "enc.")
        st.pos += 1
        codes.append(o.quantise(z))
    return np.stack(codes)


def decode_sequence(cd, weights, codes, dtype=np.float64, kv_store="bf16") -> np.ndarray:
    """The whole-sequence definition for one stream: codes int [T][8] ->
    pcm [T * samples].  The transformer runs frame by frame (it is causal by
    construction); every convolution runs once over the whole sequence with
    zeros before its start, so no state is carried between frames."""
    o = CodecOracle(cd, weights, 1, dtype, kv_store)
    st = o.slots[0]
    zs = []
    for t in range(len(codes)):
        zs.append(o.transformer(st, o.latent(codes[t])))
        st.pos += 1
    z = np.stack(zs, axis=1)  # [d][T]
    w = o.wts

    def conv(name, x):
        K = w[f"{name}.w"].shape[2]
        return causal_conv(x, w[f"{name}.w"], w[f"{name}.b"], np.zeros((x.shape[0], K - 1), o.dt))

    h = conv("conv_in", z)
    for i, s in enumerate(cd.strides):
        a = elu(h)
        u = conv_transpose_causal(a, w[f"up.{i}.w"], w[f"up.{i}.b"], np.zeros((a.shape[0], 1), o.dt), s)
        r = conv(f"res.{i}.a", elu(u))
        h = u + conv(f"res.{i}.b", elu(r))
    return conv("conv_out", elu(h))[0]
