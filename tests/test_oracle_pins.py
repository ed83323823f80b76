"""Pins of the CPU oracle against facts fixed by the pages and by mathematics:
closed forms, library routines, brute force over an unbounded history,
structural invariants and an fp64 shadow run.  Each test is built so that a
plausible slip in the oracle (a dropped term, a wrong sign, index or window
bound, a swapped operand) makes it fail."""
import numpy as np
import pytest
import scipy.special

from full_duplex_speech_moshi_amd import synth
from oracle import tick as ot
from oracle.tick import Oracle

DM = synth.TINY
W = synth.TINY_WINDOW


def bf(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


def zeros_bf(shape):
    return np.zeros(shape, np.uint16)


def teacher_frames(n, seed=11, dm=DM):
    """Fully forced frames: every text/agent row and the user rows given."""
    rng = np.random.default_rng(seed)
    f = np.empty((n, 17), np.int32)
    f[:, 0] = rng.integers(0, dm.text_card, n)
    f[:, 1:17] = rng.integers(0, dm.audio_card, (n, 16))
    return f


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


# ------------------------------------------------------------------ primitives

def test_rmsnorm_constant_input_closed_form():
    eps = 1e-5
    for c in (0.003, 0.5, 7.0):
        x = np.full(64, c, np.float64)
        y = ot.rmsnorm(x, np.ones(64), eps)
        np.testing.assert_allclose(y, 1.0 / np.sqrt(1.0 + eps / c ** 2), rtol=1e-14)


def test_rmsnorm_unit_rms_and_alpha_scaling():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(256) * 3.0
    a = 1.0 + 0.01 * rng.standard_normal(256)
    y = ot.rmsnorm(x, np.ones(256), 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-12
    # the scale multiplies elementwise after normalisation
    np.testing.assert_allclose(ot.rmsnorm(x, a, 0.0), y * a, rtol=1e-13)
    # scale invariance of the normalisation (eps negligible)
    np.testing.assert_allclose(ot.rmsnorm(1000.0 * x, a, 1e-5), ot.rmsnorm(x, a, 1e-5), rtol=1e-6)


def test_silu_identities():
    g = np.linspace(-20, 20, 401)
    s = ot.silu(g)
    # silu(x) - silu(-x) = x, silu = x * logistic(x) (scipy's expit)
    np.testing.assert_allclose(s - ot.silu(-g), g, atol=1e-12)
    np.testing.assert_allclose(s, g * scipy.special.expit(g), rtol=1e-12, atol=1e-300)
    assert ot.silu(np.array([0.0]))[0] == 0.0


def test_attention_matches_scipy_softmax_and_special_cases():
    rng = np.random.default_rng(1)
    H, Dh, n = 3, 16, 9
    q = rng.standard_normal((H, Dh))
    K = rng.standard_normal((n, H, Dh))
    V = rng.standard_normal((n, H, Dh))
    out = ot.softmax_attend(q, K, V)
    for h in range(H):
        p = scipy.special.softmax(K[:, h] @ q[h] / np.sqrt(Dh))
        np.testing.assert_allclose(out[h], p @ V[:, h], rtol=1e-12)
    # one key: the output is that key's value (softmax of one score is 1)
    np.testing.assert_allclose(ot.softmax_attend(q, K[:1], V[:1]), V[0], rtol=1e-15)
    # a zero query weights all keys equally
    np.testing.assert_allclose(ot.softmax_attend(np.zeros((H, Dh)), K, V), V.mean(axis=0), rtol=1e-12)


def test_rope_is_complex_rotation_of_adjacent_pairs():
    """Interleaved RoPE = multiply each (v[2i] + j v[2i+1]) by exp(j pos theta_i),
    theta_i = base^(-2i/Dh): an independent complex-number formulation."""
    rng = np.random.default_rng(2)
    H, Dh, base = 2, 16, 10000.0
    v = rng.standard_normal((H, Dh))
    for pos in (0, 1, 7, 2999, 123456):
        got = ot.rope_interleaved(v, pos, base)
        z = (v[:, 0::2] + 1j * v[:, 1::2]) * np.exp(1j * pos * base ** (-np.arange(0, Dh, 2) / Dh))
        np.testing.assert_allclose(got[:, 0::2], z.real, atol=1e-10)
        np.testing.assert_allclose(got[:, 1::2], z.imag, atol=1e-10)
    np.testing.assert_array_equal(ot.rope_interleaved(v, 0, base), v)


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    s = [np.dot(ot.rope_interleaved(q, p + 5, 1e4)[0], ot.rope_interleaved(k, p, 1e4)[0])
         for p in (0, 10, 1000)]
    np.testing.assert_allclose(s, s[0], rtol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(ot.rope_interleaved(q, 77, 1e4)), np.linalg.norm(q), rtol=1e-13)


def test_greedy_ties_to_lowest_index():
    assert ot.greedy(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    with pytest.raises(FloatingPointError):
        ot.greedy(np.array([0.0, np.nan]))


def test_upcast_bf16_exact():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.140625, 1e-3, 65280.0], np.float32)
    np.testing.assert_array_equal(ot.upcast_bf16(bf(vals)), synth.bf16_bits_to_f32(bf(vals)))
    np.testing.assert_array_equal(ot.upcast_bf16(bf([1.0, -2.5, 3.140625])), [1.0, -2.5, 3.140625])


# ------------------------------------------------------------------ column layout

def _digit_tables(w, dm):
    """Tables whose row t carries the 4 hex digits of t in dims 4r..4r+3 of
    column row r, zero elsewhere: the embedding sum then spells the column."""
    w = dict(w)

    def table(r, n):
        t = np.zeros((n, dm.d), np.float32)
        ids = np.arange(n)
        for j in range(4):
            t[:, 4 * r + j] = (ids >> (4 * j)) & 15
        return bf(t)

    w["emb.text"] = table(0, dm.text_card + 1)
    for r in range(1, 17):
        w[f"emb.audio.{r - 1}"] = table(r, dm.audio_card + 1)
    return w


def _read_column(x):
    digits = np.rint(x[:68]).astype(np.int64).reshape(17, 4)
    return digits @ np.array([1, 16, 256, 4096])


def test_column_layout_initial_tokens(tiny_weights):
    """17-row column: row 0 text, rows 1-8 agent, rows 9-16 user (recipe,
    Architecture); a fresh slot starts from TEXT_INITIAL_TOKEN = text vocab
    size and AUDIO_INITIAL_TOKEN = 2048 (guide, 帧 token 布局)."""
    w = _digit_tables(tiny_weights, DM)
    o = Oracle(DM, w, 1, W)
    codes = synth.user_codes(1, 3)
    o.step(codes[0:1])
    col0 = _read_column(o.taps["hidden"][0, 0])
    np.testing.assert_array_equal(col0, [DM.text_card] + [DM.audio_card] * 8 + list(codes[0]))
    chosen0 = o.taps["chosen"][0].copy()
    o.step(codes[1:2])
    np.testing.assert_array_equal(_read_column(o.taps["hidden"][0, 0]), list(chosen0) + list(codes[1]))


def test_column_layout_with_forced_frames(tiny_weights):
    w = _digit_tables(tiny_weights, DM)
    o = Oracle(DM, w, 1, W)
    f = teacher_frames(3, seed=5)
    o.prefill_forced(0, f)
    cols = []
    for t in range(3):
        o.step(np.zeros((1, 8), np.int64))  # ignored: forced frames carry the user rows
        cols.append(_read_column(o.taps["hidden"][0, 0]))
        np.testing.assert_array_equal(o.taps["chosen"][0], f[t, 0:9])
    np.testing.assert_array_equal(cols[0], [DM.text_card] + [DM.audio_card] * 8 + list(f[0, 9:]))
    np.testing.assert_array_equal(cols[1], list(f[0, 0:9]) + list(f[1, 9:]))
    np.testing.assert_array_equal(cols[2], list(f[1, 0:9]) + list(f[2, 9:]))
    # free tick: the model's own choices feed the next column
    o.step(np.full((1, 8), 3))
    chosen = o.taps["chosen"][0].copy()
    o.step(np.full((1, 8), 4))
    np.testing.assert_array_equal(_read_column(o.taps["hidden"][0, 0]), list(chosen) + [4] * 8)


# ------------------------------------------------------------------ closed-form layers

def _one_layer_dims():
    import dataclasses
    return dataclasses.replace(DM, n_layers=1)


def test_attention_block_closed_form(tiny_weights):
    """Layer with W_q = 0 (all scores equal), W_v = I, W_o = I and a zero MLP:
    x1 = x0 + mean over the window of rmsnorm(x0_p).  Pins the [q;k;v] row
    order, no rotation of values, the residual and the W-frame window that
    includes the current frame."""
    dm = _one_layer_dims()
    d = dm.d
    w = dict(tiny_weights)
    qkv = np.zeros((3 * d, d), np.float32)
    qkv[d:2 * d] = np.random.default_rng(4).standard_normal((d, d)) * 0.05   # keys: arbitrary
    qkv[2 * d:] = np.eye(d)
    w["layers.0.wqkv"] = bf(qkv)
    w["layers.0.wo"] = bf(np.eye(d))
    w["layers.0.w_in"] = zeros_bf((2 * dm.ffn, d))
    w["layers.0.w_out"] = zeros_bf((d, dm.ffn))
    Wn = 8
    o = Oracle(dm, w, 1, Wn, dtype=np.float64, kv_store="exact")
    f = teacher_frames(20, seed=6)
    o.prefill_forced(0, f)
    alpha = w["layers.0.attn_norm"].astype(np.float64)
    hist = []
    for t in range(20):
        o.step(np.zeros((1, 8)))
        x0 = o.taps["hidden"][0, 0]
        hist.append(x0 * alpha / np.sqrt(np.mean(x0 ** 2) + dm.norm_eps))
        expect = x0 + np.mean(hist[-Wn:], axis=0)
        np.testing.assert_allclose(o.taps["hidden"][1, 0], expect, rtol=1e-12, atol=1e-12)


def test_mlp_block_closed_form(tiny_weights):
    """Zero attention output (W_o = 0); gate rows = I, up rows = 2 I,
    W_out = I: x1 = x0 + silu(h) * 2h with h = rmsnorm(x0, mlp alpha).
    A swapped [gate; up] order would give silu(2h) * h."""
    dm = _one_layer_dims()
    d, F = dm.d, dm.ffn
    w = dict(tiny_weights)
    w["layers.0.wo"] = zeros_bf((d, d))
    win = np.zeros((2 * F, d), np.float32)
    win[:d] = np.eye(d)
    win[F:F + d] = 2 * np.eye(d)
    w["layers.0.w_in"] = bf(win)
    wout = np.zeros((d, F), np.float32)
    wout[:, :d] = np.eye(d)
    w["layers.0.w_out"] = bf(wout)
    o = Oracle(dm, w, 1, W, dtype=np.float64)
    o.step(synth.user_codes(1, 1))
    x0 = o.taps["hidden"][0, 0]
    a = w["layers.0.mlp_norm"].astype(np.float64)
    h = x0 * a / np.sqrt(np.mean(x0 ** 2) + dm.norm_eps)
    np.testing.assert_allclose(o.taps["hidden"][1, 0], x0 + h * scipy.special.expit(h) * 2 * h, rtol=1e-12)


def base_pows(Dh, base):
    return base ** (-np.arange(0, Dh, 2) / Dh)


# ------------------------------------------------------------------ ring = brute force

def _brute_force_hidden(dm, w, frames, window, dtype, kv_bf16=False):
    """Temporal stack over an unbounded history list, attending to the last
    `window` frames by slicing (no ring, no modulo).  kv_bf16: keep the stored
    keys/values as bf16 values (the input generator's RNE rounding)."""
    keep = (lambda a: synth.bf16_bits_to_f32(synth.to_bf16_bits(a)).astype(dtype)) if kv_bf16 else (lambda a: a)
    up = lambda n: ot.upcast_bf16(w[n], dtype) if w[n].dtype == np.uint16 else w[n].astype(dtype)
    d, H, Dh, F = dm.d, dm.n_heads, dm.head_dim, dm.ffn
    Ks = [[] for _ in range(dm.n_layers)]
    Vs = [[] for _ in range(dm.n_layers)]
    prev = [dm.text_card] + [dm.audio_card] * 8
    out = []
    for t, f in enumerate(frames):
        col = list(prev) + list(f[9:17])
        x = np.zeros(d, dtype)
        x += up("emb.text")[col[0]]
        for r in range(1, 17):
            x += up(f"emb.audio.{r - 1}")[col[r]]
        hs = [x.copy()]
        for l in range(dm.n_layers):
            h = ot.rmsnorm(x, up(f"layers.{l}.attn_norm"), dm.norm_eps)
            qkv = up(f"layers.{l}.wqkv") @ h
            q = ot.rope_interleaved(qkv[:d].reshape(H, Dh), t, dm.rope_base)
            Ks[l].append(keep(ot.rope_interleaved(qkv[d:2 * d].reshape(H, Dh), t, dm.rope_base)))
            Vs[l].append(keep(qkv[2 * d:].reshape(H, Dh)))
            o = ot.softmax_attend(q, np.stack(Ks[l][-window:]), np.stack(Vs[l][-window:]))
            x = x + up(f"layers.{l}.wo") @ o.reshape(d)
            h = ot.rmsnorm(x, up(f"layers.{l}.mlp_norm"), dm.norm_eps)
            gu = up(f"layers.{l}.w_in") @ h
            x = x + up(f"layers.{l}.w_out") @ (ot.silu(gu[:F]) * gu[F:])
            hs.append(x.copy())
        out.append(np.stack(hs))
        prev = list(f[0:9])
    return np.stack(out)


def test_ring_equals_brute_force_over_last_W_positions(tiny_weights):
    """100 ticks with W = 32 (the ring wraps three times): the ring-KV oracle
    equals full attention over the last W positions of an unbounded history,
    bit for bit in fp32 (same values, same order) and within fp64 rounding of
    an fp64 brute force."""
    n = 100
    f = teacher_frames(n, seed=8)

    def run(kv_store):
        o = Oracle(DM, tiny_weights, 1, W, kv_store=kv_store)
        o.prefill_forced(0, f)
        out = []
        for t in range(n):
            o.step(np.zeros((1, 8)))
            out.append(o.taps["hidden"][:, 0].copy())
        return np.stack(out)

    got = run("bf16")
    ref32 = _brute_force_hidden(DM, tiny_weights, f, W, np.float32, kv_bf16=True)
    np.testing.assert_array_equal(got, ref32)
    exact = run("exact")
    np.testing.assert_array_equal(exact, _brute_force_hidden(DM, tiny_weights, f, W, np.float32))
    ref64 = _brute_force_hidden(DM, tiny_weights, f, W, np.float64)
    assert rel_l2(exact, ref64) < 1e-5
    # and the window matters: an unbounded window gives different states once it wraps
    ref_inf = _brute_force_hidden(DM, tiny_weights, f[:40], 10 ** 9, np.float32, kv_bf16=True)
    assert rel_l2(got[W:40], ref_inf[W:40]) > 1e-4
    np.testing.assert_array_equal(got[:W], ref_inf[:W])


# ------------------------------------------------------------------ isolation, recycle, depformer

def test_slot_isolation_batch_equals_separate_runs(tiny_weights):
    B, n = 3, 12
    codes = [synth.user_codes(100 + b, n) for b in range(B)]
    ob = Oracle(DM, tiny_weights, B, W)
    ob.prefill_forced(1, teacher_frames(4, seed=9))
    toks_b = [ob.step(np.stack([codes[b][t] for b in range(B)])) for t in range(n)]
    for b in range(B):
        o1 = Oracle(DM, tiny_weights, 1, W)
        if b == 1:
            o1.prefill_forced(0, teacher_frames(4, seed=9))
        for t in range(n):
            tk = o1.step(codes[b][t:t + 1])
            np.testing.assert_array_equal(tk[0], toks_b[t][b])
        np.testing.assert_array_equal(o1.taps["hidden"][:, 0], ob.taps["hidden"][:, b])


def test_recycled_slot_equals_fresh_engine(tiny_weights):
    codes = synth.user_codes(1, 40)
    o = Oracle(DM, tiny_weights, 1, W)
    for t in range(37):           # wraps the ring
        o.step(codes[t:t + 1])
    o.slot_reset(0)
    fresh = Oracle(DM, tiny_weights, 1, W)
    for t in range(5):
        a = o.step(codes[t:t + 1])
        b = fresh.step(codes[t:t + 1])
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(o.taps["dep_logits"], fresh.taps["dep_logits"])


def test_depformer_reset_each_frame(tiny_weights):
    """Temporal layers zeroed, so z depends only on the column.  The same
    forced column at tick 3 and tick 9 (different positions and histories)
    must give identical depformer outputs: nothing carries across frames."""
    w = dict(tiny_weights)
    for l in range(DM.n_layers):
        w[f"layers.{l}.wo"] = zeros_bf((DM.d, DM.d))
        w[f"layers.{l}.w_out"] = zeros_bf((DM.d, DM.ffn))
    f = teacher_frames(10, seed=10)
    f[9] = f[3]
    f[8, 0:9] = f[2, 0:9]
    o = Oracle(DM, w, 1, W)
    o.prefill_forced(0, f)
    outs = []
    for t in range(10):
        o.step(np.zeros((1, 8)))
        outs.append(o.taps["dep_logits"].copy())
    np.testing.assert_array_equal(outs[3], outs[9])
    assert not np.array_equal(outs[3], outs[4])


def test_depformer_chain_closed_form(tiny_weights):
    """Depformer with zero input projections and zero layers reduces to
    y_k = table_k[tok_{k-1}], logits_k = head_k . rmsnorm(y_k): the greedy chain
    computed here by hand pins which table and head each step uses, that step 0
    is fed the chosen text token and that forced agent tokens are fed on."""
    dm = DM
    w = dict(tiny_weights)
    dd, dF = dm.dep_d, dm.dep_ffn
    for k in range(dm.dep_q):
        w[f"dep.in_proj.{k}"] = zeros_bf((dd, dm.d))
    for l in range(dm.dep_layers):
        w[f"dep.layers.{l}.wo"] = zeros_bf((dd, dd))
        w[f"dep.layers.{l}.w_out"] = zeros_bf((dd, dF))
    f = teacher_frames(1, seed=12)
    f[0, 1:9] = -1
    f[0, 3] = 1234      # agent codebook 2 forced
    o = Oracle(dm, w, 1, W, dtype=np.float64)
    o.prefill_forced(0, f)
    toks = o.step(np.zeros((1, 8)))
    up = lambda n: ot.upcast_bf16(w[n], np.float64)
    a = w["dep.out_norm"].astype(np.float64)
    tok = int(f[0, 0])
    preds = []
    for k in range(dm.dep_q):
        y = up("dep.emb.text" if k == 0 else f"dep.emb.audio.{k}")[tok]
        yn = y * a / np.sqrt(np.mean(y * y) + dm.norm_eps)
        lg = up(f"dep.head.{k}") @ yn
        np.testing.assert_allclose(o.taps["dep_logits"][0, k], lg, rtol=1e-12, atol=1e-14)
        p = int(np.argmax(lg))
        preds.append(p)
        tok = 1234 if k == 2 else p
    np.testing.assert_array_equal(toks[0, 1:], preds[:8])
    np.testing.assert_array_equal(o.taps["user_pred"][0], preds[8:])
    assert o.taps["chosen"][0, 3] == 1234 and toks[0, 3] == preds[2]


def test_depformer_attention_closed_form(tiny_weights):
    """Depformer with zero input projections, W_q = W_k = W_v = W_o = I and a
    zero MLP: step k's state is e_k + attention of h_k over h_0..h_k of this
    frame (h_j = rmsnorm(e_j), plain dot-product scores, no rotation), with
    e_k = table_k[tok_{k-1}].  Pins the per-frame causal window over steps and
    the absence of positional encoding in the depformer."""
    dm = DM
    w = dict(tiny_weights)
    dd, dF, dH, dDh = dm.dep_d, dm.dep_ffn, dm.dep_heads, dm.dep_head_dim
    for k in range(dm.dep_q):
        w[f"dep.in_proj.{k}"] = zeros_bf((dd, dm.d))
    eye3 = np.concatenate([np.eye(dd)] * 3).astype(np.float32)
    w["dep.layers.0.wqkv"] = bf(eye3)
    w["dep.layers.0.wo"] = bf(np.eye(dd))
    w["dep.layers.0.w_out"] = zeros_bf((dd, dF))
    f = teacher_frames(1, seed=17)
    o = Oracle(dm, w, 1, W, dtype=np.float64, kv_store="exact")
    o.prefill_forced(0, f)
    o.step(np.zeros((1, 8)))
    up = lambda n: ot.upcast_bf16(w[n], np.float64)
    a1 = w["dep.layers.0.attn_norm"].astype(np.float64)
    ao = w["dep.out_norm"].astype(np.float64)
    tok = int(f[0, 0])
    hs = []
    for k in range(dm.dep_q):
        e = up("dep.emb.text" if k == 0 else f"dep.emb.audio.{k}")[tok]
        hs.append((e * a1 / np.sqrt(np.mean(e * e) + dm.norm_eps)).reshape(dH, dDh))
        hk = np.stack(hs)                       # [k+1, H, Dh]
        att = np.stack([scipy.special.softmax(hk[:, h] @ hk[-1, h] / np.sqrt(dDh)) @ hk[:, h]
                        for h in range(dH)]).reshape(dd)
        y = e + att
        lg = up(f"dep.head.{k}") @ (y * ao / np.sqrt(np.mean(y * y) + dm.norm_eps))
        np.testing.assert_allclose(o.taps["dep_logits"][0, k], lg, rtol=1e-10, atol=1e-13)
        tok = int(f[0, 1 + k]) if k < 8 else int(np.argmax(lg))


def test_depformer_mlp_sublayers_closed_form():
    """Two-layer depformer with zero input projections and zero attention
    output (W_o = 0).  Layer l's MLP has gate rows = g_l I, up rows = c_l I
    and W_out = I (g = 1, 0.5; c = 2, 3; all exact in bf16), so step k is
    y = e_k; y += silu(g_l h) * c_l h with h = rmsnorm(y, mlp alpha of layer
    l), for l = 0, 1; logits = head_k . rmsnorm(y, out alpha).  A swapped
    [gate; up] order, the attention alpha in place of the MLP alpha, or layer
    0's weights reused at layer 1 each move the logits."""
    import dataclasses
    dm = dataclasses.replace(DM, dep_layers=2)
    w = synth.make_weights(dm, seed=0)
    dd, dF = dm.dep_d, dm.dep_ffn
    gains, ups = (1.0, 0.5), (2.0, 3.0)
    for k in range(dm.dep_q):
        w[f"dep.in_proj.{k}"] = zeros_bf((dd, dm.d))
    for l in range(dm.dep_layers):
        w[f"dep.layers.{l}.wo"] = zeros_bf((dd, dd))
        win = np.zeros((2 * dF, dd), np.float32)
        win[:dd] = gains[l] * np.eye(dd)
        win[dF:dF + dd] = ups[l] * np.eye(dd)
        w[f"dep.layers.{l}.w_in"] = bf(win)
        wout = np.zeros((dd, dF), np.float32)
        wout[:, :dd] = np.eye(dd)
        w[f"dep.layers.{l}.w_out"] = bf(wout)
    assert not np.array_equal(w["dep.layers.0.mlp_norm"], w["dep.layers.1.mlp_norm"])
    assert not np.array_equal(w["dep.layers.0.mlp_norm"], w["dep.layers.0.attn_norm"])
    f = teacher_frames(1, seed=19, dm=dm)
    o = Oracle(dm, w, 1, W, dtype=np.float64)
    o.prefill_forced(0, f)
    o.step(np.zeros((1, 8)))
    up = lambda n: ot.upcast_bf16(w[n], np.float64)
    ao = w["dep.out_norm"].astype(np.float64)
    tok = int(f[0, 0])
    for k in range(dm.dep_q):
        y = up("dep.emb.text" if k == 0 else f"dep.emb.audio.{k}")[tok].copy()
        for l in range(dm.dep_layers):
            a = w[f"dep.layers.{l}.mlp_norm"].astype(np.float64)
            h = y * a / np.sqrt(np.mean(y * y) + dm.norm_eps)
            g = gains[l] * h
            y = y + g * scipy.special.expit(g) * ups[l] * h
        lg = up(f"dep.head.{k}") @ (y * ao / np.sqrt(np.mean(y * y) + dm.norm_eps))
        np.testing.assert_allclose(o.taps["dep_logits"][0, k], lg, rtol=1e-10, atol=1e-13)
        tok = int(f[0, 1 + k]) if k < 8 else int(np.argmax(lg))


def test_depformer_is_causal_over_codebooks(tiny_weights):
    """Changing the table used at step 5 leaves logits of steps 0-4 unchanged."""
    o1 = Oracle(DM, tiny_weights, 1, W)
    w = dict(tiny_weights)
    w["dep.emb.audio.5"] = bf(np.random.default_rng(13).standard_normal((DM.audio_card + 1, DM.dep_d)) * 0.02)
    o2 = Oracle(DM, w, 1, W)
    c = synth.user_codes(1, 1)
    o1.step(c)
    o2.step(c)
    np.testing.assert_array_equal(o1.taps["dep_logits"][0, :5], o2.taps["dep_logits"][0, :5])
    assert not np.array_equal(o1.taps["dep_logits"][0, 5], o2.taps["dep_logits"][0, 5])


def test_heads_read_the_normalised_state(tiny_weights):
    """Temporal layers zeroed: x is the embedding sum.  Scaling every temporal
    table by 4 (exact in bf16) scales x by 4 and z = rmsnorm(x) by
    r = sqrt(ms + eps) / sqrt(ms + eps/16) only, so text logits scale by r; the
    depformer (fed z, not x) barely moves.  A head fed x would scale by 4."""
    w = dict(tiny_weights)
    for l in range(DM.n_layers):
        w[f"layers.{l}.wo"] = zeros_bf((DM.d, DM.d))
        w[f"layers.{l}.w_out"] = zeros_bf((DM.d, DM.ffn))
    w4 = dict(w)
    for n in ["emb.text"] + [f"emb.audio.{r}" for r in range(16)]:
        w4[n] = bf(synth.bf16_bits_to_f32(w[n]) * 4)
    f = teacher_frames(1, seed=16)
    a, b = Oracle(DM, w, 1, W, np.float64), Oracle(DM, w4, 1, W, np.float64)
    for o in (a, b):
        o.prefill_forced(0, f)
        o.step(np.zeros((1, 8)))
    x = a.taps["hidden"][-1, 0]
    np.testing.assert_array_equal(b.taps["hidden"][:, 0], 4 * a.taps["hidden"][:, 0])
    ms = np.mean(x * x)
    r = np.sqrt(ms + DM.norm_eps) / np.sqrt(ms + DM.norm_eps / 16)
    np.testing.assert_allclose(b.taps["text_logits"], r * a.taps["text_logits"], rtol=1e-10)
    # steps 0..8 are fed forced tokens, so their inputs match exactly
    np.testing.assert_allclose(b.taps["dep_logits"][0, :9], a.taps["dep_logits"][0, :9], rtol=5e-3, atol=1e-4)


# ------------------------------------------------------------------ ring fill, fp64 shadow, state rules

def _crot(v, pos, base):
    """Rotation of adjacent pairs as complex multiplication by exp(j pos theta_i)."""
    Dh = v.shape[1]
    z = (v[:, 0::2] + 1j * v[:, 1::2]) * np.exp(1j * pos * base_pows(Dh, base))
    out = np.empty_like(v)
    out[:, 0::2] = z.real
    out[:, 1::2] = z.imag
    return out


def test_ring_fill_then_ticks_equal_independent_brute_force(tiny_weights):
    """A fill of n = 20 frames places keys/values at positions 0..n-1 and the
    next tick runs at absolute position n; 15 teacher-forced ticks then slide
    the W = 32 window.  Checked against an independent fp64 brute force over an
    unbounded history (complex-number rotation of q and k at the absolute
    position, scipy softmax, logistic-form SiLU)."""
    k, v = synth.ring_fill(DM, 3, 20)
    o = Oracle(DM, tiny_weights, 1, W, dtype=np.float64, kv_store="exact")
    o.ring_fill(0, k, v)
    assert o.slots[0].pos == 20
    f = teacher_frames(15, seed=14)
    o.prefill_forced(0, f)
    hid = []
    for t in range(15):
        o.step(np.zeros((1, 8)))
        hid.append(o.taps["hidden"][:, 0].copy())
    # brute force: history lists start with the filled K/V
    dm, dt = DM, np.float64
    up = lambda n: ot.upcast_bf16(tiny_weights[n], dt) if tiny_weights[n].dtype == np.uint16 else tiny_weights[n].astype(dt)
    d, H, Dh, F = dm.d, dm.n_heads, dm.head_dim, dm.ffn
    Ks = [list(ot.upcast_bf16(k[l], dt)) for l in range(dm.n_layers)]
    Vs = [list(ot.upcast_bf16(v[l], dt)) for l in range(dm.n_layers)]
    prev = [dm.text_card] + [dm.audio_card] * 8
    for t in range(15):
        pos = 20 + t
        col = prev + list(f[t, 9:])
        x = up("emb.text")[col[0]].copy()
        for r in range(1, 17):
            x = x + up(f"emb.audio.{r - 1}")[col[r]]
        for l in range(dm.n_layers):
            h = x * up(f"layers.{l}.attn_norm") / np.sqrt(np.mean(x * x) + dm.norm_eps)
            qkv = up(f"layers.{l}.wqkv") @ h
            q = _crot(qkv[:d].reshape(H, Dh), pos, dm.rope_base)
            Ks[l].append(_crot(qkv[d:2 * d].reshape(H, Dh), pos, dm.rope_base))
            Vs[l].append(qkv[2 * d:].reshape(H, Dh))
            kk = np.stack(Ks[l][-W:])
            vv = np.stack(Vs[l][-W:])
            o_ = np.stack([scipy.special.softmax(kk[:, hh] @ q[hh] / np.sqrt(Dh)) @ vv[:, hh] for hh in range(H)])
            x = x + up(f"layers.{l}.wo") @ o_.reshape(d)
            h = x * up(f"layers.{l}.mlp_norm") / np.sqrt(np.mean(x * x) + dm.norm_eps)
            gu = up(f"layers.{l}.w_in") @ h
            x = x + up(f"layers.{l}.w_out") @ (gu[:F] * scipy.special.expit(gu[:F]) * gu[F:])
        np.testing.assert_allclose(hid[t][-1], x, rtol=1e-10, atol=1e-12)
        prev = list(f[t, :9])


def test_caches_hold_bf16_rounded_values(tiny_weights):
    """Default storage: each stored key/value is the nearest bf16 value (ties
    to even) of the exact one, in the ring and in the depformer's cache."""
    a = Oracle(DM, tiny_weights, 1, W)
    b = Oracle(DM, tiny_weights, 1, W, kv_store="exact")
    c = synth.user_codes(1, 1)
    a.step(c)
    b.step(c)
    # layer 0 sees identical inputs in both runs (deeper layers do not)
    for arr_a, arr_b in ((a.slots[0].K, b.slots[0].K), (a.slots[0].V, b.slots[0].V)):
        want = synth.bf16_bits_to_f32(synth.to_bf16_bits(arr_b[0, 0]))
        np.testing.assert_array_equal(arr_a[0, 0], want)
    assert not np.array_equal(a.slots[0].K[0, 0], b.slots[0].K[0, 0])
    # the first depformer step attends to its own (rounded) value only
    np.testing.assert_array_equal(ot.round_bf16(np.array([1.00390625, -1.01171875, 3.0e-3], np.float32)),
                                  synth.bf16_bits_to_f32(synth.to_bf16_bits(np.array([1.00390625, -1.01171875, 3.0e-3], np.float32))))


def test_fp64_shadow_bounds_fp32_oracle_error(tiny_weights):
    """fp32 oracle vs the same oracle in fp64, 100 teacher-forced C0 ticks:
    hidden states agree far below the 1e-2 rel-L2 GPU gate."""
    f = teacher_frames(100, seed=15)
    a = Oracle(DM, tiny_weights, 1, W, np.float32, kv_store="exact")
    b = Oracle(DM, tiny_weights, 1, W, np.float64, kv_store="exact")
    a.prefill_forced(0, f)
    b.prefill_forced(0, f)
    worst_h, worst_l = 0.0, 0.0
    for t in range(100):
        a.step(np.zeros((1, 8)))
        b.step(np.zeros((1, 8)))
        worst_h = max(worst_h, rel_l2(a.taps["hidden"], b.taps["hidden"]))
        worst_l = max(worst_l, np.abs(a.taps["text_logits"] - b.taps["text_logits"]).max(),
                      np.abs(a.taps["dep_logits"] - b.taps["dep_logits"]).max())
    assert worst_h < 1e-5
    assert worst_l < 1e-4


def test_state_rules(tiny_weights):
    o = Oracle(DM, tiny_weights, 2, W)
    k, v = synth.ring_fill(DM, 3, 5)
    o.prefill_forced(0, teacher_frames(1))
    with pytest.raises(RuntimeError):
        o.ring_fill(0, k, v)          # a fill must come before any prefill
    o.step(np.zeros((2, 8)))
    o.step(np.zeros((2, 8)))          # slot 0 now free-running: live
    with pytest.raises(RuntimeError):
        o.prefill_forced(0, teacher_frames(1))
    with pytest.raises(ValueError):
        o.slot_reset(1)
        o.ring_fill(1, *synth.ring_fill(DM, 3, W + 1))
    o.slot_reset(0)
    o.ring_fill(0, k, v)
    o.prefill_forced(0, teacher_frames(2))


# ------------------------------------------------------------------ acoustic delay, embedding-form prefill

def test_acoustic_delay_column_layout(tiny_weights):
    """Delay D: the column's user rows 10-16 (codebooks 1-7) carry the frame
    D ticks back, the initial audio token before the first; row 9 (codebook
    0) and the text row are not delayed (recipe: an 80 ms acoustic delay
    behind the 80 ms frame)."""
    w = _digit_tables(tiny_weights, DM)
    A = DM.audio_card
    codes = synth.user_codes(4, 4)
    for D in (1, 2):
        o = Oracle(DM, w, 1, W)
        o.set_acoustic_delay(D)
        for t in range(4):
            o.step(codes[t:t + 1])
            col = _read_column(o.taps["hidden"][0, 0])
            assert col[9] == codes[t, 0]
            want = list(codes[t - D, 1:]) if t >= D else [A] * 7
            np.testing.assert_array_equal(col[10:17], want)


def test_acoustic_delay_forced_agent_rows(tiny_weights):
    """With D = 1 a forced frame forces the text row and codebook 0 on its
    own tick and codebooks 1-7 one tick later; on tick 0 those are free."""
    o = Oracle(DM, tiny_weights, 1, W)
    o.set_acoustic_delay(1)
    f = teacher_frames(3, seed=9)
    o.prefill_forced(0, f)
    for t in range(3):
        tok = o.step(np.zeros((1, 8), np.int64))
        ch = o.taps["chosen"][0]
        assert ch[0] == f[t, 0] and ch[1] == f[t, 1]
        np.testing.assert_array_equal(ch[2:9], f[t - 1, 2:9] if t else tok[0, 2:9])
    # first free tick: the last forced frame's codebooks 1-7 still apply
    o.step(np.zeros((1, 8), np.int64))
    np.testing.assert_array_equal(o.taps["chosen"][0, 2:9], f[2, 2:9])


def test_acoustic_delay_equals_shifted_inputs(tiny_weights):
    """A delayed run is the undelayed model fed the shifted user frames:
    bit-identical hidden states, logits and tokens."""
    A = DM.audio_card
    codes = synth.user_codes(6, 5)
    o1 = Oracle(DM, tiny_weights, 1, W)
    o1.set_acoustic_delay(1)
    o0 = Oracle(DM, tiny_weights, 1, W)
    for t in range(5):
        shifted = np.concatenate([codes[t, :1], codes[t - 1, 1:] if t else np.full(7, A)])
        t1 = o1.step(codes[t:t + 1])
        t0 = o0.step(shifted[None])
        np.testing.assert_array_equal(t1, t0)
        for k in ("hidden", "text_logits", "dep_logits", "chosen"):
            np.testing.assert_array_equal(o1.taps[k], o0.taps[k])


def test_agent_frames_are_frame_aligned(tiny_weights):
    """Agent frame f = codebook 0 chosen at tick f, codebooks 1-7 chosen at
    tick f + D; none before tick D; with D = 0 the tick's own choice."""
    codes = synth.user_codes(8, 5)
    for D in (0, 1, 2):
        o = Oracle(DM, tiny_weights, 1, W)
        o.set_acoustic_delay(D)
        chosen = []
        for t in range(5):
            o.step(codes[t:t + 1])
            chosen.append(o.taps["chosen"][0, 1:].copy())
            assert bool(o.taps["agent_frame_valid"][0]) == (t >= D)
            if t >= D:
                np.testing.assert_array_equal(o.taps["agent_frame"][0, :1], chosen[t - D][:1])
                np.testing.assert_array_equal(o.taps["agent_frame"][0, 1:], chosen[t][1:])


def test_embedding_frame_replaces_the_gather_sum(tiny_weights):
    """An embedding-form prefill frame's x is the tick's input itself:
    with digit tables, x = the digits of a column reproduces the token frame
    bit for bit, and x = 0 leaves no trace of the column."""
    w = _digit_tables(tiny_weights, DM)
    f = teacher_frames(2, seed=13)
    ot_ = Oracle(DM, w, 1, W)
    ot_.prefill_forced(0, f)
    oe = Oracle(DM, w, 1, W)
    for t in range(2):
        ot_.step(np.zeros((1, 8), np.int64))
        x = ot_.taps["hidden"][0, 0].copy()     # integer digits: exact in fp32
        col = _read_column(x)
        np.testing.assert_array_equal(col[9:], f[t, 9:])
        oe.prefill_embed(0, x[None], f[t:t + 1, :9])
        tok = oe.step(np.zeros((1, 8), np.int64))
        for k in ("hidden", "text_logits", "dep_logits", "chosen"):
            np.testing.assert_array_equal(oe.taps[k], ot_.taps[k])
    oz = Oracle(DM, w, 1, W)
    oz.prefill_embed(0, np.zeros((1, DM.d), np.float32))
    oz.step(np.full((1, 8), 5))
    assert not oz.taps["hidden"][0, 0].any()
    # a zero input stays zero through every temporal layer (no biases)
    assert not oz.taps["hidden"].any()


def test_embedding_frame_forces_and_user_history(tiny_weights):
    """Forced choices of an embedding frame apply as for a token frame
    (-1 free); with D = 1 the frame gives no user codes, so the next
    column's delayed user rows hold the initial audio token."""
    w = _digit_tables(tiny_weights, DM)
    o = Oracle(DM, w, 1, W)
    o.set_acoustic_delay(1)
    force = np.array([[7, 1, 2, -1, -1, -1, -1, -1, -1]])
    o.prefill_embed(0, np.ones((1, DM.d), np.float32), force)
    tok = o.step(np.zeros((1, 8), np.int64))
    ch = o.taps["chosen"][0]
    assert ch[0] == 7 and ch[1] == 1
    np.testing.assert_array_equal(ch[2:], tok[0, 2:])   # codebooks 1-7: forced only a tick later
    codes = synth.user_codes(3, 1)
    o.step(codes)
    col = _read_column(o.taps["hidden"][0, 0])
    assert col[9] == codes[0, 0]
    np.testing.assert_array_equal(col[10:], [DM.audio_card] * 7)
    assert o.taps["chosen"][0, 2] == 2                  # the frame's codebook-1 force, one tick late


def test_delay_rules(tiny_weights):
    o = Oracle(DM, tiny_weights, 1, W)
    with pytest.raises(ValueError):
        o.set_acoustic_delay(5)
    o.set_acoustic_delay(2)
    o.step(np.zeros((1, 8)))
    with pytest.raises(RuntimeError):
        o.set_acoustic_delay(1)
