"""Pins of the codec oracle (oracle/codec.py, decoder and encoder) to things
outside it.

* Its causal and transposed convolutions against PyTorch's CPU routines
  (conv1d with left padding, conv_transpose1d), fp64.
* Its streaming state: frame-by-frame decoding equals the whole-sequence
  definition, which carries no state; a reset slot equals a fresh one.
* Its transformer against the tick oracle's temporal block (itself pinned in
  test_oracle_pins.py): the same weights, fed as embedding-form frames, give
  the same hidden state, over more frames than the window holds.
* The residual-quantiser sum against one-hot codebooks.
* The convolutional stack's wiring (ELU placement, upsampling, channel
  order, residual skip from the pre-activation signal, biases) against a
  closed form with pass-through weights.
* The encoder: its strided convolution against PyTorch's conv1d (stride s,
  left padding); the nearest-row search against brute force with the
  lowest index on ties; the residual quantiser against codebooks built so
  that only stage-by-stage quantisation of what is left gives the codes;
  its transformer against the tick oracle's temporal block and its own
  output norm; its streaming against the whole-sequence definition; its
  convolutional wiring against a closed form with pass-through weights.

The codec's layer structure is a reading of the pages (section
2.3 of the chenxutan.com article: a SoundStream/EnCodec-family codec with a
transformer, 12.5 Hz frames, 24 kHz audio); parity with the real Mimi codec
is unpinned: its weights and exact layers are not available."""
import dataclasses

import numpy as np
import pytest
import torch

from full_duplex_speech_moshi_amd import synth
from oracle import codec, tick

CD = synth.CODEC_TINY


def _bits(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


def test_frame_is_1920_samples_at_the_pages_rate():
    # 24 kHz / 12.5 Hz = 1920 samples per 80 ms frame
    assert synth.CODEC.samples == 24000 * 80 // 1000 == 1920
    assert synth.CODEC.n_q == 8 and synth.CODEC.card == 2048


@pytest.mark.parametrize("K", [1, 3, 7])
def test_causal_conv_matches_torch(K):
    rng = np.random.default_rng(K)
    ci, co, T = 5, 4, 9
    x, w, b = rng.normal(size=(ci, T)), rng.normal(size=(co, ci, K)), rng.normal(size=co)
    y = codec.causal_conv(x, w, b, np.zeros((ci, K - 1)))
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(torch.tensor(x)[None], (K - 1, 0)),
                                     torch.tensor(w), torch.tensor(b))[0].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a history is the inputs before x: the same as convolving the concatenation
    h = rng.normal(size=(ci, K - 1))
    y2 = codec.causal_conv(x, w, b, h)
    full = np.concatenate([h, x], axis=1)
    ref2 = torch.nn.functional.conv1d(torch.nn.functional.pad(torch.tensor(full)[None], (K - 1, 0)),
                                      torch.tensor(w), torch.tensor(b))[0].numpy()[:, K - 1:]
    np.testing.assert_allclose(y2, ref2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s", [2, 3, 5, 8])
def test_conv_transpose_matches_torch(s):
    rng = np.random.default_rng(s)
    ci, co, T = 4, 3, 6
    x, w, b = rng.normal(size=(ci, T)), rng.normal(size=(co, ci, 2 * s)), rng.normal(size=co)
    # torch's weight layout is [C_in][C_out][K]; its output has (T - 1) s + K
    # samples, of which the causal call keeps the first T s
    ref = torch.nn.functional.conv_transpose1d(torch.tensor(x)[None], torch.tensor(w.transpose(1, 0, 2)),
                                               torch.tensor(b), stride=s)[0].numpy()
    y = codec.conv_transpose_causal(x, w, b, np.zeros((ci, 1)), s)
    np.testing.assert_allclose(y, ref[:, :T * s], rtol=1e-12, atol=1e-12)
    # with the previous input given, the outputs are those of the longer
    # sequence, shifted by one input
    prev = rng.normal(size=(ci, 1))
    full = torch.nn.functional.conv_transpose1d(torch.tensor(np.concatenate([prev, x], 1))[None],
                                                torch.tensor(w.transpose(1, 0, 2)), torch.tensor(b),
                                                stride=s)[0].numpy()
    y2 = codec.conv_transpose_causal(x, w, b, prev, s)
    np.testing.assert_allclose(y2, full[:, s:s + T * s], rtol=1e-12, atol=1e-12)


def test_elu_values():
    x = np.array([-2.0, -1.0, -1e-8, 0.0, 1e-8, 0.5, 3.0])
    # e^-2 - 1, e^-1 - 1 and e^-1e-8 - 1 to 17 digits
    np.testing.assert_allclose(codec.elu(x), [-0.8646647167633873, -0.6321205588285577, -9.9999999500000002e-09,
                                              0.0, 1e-8, 0.5, 3.0], rtol=1e-15, atol=0)


def test_streaming_equals_whole_sequence_and_reset_equals_fresh():
    w = synth.make_codec_weights(CD, seed=3)
    n = 2 * CD.window + 3  # past the transformer's window
    codes = synth.agent_frames(11, n)
    o = codec.CodecOracle(CD, w, 2, np.float64)
    other = synth.agent_frames(12, 5)
    pcm = []
    for t in range(n):
        c = np.stack([codes[t], other[t % 5]])
        pcm.append(o.decode(c)[0])
    ref = codec.decode_sequence(CD, w, codes, np.float64)
    np.testing.assert_allclose(np.concatenate(pcm), ref, rtol=0, atol=1e-12)
    # slot 1 reset mid-stream, then fed the sequence: the same samples
    o.reset(1)
    got = [o.decode(np.stack([other[0], codes[t]]))[1] for t in range(6)]
    np.testing.assert_allclose(np.concatenate(got), ref[:6 * CD.samples], rtol=0, atol=1e-12)


def test_latent_is_the_codebook_sum_in_order():
    w = synth.make_codec_weights(CD, seed=0)
    for q in range(CD.n_q):
        t = np.zeros((CD.card, CD.d), np.float32)
        t[np.arange(CD.card), (np.arange(CD.card) + 3 * q) % CD.d] = 2.0 ** -q
        w[f"codebook.{q}"] = _bits(t)
    o = codec.CodecOracle(CD, w, 1, np.float64)
    codes = np.array([5, 900, 17, 17, 2047, 0, 64, 127])
    x = o.latent(codes)
    ref = np.zeros(CD.d)
    for q, c in enumerate(codes):
        ref[(c + 3 * q) % CD.d] += 2.0 ** -q
    np.testing.assert_array_equal(x, ref)


def test_transformer_is_the_temporal_block():
    """The codec's layers against the tick oracle's temporal layers with the
    same weights: embedding-form frames give the tick its input x, and the
    tick's hidden state after the last layer must equal the codec's, frame by
    frame, beyond the window (ring wrap)."""
    cw = synth.make_codec_weights(CD, seed=5)
    dm = synth.Dims(d=CD.d, n_layers=CD.n_layers, n_heads=CD.n_heads, ffn=CD.ffn, text_card=64,
                    audio_card=64, n_q=8, dep_d=32, dep_layers=1, dep_heads=1, dep_ffn=32, dep_q=16,
                    norm_eps=CD.norm_eps, rope_base=CD.rope_base)
    tw = synth.make_weights(dm, seed=1)
    for l in range(CD.n_layers):
        for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out"):
            tw[f"layers.{l}.{k}"] = cw[f"layers.{l}.{k}"]
    n = CD.window + 4
    rng = np.random.default_rng(9)
    xs = rng.normal(size=(n, CD.d))
    t = tick.Oracle(dm, tw, 1, CD.window, dtype=np.float64)
    t.prefill_embed(0, xs)
    o = codec.CodecOracle(CD, cw, 1, np.float64)
    st = o.slots[0]
    for i in range(n):
        t.step(np.zeros((1, 8), np.int64))
        got = o.blocks(st, xs[i].copy())
        st.pos += 1
        np.testing.assert_allclose(got, t.taps["hidden"][-1, 0], rtol=1e-12, atol=1e-12, err_msg=f"frame {i}")


def test_conv_stack_closed_form():
    """Pass-through weights: the first convolution picks z's channel 0 from
    its current tap, each upsampling holds channel 0 of its ELU'd input for
    `stride` samples (weights 1 on taps 0..s-1), each residual unit adds only
    its second bias beta_i (zero weights), the last convolution picks channel
    0.  Then every sample of frame t is elu(v_n), with v_0 = z_t[0] + b_in
    and v_{i+1} = elu(v_i) + b_up_i + beta_i."""
    w = synth.make_codec_weights(CD, seed=2)
    c = CD.channels
    rng = np.random.default_rng(4)

    def onehot(co, ci, K, taps):
        a = np.zeros((co, ci, K), np.float32)
        for k in taps:
            a[0, 0, k] = 1.0
        return _bits(a)

    w["conv_in.w"] = onehot(c[0], CD.d, CD.conv_k, [CD.conv_k - 1])
    w["conv_in.b"] = np.zeros(c[0], np.float32)
    w["conv_in.b"][0] = 0.25
    b_up, beta = [], []
    for i, s in enumerate(CD.strides):
        w[f"up.{i}.w"] = onehot(c[i + 1], c[i], 2 * s, range(s))
        w[f"up.{i}.b"] = np.zeros(c[i + 1], np.float32)
        b_up.append(float(np.float32(rng.normal() * 0.5)))
        w[f"up.{i}.b"][0] = b_up[-1]
        w[f"res.{i}.a.w"] = _bits(rng.normal(size=w[f"res.{i}.a.w"].shape))
        w[f"res.{i}.b.w"] = _bits(np.zeros(w[f"res.{i}.b.w"].shape))
        w[f"res.{i}.b.b"] = np.zeros(c[i + 1], np.float32)
        beta.append(float(np.float32(rng.normal() * 0.5)))
        w[f"res.{i}.b.b"][0] = beta[-1]
    w["conv_out.w"] = onehot(1, c[-1], CD.conv_k, [CD.conv_k - 1])
    w["conv_out.b"] = np.zeros(1, np.float32)
    o = codec.CodecOracle(CD, w, 1, np.float64)
    codes = synth.agent_frames(21, 4)
    for t in range(4):
        st = o.slots[0]
        z = o.transformer(st, o.latent(codes[t]))
        pcm = o.convs(st, z)
        st.pos += 1
        v = z[0] + 0.25
        for i in range(len(CD.strides)):
            v = (np.expm1(v) if v <= 0 else v) + b_up[i] + beta[i]
        v = np.expm1(v) if v <= 0 else v
        np.testing.assert_allclose(pcm, np.full(CD.samples, v), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- the encoder

@pytest.mark.parametrize("s", [2, 4, 5, 8])
def test_strided_conv_matches_torch(s):
    rng = np.random.default_rng(10 + s)
    ci, co, To = 3, 4, 5
    x, w, b = rng.normal(size=(ci, To * s)), rng.normal(size=(co, ci, 2 * s)), rng.normal(size=co)
    # causal: left padding K - s, stride s
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(torch.tensor(x)[None], (s, 0)), torch.tensor(w),
                                     torch.tensor(b), stride=s)[0].numpy()
    y = codec.strided_conv_causal(x, w, b, np.zeros((ci, s)), s)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a history is the s inputs before x
    h = rng.normal(size=(ci, s))
    full = np.concatenate([h, x], axis=1)
    ref2 = torch.nn.functional.conv1d(torch.nn.functional.pad(torch.tensor(full)[None], (s, 0)), torch.tensor(w),
                                      torch.tensor(b), stride=s)[0].numpy()[:, 1:]
    np.testing.assert_allclose(codec.strided_conv_causal(x, w, b, h, s), ref2, rtol=1e-12, atol=1e-12)


def test_nearest_is_brute_force_with_lowest_index_on_ties():
    rng = np.random.default_rng(4)
    table = rng.normal(size=(40, 6))
    table[17] = table[5]            # an exact tie: index 5 must win
    for trial in range(50):
        r = rng.normal(size=6) if trial else table[5] + 1e-3
        best, bd = None, None
        for j in range(len(table)):
            dj = sum((table[j][i] - r[i]) ** 2 for i in range(6))
            if bd is None or dj < bd:
                best, bd = j, dj
        assert codec.nearest(r, table)[0] == best


def test_quantiser_closed_form():
    """Codebooks built so that z = C_0[a] + C_1[b] exactly, codebook 0 coarse
    (rows of scale 1) and codebook 1 fine (scale 0.05), and codebooks 2..7
    each hold an exact zero row (index z_q), a copy of C_0[a] (index 77) and
    otherwise rows far away: the codes are (a, b, z_2, ..., z_7) only if each
    stage quantises what the stages before it left."""
    cd = CD
    w = synth.make_codec_weights(cd, seed=0)
    rng = np.random.default_rng(5)
    a, b = 700, 1234
    zq = [3, 2047, 0, 555, 1024, 9]
    tabs = []
    for q in range(cd.n_q):
        t = rng.normal(size=(cd.card, cd.d)).astype(np.float32) * (1.0 if q == 0 else 0.05)
        if q >= 2:
            t += 10.0                      # far from any residual left after two stages
            t[zq[q - 2]] = 0.0
            t[77] = tabs[0][a]
        tabs.append(synth.bf16_bits_to_f32(_bits(t)))
        w[f"codebook.{q}"] = _bits(t)
    z = tabs[0][a].astype(np.float64) + tabs[1][b]
    o = codec.CodecOracle(cd, w, 1, np.float64)
    np.testing.assert_array_equal(o.quantise(z), [a, b] + zq)


def test_encoder_output_norm_is_its_own():
    """With every layer's updates zero (out- and down-projections zero), the
    encoder's transformer output is the RMS-normalised latent scaled by the
    encoder's output-norm alpha, not the decoder's: the two alphas are set to
    0.5 and 2 and the ratio z / (y / rms(y)) must be 0.5 everywhere."""
    w = synth.make_codec_weights(CD, seed=9)
    for l in range(CD.n_layers):
        for k in ("wo", "w_out"):
            w[f"enc.layers.{l}.{k}"] = _bits(np.zeros(w[f"enc.layers.{l}.{k}"].shape))
    w["enc.out_norm"] = np.full(CD.d, 0.5, np.float32)
    w["out_norm"] = np.full(CD.d, 2.0, np.float32)
    o = codec.CodecOracle(CD, w, 1, np.float64)
    y = np.random.default_rng(12).normal(size=CD.d)
    z = o.transformer(o.enc_slots[0], y.copy(), "enc.")
    rms = np.sqrt(np.mean(y ** 2) + CD.norm_eps)
    np.testing.assert_allclose(z / (y / rms), 0.5, rtol=1e-12)


def test_encoder_streaming_equals_whole_sequence_and_reset_is_fresh():
    w = synth.make_codec_weights(CD, seed=6)
    n = 2 * CD.window + 3
    pcm = synth.user_audio(7, n, CD.samples)
    other = synth.user_audio(8, 5, CD.samples)
    o = codec.CodecOracle(CD, w, 2, np.float64)
    got = [o.encode(np.stack([pcm[t], other[t % 5]]))[0] for t in range(n)]
    ref = codec.encode_sequence(CD, w, pcm.reshape(-1), np.float64)
    np.testing.assert_array_equal(np.stack(got), ref)
    o.reset(1)
    got = [o.encode(np.stack([other[0], pcm[t]]))[1] for t in range(6)]
    np.testing.assert_array_equal(np.stack(got), ref[:6])


def test_encoder_transformer_is_the_temporal_block():
    cw = synth.make_codec_weights(CD, seed=7)
    dm = synth.Dims(d=CD.d, n_layers=CD.n_layers, n_heads=CD.n_heads, ffn=CD.ffn, text_card=64,
                    audio_card=64, n_q=8, dep_d=32, dep_layers=1, dep_heads=1, dep_ffn=32, dep_q=16,
                    norm_eps=CD.norm_eps, rope_base=CD.rope_base)
    tw = synth.make_weights(dm, seed=2)
    for l in range(CD.n_layers):
        for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out"):
            tw[f"layers.{l}.{k}"] = cw[f"enc.layers.{l}.{k}"]
    n = CD.window + 3
    xs = np.random.default_rng(10).normal(size=(n, CD.d))
    t = tick.Oracle(dm, tw, 1, CD.window, dtype=np.float64)
    t.prefill_embed(0, xs)
    o = codec.CodecOracle(CD, cw, 1, np.float64)
    st = o.enc_slots[0]
    for i in range(n):
        t.step(np.zeros((1, 8), np.int64))
        got = o.blocks(st, xs[i].copy(), "enc.")
        st.pos += 1
        np.testing.assert_allclose(got, t.taps["hidden"][-1, 0], rtol=1e-12, atol=1e-12, err_msg=f"frame {i}")


def test_encoder_conv_stack_closed_form():
    """Pass-through weights: the first convolution takes the current sample
    plus beta_in, each residual unit adds only its second bias beta_j, each
    strided convolution takes channel 0 of its ELU'd input at its last tap
    (the last sample of its block) plus b_j, the last convolution takes
    channel 0 plus b_out.  The latent's channel 0 for frame f is then
    elu(v_n) + b_out with v_0 = x[last sample of frame f] + beta_in and
    v_{j+1} = elu(v_j + beta_j) + b_j."""
    w = synth.make_codec_weights(CD, seed=8)
    c, n = CD.channels, len(CD.strides)
    rng = np.random.default_rng(11)

    def onehot(shape, taps):
        a = np.zeros(shape, np.float32)
        for k in taps:
            a[0, 0, k] = 1.0
        return _bits(a)

    def bias(m, v):
        b = np.zeros(m, np.float32)
        b[0] = v
        return b

    f32 = lambda v: float(np.float32(v))
    b_in = f32(0.125)
    w["enc.conv_in.w"] = onehot(w["enc.conv_in.w"].shape, [CD.conv_k - 1])
    w["enc.conv_in.b"] = bias(c[-1], b_in)
    beta, bd = [], []
    for j in range(n):
        ci = c[n - j]
        w[f"enc.res.{j}.b.w"] = _bits(np.zeros(w[f"enc.res.{j}.b.w"].shape))
        beta.append(f32(rng.normal() * 0.5))
        w[f"enc.res.{j}.b.b"] = bias(ci, beta[-1])
        K = w[f"enc.down.{j}.w"].shape[2]
        w[f"enc.down.{j}.w"] = onehot(w[f"enc.down.{j}.w"].shape, [K - 1])
        bd.append(f32(rng.normal() * 0.5))
        w[f"enc.down.{j}.b"] = bias(c[n - 1 - j], bd[-1])
    b_out = f32(-0.25)
    w["enc.conv_out.w"] = onehot(w["enc.conv_out.w"].shape, [CD.conv_k - 1])
    w["enc.conv_out.b"] = bias(CD.d, b_out)
    o = codec.CodecOracle(CD, w, 1, np.float64)
    pcm = synth.user_audio(12, 4, CD.samples)
    for t in range(4):
        y = o.enc_convs(o.enc_slots[0], pcm[t].astype(np.float64))
        v = float(pcm[t][-1]) + b_in
        for j in range(n):
            u = v + beta[j]
            v = (u if u > 0 else np.expm1(u)) + bd[j]
        v = (v if v > 0 else np.expm1(v)) + b_out
        np.testing.assert_allclose(y[0], v, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y[1:], 0.0, atol=0)


def test_convolutions_match_torch_on_random_shapes():
    """The three convolution forms against PyTorch's routines over 60 random
    shapes each (channels 1-9, kernels 1-8, strides 1-8, 1-7 frames' worth of
    inputs), each call with a random history: the output must equal the
    tail of the routine's output over (history, input)."""
    rng = np.random.default_rng(2026)
    F = torch.nn.functional
    for _ in range(60):
        ci, co = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        K, s, n = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 8))
        b = rng.normal(size=co)
        # causal, kernel K: history K - 1
        x, w, h = rng.normal(size=(ci, n)), rng.normal(size=(co, ci, K)), rng.normal(size=(ci, K - 1))
        ref = F.conv1d(torch.tensor(np.concatenate([h, x], 1))[None], torch.tensor(w), torch.tensor(b))[0].numpy()
        np.testing.assert_allclose(codec.causal_conv(x, w, b, h), ref, rtol=1e-12, atol=1e-12)
        # strided, stride s, kernel 2 s: history s, n blocks of s inputs
        x, w, h = rng.normal(size=(ci, n * s)), rng.normal(size=(co, ci, 2 * s)), rng.normal(size=(ci, s))
        ref = F.conv1d(torch.tensor(np.concatenate([h, x], 1))[None], torch.tensor(w), torch.tensor(b),
                       stride=s)[0].numpy()
        np.testing.assert_allclose(codec.strided_conv_causal(x, w, b, h, s), ref, rtol=1e-12, atol=1e-12)
        # transposed, stride s, kernel 2 s: the previous input, then n inputs;
        # the routine's outputs s .. s + n s - 1 are this call's
        x, w, p = rng.normal(size=(ci, n)), rng.normal(size=(co, ci, 2 * s)), rng.normal(size=(ci, 1))
        ref = F.conv_transpose1d(torch.tensor(np.concatenate([p, x], 1))[None], torch.tensor(w.transpose(1, 0, 2)),
                                 torch.tensor(b), stride=s)[0].numpy()[:, s:s + n * s]
        np.testing.assert_allclose(codec.conv_transpose_causal(x, w, b, p, s), ref, rtol=1e-12, atol=1e-12)
