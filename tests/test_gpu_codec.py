"""The codec's HIP path (include/codec.h), decoder and encoder, against the
codec oracle (oracle/codec.py, fp64), and its slot isolation and streaming
state.

Stored keys and values: both sides round them to bf16, the GPU from its
fp32 value and the oracle from the fp64 value, so where the two lie on
opposite sides of a rounding point the stored values differ, and either is a
correct rounding.  The GPU's error on a key or value comes from its GEMM
input's bf16 hi/lo representation (2^-17 of each input) and fp32 sums,
added over the dot product: bounded by 2^-12 of the head vector's RMS (about
18 terms' worth of |W_i h_i| at 2^-17 each, with margin), which can be many
bf16 steps of a near-zero element.  Each stored value must be within half a
bf16 step of the exact value plus that bound; values that differ from the
oracle's own rounding are counted and reported.  The oracle then takes the
GPU's stored values, so everything downstream is compared on identical
caches.

Tolerance on the samples and on the transformer output: the GPU computes in
fp32 with bf16 weights (the transformer's GEMM inputs as bf16 hi/lo pairs),
the oracle in fp64 with the same weights; the oracle's own fp32 run sits
about 3e-6 (relative L2) from its fp64 run at the full shape, and the bound
is 5e-5 relative L2 and 5e-5 of the frame's largest sample elementwise.
Encoder: the latent fed to the transformer (fp32 convolutions over 1920
samples) and the transformer output are held to the same bounds.  The
quantiser's argmin is an integer decision from floating point: the GPU's
distances are fp32 (|c|^2 - 2 r.c), the oracle's fp64 (|r - c|^2), so at a
near tie they can pick different rows.  The oracle takes the GPU's code
where it is its own choice or within 2^-14 of |r|^2 + |c|^2 of its best
distance (a near tie); such substitutions are counted and reported, and the
residual then carries on from the same row on both sides.

Parity with the real Mimi codec is unpinned: its layers and weights are not
available (the structure is a reading of the SoundStream / EnCodec family
the pages name)."""
import dataclasses

import numpy as np
import pytest

from full_duplex_speech_moshi_amd import synth
from oracle import codec as oracle_codec
from oracle.tick import upcast_bf16

pytestmark = pytest.mark.gpu

REL_L2 = 5e-5
MAX_REL = 5e-5
KV_ERR = 2.0 ** -12  # of the head vector's RMS
TIE = 2.0 ** -14     # of |r|^2 + |c|^2


def _say(msg):
    print(msg, flush=True)


def _engine(cd, w, B, dev=None):
    import torch
    from full_duplex_speech_moshi_amd import codec
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return codec.CodecEngine(cd, w, B, device_weights=dev)


def _compare(got, ref, what):
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= REL_L2 and mx <= MAX_REL, f"{what}: rel-L2 {err:.2e}, max {mx:.2e}"
    return err, mx


class _GpuCaches:
    """The oracle's store hook: checks the GPU's stored keys and values of
    the frame just decoded and hands them to the oracle."""

    def __init__(self, cd):
        self.cd, self.ring, self.flips, self.checked = cd, None, 0, 0

    def __call__(self, slot, layer, pos, k, v, ks, vs):
        out = []
        for which, exact, mine in ((0, k, ks), (1, v, vs)):
            gpu = upcast_bf16(self.ring[slot, layer, which, :, pos % self.cd.window, :], np.float64)
            rms = np.sqrt(np.mean(exact ** 2, axis=1, keepdims=True))
            # half a bf16 step at the value's magnitude: 2^(floor(log2|x|) - 8)
            half = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 8)
            bad = np.abs(gpu - exact) > half + KV_ERR * rms
            assert not bad.any(), \
                f"slot {slot} layer {layer} pos {pos} {'kv'[which]}: GPU stored {gpu[bad][:4]}, exact {exact[bad][:4]}"
            self.flips += int((gpu != mine).sum())
            self.checked += gpu.size
            out.append(gpu)
        return out[0], out[1]


def _parity_run(cd, w, B, n, seed, report):
    codes = [synth.agent_frames(seed + b, n, cd.card)[:, :cd.n_q] for b in range(B)]
    o = oracle_codec.CodecOracle(cd, w, B, np.float64)
    hook = _GpuCaches(cd)
    o.store_hook = hook
    e = _engine(cd, w, B)
    worst = [0.0, 0.0, 0.0]
    for t in range(n):
        c = np.stack([codes[b][t] for b in range(B)])
        got = e.decode(c)
        taps = e.taps()
        hook.ring = taps["ring"]
        ref = o.decode(c)
        for b in range(B):
            err, mx = _compare(got[b], ref[b], f"frame {t} slot {b}")
            zerr, _ = _compare(taps["z"][b], o.slots[b].last_z, f"frame {t} slot {b} transformer output")
            worst = [max(worst[0], err), max(worst[1], mx), max(worst[2], zerr)]
    timing = e.time(10)
    e.close()
    report(f"worst rel-L2 {worst[0]:.2e}, worst max {worst[1]:.2e}, transformer output {worst[2]:.2e}; "
           f"stored keys and values checked "
           f"{hook.checked}, of which {hook.flips} differ from the oracle's rounding; device time per call {timing:.3f} ms")


@pytest.mark.timeout(600)
def test_tiny_codec_matches_oracle_over_a_wrapping_window():
    cd = synth.CODEC_TINY
    _say(f"case: tiny codec, B=2, {3 * cd.window + 2} frames (window {cd.window})")
    _parity_run(cd, synth.make_codec_weights(cd, seed=1), 2, 3 * cd.window + 2, 30, _say)


@pytest.mark.timeout(600)
def test_full_codec_matches_oracle():
    cd = synth.CODEC
    _say("case: codec at the full shape (1920 samples per frame), B=2, 8 frames")
    _parity_run(cd, synth.make_codec_weights(cd, seed=0), 2, 8, 40, _say)


@pytest.mark.timeout(600)
def test_codec_slots_are_independent_and_reset_is_fresh():
    """B = 5 against B = 1, bit for bit: slot 3 of the batch carries the same
    stream as the single slot; slot 1 is reset mid-stream and then fed that
    stream from its start, which must give the single slot's samples; timing
    launches and a rejected call in between change nothing."""
    import torch
    from full_duplex_speech_moshi_amd import codec, pp
    cd = synth.CODEC_TINY
    w = synth.make_codec_weights(cd, seed=2)
    dev = codec.upload_codec_weights(cd, w, torch.device("cuda:0"))
    n = 2 * cd.window + 3
    mine = synth.agent_frames(50, n)
    noise = synth.agent_frames(51, 2 * n)
    single = _engine(cd, w, 1, dev)
    ref = [single.decode(mine[t][None])[0] for t in range(n)]
    single.close()
    _say("case: tiny codec, B=5 vs B=1, reset at frame 7")
    e = _engine(cd, w, 5, dev)
    t1 = 0
    for t in range(n):
        c = noise[t % len(noise)][None].repeat(5, 0)
        c[0] = noise[(t + 3) % len(noise)]
        c[3] = mine[t]
        if t == 7:
            e.reset(1)
            t1 = 0
        if t >= 7:
            c[1] = mine[t1]
        if t == 9:
            e.time(3)
            bad = c.copy()
            bad[2, 4] = cd.card
            with pytest.raises(pp.PPError) as ex:
                e.decode(bad)
            assert ex.value.code == pp.PP_EINVAL
        got = e.decode(c)
        np.testing.assert_array_equal(got[3], ref[t], err_msg=f"frame {t} slot 3")
        if t >= 7:
            np.testing.assert_array_equal(got[1], ref[t1], err_msg=f"frame {t} slot 1 (reset at 7)")
            t1 += 1
    e.close()


class _GpuCodes:
    """The oracle's quantiser hook: takes the GPU's code of the frame just
    encoded where it is the oracle's own choice or a near tie with it."""

    def __init__(self):
        self.codes, self.subs, self.checked = None, 0, 0

    def __call__(self, slot, q, r, dist, c):
        g = int(self.codes[slot, q])
        self.checked += 1
        if g != c:
            scale = float(np.dot(r, r)) + float(dist[c]) + 1e-30
            assert dist[g] - dist[c] <= TIE * scale, \
                f"slot {slot} stage {q}: GPU code {g} at distance {dist[g]:.6g}, oracle's {c} at {dist[c]:.6g}"
            self.subs += 1
        return g


def _encoder_parity_run(cd, w, B, n, seed, report):
    pcm = [synth.user_audio(seed + b, n, cd.samples) for b in range(B)]
    o = oracle_codec.CodecOracle(cd, w, B, np.float64)
    caches, codes = _GpuCaches(cd), _GpuCodes()
    o.enc_store_hook, o.code_hook = caches, codes
    e = _engine(cd, w, B)
    worst = [0.0, 0.0]
    for t in range(n):
        x = np.stack([pcm[b][t] for b in range(B)])
        got = e.encode(x)
        taps = e.taps()
        caches.ring, codes.codes = taps["enc_ring"], got
        ref = o.encode(x)
        np.testing.assert_array_equal(got, ref, err_msg=f"frame {t}")  # the hook took the GPU's only at near ties
        for b in range(B):
            ye, _ = _compare(taps["enc_y"][b], o.enc_slots[b].last_y, f"frame {t} slot {b} latent")
            ze, _ = _compare(taps["enc_z"][b], o.enc_slots[b].last_z, f"frame {t} slot {b} transformer output")
            worst = [max(worst[0], ye), max(worst[1], ze)]
    timing = e.time_encode(10)
    e.close()
    report(f"latent worst rel-L2 {worst[0]:.2e}, transformer output {worst[1]:.2e}; codes {codes.checked}, "
           f"near-tie substitutions {codes.subs}; stored keys and values {caches.checked}, of which {caches.flips} "
           f"differ from the oracle's rounding; device time per call {timing:.3f} ms")


@pytest.mark.timeout(600)
def test_tiny_encoder_matches_oracle_over_a_wrapping_window():
    cd = synth.CODEC_TINY
    _say(f"case: tiny codec encoder, B=2, {3 * cd.window + 2} frames (window {cd.window})")
    _encoder_parity_run(cd, synth.make_codec_weights(cd, seed=1), 2, 3 * cd.window + 2, 70, _say)


@pytest.mark.timeout(600)
def test_encoder_with_a_ragged_codebook_matches_oracle():
    """100 codewords: the quantiser's last tile of codewords is partly past
    the codebook's end; 3 codebooks, B=3."""
    import dataclasses
    cd = dataclasses.replace(synth.CODEC_TINY, card=100, n_q=3)
    _say(f"case: tiny codec encoder, card 100, n_q 3, B=3, {cd.window + 3} frames")
    _encoder_parity_run(cd, synth.make_codec_weights(cd, seed=2), 3, cd.window + 3, 90, _say)


@pytest.mark.timeout(600)
def test_full_encoder_matches_oracle():
    cd = synth.CODEC
    _say("case: codec encoder at the full shape (1920 samples per frame), B=2, 6 frames")
    _encoder_parity_run(cd, synth.make_codec_weights(cd, seed=0), 2, 6, 80, _say)


@pytest.mark.timeout(600)
def test_encoder_slots_are_independent_and_reset_is_fresh():
    """B = 5 against B = 1, bit for bit, as for the decoder: slot 3 carries the
    single slot's audio; slot 1 is reset mid-stream and fed it from the
    start; a timing launch and a rejected call (a NaN sample) in between."""
    import torch
    from full_duplex_speech_moshi_amd import codec, pp
    cd = synth.CODEC_TINY
    w = synth.make_codec_weights(cd, seed=3)
    dev = codec.upload_codec_weights(cd, w, torch.device("cuda:0"))
    n = 2 * cd.window + 3
    mine = synth.user_audio(90, n, cd.samples)
    noise = synth.user_audio(91, n, cd.samples)
    single = _engine(cd, w, 1, dev)
    ref = [single.encode(mine[t][None])[0] for t in range(n)]
    single.close()
    _say("case: tiny codec encoder, B=5 vs B=1, reset at frame 7")
    e = _engine(cd, w, 5, dev)
    t1 = 0
    for t in range(n):
        x = np.stack([noise[(t + b) % n] for b in range(5)])
        x[3] = mine[t]
        if t == 7:
            e.reset(1)
            t1 = 0
        if t >= 7:
            x[1] = mine[t1]
        if t == 9:
            e.time_encode(3)
            bad = x.copy()
            bad[2, cd.samples // 2] = np.nan
            with pytest.raises(pp.PPError) as ex:
                e.encode(bad)
            assert ex.value.code == pp.PP_EINVAL
        got = e.encode(x)
        np.testing.assert_array_equal(got[3], ref[t], err_msg=f"frame {t} slot 3")
        if t >= 7:
            np.testing.assert_array_equal(got[1], ref[t1], err_msg=f"frame {t} slot 1 (reset at 7)")
            t1 += 1
    e.close()


# The launch configuration the codec benchmark times: B = 32 at the full
# shape.  Two slots (the first and the last) against the oracle, with the
# stored keys and values checked and adopted as in the B = 2 runs, and one
# slot against a B = 1 handle bit for bit (every launch shape of the batch
# must give a slot the same arithmetic).
B32, PICKS, SAME = 32, (0, 31), 17


@pytest.mark.timeout(900)
def test_full_codec_b32_matches_oracle_and_b1():
    import torch
    from full_duplex_speech_moshi_amd import codec
    cd = synth.CODEC
    w = synth.make_codec_weights(cd, seed=0)
    dev = codec.upload_codec_weights(cd, w, torch.device("cuda:0"))
    n = 4
    frames = [synth.agent_frames(200 + b, n) for b in range(B32)]
    _say(f"case: codec decoder at the full shape, B=1 reference for slot {SAME}, {n} frames")
    single = _engine(cd, w, 1, dev)
    ref1 = []
    for t in range(n):
        pcm = single.decode(frames[SAME][t][None])[0]
        ref1.append((pcm, single.taps()["z"][0]))
    single.close()
    _say(f"case: codec decoder at the full shape, B={B32}, slots {PICKS} against the oracle")
    o = oracle_codec.CodecOracle(cd, w, len(PICKS), np.float64)
    hook = _GpuCaches(cd)
    o.store_hook = hook
    e = _engine(cd, w, B32, dev)
    worst = [0.0, 0.0]
    for t in range(n):
        c = np.stack([frames[b][t] for b in range(B32)])
        got = e.decode(c)
        taps = e.taps()
        np.testing.assert_array_equal(got[SAME], ref1[t][0], err_msg=f"frame {t}: B={B32} slot {SAME} vs B=1")
        np.testing.assert_array_equal(taps["z"][SAME], ref1[t][1], err_msg=f"frame {t}: transformer output")
        hook.ring = taps["ring"][list(PICKS)]
        ref = o.decode(c[list(PICKS)])
        for k, b in enumerate(PICKS):
            err, _ = _compare(got[b], ref[k], f"frame {t} slot {b}")
            zerr, _ = _compare(taps["z"][b], o.slots[k].last_z, f"frame {t} slot {b} transformer output")
            worst = [max(worst[0], err), max(worst[1], zerr)]
    e.close()
    _say(f"samples worst rel-L2 {worst[0]:.2e}, transformer output {worst[1]:.2e}; stored keys and values "
         f"{hook.checked}, {hook.flips} on the other side of a rounding point")


@pytest.mark.timeout(900)
def test_full_encoder_b32_matches_oracle_and_b1():
    import torch
    from full_duplex_speech_moshi_amd import codec
    cd = synth.CODEC
    w = synth.make_codec_weights(cd, seed=0)
    dev = codec.upload_codec_weights(cd, w, torch.device("cuda:0"))
    n = 4
    pcm = [synth.user_audio(300 + b, n, cd.samples) for b in range(B32)]
    _say(f"case: codec encoder at the full shape, B=1 reference for slot {SAME}, {n} frames")
    single = _engine(cd, w, 1, dev)
    ref1 = []
    for t in range(n):
        codes1 = single.encode(pcm[SAME][t][None])[0]
        tp = single.taps()
        ref1.append((codes1, tp["enc_y"][0], tp["enc_z"][0]))
    single.close()
    _say(f"case: codec encoder at the full shape, B={B32}, slots {PICKS} against the oracle")
    o = oracle_codec.CodecOracle(cd, w, len(PICKS), np.float64)
    caches, codes = _GpuCaches(cd), _GpuCodes()
    o.enc_store_hook, o.code_hook = caches, codes
    e = _engine(cd, w, B32, dev)
    worst = [0.0, 0.0]
    for t in range(n):
        x = np.stack([pcm[b][t] for b in range(B32)])
        got = e.encode(x)
        taps = e.taps()
        np.testing.assert_array_equal(got[SAME], ref1[t][0], err_msg=f"frame {t}: B={B32} slot {SAME} vs B=1")
        np.testing.assert_array_equal(taps["enc_y"][SAME], ref1[t][1], err_msg=f"frame {t}: latent")
        np.testing.assert_array_equal(taps["enc_z"][SAME], ref1[t][2], err_msg=f"frame {t}: transformer output")
        caches.ring, codes.codes = taps["enc_ring"][list(PICKS)], got[list(PICKS)]
        ref = o.encode(x[list(PICKS)])
        np.testing.assert_array_equal(got[list(PICKS)], ref, err_msg=f"frame {t}")
        for k, b in enumerate(PICKS):
            ye, _ = _compare(taps["enc_y"][b], o.enc_slots[k].last_y, f"frame {t} slot {b} latent")
            ze, _ = _compare(taps["enc_z"][b], o.enc_slots[k].last_z, f"frame {t} slot {b} transformer output")
            worst = [max(worst[0], ye), max(worst[1], ze)]
    e.close()
    _say(f"latent worst rel-L2 {worst[0]:.2e}, transformer output {worst[1]:.2e}; codes {codes.checked}, "
         f"near-tie substitutions {codes.subs}")


# Odd shapes that reach the convolution kernels' other branches: fewer than
# 4 output channels (one channel per thread), stride 1 (transposed and
# strided), kernels of 1 and 2 taps, a split sum over 64 lanes; then wide
# kernels (8 and 5 taps, stride 8 with 16 taps), a split sum over 256 lanes,
# channel counts that are not multiples of 8, and a codebook of 300 rows.
ODD = [dataclasses.replace(synth.CODEC_TINY, d=64, n_layers=1, n_heads=2, ffn=64, window=3, conv_k=1, res_k=2,
                           strides=(1, 5), channels=(6, 4, 2), n_q=3, card=130),
       dataclasses.replace(synth.CODEC_TINY, d=256, n_layers=1, n_heads=2, ffn=256, window=4, conv_k=8, res_k=5,
                           strides=(8, 3), channels=(96, 44, 40), n_q=4, card=300)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", range(len(ODD)))
def test_odd_codec_shapes_match_oracle_both_directions(k):
    cd = ODD[k]
    w = synth.make_codec_weights(cd, seed=10 + k)
    _say(f"case: codec shape {k}: d {cd.d}, strides {cd.strides}, channels {cd.channels}, kernels "
         f"{cd.conv_k}/{cd.res_k}, card {cd.card}, B=3, {cd.window + 3} frames, decoder")
    _parity_run(cd, w, 3, cd.window + 3, 110 + 10 * k, _say)
    _say(f"case: codec shape {k}, encoder")
    _encoder_parity_run(cd, w, 3, cd.window + 3, 120 + 10 * k, _say)


# The degenerate and the largest settings: a 1-frame window (attention sees
# the current frame only) with a single codebook of 64 rows, and the largest
# window (PP_CODEC_MAX_WINDOW = 256 frames, one full decode split) over more
# frames than it holds.
EDGE = [dataclasses.replace(synth.CODEC_TINY, window=1, n_q=1, card=64),
        dataclasses.replace(synth.CODEC_TINY, window=256)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("k", range(len(EDGE)))
def test_edge_codec_windows_match_oracle_both_directions(k):
    cd = EDGE[k]
    w = synth.make_codec_weights(cd, seed=20 + k)
    n = cd.window + 4
    B = 2 if k == 0 else 1
    _say(f"case: codec window {cd.window}, n_q {cd.n_q}, card {cd.card}, B={B}, {n} frames, decoder")
    _parity_run(cd, w, B, n, 130 + 10 * k, _say)
    _say(f"case: codec window {cd.window}, encoder")
    _encoder_parity_run(cd, w, B, n, 140 + 10 * k, _say)


def _random_dims(seed):
    """A small codec with random stage count (1-3), strides (1-8), kernels
    (1-8), channel counts (even, up to 48 after the first convolution's up to
    80) and codebooks: reaches the convolution kernels' template branches."""
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 4))
    strides = tuple(int(v) for v in r.integers(1, 9, n))
    channels = (int(r.integers(4, 81)),) + tuple(2 * int(v) for v in r.integers(1, 25, n))
    return dataclasses.replace(synth.CODEC_TINY, d=64, n_layers=1, n_heads=2, ffn=64, window=2,
                               conv_k=int(r.integers(1, 9)), res_k=int(r.integers(1, 9)), strides=strides,
                               channels=channels, n_q=int(r.integers(1, 5)), card=int(r.integers(16, 200)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", range(6))
def test_random_codec_shapes_match_oracle_both_directions(seed):
    cd = _random_dims(1000 + seed)
    w = synth.make_codec_weights(cd, seed=40 + seed)
    _say(f"case: random codec {seed}: strides {cd.strides}, channels {cd.channels}, kernels {cd.conv_k}/{cd.res_k}, "
         f"n_q {cd.n_q}, card {cd.card}, B=2, 5 frames")
    _parity_run(cd, w, 2, 5, 200 + seed, _say)
    _encoder_parity_run(cd, w, 2, 5, 300 + seed, _say)
