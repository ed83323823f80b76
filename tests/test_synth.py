"""The seeded input generator: bf16 rounding, determinism, schedules."""
import numpy as np
import torch

from full_duplex_speech_moshi_amd import synth


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 0.02,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.5e-3, 65504.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.to_bf16_bits(x), ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert synth.to_bf16_bits(np.float32(1.00390625)) == 0x3F80
    assert synth.to_bf16_bits(np.float32(1.01171875)) == 0x3F82


def test_weights_deterministic_and_thread_independent():
    a = synth.make_weights(synth.TINY, seed=0, threads=1)
    b = synth.make_weights(synth.TINY, seed=0, threads=7)
    assert a.keys() == b.keys()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    man = synth.manifest(synth.TINY)
    assert [m[0] for m in man] == list(a.keys())
    for name, shape, kind in man:
        assert a[name].shape == shape
        assert a[name].dtype == (np.uint16 if kind == "bf16" else np.float32)
    f = synth.bf16_bits_to_f32(a["layers.0.wqkv"])
    assert abs(f.std() - 0.02) < 1e-3 and abs(f.mean()) < 1e-3
    al = a["layers.0.attn_norm"]
    assert abs(al.mean() - 1.0) < 2e-3 and abs(al.std() - 0.01) < 2e-3


def test_full_manifest_byte_count():
    """Resident weight bytes of the 7B shape: 14,431,268,864."""
    total = 0
    for name, shape, kind in synth.manifest(synth.FULL):
        total += int(np.prod(shape)) * (2 if kind == "bf16" else 4)
    assert total == 14_431_268_864


def test_session_open_schedule_layout():
    f = synth.session_open(3, text_card=32000)
    assert f.shape == (92, 17)
    assert (f[:16, 0] == synth.FREE).all() and (f[:16, 1:9] >= 0).all()
    sil = synth.fixed_frame(2)
    assert (f[16:22, 1:9] == sil).all() and (f[16:22, 0] == synth.FREE).all()
    assert (f[22:86, 0] >= 0).all() and (f[22:86, 1:9] == synth.FREE).all()
    assert (f[86:92, 1:9] == sil).all()
    assert (f[:, 9:17] == synth.fixed_frame(5)).all()


def test_elastic_schedule():
    sess, ev = synth.elastic_schedule(32, 300, 3000)
    assert sorted(ev[0]) == list(range(32))
    assert len(sess) == 32 + sum(len(e) for e in ev[1:])
    for s in sess:
        assert 0 <= s["fill_n"] <= 3000
    # about 1% of slot-ticks turn over
    n_events = sum(len(e) for e in ev[1:])
    assert 40 < n_events < 160


def test_ring_fill_shapes():
    k, v = synth.ring_fill(synth.TINY, 3, 7)
    assert k.shape == v.shape == (2, 7, 4, 64)
    assert not np.array_equal(k, v)
