"""The C-ABI library on a machine without a GPU: it loads, exports every
entry point include/pp.h declares, and its pure-host calls validate their
arguments.  No compute call is made."""
import ctypes
import os
import re

import pytest

from full_duplex_speech_moshi_amd import pp, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header="pp.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pp_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pp.LIB_PATH):
        pytest.fail("libpp.so not built: run python -m full_duplex_speech_moshi_amd.build")
    return pp.load_library()


def test_exports_every_declared_entry_point(lib):
    names = declared_functions()
    assert len(names) >= 11
    assert set(names) == set(pp.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_exports_every_codec_entry_point(lib):
    from full_duplex_speech_moshi_amd import codec
    names = declared_functions("codec.h")
    assert len(names) == 11
    assert set(names) == set(codec.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_codec_limits_and_structs_match_the_header():
    from full_duplex_speech_moshi_amd import codec
    src = open(os.path.join(ROOT, "include", "codec.h")).read()
    limits = {k: int(v) for k, v in re.findall(r"#define\s+(PP_CODEC_MAX_\w+)\s+(\d+)", src)}
    assert limits == {"PP_CODEC_MAX_STAGES": codec.PP_CODEC_MAX_STAGES, "PP_CODEC_MAX_BATCH": codec.PP_CODEC_MAX_BATCH,
                      "PP_CODEC_MAX_WINDOW": codec.PP_CODEC_MAX_WINDOW}
    body = re.sub(r"/\*.*?\*/", "", src[src.index("typedef struct pp_codec_weights"):], flags=re.S)
    body = body[:body.index("}")]
    fields = re.findall(r"(\w+)(?:\[PP_CODEC_MAX_STAGES\])?;", body)
    assert fields == [f[0] for f in codec.PPCodecWeights._fields_]


def test_codec_dims_validated_on_the_host(lib):
    import dataclasses
    from full_duplex_speech_moshi_amd import codec
    assert codec.pp_codec_samples(codec.make_codec_dims(synth.CODEC)) == 1920
    assert codec.pp_codec_samples(codec.make_codec_dims(synth.CODEC_TINY)) == 24
    bad = [dict(n_heads=3), dict(d=500), dict(window=257), dict(strides=(0, 2)), dict(strides=(9, 2)),
           dict(conv_k=9), dict(channels=(8, 5, 4)),
           dict(n_q=17), dict(ffn=100), dict(card=0), dict(d=8320, n_heads=65)]
    for kw in bad:
        cd = dataclasses.replace(synth.CODEC_TINY, **kw)
        if "strides" in kw:
            cd = dataclasses.replace(cd, channels=cd.channels[:len(cd.strides) + 1])
        if "channels" in kw:
            cd = dataclasses.replace(cd, strides=cd.strides[:len(cd.channels) - 1])
        out = ctypes.c_size_t()
        assert codec._lib().pp_codec_arena_bytes(ctypes.byref(codec.make_codec_dims(cd)), 1, ctypes.byref(out)) \
            == pp.PP_EINVAL, kw
    out = ctypes.c_size_t()
    for B in (0, 33):
        assert codec._lib().pp_codec_arena_bytes(ctypes.byref(codec.make_codec_dims(synth.CODEC)), B,
                                                 ctypes.byref(out)) == pp.PP_EINVAL
    # one slot's ring: layers x {k, v} x heads x window x head_dim bf16
    n1 = codec.pp_codec_arena_bytes(codec.make_codec_dims(synth.CODEC), 1)
    n2 = codec.pp_codec_arena_bytes(codec.make_codec_dims(synth.CODEC), 2)
    assert n2 - n1 >= 8 * 2 * 8 * 250 * 64 * 2
    h = ctypes.c_void_p()
    w = codec.PPCodecWeights()
    rc = codec._lib().pp_codec_create(ctypes.byref(codec.make_codec_dims(synth.CODEC)), 1, ctypes.byref(w),
                                      ctypes.c_void_p(256), 1 << 30, None, ctypes.byref(h))
    assert rc == pp.PP_EINVAL and not h.value and b"NULL" in codec._lib().pp_codec_last_error(None)


def test_binding_limits_match_the_header():
    src = open(os.path.join(ROOT, "include", "pp.h")).read()
    limits = {k: int(v) for k, v in re.findall(r"#define\s+(PP_MAX_\w+)\s+(\d+)", src)}
    assert limits["PP_MAX_BATCH"] == pp.PP_MAX_BATCH
    assert limits["PP_MAX_WINDOW"] == pp.PP_MAX_WINDOW


def test_arena_bytes_matches_ring_layout(lib):
    dims = pp.make_dims(synth.FULL)
    n1 = pp.pp_arena_bytes(dims, 1, 3000)
    n2 = pp.pp_arena_bytes(dims, 2, 3000)
    ring_per_slot = 32 * 2 * 32 * 3000 * 128 * 2     # [L][2][H][W][Dh] bf16
    assert n1 > ring_per_slot
    assert n2 - n1 >= ring_per_slot
    assert n2 - n1 < ring_per_slot + 64 * 2**20      # activations are small beside the ring


@pytest.mark.parametrize("field,value", [("n_q", 4), ("dep_q", 8), ("n_heads", 3), ("d", 250), ("ffn", 700)])
def test_bad_dims_rejected(lib, field, value):
    import dataclasses
    dm = dataclasses.replace(synth.TINY, **{field: value})
    out = ctypes.c_size_t()
    assert lib.pp_arena_bytes(ctypes.byref(pp.make_dims(dm)), 1, 32, ctypes.byref(out)) == pp.PP_EINVAL


@pytest.mark.parametrize("B,W", [(0, 32), (33, 32), (1, 0), (1, 4097)])
def test_bad_batch_or_window_rejected(lib, B, W):
    out = ctypes.c_size_t()
    assert lib.pp_arena_bytes(ctypes.byref(pp.make_dims(synth.TINY)), B, W, ctypes.byref(out)) == pp.PP_EINVAL


def test_create_validates_before_touching_the_device(lib):
    dims = pp.make_dims(synth.TINY)
    h = ctypes.c_void_p()
    w = pp.PPWeights()            # all NULL
    rc = lib.pp_create(ctypes.byref(dims), 1, 32, ctypes.byref(w), ctypes.c_void_p(256), 1 << 20, None, ctypes.byref(h))
    assert rc == pp.PP_EINVAL and not h.value
    assert b"NULL" in lib.pp_last_error(None)
    w = pp.PPWeights(**{f: 4096 for f in pp.WEIGHT_FIELDS})
    rc = lib.pp_create(ctypes.byref(dims), 1, 32, ctypes.byref(w), ctypes.c_void_p(256), 16, None, ctypes.byref(h))
    assert rc == pp.PP_ENOSPC
    rc = lib.pp_create(ctypes.byref(dims), 1, 32, ctypes.byref(w), ctypes.c_void_p(100), 1 << 30, None, ctypes.byref(h))
    assert rc == pp.PP_EINVAL   # misaligned arena


def test_null_handle_calls_are_rejected(lib):
    assert lib.pp_step(None, None, None) == pp.PP_EINVAL
    assert lib.pp_slot_reset(None, 0) == pp.PP_EINVAL
    assert lib.pp_prefill_forced(None, 0, None, 0) == pp.PP_EINVAL
    assert lib.pp_prefill_embed(None, 0, None, None, 0) == pp.PP_EINVAL
    assert lib.pp_set_acoustic_delay(None, 1) == pp.PP_EINVAL
    assert lib.pp_agent_frames(None, None, None) == pp.PP_EINVAL
    assert lib.pp_set_sampling(None, None) == pp.PP_EINVAL
    assert lib.pp_slot_seed(None, 0, 1) == pp.PP_EINVAL
    lib.pp_destroy(None)


def test_engine_refuses_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(RuntimeError):
        pp.Engine(synth.TINY, {}, 1, 32)


def test_packed_elems(lib):
    assert pp.pp_packed_elems(1000, 256) == 1008 * 256     # ragged rows pad to a 16-row tile
    assert pp.pp_packed_elems(12288, 4096) == 12288 * 4096
    assert pp.pp_packed_elems(16, 100) == 0                 # K must be a multiple of 32
    assert pp.pp_packed_elems(0, 32) == 0
    assert lib.pp_pack_matrix(None, 16, 32, None, None) == pp.PP_EINVAL
