"""The shape and constants every part of the build uses (the seeded weights,
the oracle, the library's dimension check, the benchmark's byte counts)
against the figures the source pages state, stored with their citations in
tests/golden/personaplex_7b_shape.txt.  No GPU."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from full_duplex_speech_moshi_amd import pp, synth  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "personaplex_7b_shape.txt")


def _load():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            name, value = line.split()
            vals[name] = value
    return vals


G = _load()


def _int(name):
    return int(G[name])


def test_golden_file_holds_every_figure():
    assert set(G) == {"sample_rate_hz", "frame_rate_hz", "frame_samples", "frame_ms", "audio_codebooks",
                      "audio_card", "text_card", "column_rows", "agent_rows", "user_rows", "d_model", "n_layers",
                      "n_heads", "window", "dep_d_model", "dep_layers", "dep_heads", "dep_codebooks",
                      "silence_frames"}


def test_the_pages_figures_agree_with_each_other():
    # 24 kHz at 12.5 frames per second is 1920 samples and 80 ms per frame
    assert _int("sample_rate_hz") / float(G["frame_rate_hz"]) == _int("frame_samples")
    assert 1000.0 / float(G["frame_rate_hz"]) == _int("frame_ms")
    # one text row, then the agent and the user codebooks
    a0, a1 = (int(x) for x in G["agent_rows"].split("-"))
    u0, u1 = (int(x) for x in G["user_rows"].split("-"))
    assert (a0, a1 - a0 + 1) == (1, _int("audio_codebooks"))
    assert (u0, u1 - u0 + 1) == (a1 + 1, _int("audio_codebooks"))
    assert _int("column_rows") == u1 + 1 == 1 + 2 * _int("audio_codebooks")
    # the depformer predicts both streams' codebooks of the frame
    assert _int("dep_codebooks") == 2 * _int("audio_codebooks")
    # the silence prompt is about 0.5 s: the whole frames that fit in it
    assert _int("silence_frames") == int(0.5 * float(G["frame_rate_hz"]))


def test_the_7b_shape_is_the_pages_shape():
    dm = synth.FULL
    assert (dm.d, dm.n_layers, dm.n_heads) == (_int("d_model"), _int("n_layers"), _int("n_heads"))
    assert (dm.dep_d, dm.dep_layers, dm.dep_heads) == (_int("dep_d_model"), _int("dep_layers"), _int("dep_heads"))
    assert (dm.text_card, dm.audio_card) == (_int("text_card"), _int("audio_card"))
    assert (dm.n_q, dm.dep_q) == (_int("audio_codebooks"), _int("dep_codebooks"))
    assert 1 + 2 * dm.n_q == _int("column_rows")
    assert synth.FULL_WINDOW == _int("window")
    assert synth.SILENCE_FRAMES == _int("silence_frames")
    # head widths follow: 128 temporal, 64 depformer
    assert (dm.head_dim, dm.dep_head_dim) == (128, 64)


def test_the_library_takes_the_pages_shape_at_its_window():
    lib = pp.load_library()
    assert lib is not None
    # the window the pages give fits the library's limit, and the dimension
    # check accepts the shape (host-only call: no device is touched)
    assert _int("window") <= pp.PP_MAX_WINDOW
    n = pp.pp_arena_bytes(pp.make_dims(synth.FULL), 1, _int("window"))
    assert n > 0
