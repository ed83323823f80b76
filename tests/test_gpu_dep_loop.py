"""The fused depformer loop (one persistent launch per tick at B <= 2) against
the per-layer kernel launches, bit for bit, and against the oracle.

Small shape: the tiny temporal transformer with a depformer of width 256, 8
heads of 32, FFN 768 and 2 layers (the loop's smallest supported dims: one
head and one 96-row FFN slice per XCD).  7B shape: the configuration the
benchmark times at B = 1."""
import dataclasses

import numpy as np
import pytest

from full_duplex_speech_moshi_amd import synth
from oracle.tick import Oracle
from tests import parity

pytestmark = pytest.mark.gpu

SMALL = dataclasses.replace(synth.TINY, dep_d=256, dep_heads=8, dep_ffn=768, dep_layers=2)
W = synth.TINY_WINDOW
KEYS = ("hidden", "text_logits", "dep_logits", "tokens", "user_pred", "chosen")


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def small():
    import torch
    from full_duplex_speech_moshi_amd import pp
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    w = synth.make_weights(SMALL, seed=0)
    dev = pp.upload_weights(SMALL, w, torch.device("cuda:0"))
    torch.cuda.synchronize()
    return w, dev


def _engine(dm, wd, B, window, fused):
    from full_duplex_speech_moshi_amd import pp
    w, dev = wd
    e = pp.Engine(dm, w, B, window, device_weights=dev)
    assert not e.depformer_loop_active(), "per-layer launches are the default"
    e.set_depformer_loop(fused)
    assert e.depformer_loop_active() == fused
    return e


def _frames(dm, n, seed):
    """Forced frames: voice-like agent rows on tick 0, a persona text token on
    tick 1, free rows after."""
    rng = np.random.default_rng(seed)
    f = np.full((n, 17), -1, np.int32)
    f[:, 9:] = rng.integers(0, dm.audio_card, (n, 8))
    f[0, 1:9] = rng.integers(0, dm.audio_card, 8)
    if n > 1:
        f[1, 0] = rng.integers(0, dm.text_card)
    return f


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("taps_every_tick", [True, False])
def test_small_fused_equals_per_launch(small, B, taps_every_tick):
    """Forced then free ticks; with taps after every tick (each user half then
    runs in its own launch) or only at the end (each user half runs as extra
    columns of the next tick's launch).  Tokens every tick, taps at the end
    (and every tick when taken), bit for bit."""
    n = 7
    _say(f"case: small dims, B={B}, {n} ticks, taps every tick: {taps_every_tick}")
    codes = [synth.user_codes(300 + b, n) for b in range(B)]
    fr = [_frames(SMALL, 2, 40 + b) for b in range(B)]
    outs = []
    for fused in (True, False):
        e = _engine(SMALL, small, B, W, fused)
        for b in range(B):
            e.prefill_forced(b, fr[b])
        toks, taps = [], []
        for t in range(n):
            toks.append(e.step(np.stack([codes[b][t] for b in range(B)])))
            if taps_every_tick or t == n - 1:
                taps.append(e.taps())
        e.close()
        outs.append((toks, taps))
    (tf, pf), (tp, pp_) = outs
    for t in range(n):
        np.testing.assert_array_equal(tf[t], tp[t], err_msg=f"tick {t} tokens")
    for i, (a, r) in enumerate(zip(pf, pp_)):
        for k in KEYS:
            np.testing.assert_array_equal(a[k], r[k], err_msg=f"taps {i} {k}")


@pytest.mark.timeout(600)
def test_small_fused_matches_oracle(small):
    """Teacher-forced against the oracle at the small shape, 12 ticks (the ring
    of 32 frames is not reached; the fused loop is what differs from the
    tiny-shape parity tests)."""
    w, _ = small
    n = 12
    codes = synth.user_codes(9, n)
    o = Oracle(SMALL, w, 1, W)
    recs = parity.oracle_run(o, codes)
    e = _engine(SMALL, small, 1, W, True)
    e.prefill_forced(0, parity.teacher_frames(recs, codes))
    fails, rep = [], {}
    for t in range(n):
        e.step(np.zeros((1, 8), np.int32))
        fails += parity.compare_tick(parity.gpu_slot(e.taps(), 0), recs[t], t, rep)
    e.close()
    _say(f"worst hidden rel-L2 {max(rep['hidden_rel_l2']):.2e}, dep logit abs {max(rep['dep_logit_abs']):.2e}, "
         f"tokens checked {rep.get('tok_checked', 0)}")
    assert not fails, "\n".join(fails[:20])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("B", [1, 2])
def test_full_fused_equals_per_launch(B):
    """7B: 4 pipelined ticks (forced then free) and the last taps, fused loop
    vs per-layer launches, bit for bit; slot 1 (B = 2) holds a 700-frame ring."""
    import torch
    from full_duplex_speech_moshi_amd import pp
    dm = synth.FULL
    _say(f"case: 7B, B={B}, fused loop vs per-layer launches, 4 ticks")
    w = synth.make_weights(dm, seed=0)
    dev = pp.upload_weights(dm, w, torch.device("cuda:0"))
    n = 4
    codes = [synth.user_codes(500 + b, n) for b in range(B)]
    fill = synth.ring_fill(dm, 8, 700) if B > 1 else None
    fr = _frames(dm, 2, 77)
    outs = []
    for fused in (True, False):
        e = _engine(dm, (w, dev), B, synth.FULL_WINDOW, fused)
        if fill is not None:
            e.ring_fill(1, *fill)
        e.prefill_forced(0, fr)
        toks = [e.step(np.stack([codes[b][t] for b in range(B)])) for t in range(n)]
        outs.append((toks, e.taps()))
        if fused:
            ms = e.time_graph(10)
            _say(f"fused device tick {ms:.3f} ms")
        else:
            ms = e.time_graph(10)
            _say(f"per-launch device tick {ms:.3f} ms")
        e.close()
    for t in range(n):
        np.testing.assert_array_equal(outs[0][0][t], outs[1][0][t], err_msg=f"tick {t} tokens")
    for k in KEYS:
        np.testing.assert_array_equal(outs[0][1][k], outs[1][1][k], err_msg=k)
