"""The allocation-free entry point, pp_step_static, through the C ABI:
the same ticks as pp_step on a twin handle, bit for bit (same kernels, only
the work buffers move to the library's static array), on two handles in a
row, the second with a smaller input.  The first is the 7B shape at B = 10
(large-batch GEMM partials and multi-split decode partials in the array),
the second the tiny shape at B = 2 with a 4096-frame window (16-split
decode tickets in the array, left behind by the first)."""
import numpy as np
import pytest

from full_duplex_speech_moshi_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _twin_run(dm, w, dev, B, window, fills, n, seed, mix=False):
    from full_duplex_speech_moshi_amd import pp
    es = pp.Engine(dm, w, B, window, device_weights=dev)
    ep = pp.Engine(dm, w, B, window, device_weights=dev)
    for e in (es, ep):
        for b, f in fills.items():
            e.ring_fill(b, *f)
    codes = [synth.user_codes(seed + b, n) for b in range(B)]
    for t in range(n):
        c = np.stack([codes[b][t] for b in range(B)])
        ts = es.step(c) if (mix and t % 2) else es.step_static(c)
        tp = ep.step(c)
        np.testing.assert_array_equal(ts, tp, err_msg=f"tick {t} tokens")
        a, r = es.taps(), ep.taps()
        for key in ("hidden", "text_logits", "dep_logits", "tokens", "user_pred", "chosen"):
            np.testing.assert_array_equal(a[key], r[key], err_msg=f"tick {t} {key}")
    es.close()
    ep.close()


@pytest.mark.timeout(900)
def test_step_static_equals_step_twice_second_smaller():
    import torch
    from full_duplex_speech_moshi_amd import pp
    assert torch.cuda.is_available()
    dm = synth.FULL
    _say("case: pp_step_static vs pp_step, 7B, B=10, window 3000, one slot at 600 frames, 3 ticks")
    w = synth.make_weights(dm, seed=0)
    dev = pp.upload_weights(dm, w, torch.device("cuda:0"))
    _twin_run(dm, w, dev, 10, synth.FULL_WINDOW, {9: synth.ring_fill(dm, 31, 600)}, 3, 4000)
    del dev, w
    torch.cuda.empty_cache()
    dm = synth.TINY
    _say("case: pp_step_static vs pp_step, tiny, B=2, window 4096, rings at 4000 and 1000, 4 ticks, mixed calls")
    w = synth.make_weights(dm, seed=0)
    dev = pp.upload_weights(dm, w, torch.device("cuda:0"))
    _twin_run(dm, w, dev, 2, pp.PP_MAX_WINDOW,
              {0: synth.ring_fill(dm, 32, 4000), 1: synth.ring_fill(dm, 33, 1000)}, 4, 4100, mix=True)
