"""GPU parity of the tick at the tiny shape (d 256, 2 layers, ring window 32
so the ring wraps), through the C-ABI library, against the CPU oracle."""
import numpy as np
import pytest

from full_duplex_speech_moshi_amd import synth
from oracle.tick import Oracle
from tests import parity

pytestmark = pytest.mark.gpu

DM = synth.TINY
W = synth.TINY_WINDOW


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(tiny_weights):
    import torch
    from full_duplex_speech_moshi_amd import pp
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return pp.upload_weights(DM, tiny_weights, torch.device("cuda:0"))


def engine(tiny_weights, dev, B, window=W):
    from full_duplex_speech_moshi_amd import pp
    return pp.Engine(DM, tiny_weights, B, window, device_weights=dev)


def test_c0_teacher_forced_parity(tiny_weights, dev):
    """100 ticks, B = 1, W = 32 (three wraps); user codes uniform from seed 1;
    the text/agent rows replay the oracle's own choices."""
    _say("case: C0 teacher-forced parity, 100 ticks, B=1, W=32")
    n = 100
    codes = synth.user_codes(1, n)
    recs = parity.oracle_run(Oracle(DM, tiny_weights, 1, W), codes)
    frames = parity.teacher_frames(recs, codes)
    e = engine(tiny_weights, dev, 1)
    e.prefill_forced(0, frames)
    fails, report = [], {}
    for t in range(n):
        tok = e.step(np.zeros((1, 8), np.int32))
        tp = e.taps()
        g = parity.gpu_slot(tp, 0)
        np.testing.assert_array_equal(tok[0], g["tokens"])
        # the embedding sum is exact: same fp32 adds in the same row order
        np.testing.assert_array_equal(g["hidden"][0], recs[t]["hidden"][0])
        np.testing.assert_array_equal(g["chosen"], recs[t]["chosen"])
        fails += parity.compare_tick(g, recs[t], t, report)
    e.close()
    _say(f"worst hidden rel-L2 {max(report['hidden_rel_l2']):.3e}, text logit abs "
         f"{max(report['text_logit_abs']):.3e}, dep logit abs {max(report['dep_logit_abs']):.3e}, "
         f"tokens checked {report.get('tok_checked', 0)}")
    assert not fails, "\n".join(fails[:20])


def test_c0_free_running_matches_oracle_until_low_margin(tiny_weights, dev):
    """Free-running (no forcing): the GPU's greedy tokens equal the oracle's
    until the first tick where the oracle's top-2 margin is below 1e-2."""
    _say("case: C0 free-running agreement, B=1")
    n = 100
    codes = synth.user_codes(1, n)
    recs = parity.oracle_run(Oracle(DM, tiny_weights, 1, W), codes)
    e = engine(tiny_weights, dev, 1)
    agree = 0
    for t in range(n):
        tok = e.step(codes[t:t + 1])
        tp = e.taps()
        r = recs[t]
        low = parity.margin(r["text_logits"]) <= parity.MARGIN or any(
            parity.margin(r["dep_logits"][k]) <= parity.MARGIN for k in range(8))
        if not np.array_equal(tok[0], r["tokens"]):
            assert low, f"tick {t}: tokens differ at high margin: {tok[0]} vs {r['tokens']}"
            break
        agree += 1
        if low:
            break
    e.close()
    _say(f"free-running ticks in agreement: {agree}")
    assert agree >= 1


def test_slot_isolation_bit_exact_across_batch_and_column_tiles(tiny_weights, dev):
    """B = 17 engine (slot 16 in the second 16-wide column tile) vs B = 1
    engines: each slot's tokens and taps are bit-identical."""
    _say("case: slot isolation B=17 vs B=1")
    B, n = 17, 8
    codes = [synth.user_codes(100 + b, n) for b in range(B)]
    frames = synth.session_open(3, text_card=DM.text_card, n_voice=3, n_persona=2)
    eb = engine(tiny_weights, dev, B)
    eb.prefill_forced(5, frames)
    toks, taps = [], []
    for t in range(n):
        toks.append(eb.step(np.stack([codes[b][t] for b in range(B)])))
        taps.append(eb.taps())
    eb.close()
    for b in (0, 5, 15, 16):
        e1 = engine(tiny_weights, dev, 1)
        if b == 5:
            e1.prefill_forced(0, frames)
        for t in range(n):
            tk = e1.step(codes[b][t:t + 1])
            tp = e1.taps()
            np.testing.assert_array_equal(tk[0], toks[t][b])
            np.testing.assert_array_equal(tp["hidden"][:, 0], taps[t]["hidden"][:, b])
            np.testing.assert_array_equal(tp["text_logits"][0], taps[t]["text_logits"][b])
            np.testing.assert_array_equal(tp["dep_logits"][0], taps[t]["dep_logits"][b])
            np.testing.assert_array_equal(tp["user_pred"][0], taps[t]["user_pred"][b])
        e1.close()


def test_recycled_slot_bit_exact_with_fresh_engine(tiny_weights, dev):
    _say("case: recycle == fresh")
    codes = synth.user_codes(7, 45)
    e = engine(tiny_weights, dev, 2)
    for t in range(40):     # wraps the ring
        e.step(np.concatenate([codes[t:t + 1], codes[t:t + 1]]))
    e.slot_reset(1)
    f = engine(tiny_weights, dev, 1)
    for t in range(5):
        a = e.step(np.concatenate([codes[40 + t:41 + t], codes[t:t + 1]]))
        ta = e.taps()
        b = f.step(codes[t:t + 1])
        tb = f.taps()
        np.testing.assert_array_equal(a[1], b[0])
        np.testing.assert_array_equal(ta["hidden"][:, 1], tb["hidden"][:, 0])
        np.testing.assert_array_equal(ta["dep_logits"][1], tb["dep_logits"][0])
    e.close()
    f.close()


def test_replay_is_deterministic(tiny_weights, dev):
    """Two handles fed the same inputs produce the same bits; timing replays
    of the graph in between do not disturb the slot state."""
    _say("case: determinism across handles and replays")
    codes = synth.user_codes(9, 6)
    a, b = engine(tiny_weights, dev, 3), engine(tiny_weights, dev, 3)
    for t in range(6):
        c = np.stack([codes[t]] * 3)
        ta = a.step(c)
        tap_a = a.taps()
        a.time_graph(3)          # replays with other inputs; slot state must not move
        tb = b.step(c)
        tap_b = b.taps()
        np.testing.assert_array_equal(ta, tb)
        for k in ("hidden", "text_logits", "dep_logits", "user_pred"):
            np.testing.assert_array_equal(tap_a[k], tap_b[k])
    a.close()
    b.close()


def test_pipelined_ticks_match_tick_by_tick(tiny_weights, dev):
    """Ticks issued back to back (the depformer's user-stream codebooks of one
    tick still running beside the next tick's temporal stack) give the same
    bits as ticks whose taps are read, and so waited for, one by one; a slot
    reset and a session open in between included."""
    _say("case: pipelined ticks vs tick-by-tick, B=3, 12 ticks")
    B, n = 3, 12
    codes = [synth.user_codes(300 + b, n) for b in range(B)]
    frames = synth.session_open(4, text_card=DM.text_card, n_voice=2, n_persona=2)
    a, b = engine(tiny_weights, dev, B), engine(tiny_weights, dev, B)
    a.prefill_forced(2, frames)
    b.prefill_forced(2, frames)
    taps_b = None
    for t in range(n):
        if t == 6:
            a.slot_reset(1)
            b.slot_reset(1)
        c = np.stack([codes[s][t] for s in range(B)])
        ta = a.step(c)                 # no taps in between: overlapped
        tb = b.step(c)
        taps_b = b.taps()              # waits for this tick's user codebooks
        np.testing.assert_array_equal(ta, tb)
    taps_a = a.taps()
    for k in ("hidden", "text_logits", "dep_logits", "user_pred", "chosen"):
        np.testing.assert_array_equal(taps_a[k], taps_b[k])
    a.close()
    b.close()


@pytest.mark.parametrize("window", [1, 2])
def test_degenerate_window_teacher_forced_parity(tiny_weights, dev, window):
    """A ring of 1 or 2 frames: each tick attends to its own key (and the one
    before); 12 teacher-forced ticks against the oracle with the same window."""
    _say(f"case: window {window}, 12 teacher-forced ticks, B=1")
    n = 12
    codes = synth.user_codes(11, n)
    recs = parity.oracle_run(Oracle(DM, tiny_weights, 1, window), codes)
    e = engine(tiny_weights, dev, 1, window)
    e.prefill_forced(0, parity.teacher_frames(recs, codes))
    fails, report = [], {}
    for t in range(n):
        e.step(np.zeros((1, 8), np.int32))
        fails += parity.compare_tick(parity.gpu_slot(e.taps(), 0), recs[t], t, report)
    e.close()
    _say(f"worst hidden rel-L2 {max(report['hidden_rel_l2']):.3e}")
    assert not fails, "\n".join(fails[:20])


def test_ring_fill_then_teacher_forced_parity(tiny_weights, dev):
    """Ring pre-filled with 20 frames of N(0,1) bf16 keys/values; 15 ticks
    from position 20 slide the 32-frame window."""
    _say("case: ring fill 20 + 15 ticks")
    kb, vb = synth.ring_fill(DM, 3, 20)
    codes = synth.alternating_codes(15, block=4)
    o = Oracle(DM, tiny_weights, 1, W)
    o.ring_fill(0, kb, vb)
    recs = parity.oracle_run(o, codes)
    e = engine(tiny_weights, dev, 1)
    e.ring_fill(0, kb, vb)
    e.prefill_forced(0, parity.teacher_frames(recs, codes))
    fails, rep = [], {}
    for t in range(15):
        e.step(np.zeros((1, 8), np.int32))
        fails += parity.compare_tick(parity.gpu_slot(e.taps(), 0), recs[t], t, rep)
    e.close()
    _say(f"worst hidden rel-L2 {max(rep['hidden_rel_l2']):.3e}")
    assert not fails, "\n".join(fails[:20])


def test_max_window_ring_wraps_teacher_forced_parity(tiny_weights, dev):
    """The largest window (4096 frames: 16 splits of 256 keys per head, the
    most the decode combines) with B = 2: slot 0 pre-filled to 4090 frames,
    so the ring fills and wraps during the run; slot 1 pre-filled to 1000
    (4 splits).  10 teacher-forced ticks per slot against the oracle."""
    from full_duplex_speech_moshi_amd import pp
    Wm, n, fills = pp.PP_MAX_WINDOW, 10, (4090, 1000)
    _say(f"case: window {Wm}, fills {fills}, {n} teacher-forced ticks, B=2")
    codes = [synth.user_codes(40 + b, n) for b in range(2)]
    kv = [synth.ring_fill(DM, 50 + b, f) for b, f in enumerate(fills)]
    recs = []
    for b in range(2):
        o = Oracle(DM, tiny_weights, 1, Wm)
        o.ring_fill(0, *kv[b])
        recs.append(parity.oracle_run(o, codes[b]))
    e = engine(tiny_weights, dev, 2, Wm)
    for b in range(2):
        e.ring_fill(b, *kv[b])
        e.prefill_forced(b, parity.teacher_frames(recs[b], codes[b]))
    fails, rep = [], {}
    for t in range(n):
        e.step(np.zeros((2, 8), np.int32))
        tp = e.taps()
        for b in range(2):
            fails += parity.compare_tick(parity.gpu_slot(tp, b), recs[b][t], t, rep)
    e.close()
    _say(f"worst hidden rel-L2 {max(rep['hidden_rel_l2']):.3e}")
    assert not fails, "\n".join(fails[:20])


def test_session_open_schedule_parity(tiny_weights, dev):
    """Session-open forced schedule (voice, silence, persona, silence) then free
    ticks, B = 2 with different schedules, teacher-forced on free rows."""
    _say("case: session-open schedule, B=2")
    B, n_free = 2, 6
    sched = [synth.session_open(b, text_card=DM.text_card, n_voice=4, n_persona=5) for b in range(B)]
    n = len(sched[0]) + n_free
    codes = [synth.user_codes(1000 + b, n) for b in range(B)]
    recs = []
    for b in range(B):
        o = Oracle(DM, tiny_weights, 1, W)
        o.prefill_forced(0, sched[b])
        recs.append(parity.oracle_run(o, codes[b]))
    e = engine(tiny_weights, dev, B)
    for b in range(B):
        e.prefill_forced(b, parity.teacher_frames(recs[b], codes[b], sched[b]))
    fails, rep = [], {}
    for t in range(n):
        e.step(np.zeros((B, 8), np.int32))
        tp = e.taps()
        for b in range(B):
            np.testing.assert_array_equal(tp["chosen"][b], recs[b][t]["chosen"])
            fails += parity.compare_tick(parity.gpu_slot(tp, b), recs[b][t], t, rep)
    e.close()
    assert not fails, "\n".join(fails[:20])


def test_errors_leave_state_unchanged(tiny_weights, dev):
    from full_duplex_speech_moshi_amd import pp
    _say("case: error paths")
    e = engine(tiny_weights, dev, 2)
    ref = engine(tiny_weights, dev, 2)
    codes = synth.user_codes(11, 4).reshape(2, 2, 8)
    with pytest.raises(pp.PPError) as ei:
        e.slot_reset(2)
    assert ei.value.code == pp.PP_EINVAL
    bad = codes[0].copy()
    bad[1, 3] = DM.audio_card
    with pytest.raises(pp.PPError) as ei:
        e.step(bad)
    assert ei.value.code == pp.PP_EINVAL
    bad_frame = np.full((1, 17), -1, np.int32)
    bad_frame[0, 9:] = 0
    bad_frame[0, 0] = DM.text_card
    with pytest.raises(pp.PPError) as ei:
        e.prefill_forced(0, bad_frame)
    assert ei.value.code == pp.PP_EINVAL
    kb, vb = synth.ring_fill(DM, 3, W + 1)
    with pytest.raises(pp.PPError) as ei:
        e.ring_fill(0, kb, vb)
    assert ei.value.code == pp.PP_EINVAL
    x_bad = np.zeros((2, DM.d), np.float32)
    x_bad[1, 5] = np.nan
    with pytest.raises(pp.PPError) as ei:          # the whole call is rejected, frame 0 included
        e.prefill_embed(0, x_bad)
    assert ei.value.code == pp.PP_EINVAL
    with pytest.raises(pp.PPError) as ei:
        e.prefill_embed(0, np.zeros((1, DM.d), np.float32), np.full((1, 9), DM.audio_card, np.int32))
    assert ei.value.code == pp.PP_EINVAL
    with pytest.raises(pp.PPError) as ei:
        e.set_acoustic_delay(5)
    assert ei.value.code == pp.PP_EINVAL
    for bad in [dict(text_temperature=-1.0), dict(text_temperature=1.0, top_p=0.0),
                dict(text_temperature=1.0, top_k=-2), dict(text_temperature=1.0, repetition_penalty=0.5)]:
        with pytest.raises(pp.PPError) as ei:
            e.set_sampling(**bad)
        assert ei.value.code == pp.PP_EINVAL
    fr, ok = e.agent_frames()
    assert not ok.any()
    # nothing above changed any state: same results as an untouched handle
    np.testing.assert_array_equal(e.step(codes[0]), ref.step(codes[0]))
    with pytest.raises(pp.PPError) as ei:           # both slots now free-running
        e.prefill_forced(1, np.zeros((1, 17), np.int32))
    assert ei.value.code == pp.PP_EBUSY
    kb, vb = synth.ring_fill(DM, 3, 4)
    with pytest.raises(pp.PPError) as ei:
        e.ring_fill(0, kb, vb)
    assert ei.value.code == pp.PP_EBUSY
    with pytest.raises(pp.PPError) as ei:
        e.prefill_embed(1, np.zeros((1, DM.d), np.float32))
    assert ei.value.code == pp.PP_EBUSY
    with pytest.raises(pp.PPError) as ei:           # a slot has ticked
        e.set_acoustic_delay(1)
    assert ei.value.code == pp.PP_EBUSY
    np.testing.assert_array_equal(e.step(codes[1]), ref.step(codes[1]))
    e.close()
    ref.close()


# ------------------------------------------------------------------ acoustic delay, embedding-form prefill

def _oracle_ticks(o, codes, n):
    """Per-tick oracle records with the frame-aligned agent frames."""
    recs = []
    for t in range(n):
        tok = o.step(codes[t:t + 1])
        tp = o.taps
        recs.append(dict(tokens=tok[0].copy(), hidden=tp["hidden"][:, 0].copy(),
                         text_logits=tp["text_logits"][0].copy(), dep_logits=tp["dep_logits"][0].copy(),
                         chosen=tp["chosen"][0].copy(), user_pred=tp["user_pred"][0].copy(),
                         frame=tp["agent_frame"][0].copy(), frame_valid=bool(tp["agent_frame_valid"][0])))
    return recs


def test_acoustic_delay_teacher_forced_parity(tiny_weights, dev):
    """Delay 1 at the tiny shape, 40 ticks: frame-aligned teacher frames (the
    oracle's choices: text and codebook 0 of tick t, codebooks 1-7 of tick
    t + 1) replayed into both the oracle and the GPU; taps, choices and the
    completed agent frames compared every tick."""
    _say("case: acoustic delay 1, teacher-forced parity, 40 ticks, B=1")
    n = 40
    codes = synth.user_codes(21, n)
    free = Oracle(DM, tiny_weights, 1, W)
    free.set_acoustic_delay(1)
    first = _oracle_ticks(free, codes, n)
    frames = np.full((n, 17), -1, np.int32)
    for t in range(n):
        frames[t, 0:2] = first[t]["chosen"][0:2]
        if t + 1 < n:
            frames[t, 2:9] = first[t + 1]["chosen"][2:9]
        frames[t, 9:17] = codes[t]
    o = Oracle(DM, tiny_weights, 1, W)
    o.set_acoustic_delay(1)
    o.prefill_forced(0, frames)
    recs = _oracle_ticks(o, codes, n)
    e = engine(tiny_weights, dev, 1)
    e.set_acoustic_delay(1)
    e.prefill_forced(0, frames)
    fails, report = [], {}
    for t in range(n):
        e.step(np.zeros((1, 8), np.int32))
        g = parity.gpu_slot(e.taps(), 0)
        np.testing.assert_array_equal(g["hidden"][0], recs[t]["hidden"][0])
        if t == 0:  # codebooks 1-7 are free on tick 0: compare where the margin decides
            for k in range(1, 8):
                if parity.margin(recs[0]["dep_logits"][k]) > parity.MARGIN:
                    assert g["chosen"][1 + k] == recs[0]["chosen"][1 + k]
        np.testing.assert_array_equal(g["chosen"], recs[t]["chosen"])
        fr, ok = e.agent_frames()
        assert bool(ok[0]) == recs[t]["frame_valid"]
        np.testing.assert_array_equal(fr[0], recs[t]["frame"] if recs[t]["frame_valid"] else np.zeros(8))
        fails += parity.compare_tick(g, recs[t], t, report)
    e.close()
    _say(f"worst hidden rel-L2 {max(report['hidden_rel_l2']):.3e}, tokens checked {report.get('tok_checked', 0)}")
    assert not fails, "\n".join(fails[:20])


def test_acoustic_delay_agent_frames_on_gpu(tiny_weights, dev):
    """Delay 2, B = 2, free-running: each completed agent frame is codebook 0
    chosen two ticks back and codebooks 1-7 chosen now; none before tick 2;
    a reset slot starts over."""
    _say("case: acoustic delay 2, agent frames, 12 ticks, B=2")
    n, D = 12, 2
    codes = np.stack([synth.user_codes(31, n), synth.user_codes(32, n)], 1)   # [n][2][8]
    e = engine(tiny_weights, dev, 2)
    e.set_acoustic_delay(D)
    chosen, since_reset = [], [0, 0]
    for t in range(n):
        if t == 7:
            e.slot_reset(1)
            since_reset[1] = 0
        e.step(codes[t])
        chosen.append(e.taps()["chosen"][:, 1:9].copy())
        fr, ok = e.agent_frames()
        for b in range(2):
            since_reset[b] += 1
            assert bool(ok[b]) == (since_reset[b] > D)
            if ok[b]:
                np.testing.assert_array_equal(fr[b, 0], chosen[t - D][b, 0])
                np.testing.assert_array_equal(fr[b, 1:], chosen[t][b, 1:])
            else:
                assert not fr[b].any()
    e.close()


def test_embedding_frames_parity(tiny_weights, dev):
    """Embedding-form prefill (seeded N(0,1) fp32 inputs in place of the
    gather-sum) for slot 0 beside token frames for slot 1, then free ticks;
    all choices forced to the oracle's (a first oracle pass), taps compared."""
    _say("case: embedding-form prefill parity, B=2, 6 prefill + 6 free ticks")
    n_pre, n = 6, 12
    x = np.random.default_rng(41).standard_normal((n_pre, DM.d), dtype=np.float32)
    codes = np.stack([synth.user_codes(42, n), synth.user_codes(43, n)], 1)
    tok_frames = np.concatenate([np.full((n_pre, 9), -1), codes[:n_pre, 1]], 1).astype(np.int32)

    def run_oracle(force0, force1):
        o = Oracle(DM, tiny_weights, 2, W)
        o.prefill_embed(0, x, force0)
        f1 = tok_frames.copy()
        if force1 is not None:
            f1[:, :9] = force1
        o.prefill_forced(1, f1)
        out = []
        for t in range(n):
            tok = o.step(codes[t])
            out.append(dict({k: np.array(v) for k, v in o.taps.items()}, tokens=tok))
        return out

    first = run_oracle(None, None)
    force0 = np.stack([first[t]["chosen"][0] for t in range(n_pre)])
    force1 = np.stack([first[t]["chosen"][1] for t in range(n_pre)])
    ref = run_oracle(force0, force1)
    e = engine(tiny_weights, dev, 2)
    e.prefill_embed(0, x, force0)
    f1 = tok_frames.copy()
    f1[:, :9] = force1
    e.prefill_forced(1, f1)
    fails, report = [], {}
    for t in range(n):
        e.step(codes[t])
        tp = e.taps()
        if t < n_pre:
            np.testing.assert_array_equal(tp["hidden"][0, 0], x[t])
        for b in range(2):
            g = parity.gpu_slot(tp, b)
            r = dict(hidden=ref[t]["hidden"][:, b], text_logits=ref[t]["text_logits"][b],
                     dep_logits=ref[t]["dep_logits"][b], tokens=ref[t]["tokens"][b],
                     user_pred=ref[t]["user_pred"][b], chosen=ref[t]["chosen"][b])
            if t < n_pre:
                np.testing.assert_array_equal(g["chosen"], r["chosen"])
            fails += parity.compare_tick(g, r, t, report)
    e.close()
    _say(f"worst hidden rel-L2 {max(report['hidden_rel_l2']):.3e}, tokens checked {report.get('tok_checked', 0)}")
    assert not fails, "\n".join(fails[:20])


def test_embedding_frame_of_a_gather_sum_equals_the_token_frame(tiny_weights, dev):
    """A token frame's own embedding sum, fed back as an embedding-form frame
    with the same forced choices, reproduces that tick bit for bit."""
    _say("case: embedding frame = token frame's gather-sum, B=1, 3 ticks")
    frames = np.random.default_rng(51).integers(0, DM.audio_card, (3, 17)).astype(np.int32)
    frames[:, 0] = np.random.default_rng(52).integers(0, DM.text_card, 3)
    et = engine(tiny_weights, dev, 1)
    et.prefill_forced(0, frames)
    ee = engine(tiny_weights, dev, 1)
    for t in range(3):
        et.step(np.zeros((1, 8), np.int32))
        tt = et.taps()
        ee.prefill_embed(0, tt["hidden"][0, 0].copy()[None], frames[t:t + 1, :9])
        ee.step(np.zeros((1, 8), np.int32))
        te = ee.taps()
        for key in ("hidden", "text_logits", "dep_logits", "chosen", "user_pred", "tokens"):
            np.testing.assert_array_equal(te[key], tt[key])
    et.close()
    ee.close()


# ------------------------------------------------------------------ sampling variant

def test_sampling_with_top_k_1_equals_greedy(tiny_weights, dev):
    _say("case: sampling with top_k = 1 vs greedy, B=2, 8 ticks")
    codes = np.stack([synth.user_codes(61, 8), synth.user_codes(62, 8)], 1)
    eg = engine(tiny_weights, dev, 2)
    es = engine(tiny_weights, dev, 2)
    es.set_sampling(0.8, 0.3, top_k=1)
    es.slot_seed(0, 5)
    es.slot_seed(1, 6)
    for t in range(8):
        np.testing.assert_array_equal(es.step(codes[t]), eg.step(codes[t]))
        ts, tg = es.taps(), eg.taps()
        for key in ("hidden", "text_logits", "dep_logits", "chosen", "user_pred"):
            np.testing.assert_array_equal(ts[key], tg[key])
    eg.close()
    es.close()


def _oracle_choice_or_boundary(logits, seed, tick, row, temp, top_k, top_p, rho, hist, got):
    """The oracle sampler's token for the GPU's own logits row; a different
    GPU token is accepted only if nudging u or top_p by 1e-5 (a decision at a
    rounding boundary) yields it.  Returns (ok, exact)."""
    from oracle import sampling as sm
    u = sm.uniform(seed, tick, row)
    want = sm.sample(logits, u, temp, top_k, top_p, rho, hist)
    if want == got:
        return True, True
    for du in (-1e-5, 1e-5):
        if sm.sample(logits, min(max(u + du, 0.0), 1 - 2 ** -24), temp, top_k, top_p, rho, hist) == got:
            return True, False
    for dp in (-1e-5, 1e-5):
        if top_p < 1.0 and sm.sample(logits, u, temp, top_k, min(top_p + dp, 1.0), rho, hist) == got:
            return True, False
    return False, False


@pytest.mark.parametrize("knobs", [(0.8, 0.7, 0, 1.0, 1.0), (0.75, 0.3, 50, 0.9, 1.2), (1.3, 1.0, 7, 1.0, 1.1)])
def test_sampling_matches_oracle_sampler(tiny_weights, dev, knobs):
    """Free-running sampled ticks, B = 2 with seeds 11 and 2^40 + 12: every
    text and codebook choice (17 rows) equals the oracle sampler applied to
    the GPU's own logits with the same draw (Philox of seed, tick, row) and
    the slot's recent chosen text tokens."""
    t_text, t_audio, top_k, top_p, rho = knobs
    _say(f"case: sampling parity {knobs}, B=2, 12 ticks")
    n = 12
    seeds = [11, 2 ** 40 + 12]
    codes = np.stack([synth.user_codes(63, n), synth.user_codes(64, n)], 1)
    e = engine(tiny_weights, dev, 2)
    e.set_sampling(t_text, t_audio, top_k, top_p, rho)
    for b, sd in enumerate(seeds):
        e.slot_seed(b, sd)
    hist = [[], []]
    exact = boundary = 0
    for t in range(n):
        tok = e.step(codes[t])
        tp = e.taps()
        for b in range(2):
            rows = [(tp["text_logits"][b], t_text, rho, list(hist[b]), tok[b, 0])]
            for k in range(DM.dep_q):
                got = tok[b, 1 + k] if k < 8 else tp["user_pred"][b, k - 8]
                rows.append((tp["dep_logits"][b, k], t_audio, 1.0, [], got))
            for row, (lg, temp, r, h, got) in enumerate(rows):
                ok, ex = _oracle_choice_or_boundary(lg, seeds[b], t, row, temp, top_k, top_p, r, h, int(got))
                assert ok, f"tick {t} slot {b} row {row}: GPU {got} is not the oracle's choice"
                exact += ex
                boundary += not ex
            hist[b] = (hist[b] + [int(tp["chosen"][b, 0])])[-64:]
    e.close()
    _say(f"decisions: {exact} exact, {boundary} at a rounding boundary")
    assert boundary <= 2


def test_sampling_isolation_and_recycle(tiny_weights, dev):
    """Sampled slots keep strong isolation: B = 3 equals B = 1 engines with the
    same seeds, and a recycled slot draws as a fresh engine does."""
    _say("case: sampling isolation and recycle, B=3 vs B=1, 6 ticks")
    n = 6
    seeds = [3, 4, 5]
    codes = np.stack([synth.user_codes(70 + b, n) for b in range(3)], 1)
    knobs = (0.9, 0.8, 20, 0.95, 1.15)
    eb = engine(tiny_weights, dev, 3)
    eb.set_sampling(*knobs)
    for b, sd in enumerate(seeds):
        eb.slot_seed(b, sd)
    toks = []
    for t in range(n):
        if t == 3:
            eb.slot_reset(2)
        toks.append(eb.step(codes[t]))
    eb.close()
    for b in range(3):
        e1 = engine(tiny_weights, dev, 1)
        e1.set_sampling(*knobs)
        e1.slot_seed(0, seeds[b])
        t_from = 3 if b == 2 else 0
        for t in range(t_from, n):
            np.testing.assert_array_equal(e1.step(codes[t, b:b + 1])[0], toks[t][b])
        e1.close()
