"""CPU contract tests of the C ABI's state machine (no GPU).

The library's host code (engine.cpp) is compiled with g++ against a stub of
the HIP runtime (tests/hoststub): device memory is host memory, captured
graphs are replayed lists of launcher calls, and the finisher writes a
made-up prediction pred = (7 pos + 13 (step + 1) + 5) mod n with the forced
choice applied.  Observed: the tick input block each tick is given (position,
17-row column, forced choices), the returned tokens and the return codes.

Checked against include/pp.h: fresh slots start at position 0 with the
initial tokens [Vt, A x 8]; choices feed the next column; forced frames are
consumed one per tick in order and replace the user codes; a slot becomes
free-running on its first tick with an empty queue and then refuses
prefills (PP_EBUSY); fills are legal only before any tick or prefill; every
error except PP_EDEVICE leaves the state unchanged (validate-then-commit);
a device error poisons the handle; reset equals a fresh handle; the
acoustic delay shifts codebooks 1-7.  Test infrastructure only.

With PP_HOST_SANITIZE=1 the stub library is built with AddressSanitizer and
UndefinedBehaviorSanitizer; the interpreter then needs their runtimes
preloaded, e.g. LD_PRELOAD="$(g++ -print-file-name=libasan.so)
$(g++ -print-file-name=libubsan.so)" ASAN_OPTIONS=detect_leaks=0."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from full_duplex_speech_moshi_amd import pp, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DM = synth.TINY
W = 8
B = 3
TI_STRIDE, TI_POS, TI_COL, TI_FORCE = 32, 0, 1, 18
VT, A = DM.text_card, DM.audio_card


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("hoststub") / "libpp_hoststub.so")
    checks = ",".join(("address", "undefined"))  # host code only: the stub build has no device code
    san = (["-g", "-fsanitize=" + checks, "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
           if os.environ.get("PP_HOST_SANITIZE") == "1" else [])
    cmd = ["g++", "-O1", *san, "-std=c++17", "-shared", "-fPIC", "-I", os.path.join(ROOT, "tests", "hoststub"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "full_duplex_speech_moshi_amd", "csrc", "engine.cpp"),
           os.path.join(ROOT, "tests", "hoststub", "hoststub.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    L = ctypes.CDLL(out)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.pp_arena_bytes.argtypes = [ctypes.POINTER(pp.PPDims), I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.pp_create.argtypes = [ctypes.POINTER(pp.PPDims), I, I, ctypes.POINTER(pp.PPWeights), P, ctypes.c_size_t, P,
                            ctypes.POINTER(P)]
    for n, a in (("pp_prefill_forced", [P, I, P, I]), ("pp_prefill_embed", [P, I, P, P, I]), ("pp_step", [P, P, P]),
                 ("pp_slot_reset", [P, I]), ("pp_ring_fill", [P, I, I, P, P]),
                 ("pp_set_acoustic_delay", [P, I]), ("pp_agent_frames", [P, P, P])):
        getattr(L, n).argtypes = a
        getattr(L, n).restype = I
    L.pp_destroy.argtypes = [P]
    L.pp_destroy.restype = None
    L.pp_last_error.argtypes = [P]
    L.pp_last_error.restype = ctypes.c_char_p
    L.stub_last_tick_input.argtypes = [P, I]
    L.stub_last_tick_input.restype = I
    L.stub_ticks_run.restype = ctypes.c_long
    L.stub_fail_launches.argtypes = [I]
    return L


class Handle:
    """A handle of the stub build with a host arena and dummy weight pointers."""

    def __init__(self, L, nB=B, window=W, dm=DM):
        self.L, self.B = L, nB
        self.dims = pp.make_dims(dm)
        n = ctypes.c_size_t()
        assert L.pp_arena_bytes(ctypes.byref(self.dims), nB, window, ctypes.byref(n)) == 0
        self.buf = np.zeros(n.value + 256, np.uint8)
        self.arena = (self.buf.ctypes.data + 255) // 256 * 256
        self.nbytes = n.value
        self.wbuf = np.zeros(64, np.uint8)  # never read by the stub launchers
        self.w = pp.PPWeights(**{f: self.wbuf.ctypes.data for f in pp.WEIGHT_FIELDS})
        h = ctypes.c_void_p()
        rc = L.pp_create(ctypes.byref(self.dims), nB, window, ctypes.byref(self.w), self.arena, self.nbytes, None,
                         ctypes.byref(h))
        assert rc == 0, L.pp_last_error(None)
        self.h = h.value

    def step(self, codes):
        c = np.ascontiguousarray(codes, np.int32).reshape(self.B, 8)
        tok = np.zeros((self.B, 9), np.int32)
        rc = self.L.pp_step(self.h, c.ctypes.data, tok.ctypes.data)
        return rc, tok

    def ti(self):
        out = np.zeros(self.B * TI_STRIDE, np.int32)
        assert self.L.stub_last_tick_input(out.ctypes.data, out.size) == out.size
        return out.reshape(self.B, TI_STRIDE)

    def prefill(self, slot, frames):
        f = np.ascontiguousarray(frames, np.int32).reshape(-1, 17)
        return self.L.pp_prefill_forced(self.h, slot, f.ctypes.data, f.shape[0])

    def fill(self, slot, n, null=False):
        shape = (DM.n_layers, n, DM.n_heads, DM.head_dim)
        k = np.zeros(shape, np.uint16)
        return self.L.pp_ring_fill(self.h, slot, n, None if null else k.ctypes.data, None if null else k.ctypes.data)

    def close(self):
        self.L.pp_destroy(self.h)


def pred(pos, step, n):
    return (7 * pos + 13 * (step + 1) + 5) % n


def preds(pos):
    return np.array([pred(pos, -1, VT)] + [pred(pos, k, A) for k in range(8)], np.int32)


def codes(seed, n=1, nB=B):
    return np.random.default_rng(seed).integers(0, A, (n, nB, 8)).astype(np.int32)


def test_fresh_slots_and_feedback(lib):
    h = Handle(lib)
    c = codes(1, 4)
    for t in range(4):
        rc, tok = h.step(c[t])
        assert rc == 0
        ti = h.ti()
        for b in range(B):
            assert ti[b, TI_POS] == t
            prev = [VT] + [A] * 8 if t == 0 else list(preds(t - 1))
            np.testing.assert_array_equal(ti[b, TI_COL:TI_COL + 9], prev)
            np.testing.assert_array_equal(ti[b, TI_COL + 9:TI_COL + 17], c[t, b])
            np.testing.assert_array_equal(ti[b, TI_FORCE:TI_FORCE + 9], -1)
            np.testing.assert_array_equal(tok[b], preds(t))
    h.close()


def test_forced_frames_in_order_then_free_running(lib):
    h = Handle(lib)
    fr = np.full((3, 17), -1, np.int32)
    fr[:, 9:] = codes(2, 3, 1).reshape(3, 8)
    fr[0, 1:9] = [11, 12, 13, 14, 15, 16, 17, 18]   # voice frame: agent rows forced
    fr[1, 0] = 42                                    # persona frame: text row forced
    assert h.prefill(1, fr) == 0
    c = codes(3, 5)
    expect = [fr[0], fr[1], fr[2], fr[0]]   # fr[0] is queued again during tick 2's opening
    for t in range(5):
        assert h.step(c[t])[0] == 0
        ti = h.ti()[1]
        if t < len(expect):
            np.testing.assert_array_equal(ti[TI_COL + 9:TI_COL + 17], expect[t][9:])   # the frame's user rows
            np.testing.assert_array_equal(ti[TI_FORCE:TI_FORCE + 9], expect[t][:9])
        else:
            np.testing.assert_array_equal(ti[TI_COL + 9:TI_COL + 17], c[t, 1])
            np.testing.assert_array_equal(ti[TI_FORCE:TI_FORCE + 9], -1)
        if 1 <= t <= len(expect):   # the column carries the previous tick's choices: forced where forced
            chosen = np.where(expect[t - 1][:9] >= 0, expect[t - 1][:9], preds(t - 1))
            np.testing.assert_array_equal(ti[TI_COL:TI_COL + 9], chosen)
        if t == 2:
            assert h.prefill(1, fr[:1]) == 0          # still opening: the queue is not empty
    # tick 4 ran with an empty queue, so the slot is free-running
    assert h.prefill(1, fr[:1]) == pp.PP_EBUSY
    assert h.fill(1, 2) == pp.PP_EBUSY
    h.close()


def test_errors_leave_state_unchanged(lib):
    """Every rejected call on handle a is absent from handle b; the two must
    then see identical tick inputs and tokens."""
    a, b = Handle(lib), Handle(lib)
    good = np.full((2, 17), -1, np.int32)
    good[:, 9:] = 5
    c = codes(4, 6)
    for hh in (a, b):
        assert hh.prefill(2, good) == 0
    runs_before = lib.stub_ticks_run()
    # rejected calls on a
    bad_codes = c[0].copy()
    bad_codes[1, 4] = A
    assert a.step(bad_codes)[0] == pp.PP_EINVAL
    neg = c[0].copy()
    neg[0, 0] = -1
    assert a.step(neg)[0] == pp.PP_EINVAL
    assert lib.stub_ticks_run() == runs_before          # no tick ran
    assert lib.pp_slot_reset(a.h, B) == pp.PP_EINVAL
    assert lib.pp_slot_reset(a.h, -1) == pp.PP_EINVAL
    bad = good.copy()
    bad[1, 0] = VT                                     # text token out of range (valid: -1..Vt-1)
    assert a.prefill(0, bad) == pp.PP_EINVAL
    bad = good.copy()
    bad[0, 12] = -1                                    # user rows may not be free
    assert a.prefill(0, bad) == pp.PP_EINVAL
    assert a.prefill(0, np.zeros((0, 17))) == 0       # an empty prefill is a no-op
    assert lib.pp_prefill_forced(a.h, 0, None, 1) == pp.PP_EINVAL
    big = np.tile(good[:1], (pp.PP_MAX_QUEUE, 1))
    assert a.prefill(2, big) == pp.PP_ENOSPC           # 2 queued + 4096 > PP_MAX_QUEUE
    assert a.fill(0, W + 1) == pp.PP_EINVAL
    assert a.fill(0, 3, null=True) == pp.PP_EINVAL
    assert a.fill(2, 3) == pp.PP_EBUSY                 # slot 2 has queued frames
    assert lib.pp_set_acoustic_delay(a.h, 5) == pp.PP_EINVAL
    tok = np.zeros((B, 9), np.int32)
    assert lib.pp_step(a.h, None, tok.ctypes.data) == pp.PP_EINVAL
    for t in range(6):
        ra, ta = a.step(c[t])
        tia = a.ti()        # the stub keeps the last tick input of the process
        rb, tb = b.step(c[t])
        np.testing.assert_array_equal(tia, b.ti())
        assert ra == rb == 0
        np.testing.assert_array_equal(ta, tb)
        if t == 0:
            assert lib.pp_set_acoustic_delay(a.h, 1) == pp.PP_EBUSY   # slots have ticked
    a.close()
    b.close()


def test_fill_sets_position_and_reset_equals_fresh(lib):
    h = Handle(lib)
    assert h.fill(0, 5) == 0
    assert h.fill(0, 5) == 0                            # refilling before any tick is allowed
    c = codes(5, 4)
    h.step(c[0])
    assert h.ti()[0, TI_POS] == 5 and h.ti()[1, TI_POS] == 0
    assert h.fill(0, 2) == pp.PP_EBUSY                  # after a tick
    h.step(c[1])
    fr = np.full((1, 17), -1, np.int32)
    fr[0, 9:] = 7
    assert h.prefill(0, fr) == pp.PP_EBUSY              # live
    assert lib.pp_slot_reset(h.h, 0) == 0
    assert h.prefill(0, fr) == 0                        # open again
    assert lib.pp_slot_reset(h.h, 0) == 0               # reset clears the queue
    assert h.fill(0, 3) == 0
    h.step(c[2])
    f = Handle(lib)
    assert f.fill(0, 3) == 0
    f.step(c[2])
    ti_f = f.ti()[0]
    h.step(c[3])
    f2 = h.ti()[0]
    f.step(c[3])
    np.testing.assert_array_equal(f2, f.ti()[0])        # recycled slot 0 == fresh slot 0
    assert ti_f[TI_POS] == 3 and list(ti_f[TI_COL:TI_COL + 9]) == [VT] + [A] * 8
    h.close()
    f.close()


def test_acoustic_delay_rows(lib):
    h = Handle(lib)
    assert lib.pp_set_acoustic_delay(h.h, 1) == 0
    c = codes(6, 3)
    fr_seen = []
    for t in range(3):
        h.step(c[t])
        fr_seen.append(h.ti().copy())
    for b in range(B):
        # codebook 0 of the user frame is on time; codebooks 1-7 come one tick later
        assert fr_seen[0][b, TI_COL + 9] == c[0, b, 0]
        np.testing.assert_array_equal(fr_seen[0][b, TI_COL + 10:TI_COL + 17], A)
        for t in (1, 2):
            assert fr_seen[t][b, TI_COL + 9] == c[t, b, 0]
            np.testing.assert_array_equal(fr_seen[t][b, TI_COL + 10:TI_COL + 17], c[t - 1, b, 1:])
    frames = np.zeros((B, 8), np.int32)
    valid = np.zeros(B, np.int32)
    assert lib.pp_agent_frames(h.h, frames.ctypes.data, valid.ctypes.data) == 0
    assert valid.all()
    # frame 1: codebook 0 chosen at tick 1, codebooks 1-7 chosen at tick 2
    np.testing.assert_array_equal(frames[0], np.concatenate([preds(1)[1:2], preds(2)[2:9]]))
    h.close()


def test_device_error_poisons_the_handle(lib):
    h = Handle(lib)
    c = codes(7, 2)
    assert h.step(c[0])[0] == 0
    lib.stub_fail_launches(1)
    assert h.step(c[1])[0] == pp.PP_EDEVICE
    assert b"hipGraphLaunch" in lib.pp_last_error(h.h) or lib.pp_last_error(h.h)
    assert h.step(c[1])[0] == pp.PP_EDEVICE
    assert lib.pp_slot_reset(h.h, 0) == pp.PP_EDEVICE
    assert h.prefill(0, np.full((1, 17), 0, np.int32)) == pp.PP_EDEVICE
    h.close()


def test_create_arguments(lib):
    dims = pp.make_dims(DM)
    n = ctypes.c_size_t()
    assert lib.pp_arena_bytes(ctypes.byref(dims), 0, W, ctypes.byref(n)) == pp.PP_EINVAL
    assert lib.pp_arena_bytes(ctypes.byref(dims), pp.PP_MAX_BATCH + 1, W, ctypes.byref(n)) == pp.PP_EINVAL
    assert lib.pp_arena_bytes(ctypes.byref(dims), 1, pp.PP_MAX_WINDOW + 1, ctypes.byref(n)) == pp.PP_EINVAL
    assert lib.pp_arena_bytes(ctypes.byref(dims), 2, W, ctypes.byref(n)) == 0
    buf = np.zeros(n.value + 512, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    wbuf = np.zeros(64, np.uint8)
    w = pp.PPWeights(**{f: wbuf.ctypes.data for f in pp.WEIGHT_FIELDS})
    h = ctypes.c_void_p()
    assert lib.pp_create(ctypes.byref(dims), 2, W, ctypes.byref(w), base, n.value - 1, None,
                         ctypes.byref(h)) == pp.PP_ENOSPC
    assert lib.pp_create(ctypes.byref(dims), 2, W, ctypes.byref(w), base + 16, n.value, None,
                         ctypes.byref(h)) == pp.PP_EINVAL                       # not 256-byte aligned
    w0 = pp.PPWeights(**{f: wbuf.ctypes.data for f in pp.WEIGHT_FIELDS})
    w0.dep_heads = None
    assert lib.pp_create(ctypes.byref(dims), 2, W, ctypes.byref(w0), base, n.value, None,
                         ctypes.byref(h)) == pp.PP_EINVAL
    bad = pp.make_dims(DM)
    bad.n_q = 7
    assert lib.pp_create(ctypes.byref(bad), 2, W, ctypes.byref(w), base, n.value, None,
                         ctypes.byref(h)) == pp.PP_EINVAL
    assert lib.pp_create(ctypes.byref(dims), 2, W, ctypes.byref(w), base, n.value, None, ctypes.byref(h)) == 0
    lib.pp_destroy(h.value)


def test_step_static_same_state_machine_and_size_limit(lib):
    """pp_step_static gives the ticks pp_step gives; a handle whose work
    buffers exceed PP_STATIC_SCRATCH_BYTES is refused with PP_ENOSPC and no
    state change (B = 9 with a 70000-token text head: 70 MB of partials)."""
    lib.pp_step_static.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.pp_step_static.restype = ctypes.c_int
    a, b = Handle(lib), Handle(lib)
    c = codes(8, 3)
    tok = np.zeros((B, 9), np.int32)
    for t in range(3):
        cc = np.ascontiguousarray(c[t])
        assert lib.pp_step_static(a.h, cc.ctypes.data, tok.ctypes.data) == 0
        tia = a.ti()
        rb, tb = b.step(c[t])
        np.testing.assert_array_equal(tok, tb)
        np.testing.assert_array_equal(tia, b.ti())
    a.close()
    b.close()
    import dataclasses
    big = dataclasses.replace(DM, text_card=70000)
    dims = pp.make_dims(big)
    n = ctypes.c_size_t()
    assert lib.pp_arena_bytes(ctypes.byref(dims), 9, W, ctypes.byref(n)) == 0
    buf = np.zeros(n.value + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    wbuf = np.zeros(64, np.uint8)
    w = pp.PPWeights(**{f: wbuf.ctypes.data for f in pp.WEIGHT_FIELDS})
    h = ctypes.c_void_p()
    assert lib.pp_create(ctypes.byref(dims), 9, W, ctypes.byref(w), base, n.value, None, ctypes.byref(h)) == 0
    cc = np.zeros((9, 8), np.int32)
    tok = np.zeros((9, 9), np.int32)
    runs = lib.stub_ticks_run()
    assert lib.pp_step_static(h.value, cc.ctypes.data, tok.ctypes.data) == pp.PP_ENOSPC
    assert b"static array" in lib.pp_last_error(h.value)
    assert lib.stub_ticks_run() == runs
    assert lib.pp_step(h.value, cc.ctypes.data, tok.ctypes.data) == 0
    out = np.zeros(9 * TI_STRIDE, np.int32)
    lib.stub_last_tick_input(out.ctypes.data, out.size)
    assert out[TI_POS] == 0      # the refused call did not advance the slot
    lib.pp_destroy(h.value)


def test_fused_loop_toggle_same_state_machine(lib):
    """pp_set_depformer_loop: off by default; refused with PP_EINVAL and no
    change where the fused loop cannot apply (3 slots; a depformer width that
    is not a multiple of 256); where it applies, ticks give the tokens and
    tick inputs of the per-layer launches, with forced frames, taps between
    ticks (which launch the pending user half on its own) and the loop turned
    off and on between ticks; an error code left by a loop launch poisons the
    handle (PP_EDEVICE)."""
    import dataclasses
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.pp_set_depformer_loop.argtypes = [P, I]
    lib.pp_set_depformer_loop.restype = I
    lib.pp_depformer_loop_active.argtypes = [P]
    lib.pp_depformer_loop_active.restype = I
    lib.pp_taps.argtypes = [P, ctypes.POINTER(pp.PPTaps)]
    lib.pp_taps.restype = I
    lib.stub_loop_text_card.argtypes = [I]
    lib.stub_loop_error.argtypes = [I]
    lib.stub_loop_launches.restype = ctypes.c_long
    lib.stub_loop_text_card(VT)

    h3 = Handle(lib)
    assert lib.pp_depformer_loop_active(h3.h) == 0
    assert lib.pp_set_depformer_loop(h3.h, 1) == pp.PP_EINVAL
    assert lib.pp_depformer_loop_active(h3.h) == 0
    assert lib.pp_set_depformer_loop(h3.h, 0) == 0
    h3.close()
    h1 = Handle(lib, nB=1)  # depformer width 128
    assert lib.pp_set_depformer_loop(h1.h, 1) == pp.PP_EINVAL
    assert b"fused depformer loop" in lib.pp_last_error(h1.h)
    h1.close()

    small = dataclasses.replace(DM, dep_d=256, dep_heads=8, dep_ffn=768, dep_layers=2)
    a, b = Handle(lib, nB=2, dm=small), Handle(lib, nB=2, dm=small)
    assert lib.pp_depformer_loop_active(a.h) == 0
    assert lib.pp_set_depformer_loop(a.h, 1) == 0
    assert lib.pp_depformer_loop_active(a.h) == 1
    rng = np.random.default_rng(3)
    fr = np.full((2, 17), -1, np.int32)
    fr[:, 1:9] = rng.integers(0, A, (2, 8))
    fr[:, 9:] = rng.integers(0, A, (2, 8))
    fr[1, 0] = 17
    for h in (a, b):
        assert h.prefill(1, fr) == 0
    c = codes(11, 8, 2)
    n0 = lib.stub_loop_launches()
    taps = pp.PPTaps()
    for t in range(7):
        if t == 3:
            assert lib.pp_set_depformer_loop(a.h, 0) == 0
            assert lib.pp_depformer_loop_active(a.h) == 0
        if t == 5:
            assert lib.pp_set_depformer_loop(a.h, 1) == 0
        ra, ta = a.step(c[t])
        rb, tb = b.step(c[t])
        assert ra == 0 and rb == 0
        np.testing.assert_array_equal(ta, tb, err_msg=f"tick {t}")
        np.testing.assert_array_equal(a.ti(), b.ti(), err_msg=f"tick {t}")
        if t in (1, 5):
            assert lib.pp_taps(a.h, ctypes.byref(taps)) == 0
    assert lib.stub_loop_launches() - n0 >= 5
    lib.stub_loop_error(2)
    assert a.step(c[7])[0] == pp.PP_EDEVICE
    assert b"fused depformer loop" in lib.pp_last_error(a.h)
    assert a.step(c[7])[0] == pp.PP_EDEVICE
    a.close()
    b.close()
