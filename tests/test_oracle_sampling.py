"""Pins of the sampling variant's CPU oracle: the counter-based generator
against its published known-answer vectors, the sampler against brute-force
definitions and library routines, and the tick with sampling against its
greedy special case."""
import os

import numpy as np
import pytest
import scipy.special

from full_duplex_speech_moshi_amd import synth
from oracle import sampling as sm
from oracle.tick import Oracle

DM = synth.TINY
W = synth.TINY_WINDOW


def test_philox4x32_10_known_answers():
    """Known-answer vectors published with the Random123 reference
    implementation of Philox4x32-10 (Salmon et al., SC 2011), stored with
    their citation in tests/golden/philox4x32_10_kat.txt: counter and key all
    zeros, all ones, and the hexadecimal digits of pi."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.txt")
    kat = []
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if line:
            words = [int(w, 16) for w in line]
            kat.append((words[0:4], words[4:6], words[6:10]))
    assert len(kat) == 3
    for ctr, key, want in kat:
        assert sm.philox4x32_10(ctr, key) == want


def test_uniform_draws():
    us = [sm.uniform(s, t, r) for s in (0, 1, 2 ** 40 + 3) for t in (0, 1, 2 ** 33) for r in range(17)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(np.float32(u)) == u and (u * 2 ** 24) == int(u * 2 ** 24) for u in us)
    assert len(set(us)) == len(us)          # seed, tick (both 32-bit halves) and row all enter the counter/key


def _grid(n):
    return (np.arange(n) + 0.5) / n


def test_top_k_1_and_zero_temperature_are_greedy():
    rng = np.random.default_rng(0)
    for _ in range(20):
        z = rng.standard_normal(300).astype(np.float32)
        z[rng.integers(0, 300)] = z.max()    # a tie for the maximum: the lower index wins
        g = int(np.argmax(z))
        assert sm.sample(z, 0.37, 0.0) == g
        for u in (0.0, 0.5, 0.999):
            assert sm.sample(z, u, 1.3, top_k=1) == g


def test_inverse_cdf_frequencies_equal_softmax():
    """Over a fine grid of u the sampler's frequencies are the softmax of
    z / T (to the grid's resolution): the inverse CDF is exact."""
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4], np.float32)
    T = 0.7
    N = 200_000
    counts = np.bincount([sm.sample(z, u, T) for u in _grid(N)], minlength=z.size)
    np.testing.assert_allclose(counts / N, scipy.special.softmax(z.astype(np.float64) / T), atol=2.0 / N + 1e-6)


def _brute_top_k(z, k):
    order = sorted(range(z.size), key=lambda i: (-float(z[i]), i))
    return set(order[:k])


def _brute_top_p(z, keep, top_p):
    idx = sorted(keep, key=lambda i: (-float(z[i]), i))
    p = scipy.special.softmax(np.array([float(z[i]) for i in idx], np.float64))
    out, c = set(), 0.0
    for i, pi in zip(idx, p):
        out.add(i)
        c += pi
        if c >= top_p:
            break
    return out, np.cumsum(p)


def test_top_k_top_p_kept_sets_equal_brute_force():
    rng = np.random.default_rng(1)
    N = 4000
    for trial in range(12):
        n = int(rng.integers(5, 60))
        z = np.round(rng.standard_normal(n) * 2, 1).astype(np.float32)   # coarse values: ties occur
        k = int(rng.integers(0, n + 2))
        top_p = float(rng.choice([1.0, 0.9, 0.5, 0.2]))
        keep = _brute_top_k(z, k) if 0 < k < n else set(range(n))
        kept, cum = _brute_top_p(z, keep, top_p)
        if top_p < 1.0 and np.min(np.abs(cum - top_p)) < 1e-4:
            continue                                                      # boundary too close to call
        seen = {sm.sample(z, u, 1.0, top_k=k, top_p=top_p) for u in _grid(N)}
        assert seen == kept, (trial, sorted(seen), sorted(kept))


def test_repetition_penalty_closed_form():
    z = np.array([2.0, -1.0, 1.5, 0.5, -3.0], np.float32)
    zp = sm.penalise(z, [0, 1, 1, 4], 1.25)
    np.testing.assert_array_equal(zp, np.array([1.6, -1.25, 1.5, 0.5, -3.75], np.float32))
    # greedy under the penalty: token 0 (2.0 / 1.25 = 1.6) still beats 1.5; with 1.5 it does not
    assert sm.sample(z, 0.5, 0.0, rho=1.25, history=[0]) == 0
    assert sm.sample(z, 0.5, 0.0, rho=1.5, history=[0]) == 2


def test_tick_with_top_k_1_equals_greedy_tick(tiny_weights):
    codes = synth.user_codes(1, 4)
    og = Oracle(DM, tiny_weights, 1, W)
    os_ = Oracle(DM, tiny_weights, 1, W)
    os_.set_sampling(0.8, 0.3, top_k=1)
    os_.slot_seed(0, 99)
    for t in range(4):
        np.testing.assert_array_equal(og.step(codes[t:t + 1]), os_.step(codes[t:t + 1]))
        for k in ("hidden", "text_logits", "dep_logits", "chosen", "user_pred"):
            np.testing.assert_array_equal(og.taps[k], os_.taps[k])


def test_tick_sampling_reproducible_isolated_and_seeded(tiny_weights):
    """Same seed: same tokens; a B = 2 run equals two B = 1 runs with the
    slots' seeds; a reset slot draws again from tick 0; another seed differs."""
    codes = synth.user_codes(2, 6)

    def run(B, seeds, t0=0, n=6, reset_at=None):
        o = Oracle(DM, tiny_weights, B, W)
        o.set_sampling(1.0, 1.0, top_p=0.95, rho=1.1)
        for b, sd in enumerate(seeds):
            o.slot_seed(b, sd)
        out = []
        for t in range(t0, t0 + n):
            if reset_at is not None and t == reset_at:
                o.slot_reset(0)
            out.append(o.step(np.repeat(codes[t:t + 1], B, 0)))
        return np.stack(out)

    a = run(2, [5, 7])
    np.testing.assert_array_equal(a[:, 0], run(1, [5])[:, 0])
    np.testing.assert_array_equal(a[:, 1], run(1, [7])[:, 0])
    assert not np.array_equal(a[:, 0], a[:, 1])
    # recycle = fresh: after a reset at tick 3 the slot equals a fresh one fed codes 3..5
    np.testing.assert_array_equal(run(1, [5], reset_at=3)[3:, 0], run(1, [5], t0=3, n=3)[:, 0])
