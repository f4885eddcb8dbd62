"""The library's draft-depth controller (host code, no GPU) against the
oracle: the chosen depth and every rate match exactly on random acceptance
profiles and cost curves, the per-position estimator matches on random
step sequences, and bad arguments are refused."""
import ctypes

import numpy as np
import pytest

import bit_verify_gemm_amd as bv
import oracle


def test_choice_matches_oracle():
    rng = np.random.default_rng(4)
    for trial in range(500):
        dmax = int(rng.integers(0, 64))
        a = rng.random(dmax) ** rng.uniform(0.1, 2)
        # cost per step: a fixed part and a part growing with the width
        cost = rng.uniform(0.5, 2) + rng.uniform(0, 0.3) * np.arange(dmax + 1) ** rng.uniform(0.5, 1.5)
        d, r = bv.choose_draft_depth(a, cost)
        do, ro = oracle.choose_draft_depth(a, cost)
        assert d == do and np.array_equal(r, ro), trial


def test_choice_on_a_measured_curve():
    # microseconds per verify pass at M = 1, 2, 4, 8 (nvfp4 4096 x 14336),
    # linear in between, plus 3 us of drafting per draft token
    m_us = {1: 8.42, 2: 8.48, 4: 8.65, 8: 9.49}
    verify = np.interp(np.arange(1, 9), list(m_us), list(m_us.values()))
    cost = verify + 3.0 * np.arange(8)
    for a in (0.3, 0.6, 0.9):
        d, r = bv.choose_draft_depth(np.full(7, a), cost)
        assert (d, r.tolist()) == (oracle.choose_draft_depth(np.full(7, a), cost)[0], r.tolist())
        assert r[d] >= r[0]          # never worse than plain decoding


def test_estimator_matches_oracle():
    rng = np.random.default_rng(9)
    for keep in (1.0, 0.9):
        s = bv.DepthStats(10, keep)
        ro, ao = np.zeros(10), np.zeros(10)
        for _ in range(300):
            depth = int(rng.integers(0, 11))
            acc = int(rng.integers(0, depth + 1))
            s.observe(depth, acc)
            oracle.depth_observe(ro, ao, depth, acc, keep)
        assert np.array_equal(s.reached, ro) and np.array_equal(s.accepted, ao)
        assert np.array_equal(s.estimate(), oracle.depth_estimate(ro, ao))


def test_bad_arguments():
    L = bv.lib()
    c = np.ones(3)
    a = np.full(2, 0.5)
    P = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert L.mtp_choose_draft_depth(P(a), None, 2, None) == -1
    assert L.mtp_choose_draft_depth(P(a), P(c), 64, None) == -2
    assert L.mtp_choose_draft_depth(P(a), P(c), -1, None) == -2
    assert L.mtp_choose_draft_depth(P(np.array([0.5, 1.5])), P(c), 2, None) == -7
    assert L.mtp_choose_draft_depth(P(a), P(np.array([1.0, 0.0, 1.0])), 2, None) == -7
    assert L.mtp_choose_draft_depth(P(a), P(np.array([1.0, np.nan, 1.0])), 2, None) == -7
    assert L.mtp_choose_draft_depth(None, P(c[:1]), 0, None) == 0   # plain decoding only
    r = np.zeros(2)
    assert L.mtp_depth_observe(P(r), P(r), 2, 3, 0, ctypes.c_double(1.0)) == 0
    assert L.mtp_depth_observe(P(r), P(r), 2, 1, 2, ctypes.c_double(1.0)) == -2
    assert L.mtp_depth_observe(P(r), P(r), 2, 1, 0, ctypes.c_double(1.5)) == -7
    assert L.mtp_depth_estimate(P(r), P(r), 0, P(r)) == -2
