"""Pins for the oracle's draft-depth controller.

Ollama mtp.go commit log: the controller drafts the depth that maximises
committed tokens per wall-clock from live per-position acceptance and the
per-width forward cost; MTPLX blog post: plain decoding stays the baseline.
Pinned against a hand-worked case, the closed form of the expected committed
tokens for a constant acceptance rate (a geometric series), a simulation of
the committed run, the degenerate cases, and a hand-worked run of the
per-position estimator.
"""
import numpy as np
import pytest

import oracle


def test_hand_worked_choice():
    # a = .9, .5: E = 1, 1.9, 2.35; rates with costs 1, 1.2, 1.3:
    # 1, 1.5833, 1.8077 -> depth 2; with cost[2] = 1.5, 1.5667 < 1.5833 -> depth 1
    d, r = oracle.choose_draft_depth([0.9, 0.5], [1.0, 1.2, 1.3])
    assert d == 2 and np.allclose(r, [1.0, 1.9 / 1.2, 2.35 / 1.3], rtol=1e-15)
    d, r = oracle.choose_draft_depth([0.9, 0.5], [1.0, 1.2, 1.5])
    assert d == 1


@pytest.mark.parametrize("a", [0.0, 0.3, 0.77, 0.99])
def test_constant_rate_closed_form(a):
    dmax = 12
    cost = np.ones(dmax + 1)
    _, r = oracle.choose_draft_depth(np.full(dmax, a), cost)
    d = np.arange(dmax + 1)
    e = 1 + (a * (1 - a ** d) / (1 - a) if a < 1 else d)
    assert np.allclose(r, e, rtol=1e-13)


def test_expected_tokens_match_a_simulated_run():
    rng = np.random.default_rng(1)
    a = np.array([0.9, 0.8, 0.6, 0.5, 0.3])
    _, r = oracle.choose_draft_depth(a, np.ones(6))
    n = 200000
    acc = rng.random((n, 5)) < a          # per-position acceptance given the ones before
    run = np.argmin(np.concatenate([acc, np.zeros((n, 1), bool)], axis=1), axis=1)  # leading accepts
    for d in range(6):
        committed = np.minimum(run, d) + 1
        se = committed.std() / np.sqrt(n)
        assert abs(committed.mean() - r[d]) < 4 * se + 1e-12


def test_degenerate_cases():
    # nothing is ever accepted: plain decoding
    assert oracle.choose_draft_depth(np.zeros(8), np.linspace(1, 2, 9))[0] == 0
    # everything is accepted and a step costs the same at every width: deepest
    assert oracle.choose_draft_depth(np.ones(8), np.ones(9))[0] == 8
    # everything accepted, cost proportional to the width: all rates equal,
    # the smallest depth wins the tie
    assert oracle.choose_draft_depth(np.ones(8), np.arange(1, 10, dtype=float))[0] == 0
    with pytest.raises(ValueError):
        oracle.choose_draft_depth([0.5], [1.0, 0.0])
    with pytest.raises(ValueError):
        oracle.choose_draft_depth([1.5], [1.0, 1.0])


def test_estimator_hand_worked():
    reached, accepted = np.zeros(3), np.zeros(3)
    # depth 3, 1 accepted: positions 1, 2 reached, position 1 accepted
    oracle.depth_observe(reached, accepted, 3, 1)
    # depth 2, 2 accepted: positions 1, 2 reached and accepted
    oracle.depth_observe(reached, accepted, 2, 2)
    # depth 3, 0 accepted: position 1 reached
    oracle.depth_observe(reached, accepted, 3, 0)
    assert np.array_equal(reached, [3, 2, 0]) and np.array_equal(accepted, [2, 1, 0])
    assert np.allclose(oracle.depth_estimate(reached, accepted), [3 / 5, 2 / 4, 1 / 2])
    # decay: counts are multiplied by keep before each step's evidence
    oracle.depth_observe(reached, accepted, 1, 1, keep=0.5)
    assert np.allclose(reached, [2.5, 1, 0]) and np.allclose(accepted, [2, 0.5, 0])
