"""Pins for the oracle's sampled acceptance (the full sampler pipeline).

Ollama mtp.go commit log, the MLX sampler rework: penalties -> top-k ->
temperature/softmax -> top-p -> min-p -> normalize -> categorical, with the
target (and draft) distributions reused for acceptance, residual and bonus
draws.  Pinned against: worked examples whose cut positions and
probabilities are derived by hand from the readings stated in oracle.c,
reductions to the greedy and the plain rejection oracles (each pinned on its
own), and the distribution law of Leviathan/Chen rejection sampling (the
committed tokens follow the target distribution) by chi-square tests.
"""
import numpy as np
import pytest
from scipy import stats

import oracle

S = oracle.sampler


def one(z, params, **kw):
    """Target p' of a single row (B = M = 1)."""
    z = np.asarray(z, np.float32)[None, None, :]
    u = np.array([[0.5]], np.float32)
    _, _, _, tp = oracle.accept_sampled(z, np.zeros((1, 0), np.int32), u, params,
                                        with_target=True, **kw)
    return tp[0, 0]


def test_cuts_worked_example():
    # weights 8, 4, 2, 1, 1, 0.5 as logits ln(w) at T = 1: e = 1, .5, .25,
    # .125, .125, .0625 (ties at e = .125 ranked by index)
    w = np.array([8, 4, 2, 1, 1, 0.5])
    z = np.log(w).astype(np.float32)
    # top-k 5 keeps ids 0..4 (id 5 is last); sum of e = 2.0
    p = one(z, S(top_k=5))
    assert p[5] == 0.0 and np.allclose(p[:5], np.array([8, 4, 2, 1, 1]) / 16, rtol=1e-6)
    # top-p 0.8 of 2.0 = 1.6: cumulative 1, 1.5, 1.75 -> ids 0..2, mass 1.75
    p = one(z, S(top_k=5, top_p=0.8))
    assert np.allclose(p, np.array([8, 4, 2, 0, 0, 0]) / 14, rtol=1e-6, atol=0)
    # top-p measures mass within the top-k set: top-k 2 has mass 1.5, so
    # top-p 0.6 (threshold 0.9) keeps id 0 alone (over all six entries the
    # threshold would be 1.2375 and id 1 would stay)
    p = one(z, S(top_k=2, top_p=0.6))
    assert p[0] == 1.0 and np.count_nonzero(p) == 1
    # then min-p 0.3 drops e = .25: ids 0, 1 -> 2/3, 1/3
    p = one(z, S(top_k=5, top_p=0.8, min_p=0.3))
    assert np.allclose(p, [2 / 3, 1 / 3, 0, 0, 0, 0], rtol=1e-6, atol=0)
    # min-p alone at 0.125 keeps both tied entries (e = .125 is not below it)
    p = one(z, S(min_p=0.124))
    assert np.count_nonzero(p) == 5
    # top-k 4 splits the tie by index: id 3 stays, id 4 goes
    p = one(z, S(top_k=4))
    assert p[3] > 0 and p[4] == 0
    # min-p above 1 still keeps the first entry
    p = one(z, S(min_p=3.0))
    assert p[0] == 1.0 and np.count_nonzero(p) == 1


def test_penalties_worked_example():
    # logits 2, -1, 0.5, 3; history 0, 0, 1; repeat 2, frequency .25, presence .5:
    # id 0 (seen twice): 2 / 2 = 1, 1 - 2 * .25 = .5, .5 - .5 = 0
    # id 1 (seen once): -1 * 2 = -2, -2 - .25 = -2.25, -2.25 - .5 = -2.75
    z = [2.0, -1.0, 0.5, 3.0]
    par = S(repeat_penalty=2.0, frequency_penalty=0.25, presence_penalty=0.5, penalty_last_n=64)
    p = one(z, par, history=[[0, 0, 1]])
    zp = np.array([0.0, -2.75, 0.5, 3.0])
    ref = np.exp(zp - zp.max())
    assert np.allclose(p, ref / ref.sum(), rtol=1e-12)
    # a window of the last 1 token sees only id 1
    p = one(z, dict(par, penalty_last_n=1), history=[[0, 0, 1]])
    zp = np.array([2.0, -2.75, 0.5, 3.0])
    ref = np.exp(zp - zp.max())
    assert np.allclose(p, ref / ref.sum(), rtol=1e-12)


def test_penalty_window_takes_the_drafts_before_each_row():
    # rows 0 and 1 share their logits; history [3], draft 0 = 3: row 0 counts
    # id 3 once, row 1 twice, so with a frequency penalty of .5 alone the
    # log-odds of id 3 against id 0 drop by exactly .5 from row 0 to row 1
    z = np.array([[[1.0, 0.0, 0.0, 1.0]] * 2], np.float32)
    par = S(frequency_penalty=0.5, penalty_last_n=8)
    q = np.full((1, 1, 4), 0.25, np.float32)
    _, _, _, tp = oracle.accept_sampled(z, np.array([[3]], np.int32),
                                        np.array([[0.5, 0.5]], np.float32), par, q=q,
                                        history=[[3]], with_target=True)
    lo0 = np.log(tp[0, 0, 3] / tp[0, 0, 0])
    lo1 = np.log(tp[0, 1, 3] / tp[0, 1, 0])
    assert abs(lo0 - (-0.5)) < 1e-12 and abs(lo1 - (-1.0)) < 1e-12


def penalised(z, window, rp, fp, pp):
    z = np.array(z, np.float32)
    for t in set(window):
        c = window.count(t)
        x = np.float32(z[t])
        if rp != 1.0:
            x = np.float32(x / np.float32(rp)) if x > 0 else np.float32(x * np.float32(rp))
        x = np.float32(x - np.float32(np.float32(c) * np.float32(fp)))
        z[t] = np.float32(x - np.float32(pp))
    return z


@pytest.mark.parametrize("how", ["top_k1", "t0", "min_p"])
def test_point_mass_cases_are_greedy_on_penalised_logits(how):
    rng = np.random.default_rng(3)
    B, M, V = 3, 4, 50
    z = rng.integers(-3, 4, size=(B, M, V)).astype(np.float32)   # ties
    hist = [list(rng.integers(0, V, 5)) for _ in range(B)]
    par = dict(S(repeat_penalty=1.3, frequency_penalty=0.2, presence_penalty=0.1,
                 penalty_last_n=6, top_p=0.9, temperature=0.7))
    par.update(top_k=1) if how == "top_k1" else par.update(temperature=0.0) if how == "t0" \
        else par.update(min_p=2.0)
    drafts = np.zeros((B, M - 1), np.int32)
    for b in range(B):
        # drafts follow greedy decoding of the penalised rows until position b
        ctx = list(hist[b])
        for i in range(M - 1):
            zp = penalised(z[b, i], ctx[-6:], 1.3, 0.2, 0.1)
            g = int(np.flatnonzero(zp == zp.max())[0])
            drafts[b, i] = g if i < b + 1 else (g + 1) % V
            ctx.append(int(drafts[b, i]))
    q = rng.dirichlet(np.ones(V), size=(B, M - 1)).astype(np.float32)
    u = rng.random((B, M)).astype(np.float32)
    tok, cnt, rb = oracle.accept_sampled(z, drafts, u, par, q=q, history=hist,
                                         base_len=np.array([10, 20, 30]))
    for b in range(B):
        ctx = list(hist[b])
        rows = []
        for i in range(M):
            zp = penalised(z[b, i], ctx[-6:], 1.3, 0.2, 0.1)
            rows.append(zp)
            if i < M - 1:
                ctx.append(int(drafts[b, i]))
        ref = oracle.accept_greedy(np.array(rows), drafts[b], 10 * (b + 1))
        assert np.array_equal(tok[b], ref[0]) and np.array_equal(cnt[b], ref[1])
        assert rb[b] == ref[2]


def test_plain_settings_match_the_rejection_oracle():
    rng = np.random.default_rng(11)
    for trial in range(20):
        M, V = int(rng.integers(1, 6)), int(rng.integers(2, 300))
        z = (rng.standard_normal((M, V)) * (1 + trial % 3)).astype(np.float32)
        q = rng.dirichlet(np.full(V, 0.3), size=max(M - 1, 1)).astype(np.float32)[:M - 1]
        d = rng.integers(0, V, M - 1).astype(np.int32)
        u = rng.random(M).astype(np.float32)
        T, P = float(rng.choice([0.0, 0.6, 1.0])), float(rng.choice([0.5, 0.95, 1.0]))
        ref = oracle.accept_rejection(z, q, d, u, T, P, 7)
        got = oracle.accept_sampled(z[None], d[None], u[None], S(temperature=T, top_p=P),
                                    q=q[None] if M > 1 else None,
                                    q_sparse=None if M > 1 else (np.zeros((1, 0, 1)),) * 2,
                                    base_len=np.array([7]))
        assert np.array_equal(got[0][0], ref[0]) and np.array_equal(got[1][0], ref[1])
        assert got[2][0] == ref[2]


def test_sparse_q_equals_dense_q_with_zeros():
    rng = np.random.default_rng(5)
    B, M, V, K = 2, 5, 200, 12
    z = rng.standard_normal((B, M, V)).astype(np.float32) * 2
    ids = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(M - 1)])
                    for _ in range(B)]).astype(np.int32)
    pr = rng.dirichlet(np.ones(K), size=(B, M - 1)).astype(np.float32)
    dense = np.zeros((B, M - 1, V), np.float32)
    for b in range(B):
        for i in range(M - 1):
            dense[b, i, ids[b, i]] = pr[b, i]
    d = ids[:, :, 0].copy()
    par = S(temperature=0.8, top_k=20, top_p=0.9, min_p=0.05)
    for s in range(10):
        u = np.random.default_rng(s).random((B, M)).astype(np.float32)
        a = oracle.accept_sampled(z, d, u, par, q=dense)
        b_ = oracle.accept_sampled(z, d, u, par, q_sparse=(ids, pr))
        for x, y in zip(a, b_):
            assert np.array_equal(x, y)


def test_sequences_are_independent():
    rng = np.random.default_rng(8)
    B, M, V = 4, 3, 64
    z = rng.standard_normal((B, M, V)).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=(B, M - 1)).astype(np.float32)
    d = rng.integers(0, V, (B, M - 1)).astype(np.int32)
    u = rng.random((B, M)).astype(np.float32)
    hist = [list(rng.integers(0, V, n)) for n in (0, 3, 7, 1)]
    par = S(temperature=0.9, top_k=10, top_p=0.95, repeat_penalty=1.2, penalty_last_n=4)
    bl = np.array([1, 2, 3, 4])
    tok, cnt, rb = oracle.accept_sampled(z, d, u, par, q=q, history=hist, base_len=bl)
    for b in range(B):
        t1, c1, r1 = oracle.accept_sampled(z[b:b + 1], d[b:b + 1], u[b:b + 1], par,
                                           q=q[b:b + 1], history=[hist[b]], base_len=bl[b:b + 1])
        assert np.array_equal(t1[0], tok[b]) and np.array_equal(c1[0], cnt[b]) and r1[0] == rb[b]


def _chi2_ok(samples, p, V):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = p * len(samples)
    keep = exp > 5
    assert counts[~keep].sum() <= max(10, 5 * (~keep).sum()), "mass where the target has none"
    if keep.sum() <= 1:
        return True
    stat = ((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum()
    return stats.chi2.sf(stat, keep.sum() - 1) > 1e-4


@pytest.mark.parametrize("sparse", [False, True])
def test_committed_tokens_follow_the_target(sparse):
    rng = np.random.default_rng(21 + sparse)
    M, V, n = 3, 12, 30000
    z = rng.standard_normal((1, M, V)).astype(np.float32)
    par = S(temperature=0.8, top_k=8, top_p=0.9, min_p=0.05, repeat_penalty=1.5,
            presence_penalty=0.3, penalty_last_n=4)
    hist = [[1, 2, 2]]
    _, _, _, tp = oracle.accept_sampled(z, np.array([[0, 0]], np.int32),
                                        np.full((1, M), 0.5, np.float32), par,
                                        q=np.full((1, M - 1, V), 1 / V, np.float32),
                                        history=hist, with_target=True)
    p0 = tp[0, 0]
    # draft 0 ~ q_0 (sparse: 5 listed ids), draft 1 fixed: the first committed
    # token follows p'_0 whatever q_0 is
    K = 5
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(M - 1)])[None].astype(np.int32)
    pr = rng.dirichlet(np.ones(K), size=(1, M - 1)).astype(np.float32)
    dense = np.zeros((1, M - 1, V), np.float32)
    for i in range(M - 1):
        dense[0, i, ids[0, i]] = pr[0, i]
    q0 = pr[0, 0].astype(np.float64)
    q0 /= q0.sum()
    first = np.zeros(n, np.int64)
    acc = 0
    for t in range(n):
        x0 = int(rng.choice(ids[0, 0], p=q0))
        d = np.array([[x0, ids[0, 1, 0]]], np.int32)
        u = rng.random((1, M)).astype(np.float32)
        kw = dict(q_sparse=(ids, pr)) if sparse else dict(q=dense)
        tok, cnt, _ = oracle.accept_sampled(z, d, u, par, history=hist, **kw)
        first[t] = tok[0, 0]
        acc += cnt[0, 0] >= 1
    assert _chi2_ok(first, p0, V)
    rate = np.minimum(p0, dense[0, 0].astype(np.float64)).sum()
    assert stats.binomtest(int(acc), n, rate).pvalue > 1e-4
