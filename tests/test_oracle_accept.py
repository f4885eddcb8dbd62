"""Pins for the oracle's acceptance step (greedy and rejection sampling).

Pinned against: exhaustive enumeration on tiny vocabularies, the invariant
that greedy verification commits exactly what plain greedy decoding would,
the temperature-0 reduction of rejection sampling to argmax matching, and the
distribution law of Leviathan/Chen rejection sampling (the committed tokens
follow the target distribution), checked by chi-square tests on small
vocabularies with a target distribution computed here independently.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle


def first_argmax(row):
    """Lowest index of the largest non-NaN value (0 if all NaN)."""
    row = np.asarray(row, dtype=np.float64)
    if np.all(np.isnan(row)):
        return 0
    r = np.where(np.isnan(row), -np.inf, row)
    best = np.max(r)
    cand = np.flatnonzero(r == best)
    if best == -np.inf:
        # -inf ranks above NaN: first non-NaN entry
        cand = np.flatnonzero(~np.isnan(row))
    return int(cand[0])


# --------------------------------------------------------------------------
# greedy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,V", [(1, 3), (2, 4), (3, 3), (3, 4)])
def test_greedy_exhaustive_over_drafts(M, V):
    rng = np.random.default_rng(M * 10 + V)
    z = rng.integers(-2, 3, size=(M, V)).astype(np.float32)   # ties happen
    g = [first_argmax(z[i]) for i in range(M)]
    for drafts in itertools.product(range(-1, V + 1), repeat=M - 1):
        d = np.array(drafts, dtype=np.int32)
        a = 0
        while a < M - 1 and d[a] == g[a]:
            a += 1
        tok, cnt, rb = oracle.accept_greedy(z, d, base_len=17)
        assert list(tok[:a + 1]) == g[:a + 1]
        assert all(t == -1 for t in tok[a + 1:])
        assert list(cnt) == [a, a + 1]
        assert rb == 17 + a + 1


def test_greedy_equals_plain_greedy_decoding():
    # A toy target: the next-token logits depend only on the previous token
    # through a fixed table.  Plain greedy decoding follows the table's argmax
    # chain; verification of any draft must commit a prefix of that chain.
    V, M = 12, 6
    rng = np.random.default_rng(0)
    table = rng.standard_normal((V, V)).astype(np.float32)
    for trial in range(200):
        t0 = int(rng.integers(V))
        chain = [t0]
        for _ in range(M):
            chain.append(first_argmax(table[chain[-1]]))
        plain = chain[1:]                 # what plain greedy decoding emits
        L = int(rng.integers(0, M))
        drafts = list(plain[:L]) + [int(x) for x in rng.integers(0, V, M - 1 - L)]
        drafts = drafts[:M - 1]
        inputs = [t0] + drafts            # row i is the target after inputs[i]
        logits = np.stack([table[t] for t in inputs])
        tok, cnt, rb = oracle.accept_greedy(logits, np.array(drafts, np.int32), base_len=5)
        a = cnt[0]
        assert a >= min(L, M - 1)
        assert list(tok[:a + 1]) == plain[:a + 1]
        assert cnt[1] == a + 1 >= 1       # at least one token per pass
        assert rb == 5 + a + 1


def test_greedy_nan_and_ties():
    nan = np.float32(np.nan)
    z = np.array([[nan, nan, nan],
                  [1.0, 3.0, 3.0],
                  [nan, -np.inf, nan],
                  [nan, 2.0, 5.0]], dtype=np.float32)
    for i, want in enumerate([0, 1, 1, 2]):
        assert oracle.argmax(z[i]) == want == first_argmax(z[i])
    tok, cnt, rb = oracle.accept_greedy(z, np.array([0, 1, 1], np.int32))
    assert list(tok) == [0, 1, 1, 2] and list(cnt) == [3, 4] and rb == 4


# --------------------------------------------------------------------------
# rejection sampling
# --------------------------------------------------------------------------

def target_dist(z, T, top_p):
    """Independent numpy target: softmax(z/T), then the shortest prefix in
    (probability desc, index asc) order with mass >= top_p, renormalised."""
    z = np.asarray(z, dtype=np.float64)
    p = np.exp((z - z.max()) / T)
    p /= p.sum()
    if top_p >= 1:
        return p
    order = sorted(range(len(z)), key=lambda j: (-z[j], j))
    keep, mass = [], 0.0
    for j in order:
        keep.append(j)
        mass += p[j]
        if mass >= top_p or top_p <= 0:
            break
    out = np.zeros_like(p)
    out[keep] = p[keep]
    return out / out.sum()


def test_temperature_zero_is_greedy_bitwise():
    rng = np.random.default_rng(1)
    for trial in range(300):
        M, V = int(rng.integers(1, 6)), int(rng.integers(1, 9))
        z = rng.integers(-3, 4, size=(M, V)).astype(np.float32)
        q = rng.random((M - 1, V)).astype(np.float32) if M > 1 else None
        d = rng.integers(0, V, M - 1).astype(np.int32) if M > 1 else None
        u = rng.random(M).astype(np.float32)
        g = oracle.accept_greedy(z, d if d is not None else np.zeros(0, np.int32), 3)
        r = oracle.accept_rejection(z, q, d, u, 0.0, float(rng.random()), 3)
        assert np.array_equal(g[0], r[0]) and np.array_equal(g[1], r[1]) and g[2] == r[2]


def test_p_equals_q_accepts_every_draft():
    rng = np.random.default_rng(2)
    V, M, T, top_p = 16, 5, 0.6, 0.9
    z = rng.standard_normal((M, V)).astype(np.float32)
    q = np.stack([target_dist(z[i], T, top_p) for i in range(M - 1)]).astype(np.float32)
    for _ in range(200):
        qd = q.astype(np.float64)
        d = np.array([rng.choice(V, p=qd[i] / qd[i].sum()) for i in range(M - 1)], np.int32)
        u = (rng.random(M) * 0.999).astype(np.float32)
        tok, cnt, rb = oracle.accept_rejection(z, q, d, u, T, top_p)
        # q was rounded to fp32, so u*q < p' can fail only when u is within
        # fp32 rounding of 1; u <= 0.999 keeps every test an acceptance.
        assert cnt[0] == M - 1, (tok, cnt)
        assert list(tok[:M - 1]) == list(d)


def test_zero_target_mass_always_rejects_and_out_of_range():
    V = 6
    z = np.array([[5.0, 4.0, -30.0, -30.0, -30.0, -30.0]] * 2, np.float32)
    q = np.full((1, V), 1.0 / V, np.float32)
    for x in (3, -1, V, 10 ** 6):
        tok, cnt, _ = oracle.accept_rejection(z, q, np.array([x], np.int32),
                                              np.zeros(2, np.float32), 1.0, 0.5)
        assert cnt[0] == 0
        assert tok[0] == 0           # nucleus at top_p=0.5 is {0}: the draw lands there
    # q(x) = 0 with p'(x) > 0 always accepts (0 < p')
    q0 = np.zeros((1, V), np.float32)
    tok, cnt, _ = oracle.accept_rejection(z, q0, np.array([1], np.int32),
                                          np.array([0.99, 0.5], np.float32), 1.0, 1.0)
    assert cnt[0] == 1 and tok[0] == 1


def test_nucleus_cut_ties_and_degenerate_top_p():
    # logits 2,1,1,1,0: with T=1 the three tied tokens enter the nucleus in
    # index order.  Bonus draws over a sweep of u reveal the support.
    z = np.array([[2.0, 1.0, 1.0, 1.0, 0.0]], np.float32)
    p = np.exp(z[0].astype(np.float64) - 2.0)
    p /= p.sum()

    def support(top_p):
        s = set()
        for u in np.linspace(0, 1, 4001, endpoint=False):
            tok, _, _ = oracle.accept_rejection(z, None, None, np.array([u], np.float32),
                                                1.0, top_p)
            s.add(int(tok[0]))
        return s

    assert support(0.0) == {0}
    assert support(-1.0) == {0}
    assert support(p[0] * 0.999) == {0}
    assert support(p[0] + p[1] * 0.5) == {0, 1}
    assert support(p[0] + p[1] + p[2] * 0.5) == {0, 1, 2}
    assert support(1.0) == {0, 1, 2, 3, 4}
    assert support(2.0) == {0, 1, 2, 3, 4}
    # V = 1: always token 0
    tok, cnt, rb = oracle.accept_rejection(np.zeros((3, 1), np.float32),
                                           np.ones((2, 1), np.float32),
                                           np.zeros(2, np.int32),
                                           np.array([0.5, 0.5, 0.5], np.float32), 0.7, 0.95, 9)
    assert list(tok) == [0, 0, 0] and list(cnt) == [2, 3] and rb == 12


def test_draw_boundaries_follow_index_order_cdf():
    # bonus draw at M=1: smallest j with cumulative mass > u (index order)
    z = np.log(np.array([[0.1, 0.2, 0.3, 0.4]])).astype(np.float32)
    pd = target_dist(z[0], 1.0, 1.0)
    cdf = np.cumsum(pd)
    for j, c in enumerate(cdf[:-1]):
        below = np.float32(c) - np.float32(1e-6)
        above = np.float32(c) + np.float32(1e-6)
        assert oracle.accept_rejection(z, None, None, np.array([below], np.float32), 1.0, 1.0)[0][0] == j
        assert oracle.accept_rejection(z, None, None, np.array([above], np.float32), 1.0, 1.0)[0][0] == j + 1


def _run_trials(z, q, T, top_p, n, seed):
    """Draft ids ~ q, uniforms U[0,1); returns committed tokens and counts."""
    rng = np.random.default_rng(seed)
    M, V = z.shape
    qd = q.astype(np.float64)
    d = np.stack([rng.choice(V, size=n, p=qd[i] / qd[i].sum())
                  for i in range(M - 1)], axis=1).astype(np.int32)
    u = rng.random((n, M)).astype(np.float32)
    toks = np.zeros((n, M), np.int32)
    acc = np.zeros(n, np.int32)
    for t in range(n):
        tok, cnt, _ = oracle.accept_rejection(z, q, d[t], u[t], T, top_p)
        toks[t] = tok
        acc[t] = cnt[0]
    return toks, acc


def _chi2_ok(samples, p, V):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    keep = p > 0
    assert counts[~keep].sum() == 0, "sampled outside the target support"
    exp = p[keep] * len(samples)
    if keep.sum() == 1:
        return True
    stat = ((counts[keep] - exp) ** 2 / exp).sum()
    pval = stats.chi2.sf(stat, keep.sum() - 1)
    return pval > 1e-4


@pytest.mark.parametrize("V,alpha,top_p", [(8, 0.1, 0.95), (8, 1.0, 1.0), (32, 1.0, 0.95),
                                           (32, 0.1, 1.0)])
def test_rejection_sampling_preserves_target_distribution(V, alpha, top_p):
    rng = np.random.default_rng(V + int(alpha * 10) + int(top_p * 100))
    M, T, n = 3, 0.6, 40000
    z = rng.standard_normal((M, V)).astype(np.float32)
    q = rng.dirichlet(np.full(V, alpha), size=M - 1).astype(np.float32)
    q = np.maximum(q, 0)
    toks, acc = _run_trials(z, q, T, top_p, n, seed=V)
    p = [target_dist(z[i], T, top_p) for i in range(M)]
    # first committed token ~ p'_0 whatever happens
    assert _chi2_ok(toks[:, 0], p[0], V)
    # second committed token, given draft 0 accepted, ~ p'_1
    sel = acc >= 1
    assert _chi2_ok(toks[sel, 1], p[1], V)
    # bonus token, given every draft accepted, ~ p'_{M-1}
    sel = acc == M - 1
    if sel.sum() > 200:
        assert _chi2_ok(toks[sel, M - 1], p[M - 1], V)
    # acceptance rate of draft 0 = sum_x min(p'_0(x), q_0(x))  (binomial test)
    rate = np.minimum(p[0], q[0].astype(np.float64)).sum()
    k = int((acc >= 1).sum())
    assert stats.binomtest(k, n, rate).pvalue > 1e-4


def test_same_uniforms_reproduce():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((4, 50)).astype(np.float32)
    q = rng.dirichlet(np.full(50, 0.3), size=3).astype(np.float32)
    d = rng.integers(0, 50, 3).astype(np.int32)
    u = rng.random(4).astype(np.float32)
    r1 = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 0, with_margins=True)
    r2 = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 0, with_margins=True)
    for a, b in zip(r1, r2):
        assert np.array_equal(np.asarray(a), np.asarray(b))


def test_negative_temperature_rejected():
    with pytest.raises(ValueError):
        oracle.accept_rejection(np.zeros((1, 4), np.float32), None, None,
                                np.zeros(1, np.float32), -0.5, 0.9)
