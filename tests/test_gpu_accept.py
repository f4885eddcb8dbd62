"""GPU parity of mtp_accept_greedy / mtp_accept_rejection against the oracle.

Bar: committed tokens, counts and the rollback index match bit for bit.  Both
sides take every decision in fp64 from the same fp32 inputs; the oracle's
margins are printed when a case disagrees (a mismatch can only come from a
decision within ~1e-15 of its boundary).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import DEV, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")


def gpu_greedy(z, d, base):
    t, c, r = bv.accept_greedy(dev(z), dev(d) if d is not None and len(d) else None, base)
    return host(t), host(c), int(host(r)[0])


def gpu_rej(z, q, d, u, T, top_p, base):
    M = z.shape[0]
    qt = dev(q) if M > 1 else None
    dt = dev(d) if M > 1 else None
    t, c, r = bv.accept_rejection(dev(z), qt, dt, dev(u), T, top_p, base)
    return host(t), host(c), int(host(r)[0])


def check_same(g, o, what, margins=None):
    ok = np.array_equal(g[0], o[0]) and np.array_equal(g[1], o[1]) and g[2] == o[2]
    if not ok:
        raise AssertionError(f"{what}: gpu={g[0].tolist()} {g[1].tolist()} {g[2]} "
                             f"oracle={o[0].tolist()} {o[1].tolist()} {o[2]} margins={margins}")


@pytest.mark.parametrize("M,V", [(1, 1), (1, 7), (2, 5), (4, 1024), (8, 4097), (8, 262144),
                                 (16, 300), (64, 33)])
def test_greedy_matches_oracle(M, V):
    rng = np.random.default_rng(M * 7 + V)
    for trial in range(6):
        if trial % 2:
            z = rng.integers(-3, 4, size=(M, V)).astype(np.float32)     # many ties
        else:
            z = rng.standard_normal((M, V)).astype(np.float32)
        if trial == 3 and V > 2:
            z[0, :] = np.nan
            z[min(1, M - 1), ::2] = np.nan
        g = np.array([oracle.argmax(z[i]) for i in range(M)], np.int32)
        L = int(rng.integers(0, M))
        d = rng.integers(0, V, M - 1).astype(np.int32)
        d[:L] = g[:L]
        o = oracle.accept_greedy(z, d, 100 + trial)
        check_same(gpu_greedy(z, d, 100 + trial), o, f"greedy M={M} V={V} trial={trial}")


CASES = [
    # M, V, T, top_p, alpha
    (1, 5, 0.6, 0.95, 1.0), (2, 5, 1.0, 1.0, 1.0), (4, 64, 0.6, 0.95, 0.1), (4, 64, 1.7, 0.5, 1.0),
    (8, 1000, 0.6, 0.95, 0.1), (8, 1000, 0.6, 0.0, 0.3), (3, 4099, 0.9, 0.999, 0.5),
    (8, 262144, 0.6, 0.95, 0.1), (8, 262144, 1.0, 1.0, 0.1), (16, 2048, 0.3, 0.7, 1.0),
]


@pytest.mark.parametrize("M,V,T,top_p,alpha", CASES)
def test_rejection_matches_oracle(M, V, T, top_p, alpha):
    rng = np.random.default_rng(M + V + int(100 * T) + int(1000 * top_p))
    log("rejection", M, V, T, top_p, alpha)
    for trial in range(4 if V > 100000 else 12):
        z = rng.standard_normal((M, V)).astype(np.float32) * np.float32(1 + trial % 3)
        q = W.rand_dirichlet_rows(rng, max(M - 1, 1), V, alpha)[:M - 1]
        d = np.zeros(M - 1, np.int32)
        for i in range(M - 1):
            if trial % 3 == 0:
                d[i] = oracle.argmax(z[i])                     # likely accepted
            else:
                qd = q[i].astype(np.float64)
                d[i] = rng.choice(V, p=qd / qd.sum())         # drafted from q
        u = W.rand_uniforms(rng, M)
        o = oracle.accept_rejection(z, q, d, u, T, top_p, 7, with_margins=True)
        check_same(gpu_rej(z, q, d, u, T, top_p, 7), o[:3], f"rej trial={trial}", o[3])


def test_rejection_ties_at_the_nucleus_cut():
    rng = np.random.default_rng(4)
    for trial in range(20):
        M, V = 4, int(rng.integers(20, 3000))
        z = rng.integers(-2, 3, size=(M, V)).astype(np.float32)   # heavy ties
        q = W.rand_dirichlet_rows(rng, M - 1, V, 1.0)
        d = rng.integers(0, V, M - 1).astype(np.int32)
        u = W.rand_uniforms(rng, M)
        top_p = float(rng.uniform(0.05, 0.99))
        o = oracle.accept_rejection(z, q, d, u, 0.8, top_p, 0, with_margins=True)
        check_same(gpu_rej(z, q, d, u, 0.8, top_p, 0), o[:3], f"ties trial={trial}", o[3])


def test_temperature_zero_is_greedy_on_gpu():
    rng = np.random.default_rng(5)
    for trial in range(10):
        M, V = 6, 777
        z = rng.integers(-5, 5, size=(M, V)).astype(np.float32)
        q = W.rand_dirichlet_rows(rng, M - 1, V, 1.0)
        d = rng.integers(0, V, M - 1).astype(np.int32)
        g = np.array([oracle.argmax(z[i]) for i in range(M)], np.int32)
        d[:trial % M] = g[:trial % M]
        u = W.rand_uniforms(rng, M)
        check_same(gpu_rej(z, q, d, u, 0.0, 0.9, 3), gpu_greedy(z, d, 3), f"T0 trial={trial}")
        check_same(gpu_rej(z, q, d, u, 0.0, 0.9, 3), oracle.accept_greedy(z, d, 3), "T0 oracle")


def test_out_of_range_and_zero_probability_drafts():
    V = 50
    z = np.zeros((3, V), np.float32)
    z[:, 0] = 10.0
    q = np.full((2, V), 1.0 / V, np.float32)
    u = np.array([0.5, 0.5, 0.3], np.float32)
    for d in ([-1, 0], [V, 0], [7, 0], [0, 10 ** 6]):
        d = np.array(d, np.int32)
        o = oracle.accept_rejection(z, q, d, u, 1.0, 0.5, 0)
        check_same(gpu_rej(z, q, d, u, 1.0, 0.5, 0), o, f"drafts {d.tolist()}")


def test_draw_at_the_top_of_the_range_picks_the_last_positive_weight():
    # u = 1 (one past the documented range) puts the draw target at the total
    # weight: no prefix passes it, and both sides pick the last entry with a
    # positive weight; the nucleus ends well before the last id
    rng = np.random.default_rng(13)
    for trial in range(6):
        M, V = 4, 3000 + 997 * trial
        z = rng.standard_normal((M, V)).astype(np.float32)
        z[:, V // 2:] -= 40.0                       # the upper half is outside the nucleus
        q = W.rand_dirichlet_rows(rng, M - 1, V, 1.0)
        d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
        if trial % 2:
            d[1] = V - 1                            # a rejection: the residual draw
        u = np.array([0.0, 0.0, 0.0, 1.0], np.float32)
        o = oracle.accept_rejection(z, q, d, u, 0.7, 0.9, 0)
        check_same(gpu_rej(z, q, d, u, 0.7, 0.9, 0), o, f"u=1 trial={trial}")


@pytest.mark.parametrize("V", [1000, 262144])
def test_rejection_on_peaked_logits(V):
    # logits of the spread an LM head produces (std ~300): almost every weight
    # is below the fixed-point resolution and its exponential is skipped
    rng = np.random.default_rng(V)
    M = 8
    for trial in range(3):
        z = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
        z[:, rng.integers(0, V, 5)] = z.max() - np.float32(0.5)   # a few near the top
        q = W.rand_dirichlet_rows(rng, M - 1, V, 0.1)
        d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
        d[trial + 2] = int(rng.integers(0, V))
        u = W.rand_uniforms(rng, M)
        o = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 5, with_margins=True)
        check_same(gpu_rej(z, q, d, u, 0.6, 0.95, 5), o[:3], f"peaked V={V} trial={trial}", o[3])


def u_zero_case(path, trial):
    """Std-300 logits (an LM head's spread) with u_{M-1} = 0: at T = 0.6 every
    weight below the top one lies far under 2^-100 but is positive in fp64
    (logit gaps below about 446), so the pick, the smallest index with a
    positive weight, is usually not the argmax."""
    rng = np.random.default_rng(900 + 10 * trial + (path == "residual"))
    M, V = 8, 262144
    z = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
    q = W.rand_dirichlet_rows(rng, M - 1, V, 0.1)
    d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
    if path == "residual":
        a = trial + 1
        d[a] = int(rng.integers(0, V))              # p'(x) ~ 0 < u * q(x): rejected
        # a draft that gives no mass to a few ids the target still reaches:
        # their residual is p' itself, positive but far below 2^-100
        near = np.flatnonzero((z[a].max() - z[a]) < 300.0)
        q[a, near[:3]] = 0.0
    u = W.rand_uniforms(rng, M)
    u[:M - 1] = 0.5
    u[M - 1] = 0.0
    return z, q, d, u


@pytest.mark.parametrize("path", ["bonus", "residual"])
def test_draw_with_u_zero_takes_the_first_positive_weight(path):
    picks_off_argmax = 0
    for trial in range(3):
        z, q, d, u = u_zero_case(path, trial)
        o = oracle.accept_rejection(z, q, d, u, 0.6, 1.0, 9, with_margins=True)
        a = int(o[1][0])
        assert (a < len(d)) == (path == "residual")
        picks_off_argmax += int(o[0][a] != oracle.argmax(z[a]))
        check_same(gpu_rej(z, q, d, u, 0.6, 1.0, 9), o[:3], f"u=0 {path} trial={trial}", o[3])
    assert picks_off_argmax > 0     # the case exercises weights below 2^-100


@pytest.mark.parametrize("path", ["bonus", "residual"])
def test_small_nucleus_draw_with_u_zero(path):
    # top_p < 1 on std-300 logits with a few entries planted near the top: the
    # nucleus holds a handful of entries, so the workgroup that resolves a
    # row's cut draws its token itself; u_{M-1} = 0 takes the smallest kept
    # index with a positive weight (rarely the argmax), the residual path
    # also with no draft mass on some of them
    off = 0
    for trial in range(3):
        rng = np.random.default_rng(1300 + 10 * trial + (path == "residual"))
        M, V = 8, 262144
        z = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
        for i in range(M):
            near = rng.integers(0, V, 6)
            z[i, near] = z[i].max() - np.float32(0.5) * np.arange(1, 7, dtype=np.float32)
        q = W.rand_dirichlet_rows(rng, M - 1, V, 0.1)
        d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
        if path == "residual":
            a = trial + 1
            d[a] = int(rng.integers(0, V))
            kept = np.argsort(-z[a], kind="stable")[:4]
            q[a, kept[1:3]] = 0.0
        u = W.rand_uniforms(rng, M)
        u[:M - 1] = 0.5
        u[M - 1] = 0.0
        o = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 2, with_margins=True)
        a = int(o[1][0])
        assert (a < M - 1) == (path == "residual")
        off += int(o[0][a] != oracle.argmax(z[a]))
        check_same(gpu_rej(z, q, d, u, 0.6, 0.95, 2), o[:3], f"small u=0 {path} {trial}", o[3])
    assert off > 0


def test_same_trials_as_the_oracle_law():
    # The GPU reproduces the oracle trial by trial on the uniforms the oracle's
    # chi-square tests use, so the sampling law checked there holds here too.
    rng = np.random.default_rng(11)
    V, M, n = 8, 3, 400
    z = rng.standard_normal((M, V)).astype(np.float32)
    q = rng.dirichlet(np.full(V, 0.3), size=M - 1).astype(np.float32)
    for t in range(n):
        qd = q.astype(np.float64)
        d = np.array([rng.choice(V, p=qd[i] / qd[i].sum()) for i in range(M - 1)], np.int32)
        u = rng.random(M).astype(np.float32)
        o = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 0)
        check_same(gpu_rej(z, q, d, u, 0.6, 0.95, 0), o, f"law trial {t}")


def test_lm_head_acceptance_staged():
    # C3 shape: logits from the oracle's own fp64 head (rounded to fp32) feed
    # both acceptance implementations; drafts planted on the oracle's argmax.
    c = W.config3_inputs()
    cols = None
    log("C3 oracle logits (full head, fp64)")
    y_ref, _ = oracle.gemm(c["w"], c["x"], cols=cols, with_bound=False)
    z = y_ref.astype(np.float32)
    g = np.array([oracle.argmax(z[i]) for i in range(c["M"])], np.int32)
    d = W.plant_drafts(g, c["L"], c["filler"], c["miss"], c["V"])
    o = oracle.accept_greedy(z, d, 4096)
    assert o[1][0] == min(c["L"], c["M"] - 1)
    check_same(gpu_greedy(z, d, 4096), o, "C3 greedy")
    o = oracle.accept_rejection(z, c["q"], d, c["u"], c["temperature"], c["top_p"], 4096,
                                with_margins=True)
    check_same(gpu_rej(z, c["q"], d, c["u"], c["temperature"], c["top_p"], 4096), o[:3],
               "C3 rejection", o[3])
    # the same shape with spread logits (a nucleus of many thousand tokens)
    zs = W.spread_logits(3, c["M"], c["V"])
    gs = np.array([oracle.argmax(zs[i]) for i in range(c["M"])], np.int32)
    ds = W.plant_drafts(gs, c["L"], c["filler"], c["miss"], c["V"])
    o = oracle.accept_rejection(zs, c["q"], ds, c["u"], 0.6, 0.95, 4096, with_margins=True)
    check_same(gpu_rej(zs, c["q"], ds, c["u"], 0.6, 0.95, 4096), o[:3], "C3 spread", o[3])


def test_repeatable():
    rng = np.random.default_rng(8)
    M, V = 8, 100000
    z = rng.standard_normal((M, V)).astype(np.float32)
    q = W.rand_dirichlet_rows(rng, M - 1, V, 0.1)
    d = rng.integers(0, V, M - 1).astype(np.int32)
    u = W.rand_uniforms(rng, M)
    a = gpu_rej(z, q, d, u, 0.6, 0.95, 0)
    for _ in range(3):
        check_same(gpu_rej(z, q, d, u, 0.6, 0.95, 0), a, "repeat")


def test_one_workspace_across_calls_and_shapes():
    # one workspace serves greedy and rejection calls of different shapes in
    # any order (nothing a call leaves in it may affect the next)
    rng = np.random.default_rng(77)
    ws = bv.accept_workspace(8, 262144, DEV)
    for i, (M, V) in enumerate([(8, 262144), (4, 1000), (8, 262144), (1, 7), (16, 2048),
                                (8, 4097), (64, 33), (8, 262144)]):
        z = rng.standard_normal((M, V)).astype(np.float32)
        d = np.array([oracle.argmax(z[k]) for k in range(M - 1)], np.int32)
        if M > 2:
            d[M // 2] = (d[M // 2] + 1) % V
        dt = dev(d) if M > 1 else None
        t, c, r = bv.accept_greedy(dev(z), dt, 5, ws=ws)
        check_same((host(t), host(c), int(host(r)[0])), oracle.accept_greedy(z, d, 5),
                   f"greedy call {i} M={M} V={V}")
        q = W.rand_dirichlet_rows(rng, max(M - 1, 1), V, 0.5)[:M - 1]
        u = rng.random(M).astype(np.float32)
        t, c, r = bv.accept_rejection(dev(z), dev(q) if M > 1 else None, dt, dev(u), 0.8, 0.9,
                                      5, ws=ws)
        check_same((host(t), host(c), int(host(r)[0])),
                   oracle.accept_rejection(z, q, d, u, 0.8, 0.9, 5),
                   f"rejection call {i} M={M} V={V}")


ONE_LAUNCH_CASES = [
    # name, M, V, logits: the one-launch path's branches and the shapes past it
    ("flat rows (every entry a candidate, ties beyond the LDS room)", 2, 262144, "flat"),
    ("integer logits (a fine bin too large to sort directly)", 4, 262144, "int"),
    ("peaked rows (a handful of candidates)", 8, 262144, "peaked"),
    ("N(0,1) rows (thousands of candidates)", 8, 262144, "normal"),
    ("one row over 256 workgroups", 1, 262144, "normal"),
    ("rows of every kind at once", 6, 65536, "mixed"),
    ("too many workgroups for one launch (the chained kernels)", 16, 262144, "normal"),
]


@pytest.mark.parametrize("name,M,V,kind", ONE_LAUNCH_CASES)
def test_rejection_one_launch_paths(name, M, V, kind):
    rng = np.random.default_rng(M * 131 + V % 977 + len(kind))
    log("rejection path:", name)
    for trial in range(2):
        if kind == "flat":
            z = np.full((M, V), 0.75, np.float32)
        elif kind == "int":
            z = rng.integers(-3, 4, size=(M, V)).astype(np.float32)
        elif kind == "peaked":
            z = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
        elif kind == "normal":
            z = rng.standard_normal((M, V)).astype(np.float32)
        else:
            z = rng.standard_normal((M, V)).astype(np.float32)
            z[1] *= np.float32(300.0)
            z[2] = np.float32(1.25)
            z[3] = rng.integers(-2, 3, size=V).astype(np.float32)
        q = W.rand_dirichlet_rows(rng, max(M - 1, 1), V, 0.3)[:M - 1]
        d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
        if M > 2:
            d[M // 2] = int(rng.integers(0, V))
        u = W.rand_uniforms(rng, M)
        top_p = (0.95, 0.5)[trial]
        o = oracle.accept_rejection(z, q, d, u, 0.6, top_p, 3, with_margins=True)
        check_same(gpu_rej(z, q, d, u, 0.6, top_p, 3), o[:3], f"{name} trial={trial}", o[3])


def test_rejection_back_to_back_calls_on_one_workspace():
    # counters and tags left in the workspace by one call must serve the next:
    # the same inputs forty times, then other inputs, all on one workspace
    rng = np.random.default_rng(21)
    M, V = 8, 262144
    ws = bv.accept_workspace(M, V, DEV)
    z = rng.standard_normal((M, V)).astype(np.float32)
    q = W.rand_dirichlet_rows(rng, M - 1, V, 0.3)
    d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
    d[4] = 11
    u = W.rand_uniforms(rng, M)
    o = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 1)
    zt, qt, dt, ut = dev(z), dev(q), dev(d), dev(u)
    outs = [bv.accept_rejection(zt, qt, dt, ut, 0.6, 0.95, 1, ws=ws) for _ in range(40)]
    for i, (t, c, r) in enumerate(outs):
        check_same((host(t), host(c), int(host(r)[0])), o, f"call {i}")
    z2 = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
    o2 = oracle.accept_rejection(z2, q, d, u, 0.6, 0.95, 1)
    t, c, r = bv.accept_rejection(dev(z2), qt, dt, ut, 0.6, 0.95, 1, ws=ws)
    check_same((host(t), host(c), int(host(r)[0])), o2, "other inputs")


SETTLE_CASES = [
    # name, M, V: rows whose cut the workgroups' top entries may settle
    ("threshold on a prefix (the bracket straddles it: steps 2 and 3 decide)", 4, 262144),
    ("ties in the cut group (t below the group size)", 4, 262144),
    ("five maxima in one chunk (the top set is not complete)", 4, 262144),
    ("more top entries than a wave holds", 4, 262144),
    ("u below the fixed-point resolution", 8, 262144),
    ("a short last chunk", 5, 70001),
    ("one row over 256 workgroups", 1, 262144),
]


@pytest.mark.parametrize("name,M,V", SETTLE_CASES)
def test_rejection_settled_by_top_entries(name, M, V):
    rng = np.random.default_rng(sum(map(ord, name)))
    log("settle:", name)
    T = 0.6
    for trial in range(3):
        z = (rng.standard_normal((M, V)) * 300.0).astype(np.float32)
        zt = z.max(axis=1)
        top_p = 0.95
        u = W.rand_uniforms(rng, M)
        if name.startswith("threshold"):
            # two entries at the top: S = 1 + e1 (+ far less), and top_p puts
            # the threshold on the first prefix, just below or above it
            e1 = 0.25 + 0.1 * trial
            for i in range(M):
                j = int(rng.integers(0, V))
                z[i, j] = zt[i] + np.float32(T * np.log(e1))
            S = 1.0 + 0.25 + 0.1 * trial
            top_p = (1.0 / S) * (1.0 + (-1e-7, 0.0, 1e-7)[trial])
        elif name.startswith("ties"):
            for i in range(M):
                z[i, rng.choice(V, 3, replace=False)] = zt[i] + np.float32(1.0)
            top_p = (0.5, 0.34, 0.9)[trial]
        elif name.startswith("five"):
            for i in range(M):
                z[i, 100 + 512 * np.arange(5)] = zt[i] + np.float32(1.0)   # (chunks of 4096)
        elif name.startswith("more"):
            # 4 distinct near-top entries in each of the 64 chunks of 4096
            for i in range(M):
                for c in range(64):
                    z[i, c * 4096 + 7 * np.arange(4)] = zt[i] - np.float32(0.01) * (4 * c + np.arange(4))
            top_p = 0.9
        elif name.startswith("u below"):
            u[M - 1] = np.float32((1e-33, 1e-40, 3e-31)[trial])
            if trial == 1:
                u[:M - 1] = 0.999                                # residual path
        q = W.rand_dirichlet_rows(rng, max(M - 1, 1), V, 0.1)[:M - 1]
        d = np.array([oracle.argmax(z[i]) for i in range(M - 1)], np.int32)
        if M > 2:
            d[M // 2] = int(rng.integers(0, V))
        o = oracle.accept_rejection(z, q, d, u, T, top_p, 4, with_margins=True)
        check_same(gpu_rej(z, q, d, u, T, top_p, 4), o[:3], f"{name} trial={trial}", o[3])
