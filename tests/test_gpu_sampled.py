"""GPU parity of mtp_accept_sampled (the full sampler pipeline on the sparse
top-k path) against the oracle.

Bar: committed tokens, counts and rollback indices match bit for bit; each
row's kept target entries match in id and order, with probabilities within
2e-6 relative (the GPU reports p' in fp32).  Both sides take every decision
in fp64 from the same fp32 (penalised) logits; the oracle's margins are
printed when a case disagrees.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import DEV, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")


def run_both(z, drafts, u, par, q=None, q_sparse=None, history=None, base_len=None):
    B, M, V = z.shape
    sp = bv.Sampler(**par)
    ht = hl = None
    if history is not None:
        ldh = max(1, max(len(h) for h in history))
        harr = np.zeros((B, ldh), np.int32)
        for b, h in enumerate(history):
            harr[b, :len(h)] = h
        ht, hl = dev(harr), dev(np.array([len(h) for h in history], np.int32))
    bl = dev(np.asarray(base_len, np.int64)) if base_len is not None else None
    kw = {}
    if M > 1:
        kw = dict(draft_probs=dev(q)) if q is not None else \
            dict(draft_topk=(dev(q_sparse[0]), dev(q_sparse[1])))
    g = bv.accept_sampled(dev(z), dev(drafts) if M > 1 else None, dev(u), sp, history=ht,
                          history_len=hl, base_len=bl, want_target=True, **kw)
    g = [host(t) for t in g]
    o = oracle.accept_sampled(z, drafts, u, par, q=q, q_sparse=q_sparse, history=history,
                              base_len=base_len, with_target=True, with_margins=True)
    return g, o


def check(z, drafts, u, par, what, **kw):
    (gt, gc, gr, gid, gp), (ot, oc, orb, otp, om) = run_both(z, drafts, u, par, **kw)
    B, M, V = z.shape
    K = min(par["top_k"], V)
    # each row's kept entries, in order of probability (value desc, id asc)
    for b in range(B):
        for i in range(M):
            p = otp[b, i]
            ids = np.flatnonzero(p > 0)
            order = ids[np.lexsort((ids, -p[ids]))] if len(ids) else ids
            n = len(order)
            got = gid[b, i]
            if not (np.array_equal(got[:n], order) and np.all(got[n:] == -1)):
                raise AssertionError(f"{what}: row ({b},{i}) kept {got[:n + 2].tolist()} "
                                     f"oracle {order[:n + 2].tolist()} margins {om[b].tolist()}")
            # (fp32 output: below its subnormal range a probability reads 0)
            assert np.allclose(gp[b, i, :n], p[order], rtol=2e-6, atol=2.0 ** -149), what
            assert np.all(gp[b, i, n:] == 0) and n <= K
    ok = np.array_equal(gt, ot) and np.array_equal(gc, oc) and np.array_equal(gr, orb)
    if not ok:
        raise AssertionError(f"{what}: gpu {gt.tolist()} {gc.tolist()} {gr.tolist()} oracle "
                             f"{ot.tolist()} {oc.tolist()} {orb.tolist()} margins {om.tolist()}")


def drafts_for(rng, z, par, likely):
    """Drafts that are often accepted (the row argmax) or random."""
    B, M, V = z.shape
    d = rng.integers(0, V, (B, max(M - 1, 0))).astype(np.int32)
    if likely:
        d = np.argmax(z[:, :M - 1], axis=2).astype(np.int32)
    return d


CASES = [
    # B, M, V, params
    (1, 1, 7, dict(temperature=0.8, top_k=3)),
    (2, 2, 5, dict(temperature=1.0, top_k=8)),                       # top_k > V
    (1, 4, 64, dict(temperature=0.6, top_p=0.95, top_k=40)),
    (3, 5, 1000, dict(temperature=0.6, top_p=0.9, min_p=0.05, top_k=40)),
    (2, 8, 4099, dict(temperature=1.3, top_p=0.8, top_k=200, repeat_penalty=1.3,
                      frequency_penalty=0.1, presence_penalty=0.2, penalty_last_n=16)),
    (1, 8, 2048, dict(temperature=0.0, top_k=20, repeat_penalty=1.1, penalty_last_n=64)),
    (4, 3, 3000, dict(temperature=0.9, top_k=1024, min_p=0.02)),
    (1, 8, 262144, dict(temperature=0.6, top_p=0.95, top_k=40, repeat_penalty=1.1,
                        penalty_last_n=64)),
    (2, 6, 777, dict(temperature=0.7, top_k=1, repeat_penalty=1.5, penalty_last_n=8)),
    (1, 5, 500, dict(temperature=2.0, top_p=0.0, top_k=50)),
    # 64 rows over 2048 workgroups of the one-launch kernel
    (8, 8, 262144, dict(temperature=0.6, top_p=0.95, min_p=0.01, top_k=64)),
    # top_k 600 over 262144 entries: the chained kernels
    (1, 4, 262144, dict(temperature=0.8, top_p=0.9, top_k=600, repeat_penalty=1.2,
                        penalty_last_n=32)),
]


@pytest.mark.parametrize("B,M,V,par", CASES)
def test_sampled_matches_oracle(B, M, V, par):
    par = oracle.sampler(**par)
    rng = np.random.default_rng(B * 1000 + M * 100 + V)
    log("sampled", B, M, V, par)
    for trial in range(3 if V > 100000 else 8):
        if trial % 3 == 2:
            z = rng.integers(-4, 5, size=(B, M, V)).astype(np.float32)     # ties
        else:
            z = (rng.standard_normal((B, M, V)) * (1 + trial % 4)).astype(np.float32)
        d = drafts_for(rng, z, par, trial % 2 == 0)
        u = rng.random((B, M)).astype(np.float32)
        hist = [list(rng.integers(0, V, int(rng.integers(0, 40)))) for _ in range(B)]
        if trial % 2 == 0 and V > 8:   # repeat the drafts' own ids in the history
            hist = [h + list(d[b]) for b, h in enumerate(hist)]
        bl = rng.integers(0, 1000, B)
        if M > 1 and trial % 2 == 1:
            Kq = min(V, 30)
            ids = np.stack([np.stack([rng.choice(V, Kq, replace=False) for _ in range(M - 1)])
                            for _ in range(B)]).astype(np.int32)
            ids[..., 0] = d   # the draft is listed
            pr = rng.dirichlet(np.ones(Kq), size=(B, M - 1)).astype(np.float32)
            check(z, d, u, par, f"sparse q trial {trial}", q_sparse=(ids, pr), history=hist,
                  base_len=bl)
        else:
            q = rng.dirichlet(np.full(V, 0.3), size=(B, max(M - 1, 1))).astype(np.float32)
            q = q[:, :M - 1]
            check(z, d, u, par, f"dense q trial {trial}", q=q if M > 1 else None,
                  q_sparse=None if M > 1 else (np.zeros((B, 0, 1), np.int32),) * 2,
                  history=hist, base_len=bl)


@pytest.mark.parametrize("top_k", [1024, 256, 64])
@pytest.mark.parametrize("path", ["bonus", "residual"])
def test_sampled_draw_with_u_zero_takes_the_first_positive_weight(path, top_k):
    # u_{M-1} = 0: the pick is the kept id of smallest index whose weight is
    # positive in fp64.  Std-100 logits at T = 0.6 with the top 1024 (the
    # chained kernels), 256 (one launch) or 64 (one launch, one wave per row
    # after the sort) kept put nearly every kept weight far below 2^-100
    # while still positive.
    par = oracle.sampler(temperature=0.6, top_k=top_k)
    off = 0
    for trial in range(3):
        rng = np.random.default_rng(700 + 10 * trial + (path == "residual"))
        B, M, V = 2, 8, 65536
        z = (rng.standard_normal((B, M, V)) * 100.0).astype(np.float32)
        d = np.argmax(z[:, :M - 1], axis=2).astype(np.int32)
        if path == "residual":
            d[:, trial + 1] = rng.integers(0, V, B)
        q = np.stack([W.rand_dirichlet_rows(rng, M - 1, V, 0.1) for _ in range(B)])
        if path == "residual":
            # no draft mass on the three smallest kept ids: their residual is
            # p' itself, positive but far below 2^-100
            for b in range(B):
                kept = np.argsort(-z[b, trial + 1], kind="stable")[:top_k]
                q[b, trial + 1, np.sort(kept)[:3]] = 0.0
        u = np.full((B, M), 0.5, np.float32)
        u[:, M - 1] = 0.0
        o = oracle.accept_sampled(z, d, u, par, q=q)
        for b in range(B):
            a = int(o[1][b][0])
            off += int(o[0][b][a] != np.argmax(z[b, a]))
        check(z, d, u, par, f"u=0 {path} trial {trial}", q=q)
    assert off > 0


def test_draft_ids_out_of_range_are_rejected():
    rng = np.random.default_rng(3)
    B, M, V = 2, 4, 300
    z = rng.standard_normal((B, M, V)).astype(np.float32)
    d = np.array([[-1, 5, 7], [V, 0, 1]], np.int32)
    q = rng.dirichlet(np.ones(V), size=(B, M - 1)).astype(np.float32)
    u = rng.random((B, M)).astype(np.float32)
    check(z, d, u, oracle.sampler(temperature=0.8, top_k=30), "bad ids", q=q)


def test_sampled_on_lm_head_logits():
    # the 5376 -> 262144 head's own logits (8 rows), drafts planted along the
    # argmax, q ~ Dirichlet(0.1), Gemma-like sampler settings
    c = W.config3_inputs(M=8)
    w = c["w"]
    z = oracle.gemm(w, c["x"])[0].astype(np.float32)[None]
    d = np.argmax(z[0, :7], axis=1).astype(np.int32)[None]
    d[0, 5] = (d[0, 5] + 1) % c["V"]
    par = oracle.sampler(temperature=0.6, top_p=0.95, top_k=64, min_p=0.01,
                         repeat_penalty=1.1, penalty_last_n=64)
    check(z, d, c["u"][None], par, "LM head", q=c["q"][None], history=[[1, 2, 3]],
          base_len=[100])


def test_sampled_calls_share_one_workspace():
    # one workspace through one-launch and chained calls of several shapes:
    # each call must leave the head's counters ready for the next
    rng = np.random.default_rng(41)
    shapes = [(1, 8, 262144, 64), (2, 4, 262144, 600), (3, 5, 4099, 40), (1, 8, 262144, 64),
              (2, 3, 777, 1)]
    need = max(bv.accept_sampled_workspace_bytes(B, M, V, k, True) for B, M, V, k in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for rep, (B, M, V, k) in enumerate(shapes):
        par = oracle.sampler(temperature=0.7, top_p=0.9, top_k=k, repeat_penalty=1.1,
                             penalty_last_n=16)
        z = (rng.standard_normal((B, M, V)) * 2.0).astype(np.float32)
        d = drafts_for(rng, z, par, rep % 2 == 0)
        u = rng.random((B, M)).astype(np.float32)
        q = rng.dirichlet(np.full(V, 0.3), size=(B, M - 1)).astype(np.float32)
        hist = [list(rng.integers(0, V, 20)) for _ in range(B)]
        log("shared workspace", rep, B, M, V, k)
        ldh = max(len(h) for h in hist)
        harr = np.array([h + [0] * (ldh - len(h)) for h in hist], np.int32)
        g = bv.accept_sampled(dev(z), dev(d), dev(u), bv.Sampler(**par), draft_probs=dev(q),
                              history=dev(harr), history_len=dev(np.array([len(h) for h in hist],
                                                                           np.int32)), ws=ws)
        g = [host(t) for t in g]
        o = oracle.accept_sampled(z, d, u, par, q=q, history=hist)
        assert np.array_equal(g[0], o[0]) and np.array_equal(g[1], o[1]), (rep, g, o[:2])
    # the head is back to zero
    assert int(ws[:20480].count_nonzero()) == 0


@pytest.mark.parametrize("kind", ["all_equal", "few_values", "masked", "ragged_k_over_chunk",
                                  "spike_in_one_chunk"])
def test_sampled_one_launch_edge_rows(kind):
    # rows that take the one-launch kernel's slow paths: a cut bin too full
    # to sort (all equal, few distinct values), candidate sets larger than
    # the resolver keeps in LDS, a last chunk shorter than top_k, all the
    # large logits in one chunk, rows of -1e30 with a few finite entries
    rng = np.random.default_rng(sum(map(ord, kind)))   # (a fixed seed per case)
    B, M, V = 2, 4, 40000
    K = 64
    if kind == "ragged_k_over_chunk":
        V, K = 5000 + 37, 1024         # chunks of 1008 (the last 1005): none holds K
    par = oracle.sampler(temperature=0.8, top_p=0.9, min_p=0.01, top_k=K, repeat_penalty=1.2,
                         penalty_last_n=16)
    if kind == "all_equal":
        z = np.full((B, M, V), 1.5, np.float32)
    elif kind == "few_values":
        z = rng.integers(0, 3, size=(B, M, V)).astype(np.float32) * 0.5
    elif kind == "masked":
        z = np.full((B, M, V), -1e30, np.float32)
        for b in range(B):
            for i in range(M):
                keep = rng.choice(V, 100, replace=False)
                z[b, i, keep] = rng.standard_normal(100).astype(np.float32) * 2
    elif kind == "spike_in_one_chunk":
        z = rng.standard_normal((B, M, V)).astype(np.float32)
        z[:, :, 2000:2500] += 6.0
    else:
        z = (rng.standard_normal((B, M, V)) * 3).astype(np.float32)
    d = drafts_for(rng, z, par, True)
    u = rng.random((B, M)).astype(np.float32)
    q = rng.dirichlet(np.full(V, 0.3), size=(B, M - 1)).astype(np.float32)
    hist = [list(rng.integers(0, V, 10)) for _ in range(B)]
    log("sampled edge", kind, B, M, V, K)
    check(z, d, u, par, kind, q=q, history=hist)
