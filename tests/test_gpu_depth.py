"""The draft-depth controller on the device in a closed loop: each step runs
the verify GEMM (the LM head of the tiny pass) for depth + 1 rows, an accept
call, then mtp_depth_observe_device on the accept call's counts, and takes
the next depth from the device's choice.  The oracle runs the same loop on
the same logits (its acceptance, its observe, its estimate, its choice);
the two match step by step: counts and tokens exactly, the statistics and
probabilities bit for bit, the chosen depth exactly.  (The test reads the
device state every step to compare it; the library path needs no read.)"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import DEV, dev, host, log, pack_gpu

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")


def test_closed_loop_verify_accept_observe_choose():
    c = W.config0()
    K, V = 2048, c["V"]
    packed = pack_gpu(bv, c["head"])
    rng = np.random.default_rng(31)
    dmax, keep = 6, 0.9
    cost = np.array([20.0 + 3.0 * d for d in range(dmax + 1)])   # verify + drafting, per depth
    st = bv.DepthStatsDevice(dmax, cost, DEV, keep)
    ro, ao = np.zeros(dmax), np.zeros(dmax)
    depth, depths = 2, []
    for step in range(32):
        M = depth + 1
        x = W.rand_bf16(rng, (M, K))
        logits, _ = bv.verify_gemm(W.FMT_NVFP4, dev(x), packed, V, K)
        z = host(logits)
        g = np.array([oracle.argmax(z[i]) for i in range(M)], np.int32)
        hit = 0.85 if step < 16 else 0.3          # acceptance falls: the depth should follow
        d = np.array([g[i] if rng.random() < hit else (g[i] + 1) % V for i in range(depth)],
                     np.int32)
        dt = dev(d) if depth else None
        if step % 2:
            t, cnt, rb = bv.accept_greedy(logits, dt, 100 + step)
            o = oracle.accept_greedy(z, d, 100 + step)
        else:
            q = W.rand_dirichlet_rows(rng, max(depth, 1), V, 0.5)[:depth]
            u = W.rand_uniforms(rng, M)
            t, cnt, rb = bv.accept_rejection(logits, dev(q) if depth else None, dt, dev(u), 0.8,
                                             0.95, 100 + step)
            o = oracle.accept_rejection(z, q, d, u, 0.8, 0.95, 100 + step)
        st.observe(depth, cnt)
        oracle.depth_observe(ro, ao, depth, int(o[1][0]), keep)
        p_o = oracle.depth_estimate(ro, ao)
        d_o, _ = oracle.choose_draft_depth(p_o, cost)
        assert host(t).tolist() == o[0].tolist() and host(cnt).tolist() == o[1].tolist(), step
        assert np.array_equal(host(st.reached), ro) and np.array_equal(host(st.accepted), ao), step
        assert np.array_equal(host(st.prob), p_o), step
        assert int(host(st.err)[0]) == 0
        depth = int(host(st.choice)[0])
        assert depth == d_o, (step, depth, d_o)
        depths.append(depth)
    log("depths chosen:", depths)
    assert max(depths[:16]) > min(depths[16:])   # the controller backs off as acceptance falls


def test_counts_outside_the_step_leave_the_statistics():
    st = bv.DepthStatsDevice(4, [1.0, 1.2, 1.4, 1.6, 1.8], DEV)
    st.observe(3, torch.tensor([2, 3], dtype=torch.int32, device=DEV))
    before = (host(st.reached).copy(), host(st.accepted).copy())
    st.observe(2, torch.tensor([3, 4], dtype=torch.int32, device=DEV))   # 3 accepted of 2
    assert int(host(st.err)[0]) == 1
    assert np.array_equal(host(st.reached), before[0])
    assert np.array_equal(host(st.accepted), before[1])
