"""mtp_accept_greedy_static (greedy acceptance on the library's static device
scratch, for callers that cannot allocate) against mtp_accept_greedy, called
through the C ABI: tokens, counts and the rollback index bit for bit, on two
calls in a row (the second smaller), after calls of the workspace entry
point have used other memory, and against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def static_call(zt, dt, base):
    """The no-allocation entry point through ctypes (outputs pre-filled)."""
    M, V = zt.shape
    tok = torch.full((M,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((2,), -7, dtype=torch.int32, device=DEV)
    rb = torch.full((1,), -7, dtype=torch.int64, device=DEV)
    L = bv.lib()
    rc = L.mtp_accept_greedy_static(_p(zt), M, V, zt.stride(0), _p(dt), base, _p(tok), _p(cnt),
                                    _p(rb), None)
    assert rc == 0, L.mtp_last_error().decode()
    return host(tok), host(cnt), int(host(rb)[0])


def workspace_call(zt, dt, base):
    M, V = zt.shape
    ws = torch.full((bv.accept_workspace_bytes(M, V),), 0x5A, dtype=torch.uint8, device=DEV)
    tok, cnt, rb = bv.accept_greedy(zt, dt, base, ws=ws)
    return host(tok), host(cnt), int(host(rb)[0])


def case(seed, M, V, ties):
    rng = np.random.default_rng(seed)
    if ties:
        z = rng.integers(-3, 4, size=(M, V)).astype(np.float32)
    else:
        z = rng.standard_normal((M, V)).astype(np.float32)
    z[M // 2, ::3] = np.nan
    g = np.array([oracle.argmax(z[i]) for i in range(M)], np.int32)
    d = rng.integers(0, V, M - 1).astype(np.int32)
    L = M // 2
    d[:L] = g[:L]
    return z, d


def test_static_scratch_matches_the_workspace_entry_point():
    # two calls in a row, the second with a smaller input: the first leaves
    # its partial maxima in the scratch, which the second must not read
    for i, (M, V, ties) in enumerate([(16, 262144, False), (3, 1000, True), (64, 4097, False),
                                      (1, 7, True)]):
        log("static greedy call", i, M, V)
        z, d = case(100 + i, M, V, ties)
        zt = dev(z)
        dt = dev(d) if M > 1 else None
        want = workspace_call(zt, dt, 40 + i)
        got = static_call(zt, dt, 40 + i)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), (i, got, want)
        assert got[2] == want[2], i
        o = oracle.accept_greedy(z, d, 40 + i)
        assert got[0].tolist() == o[0].tolist() and got[1].tolist() == o[1].tolist()
        assert got[2] == o[2]


def test_static_scratch_in_a_graph_replayed_twice():
    # captured in a HIP graph (the caller allocates nothing inside it) and
    # replayed twice with eager calls of other shapes in between
    z, d = case(7, 8, 50000, False)
    zt, dt = dev(z), dev(d)
    tok = torch.empty(8, dtype=torch.int32, device=DEV)
    cnt = torch.empty(2, dtype=torch.int32, device=DEV)
    rb = torch.empty(1, dtype=torch.int64, device=DEV)
    bv.accept_greedy_static(zt, dt, 5, outs=(tok, cnt, rb))   # address lookup outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bv.accept_greedy_static(zt, dt, 5, outs=(tok, cnt, rb))
    o = oracle.accept_greedy(z, d, 5)
    for rep in range(2):
        tok.fill_(-1)
        cnt.fill_(-1)
        rb.fill_(-1)
        z2, d2 = case(20 + rep, 5, 3000, True)
        static_call(dev(z2), dev(d2), 0)                     # other contents in the scratch
        g.replay()
        torch.cuda.synchronize()
        assert host(tok).tolist() == o[0].tolist() and host(cnt).tolist() == o[1].tolist()
        assert int(host(rb)[0]) == o[2]
