"""Host-side checks of the dense GEMM launch plan (no GPU work).

The plan comes from the library itself (mtp_gemm_plan_info).  These tests
check the invariants the kernel relies on, and replay the kernel's index
arithmetic for every workgroup and wave in numpy, so that every weight block,
LDS offset, partial-sum slot and arrival counter a launch touches is shown to
lie inside its buffer before any kernel runs.
"""
import numpy as np
import pytest

import bit_verify_gemm_amd as bv
import workloads as W

MAX_LDS = 160 * 1024
PAIR_BYTES = 2304
SHAPES = [(16, 32), (37, 96), (100, 256), (130, 1056), (70, 2080), (2048, 2048), (1024, 2048),
          (14336, 4096), (262144, 5376), (8192, 5120), (2176 * 16, 5120), (65536, 5376),
          (65536, 1536)] + \
    [(n, k) for _, k, n in W.LAYER_27B]


def row_bytes(np_):
    return (np_ + 1) * 512 + 16


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
@pytest.mark.parametrize("N,K", SHAPES)
def test_plan_invariants(fmt, N, K):
    slices = set()
    for M in range(1, 17):
        p = bv.gemm_plan_info(fmt, M, N, K)
        T, P, S, ppj, J, KG, TW = (p[k] for k in ("T", "P", "S", "ppj", "J", "KG", "TW"))
        assert T == -(-N // 16) and P == -(-K // 256)
        assert 1 <= ppj <= 16 and S * ppj >= P and (S - 1) * ppj < P
        assert 1 <= J <= 16 and J * KG >= S and (KG - 1) * J < S
        waves = TW * J
        assert TW >= 1 and TW & (TW - 1) == 0 and waves <= 8 and p["threads"] == waves * 64
        assert p["TG"] == -(-T // TW) and p["grid"] == p["G"] * KG and 1 <= p["G"] <= p["TG"]
        np_ = min(J * ppj, P)
        lds = M * row_bytes(np_) + (fmt == W.FMT_Q4_0) * (np_ + 1) * 128 * 4 + waves * 1024
        assert p["lds"] == lds and lds + 16 <= MAX_LDS
        assert p["ws_bytes"] <= bv.gemm_workspace_bytes(N, K)
        assert (p["ws_bytes"] > 0) == (KG > 1)
        # blocks in flight: 2 when two persistent workgroups share a CU (their
        # registers must fit together); one round of workgroups takes 3 or 4,
        # whichever pads a wave's positions per tile group less, 4 on a tie; a
        # persistent workgroup alone on its CU takes whichever of 3, 4, 5, 6, 8
        # pads least, the deeper on a tie
        one_round = p["grid"] <= 256 and p["G"] == p["TG"]
        pad = {pp: -(-ppj // pp) * pp - ppj for pp in (3, 4, 5, 6, 8)}
        per_cu = min(MAX_LDS // (p["lds"] + 1024), 16 // waves)
        if one_round:
            want = 3 if pad[3] < pad[4] else 4
        elif per_cu >= 2:
            want = 2
        else:
            want = min((pad[pp], -pp) for pp in (3, 4, 5, 6, 8))[1] * -1
        assert p["PP"] == want
        slices.add((S, ppj))
    assert len(slices) == 1, "the K split must not depend on M"


def replay(p, M, N, K):
    """Index ranges one launch touches, from the kernel's own arithmetic."""
    T, P, S, ppj, J, KG, TW, TG, G = (p[k] for k in
                                      ("T", "P", "S", "ppj", "J", "KG", "TW", "TG", "G"))
    hi = dict(block=-1, pair_lo=P, slot=-1, part=-1, cnt=-1, tiles=set(), cover=np.zeros((T, P), int))
    for b in range(p["grid"]):
        kg, wt = b % KG, b // KG
        count = -(-(TG - wt) // G)
        pa = kg * J * ppj
        np_ = min(J * ppj, P - pa)
        assert np_ >= 1
        for u in range(count):
            tg = wt + u * G
            hi["cnt"] = max(hi["cnt"], tg)
            for tw in range(TW):
                t = tg * TW + tw
                tile = t if t < T else -1
                for j in range(J):
                    js = min(np_, j * ppj)
                    n = min(np_, js + ppj) - js
                    # stream positions past the slice or the matrix read
                    # nothing (empty buffer windows)
                    if tile >= 0 and n > 0:
                        hi["block"] = max(hi["block"], tile * P + pa + js + n - 1)
                        hi["pair_lo"] = min(hi["pair_lo"], pa + js)
                    hi["slot"] = max(hi["slot"], js + n if n else np_)
                    assert js + n <= np_
                    if tile >= 0 and n > 0:
                        hi["cover"][tile, pa + js:pa + js + n] += 1
                    slice_ = kg * J + j
                    if KG > 1 and tile >= 0 and slice_ < S:
                        hi["part"] = max(hi["part"], tile * S + slice_)
    return hi


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_launch_stays_in_bounds(fmt, M, N, K):
    p = bv.gemm_plan_info(fmt, M, N, K)
    h = replay(p, M, N, K)
    T, P, S = p["T"], p["P"], p["S"]
    assert h["block"] < T * P and h["pair_lo"] >= 0
    # every (tile, pair) block is read by exactly one wave stream
    assert (h["cover"] == 1).all()
    if p["KG"] > 1:
        cnt_bytes = max(256 * 1024, -(-T * 4 // 256) * 256)   # counter header, then partials
        assert h["cnt"] < T and cnt_bytes + (h["part"] + 1) * 1024 <= p["ws_bytes"]
