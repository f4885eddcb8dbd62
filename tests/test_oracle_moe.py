"""Pins for the oracle's routed-MoE verify pass.

The MoE oracle is checked against an independent composition written here
(library element decoders, numpy products, an independent bf16 rounding) and
against structural invariants: slot-order combine, deduplication not
changing results, duplicated experts counted twice, out-of-range ids
contributing nothing.  The choice of SiLU and of the bf16 rounding of the
intermediate is a reading of the pages, not something they fix; what is
pinned here is the oracle's arithmetic for that reading.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_oracle_gemm import dense_weights, lib_bf16


def bf16_round_independent(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, nearest-even, via torch's fp32 path with a guard
    for the double-rounding case (an fp32 result exactly halfway between two
    bf16 values while the fp64 input is not)."""
    v = np.asarray(v, np.float64)
    f32 = v.astype(np.float32)
    bits32 = f32.view(np.uint32)
    out = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    mid = ((bits32 & 0xFFFF) == 0x8000) & (f32.astype(np.float64) != v)
    for i in np.flatnonzero(mid):
        up = abs(v[i]) > abs(float(f32[i]))
        base = int(bits32[i] >> 16)
        out[i] = base + 1 if up else base
    return out


def tiny_cfg(seed=0, T=3, E=5, topk=2, H=64, F=32, fmt=W.FMT_NVFP4):
    rng = np.random.default_rng(seed)
    gu = W.rand_weight(fmt, rng, rng, E * 2 * F, H)
    dn = W.rand_weight(fmt, rng, rng, E * H, F)
    ids, gw = W.rand_routing(rng, T, E, topk)
    return {"T": T, "E": E, "topk": topk, "H": H, "F": F, "x": W.rand_bf16(rng, (T, H)),
            "gate_up": {"format": fmt, "codes": gu["codes"].reshape(E, 2 * F, H // 2),
                        "scales": gu["scales"].reshape(E, 2 * F, -1),
                        "g": rng.uniform(0.5, 2, E).astype(np.float32)},
            "down": {"format": fmt, "codes": dn["codes"].reshape(E, H, F // 2),
                     "scales": dn["scales"].reshape(E, H, -1),
                     "g": rng.uniform(0.5, 2, E).astype(np.float32)},
            "ids": ids, "gw": gw}


def expert_dense(part, e, N, K):
    return dense_weights({"format": part["format"], "codes": part["codes"][e],
                          "scales": part["scales"][e], "g": float(part["g"][e]), "N": N, "K": K})


def independent_moe(cfg):
    T, H, F, E, topk = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["topk"]
    x = lib_bf16(cfg["x"])
    out = np.zeros((T, H))
    hs = np.zeros((T * topk, F), np.uint16)
    for t in range(T):
        for s in range(topk):
            e = int(cfg["ids"][t, s])
            if not 0 <= e < E:
                continue
            a = expert_dense(cfg["gate_up"], e, 2 * F, H) @ x[t]
            hval = a[:F] / (1.0 + np.exp(-a[:F])) * a[F:]
            hb = bf16_round_independent(hval)
            hs[t * topk + s] = hb
            y = expert_dense(cfg["down"], e, H, F) @ lib_bf16(hb)
            out[t] += float(cfg["gw"][t, s]) * y
    return out, hs


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_moe_matches_independent_composition(fmt):
    cfg = tiny_cfg(seed=3, fmt=fmt)
    out, outb, h = oracle.moe(cfg)
    ref, href = independent_moe(cfg)
    # h: identical bf16 unless the pre-rounding value sits on a rounding tie
    # within the fp64 summation-order difference (not the case here).
    assert np.array_equal(h, href)
    assert np.all(np.abs(out - ref) <= 1e-12 * outb + 1e-300)


def test_moe_duplicate_and_out_of_range_ids():
    cfg = tiny_cfg(seed=4, T=2, topk=3)
    cfg["ids"] = np.array([[1, 1, 7], [-1, 2, 2]], np.int32)      # E = 5
    cfg["gw"] = np.array([[0.5, 0.5, 9.0], [9.0, 0.25, 0.75]], np.float32)
    out, outb, h = oracle.moe(cfg)
    ref, href = independent_moe(cfg)
    assert np.array_equal(h, href)
    assert np.all(h[2] == 0) and np.all(h[3] == 0)
    assert np.all(np.abs(out - ref) <= 1e-12 * outb + 1e-300)
    # token 0: the same expert twice with weights 0.5 + 0.5 == once with 1.0
    single = dict(cfg, ids=np.array([[1, 7, 7], [-1, 2, 2]], np.int32),
                  gw=np.array([[1.0, 9.0, 9.0], [9.0, 0.25, 0.75]], np.float32))
    out1, _, _ = oracle.moe(single)
    np.testing.assert_allclose(out1[0], out[0], rtol=1e-13, atol=1e-13)


def test_moe_slot_order_and_dense_equivalence():
    cfg = tiny_cfg(seed=5, T=2, topk=3, E=4)
    out, outb, h = oracle.moe(cfg)
    # recompute each pair's down projection with the dense oracle GEMM on the
    # oracle's own h, then combine in slot order
    H, F, topk = cfg["H"], cfg["F"], cfg["topk"]
    for t in range(cfg["T"]):
        acc = 0.0
        for s in range(topk):
            e = int(cfg["ids"][t, s])
            dn = {"format": cfg["down"]["format"], "N": H, "K": F,
                  "codes": cfg["down"]["codes"][e], "scales": cfg["down"]["scales"][e],
                  "g": float(cfg["down"]["g"][e])}
            y, _ = oracle.gemm(dn, h[t * topk + s][None, :])
            acc = acc + float(cfg["gw"][t, s]) * y[0]
        assert np.array_equal(acc, out[t])
