"""GPU parity of mtp_verify_moe against the oracle.

Bar: out within 1e-3 * B + 1e-5 per element, B = sum_s |w| * sum_f |h * w_d|
(the oracle's error scale); the bf16 intermediate h within one bf16 step of
the oracle's (its rounding decision sees fp32 vs fp64 pre-activations).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import DEV, assert_gemm_close, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")

import torch  # noqa: E402


def run_moe(cfg):
    T, H, F, E = cfg["T"], cfg["H"], cfg["F"], cfg["E"]
    gu, dn = cfg["gate_up"], cfg["down"]
    h = torch.full((T * cfg["topk"], F), -1, dtype=torch.int16, device=DEV)
    gug = dev(gu["g"]) if gu.get("g") is not None else None
    dng = dev(dn["g"]) if dn.get("g") is not None else None
    out, _ = bv.verify_moe(gu["format"], dev(cfg["x"]), dev(cfg["ids"]), dev(cfg["gw"]),
                           dev(gu["codes"]), dev(gu["scales"]), dev(dn["codes"]),
                           dev(dn["scales"]), E, F, gu_global=gug, dn_global=dng, h_out=h)
    return host(out).astype(np.float64), host(h).view(np.uint16)


def bf16_steps_apart(a, b):
    """Distance in representable bf16 steps (same-sign finite values)."""
    ai = a.astype(np.int32)
    bi = b.astype(np.int32)
    ai = np.where(ai & 0x8000, 0x8000 - ai, ai)
    bi = np.where(bi & 0x8000, 0x8000 - bi, bi)
    return np.abs(ai - bi)


def check(cfg, what):
    out, h = run_moe(cfg)
    o_out, o_b, o_h = oracle.moe(cfg)
    steps = bf16_steps_apart(h, o_h)
    assert steps.max() <= 1, f"{what}: h differs by {steps.max()} bf16 steps"
    log(what, "h mismatches:", int((steps > 0).sum()), "of", steps.size)
    assert_gemm_close(out, o_out, o_b, what)


def tiny(seed, T=3, E=5, topk=2, H=64, F=32, fmt=W.FMT_NVFP4):
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


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
@pytest.mark.parametrize("T,E,topk,H,F", [(1, 4, 1, 64, 32), (3, 5, 2, 64, 32),
                                          (8, 16, 4, 256, 96), (20, 6, 3, 128, 64)])
def test_small(fmt, T, E, topk, H, F):
    check(tiny(T * 31 + E, T=T, E=E, topk=topk, H=H, F=F, fmt=fmt), f"moe {fmt} {T},{E},{topk}")


def test_duplicates_and_invalid_ids():
    cfg = tiny(9, T=4, E=6, topk=3, H=128, F=64)
    cfg["ids"] = np.array([[1, 1, 7], [-1, 2, 2], [5, 5, 5], [0, 3, 4]], np.int32)
    out, h = run_moe(cfg)
    assert np.all(h[2] == 0) and np.all(h[3] == 0)
    check(cfg, "dup/invalid")


def test_all_tokens_same_experts():
    cfg = tiny(10, T=8, E=32, topk=8, H=256, F=64)
    cfg["ids"] = np.tile(np.arange(8, dtype=np.int32), (8, 1))
    check(cfg, "shared experts")


def test_moe_128_experts_top8_full_size():
    cfg = W.config4()
    log("C4 unique experts", len(np.unique(cfg["ids"])))
    check(cfg, "C4")
