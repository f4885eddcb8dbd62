"""GPU parity of mtp_verify_moe against the oracle.

Bar: out within 1e-3 * B + 1e-5 per element, B = sum_s |w| * sum_f |h * w_d|
(the oracle's error scale).  The bf16 intermediate h = bf16(silu(g) * u) is
checked against the oracle's within the GEMM tolerance of its inputs carried
through the activation: with dg = 1e-3 * B_g + 1e-5 (likewise du) and
|silu'| <= 1.1, |dh| <= 1.1 dg (|u| + du) + (|silu(g)| + 1.1 dg) du, plus one
bf16 rounding step and 2^-126 (values below the fp32 normal range).
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
    gup = bv.pack_weights(gu["format"], dev(gu["codes"]), dev(gu["scales"]), 2 * F, H, count=E)
    dnp = bv.pack_weights(dn["format"], dev(dn["codes"]), dev(dn["scales"]), H, F, count=E)
    out, _ = bv.verify_moe(gu["format"], dev(cfg["x"]), dev(cfg["ids"]), dev(cfg["gw"]),
                           gup, dnp, E, F, gu_global=gug, dn_global=dng, h_out=h)
    return host(out).astype(np.float64), host(h).view(np.uint16)


def bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def silu(v):
    e = np.exp(-np.abs(v))
    return np.where(v >= 0, v / (1 + e), v * e / (1 + e))


def h_allowed(a, ab, F, h_or):
    g, u = a[:, :F], a[:, F:]
    dg = 1e-3 * ab[:, :F] + 1e-5
    du = 1e-3 * ab[:, F:] + 1e-5
    prop = 1.1 * dg * (np.abs(u) + du) + (np.abs(silu(g)) + 1.1 * dg) * du
    mag = np.abs(h_or) + prop
    step = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -133))) - 7)
    return prop + step + 2.0 ** -126


def check(cfg, what):
    out, h = run_moe(cfg)
    o_out, o_b, o_h, a, ab = oracle.moe(cfg, with_preact=True)
    hv, ov = bf16_value(h), bf16_value(o_h)
    diff = np.abs(hv - ov)
    allowed = h_allowed(a, ab, cfg["F"], ov)
    bad = ~(diff <= allowed)
    assert not bad.any(), (f"{what}: h outside bound at {np.argwhere(bad)[:4].tolist()}: "
                           f"gpu {hv[bad][:4]} oracle {ov[bad][:4]}")
    log(what, "h entries differing:", int((h != o_h).sum()), "of", h.size)
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


def test_c4_one_token():
    # the one-token baseline of the MoE workload at full size (its 8 experts,
    # the quick routing path): every weight block of those experts must be read
    cfg = W.config4()
    one = dict(cfg, T=1, x=cfg["x"][:1], ids=cfg["ids"][:1], gw=cfg["gw"][:1])
    check(one, "C4 one token")


def test_many_pairs():
    # 1024 (token, slot) pairs, the most the call takes: every workgroup ranks
    # all of them, and an expert's 60-odd rows take several staging passes
    check(tiny(77, T=128, E=16, topk=8, H=64, F=32), "moe 1024 pairs")


def test_token_with_no_valid_expert():
    cfg = tiny(12, T=3, E=4, topk=2, H=64, F=32)
    cfg["ids"] = np.array([[0, 1], [-1, 9], [1, 1]], np.int32)
    out, _ = run_moe(cfg)
    assert np.all(out[1] == 0.0)
    check(cfg, "token without a valid expert")


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_k_split_over_waves(fmt):
    # H = 4096 and F = 3072 cut each expert's K into two slices per tile
    # (gate and up tiles in separate waves, the slice sums meeting in LDS)
    check(tiny(13, T=2, E=3, topk=2, H=4096, F=3072, fmt=fmt), f"moe {fmt} K split")


def test_one_workspace_across_calls_and_shapes():
    # calls of different token counts and shapes in a row on one workspace
    # (each call sets up its own counters), each matched with the oracle,
    # then the first again
    cfgs = [tiny(71, T=8, E=16, topk=4, H=256, F=128), tiny(72, T=1, E=16, topk=4, H=256, F=128),
            tiny(73, T=5, E=9, topk=3, H=128, F=64), tiny(71, T=8, E=16, topk=4, H=256, F=128)]
    need = max(bv.moe_workspace_bytes(c["T"], c["H"], c["F"], c["E"], c["topk"]) for c in cfgs)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, cfg in enumerate(cfgs):
        T, H, F, E = cfg["T"], cfg["H"], cfg["F"], cfg["E"]
        gu, dn = cfg["gate_up"], cfg["down"]
        gup = bv.pack_weights(gu["format"], dev(gu["codes"]), dev(gu["scales"]), 2 * F, H, count=E)
        dnp = bv.pack_weights(dn["format"], dev(dn["codes"]), dev(dn["scales"]), H, F, count=E)
        out, _ = bv.verify_moe(gu["format"], dev(cfg["x"]), dev(cfg["ids"]), dev(cfg["gw"]),
                               gup, dnp, E, F, gu_global=dev(gu["g"]), dn_global=dev(dn["g"]),
                               ws=ws)
        o_out, o_b, _ = oracle.moe(cfg)[:3]
        assert_gemm_close(host(out).astype(np.float64), o_out, o_b, f"call {i} (T={T})")
