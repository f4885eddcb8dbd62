"""Seeded synthetic inputs for the verification pass.

This module only draws random bytes and values; it holds none of the verify
arithmetic (no dequantisation, no dot products, no acceptance logic).  Both
the CPU oracle (tests, bench baseline) and the HIP path consume what it makes,
so the stored bytes are the single ground truth for both.

Distributions follow the workloads the pages describe for the verify pass:
* activations: bf16 rows ~ N(0,1), rounded to nearest-even from fp32;
* nvfp4 weights: E2M1 codes uniform over all 16 values (uniform bytes give
  independent uniform nibbles), one E4M3 scale per 16 weights along K drawn
  log-uniform in [2^-4, 2^2] and rounded to E4M3 (nearest-even), fp32
  global scale 1.0;
* Q4_0-style weights: offset-binary codes uniform over 0..15 (value u-8, i.e.
  int4 in [-8, 7]), one fp16 scale per 32 weights along K, |N(0, 0.02)|;
* draft ids uniform over the vocabulary; draft distributions Dirichlet(0.1);
  uniforms U[0,1) supplied by the caller;
* MoE routing: per token, top-k expert ids drawn without replacement, gate
  weights = softmax of N(0,1) router logits over the selected experts.

Seeds: numpy ``default_rng(SeedSequence(1234 + cfg))`` with child streams
spawned in a fixed order (x, codes, scales, head, drafts, q, uniforms, routing)
so that every config is reproducible byte for byte.
"""
from __future__ import annotations

import numpy as np
import torch

FMT_NVFP4 = 1
FMT_Q4_0 = 2

_STREAMS = ("x", "codes", "scales", "head", "drafts", "q", "uniforms", "routing")


def streams(cfg: int, seed_offset: int = 0) -> dict:
    """Child generators for config ``cfg`` in a fixed spawn order."""
    ss = np.random.SeedSequence(1234 + cfg + seed_offset)
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}


# ----------------------------------------------------------------------------
# element encoders (inputs only: fp32 -> stored bits)
# ----------------------------------------------------------------------------

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> bf16 bit patterns (uint16), nearest-even via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 (OCP 'FN' variant) bytes, nearest-even via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64).astype(np.float16).view(np.uint16).copy()


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

def rand_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def rand_codes(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """[N][K/2] bytes; element k of row n is the low nibble of byte k/2 for
    even k and the high nibble for odd k."""
    return rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)


def rand_nvfp4_scales(rng: np.random.Generator, N: int, K: int,
                      lo: float = -4.0, hi: float = 2.0) -> np.ndarray:
    e = rng.uniform(lo, hi, size=(N, K // 16))
    return to_e4m3_bits(np.exp2(e).astype(np.float32))


def rand_q4_scales(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    d = np.abs(rng.normal(0.0, std, size=(N, K // 32)))
    return to_f16_bits(d)


def rand_weight(fmt: int, rng_codes, rng_scales, N: int, K: int) -> dict:
    codes = rand_codes(rng_codes, N, K)
    if fmt == FMT_NVFP4:
        scales = rand_nvfp4_scales(rng_scales, N, K)
    elif fmt == FMT_Q4_0:
        scales = rand_q4_scales(rng_scales, N, K)
    else:
        raise ValueError(f"unknown format {fmt}")
    return {"format": fmt, "N": N, "K": K, "codes": codes, "scales": scales, "g": 1.0}


def rand_uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    u = rng.random(n, dtype=np.float32)
    return np.minimum(u, np.float32(1.0) - np.float32(2.0 ** -24)).astype(np.float32)


def rand_dirichlet_rows(rng: np.random.Generator, rows: int, V: int, alpha: float) -> np.ndarray:
    """rows x V fp32 probability rows ~ Dirichlet(alpha), drawn via normalised
    Gamma(alpha) variates (the standard construction)."""
    g = rng.standard_gamma(alpha, size=(rows, V))
    s = g.sum(axis=1, keepdims=True)
    s[s == 0] = 1.0
    return (g / s).astype(np.float32)


def rand_routing(rng: np.random.Generator, T: int, E: int, topk: int):
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.standard_normal((T, topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


# ----------------------------------------------------------------------------
# configs
# ----------------------------------------------------------------------------

# Shapes of the single 27B-class decoder layer (hidden 5120), Q4_0-style.
LAYER_27B = (
    ("q", 5120, 6144),
    ("k", 5120, 1024),
    ("v", 5120, 1024),
    ("o", 6144, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
)


def config0(seed_offset: int = 0) -> dict:
    """Tiny verify pass: M=4 rows x nvfp4 2048x2048, then a 2048->1024 nvfp4
    head and 3 uniform draft ids over the 1024-entry vocabulary."""
    r = streams(0, seed_offset)
    M, K, N, V = 4, 2048, 2048, 1024
    x = rand_bf16(r["x"], (M, K))
    w1 = rand_weight(FMT_NVFP4, r["codes"], r["scales"], N, K)
    head = rand_weight(FMT_NVFP4, r["head"], r["head"], V, N)
    drafts = r["drafts"].integers(0, V, size=M - 1, dtype=np.int64).astype(np.int32)
    return {"M": M, "x": x, "w1": w1, "head": head, "drafts": drafts, "V": V}


def config1(seed_offset: int = 0, M: int = 8, K: int = 4096, N: int = 14336) -> dict:
    """Dense FFN-up verify GEMM: x[M][4096] bf16, nvfp4 4096 -> 14336."""
    r = streams(1, seed_offset)
    x = rand_bf16(r["x"], (M, K))
    w = rand_weight(FMT_NVFP4, r["codes"], r["scales"], N, K)
    return {"M": M, "x": x, "w": w}


def config2(seed_offset: int = 0, M: int = 8, shapes=LAYER_27B) -> dict:
    """One 27B-class decoder layer's projections, Q4_0-style weights."""
    r = streams(2, seed_offset)
    out = {"M": M, "proj": {}}
    for name, K, N in shapes:
        out["proj"][name] = {
            "x": rand_bf16(r["x"], (M, K)),
            "w": rand_weight(FMT_Q4_0, r["codes"], r["scales"], N, K),
        }
    return out


def config3_inputs(seed_offset: int = 0, M: int = 8, K: int = 5376, V: int = 262144,
                   alpha: float = 0.1) -> dict:
    """LM-head verification + acceptance inputs.  The planted match length L
    and the filler ids are drawn here; turning L into draft ids needs the
    target's argmax, which the caller supplies (the oracle's in the tests)."""
    r = streams(3, seed_offset)
    x = rand_bf16(r["x"], (M, K))
    w = rand_weight(FMT_NVFP4, r["codes"], r["scales"], V, K)
    L = int(r["drafts"].integers(0, M))          # uniform over 0..M-1
    filler = r["drafts"].integers(0, V, size=M - 1, dtype=np.int64).astype(np.int32)
    miss = r["drafts"].integers(1, V, size=M - 1, dtype=np.int64).astype(np.int32)
    q = rand_dirichlet_rows(r["q"], M - 1, V, alpha)
    u = rand_uniforms(r["uniforms"], M)
    return {"M": M, "K": K, "V": V, "x": x, "w": w, "L": L, "filler": filler,
            "miss": miss, "q": q, "u": u, "temperature": 0.6, "top_p": 0.95}


def plant_drafts(argmax_rows: np.ndarray, L: int, filler: np.ndarray, miss: np.ndarray,
                 V: int) -> np.ndarray:
    """Draft ids whose first L entries equal the given per-row argmax, whose
    entry L differs from it (argmax + miss offset, mod V), and whose later
    entries are the uniform filler ids."""
    n = len(filler)
    d = filler.copy()
    for i in range(min(L, n)):
        d[i] = argmax_rows[i]
    if L < n:
        d[L] = (int(argmax_rows[L]) + int(miss[L])) % V
    return d.astype(np.int32)


def config4(seed_offset: int = 0, T: int = 8, E: int = 128, topk: int = 8,
            H: int = 2048, F: int = 768) -> dict:
    """MoE verify pass: T tokens, E experts, top-k routing, each expert a
    gated FFN H -> F -> H with nvfp4 weights (gate and up stacked along N)."""
    r = streams(4, seed_offset)
    x = rand_bf16(r["x"], (T, H))
    gu_codes = rand_codes(r["codes"], E * 2 * F, H).reshape(E, 2 * F, H // 2)
    gu_scales = rand_nvfp4_scales(r["scales"], E * 2 * F, H).reshape(E, 2 * F, H // 16)
    dn_codes = rand_codes(r["head"], E * H, F).reshape(E, H, F // 2)
    dn_scales = rand_nvfp4_scales(r["head"], E * H, F).reshape(E, H, F // 16)
    ids, gw = rand_routing(r["routing"], T, E, topk)
    return {"T": T, "E": E, "topk": topk, "H": H, "F": F, "x": x,
            "gate_up": {"format": FMT_NVFP4, "codes": gu_codes, "scales": gu_scales,
                        "g": np.ones(E, np.float32)},
            "down": {"format": FMT_NVFP4, "codes": dn_codes, "scales": dn_scales,
                     "g": np.ones(E, np.float32)},
            "ids": ids, "gw": gw}


def spread_logits(seed: int, M: int, V: int) -> np.ndarray:
    """Logits ~ N(0,1) fp32 (a wide nucleus at T=0.6, top_p=0.95)."""
    rng = np.random.default_rng(np.random.SeedSequence(99_000 + seed))
    return rng.standard_normal((M, V), dtype=np.float32)


def weight_bytes(N: int, K: int) -> int:
    """Algorithmic weight bytes: 4-bit codes plus block scales (both formats
    carry 9/16 byte per weight)."""
    return N * K // 2 + N * K // 16
