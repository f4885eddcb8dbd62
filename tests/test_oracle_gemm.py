"""Pins for the oracle's verify GEMM.

Each test checks the oracle against something other than itself: exact
rational arithmetic, library element decoders with an independently written
nibble packer, closed forms, and algebraic invariants.  Together they catch a
swapped nibble order, a wrong scale index, a dropped offset or global scale, a
transposed operand, a dropped term or a wrong sign.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "e2m1_table.json")) as _f:
    E2M1 = np.array(json.load(_f)["values"], dtype=np.float64)


# --------------------------------------------------------------------------
# independent helpers (library decoders + a packer written from the layout)
# --------------------------------------------------------------------------

def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[N][K] nibble values -> [N][K/2] bytes, element k in byte k/2, low
    nibble for even k."""
    nib = nib.astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def lib_e4m3(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def lib_f16(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def lib_bf16(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def unpack_for_test(codes):
    lo = codes & 15
    hi = codes >> 4
    N, H = codes.shape
    nib = np.empty((N, 2 * H), np.int64)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    return nib


def dense_weights(w) -> np.ndarray:
    """[N][K] float64 weight values via library decoders."""
    nib = unpack_for_test(w["codes"])
    N, K = nib.shape
    if w["format"] == W.FMT_NVFP4:
        s = np.repeat(lib_e4m3(w["scales"]), 16, axis=1)
        return float(w.get("g", 1.0)) * s * E2M1[nib]
    d = np.repeat(lib_f16(w["scales"]), 32, axis=1)
    return float(w.get("g", 1.0)) * d * (nib - 8)


def small_weight(fmt, N, K, seed, g=1.0):
    rng = np.random.default_rng(seed)
    w = W.rand_weight(fmt, rng, rng, N, K)
    w["g"] = g
    return w


# --------------------------------------------------------------------------
# G-1: brute force in exact rationals
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (3, 64, 4), (8, 32, 3), (16, 64, 2)])
def test_gemm_matches_exact_rationals(fmt, M, K, N):
    w = small_weight(fmt, N, K, seed=M * 100 + K + N, g=0.75)
    rng = np.random.default_rng(K + M)
    x = W.rand_bf16(rng, (M, K))
    y, b = oracle.gemm(w, x)
    wd = dense_weights(w)
    xd = lib_bf16(x)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(xd[m, k]) * Fraction(wd[n, k]) for k in range(K)), Fraction(0))
            mag = sum((abs(Fraction(xd[m, k]) * Fraction(wd[n, k])) for k in range(K)), Fraction(0))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(K * 2.0 ** -52) * mag
            assert abs(Fraction(b[m, n]) - mag) <= Fraction(K * 2.0 ** -52) * mag


# --------------------------------------------------------------------------
# G-2: one-hot readout pins layout, scale indexing, offset and global scale
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_one_hot_readout_recovers_each_weight(fmt):
    N, K = 5, 96
    rng = np.random.default_rng(11)
    nib = rng.integers(0, 16, size=(N, K))
    if fmt == W.FMT_NVFP4:
        sbits = W.to_e4m3_bits(np.exp2(rng.uniform(-4, 2, size=(N, K // 16))))
        sval = np.repeat(lib_e4m3(sbits), 16, axis=1)
        val = sval * E2M1[nib]
    else:
        sbits = W.to_f16_bits(np.abs(rng.normal(0, 0.02, size=(N, K // 32))))
        sval = np.repeat(lib_f16(sbits), 32, axis=1)
        val = sval * (nib - 8)
    g = 1.5
    w = {"format": fmt, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sbits, "g": g}
    one = W.to_bf16_bits(np.eye(K, dtype=np.float32))      # K one-hot rows
    for k0 in range(0, K, 16):
        y, _ = oracle.gemm(w, one[k0:k0 + 16])
        assert np.array_equal(y, g * val[:, k0:k0 + 16].T)


# --------------------------------------------------------------------------
# G-4: exact regime -- integer activations and power-of-two scales
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_exact_regime_is_exact(fmt):
    M, N, K = 8, 7, 256
    rng = np.random.default_rng(5)
    x = W.to_bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    nib = rng.integers(0, 16, size=(N, K))
    if fmt == W.FMT_NVFP4:
        sbits = W.to_e4m3_bits(np.exp2(rng.integers(-1, 3, size=(N, K // 16))).astype(np.float32))
    else:
        sbits = W.to_f16_bits(np.exp2(rng.integers(-3, 2, size=(N, K // 32))))
    w = {"format": fmt, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sbits, "g": 1.0}
    y, _ = oracle.gemm(w, x)
    exact = lib_bf16(x) @ dense_weights(w).T          # every partial sum exact in fp64
    assert np.array_equal(y, exact)


# --------------------------------------------------------------------------
# G-5: closed forms and invariants
# --------------------------------------------------------------------------

def test_constant_code_and_scale_closed_form():
    M, N, K = 4, 3, 128
    rng = np.random.default_rng(2)
    x = W.rand_bf16(rng, (M, K))
    sx = lib_bf16(x).sum(axis=1)
    # nvfp4: code 0x3 (=1.5) everywhere, scale 0x40 (=2.0), g = 0.5
    w = {"format": W.FMT_NVFP4, "N": N, "K": K, "codes": np.full((N, K // 2), 0x33, np.uint8),
         "scales": np.full((N, K // 16), 0x40, np.uint8), "g": 0.5}
    y, _ = oracle.gemm(w, x)
    for n in range(N):
        np.testing.assert_allclose(y[:, n], 0.5 * 2.0 * 1.5 * sx, rtol=1e-13, atol=1e-13)
    # Q4_0: code 0xA (=+2) everywhere, scale 0.25
    wq = {"format": W.FMT_Q4_0, "N": N, "K": K, "codes": np.full((N, K // 2), 0xAA, np.uint8),
          "scales": W.to_f16_bits(np.full((N, K // 32), 0.25)), "g": 1.0}
    y, _ = oracle.gemm(wq, x)
    for n in range(N):
        np.testing.assert_allclose(y[:, n], 0.25 * 2 * sx, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_doubling_and_block_permutation(fmt):
    M, N, K = 3, 6, 256
    w = small_weight(fmt, N, K, seed=9)
    rng = np.random.default_rng(4)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    x = W.to_bf16_bits(xf)
    x2 = W.to_bf16_bits(2 * lib_bf16(x).astype(np.float32))
    y, _ = oracle.gemm(w, x)
    y2, _ = oracle.gemm(w, x2)
    assert np.array_equal(y2, 2 * y)                   # exact: scaling by 2
    # permute whole 32-wide blocks along K in x and W consistently
    perm = rng.permutation(K // 32)
    kidx = (perm[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    nib = unpack_for_test(w["codes"])[:, kidx]
    bs = 16 if fmt == W.FMT_NVFP4 else 32
    sidx = (perm[:, None] * (32 // bs) + np.arange(32 // bs)[None, :]).reshape(-1)
    wp = dict(w, codes=pack_nibbles(nib), scales=np.ascontiguousarray(w["scales"][:, sidx]))
    yp, bp = oracle.gemm(wp, np.ascontiguousarray(x[:, kidx]))
    _, b = oracle.gemm(w, x)
    np.testing.assert_allclose(yp, y, rtol=0, atol=K * 2.0 ** -52 * b.max())


def test_m_rows_equal_m_gemvs_and_column_subsets():
    M, N, K = 8, 20, 512
    w = small_weight(W.FMT_NVFP4, N, K, seed=21)
    x = W.rand_bf16(np.random.default_rng(8), (M, K))
    y, b = oracle.gemm(w, x)
    for m in range(M):
        ym, _ = oracle.gemm(w, x[m:m + 1])
        assert np.array_equal(ym[0], y[m])
    cols = [19, 0, 7, 7, 3]
    yc, bc = oracle.gemm(w, x, cols=cols)
    assert np.array_equal(yc, y[:, cols])
    assert np.array_equal(bc, b[:, cols])


def test_threads_do_not_change_results():
    w = small_weight(W.FMT_Q4_0, 33, 128, seed=1)
    x = W.rand_bf16(np.random.default_rng(1), (5, 128))
    y1, _ = oracle.gemm(w, x, nthreads=1)
    y7, _ = oracle.gemm(w, x, nthreads=7)
    assert np.array_equal(y1, y7)


def test_bad_shapes_rejected():
    w = small_weight(W.FMT_NVFP4, 4, 64, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm(w, W.rand_bf16(np.random.default_rng(0), (17, 64)))
