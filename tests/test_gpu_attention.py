"""GPU parity of mtp_verify_attention against the oracle.

Bar, per element: |out - oracle| <= 1e-3 * sum_j p_j |v_j| + 1e-6, the
accuracy the verify GEMMs are held to (1e-3 of the magnitude sum of the
products), set by that requirement rather than by the kernel.  (The kernel
holds each probability as two bf16 parts, 16 significant bits, so its
products carry relative errors below 2^-17; its fp32 scores, softmax and
accumulation stay far inside the bar.)"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import DEV, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")


def case(seed, M, Hq, Hkv, D, L, extra=5, spread=1.0):
    rng = np.random.default_rng(seed)
    q = W.to_bf16_bits((rng.standard_normal((M, Hq, D)) * spread).astype(np.float32))
    k = W.to_bf16_bits(rng.standard_normal((Hkv, L + M + extra, D)).astype(np.float32))
    v = W.to_bf16_bits(rng.standard_normal((Hkv, L + M + extra, D)).astype(np.float32))
    return q, k, v


def check(q, k, v, L, what, scale=None):
    M, Hq, D = q.shape
    o = host(bv.verify_attention(dev(q), dev(k), dev(v), L, scale))
    ro, rb = oracle.verify_attention(q, k, v, L, scale)
    err = np.abs(o - ro)
    bar = 1e-3 * rb + 1e-6
    bad = err > bar
    log(what, "max err / bound", float((err / bar).max()))
    assert not bad.any(), f"{what}: {np.argwhere(bad)[:4].tolist()} gpu {o[bad][:4]} oracle {ro[bad][:4]}"


@pytest.mark.parametrize("M,Hq,Hkv,D,L", [
    (1, 1, 1, 64, 0), (1, 2, 2, 128, 31), (4, 8, 8, 128, 100), (8, 16, 2, 128, 1000),
    (16, 8, 1, 64, 37), (8, 32, 4, 256, 2048), (5, 6, 3, 64, 777), (16, 16, 2, 64, 300),
    (8, 4, 4, 256, 33), (2, 64, 1, 64, 500)])
def test_attention_matches_oracle(M, Hq, Hkv, D, L):
    q, k, v = case(M * 100 + Hq + D + L, M, Hq, Hkv, D, L)
    check(q, k, v, L, f"attn M={M} Hq={Hq} Hkv={Hkv} D={D} L={L}")


def test_peaked_scores_and_padded_cache():
    # large scores (a few keys dominate) and a cache with unused positions
    # holding non-finite garbage after L + M: they must never be read
    q, k, v = case(7, 8, 8, 2, 128, 500, extra=64, spread=4.0)
    nan = np.uint16(0x7FC0)
    k[:, 500 + 8:] = nan
    v[:, 500 + 8:] = nan
    check(q, k, v, 500, "peaked, NaN past the keys")


def test_long_context_gqa():
    # 8 verify rows, 32 query heads over 8 KV heads of dim 128, 32768 keys
    q, k, v = case(11, 8, 32, 8, 128, 32768 - 8, extra=0)
    check(q, k, v, 32768 - 8, "long context")
