"""Pins for the oracle's multi-row verify attention (Qiita roofline article,
§2-3: the verify candidates share one read of the KV prefix).

Pinned against: scipy's softmax with numpy's products on small cases (a
library routine), the closed form for identical keys (the mean of the
visible values), causality (keys after a row's position never change it,
earlier ones do), the equivalence of grouped heads with repeated KV heads,
and the error-scale bound."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W


def bf16(x):
    return W.to_bf16_bits(np.asarray(x, np.float32))


def val(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_case(rng, M, Hq, Hkv, D, L, extra=3):
    q = bf16(rng.standard_normal((M, Hq, D)).astype(np.float32))
    k = bf16(rng.standard_normal((Hkv, L + M + extra, D)).astype(np.float32))
    v = bf16(rng.standard_normal((Hkv, L + M + extra, D)).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("M,Hq,Hkv,D,L", [(1, 1, 1, 8, 0), (3, 4, 2, 16, 5), (4, 6, 3, 32, 40)])
def test_matches_scipy_softmax(M, Hq, Hkv, D, L):
    rng = np.random.default_rng(M + Hq + D + L)
    q, k, v = rand_case(rng, M, Hq, Hkv, D, L)
    o, ob = oracle.verify_attention(q, k, v, L, scale=0.3)
    G = Hq // Hkv
    for i in range(M):
        for h in range(Hq):
            n = L + i + 1
            s = 0.3 * val(k[h // G, :n]) @ val(q[i, h])
            p = softmax(s)
            assert np.allclose(o[i, h], p @ val(v[h // G, :n]), rtol=1e-12, atol=1e-14)
            assert np.allclose(ob[i, h], p @ np.abs(val(v[h // G, :n])), rtol=1e-12, atol=1e-14)


def test_identical_keys_average_the_visible_values():
    rng = np.random.default_rng(2)
    M, D, L = 4, 16, 9
    q, k, v = rand_case(rng, M, 2, 1, D, L)
    k[:] = k[:, :1]                       # every key equal: uniform weights
    o, _ = oracle.verify_attention(q, k, v, L)
    for i in range(M):
        ref = val(v[0, :L + i + 1]).mean(axis=0)
        assert np.allclose(o[i, 0], ref, rtol=1e-13) and np.allclose(o[i, 1], ref, rtol=1e-13)


def test_causality():
    rng = np.random.default_rng(3)
    M, D, L = 5, 16, 7
    q, k, v = rand_case(rng, M, 2, 1, D, L, extra=0)
    o, _ = oracle.verify_attention(q, k, v, L)
    k2, v2 = k.copy(), v.copy()
    k2[:, L + 2:] = bf16(rng.standard_normal((1, M - 2, D)).astype(np.float32))
    v2[:, L + 2:] = bf16(rng.standard_normal((1, M - 2, D)).astype(np.float32))
    o2, _ = oracle.verify_attention(q, k2, v2, L)
    assert np.array_equal(o[:2], o2[:2])          # rows 0, 1 see up to L + 1
    assert not np.allclose(o[2:], o2[2:])


def test_grouped_heads_equal_repeated_kv_heads():
    rng = np.random.default_rng(4)
    M, Hq, Hkv, D, L = 3, 6, 2, 16, 11
    q, k, v = rand_case(rng, M, Hq, Hkv, D, L)
    o, ob = oracle.verify_attention(q, k, v, L)
    G = Hq // Hkv
    o2, ob2 = oracle.verify_attention(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), L)
    assert np.array_equal(o, o2) and np.array_equal(ob, ob2)
    assert np.all(np.abs(o) <= ob * (1 + 1e-12))
