"""GPU parity of mtp_verify_gemm against the fp64 oracle.

Bar: |y_gpu - y_oracle| <= 1e-3 * sum_k |x*w| + 1e-5 per output, and bitwise
equality where the exact result is representable and every fp32 partial sum
is exact (one-hot readout, integer activations with power-of-two scales).
Shapes span several tiles, several LDS chunks and K splits, ragged N and K
tails, M = 1..16, and the full workload sizes (sampled columns).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import DEV, assert_gemm_close, dev, gemm_gpu, host, log, pack_gpu

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")
FMTS = [W.FMT_NVFP4, W.FMT_Q4_0]
FNAME = {W.FMT_NVFP4: "nvfp4", W.FMT_Q4_0: "q4_0"}


def weight(fmt, N, K, seed, g=1.0):
    rng = np.random.default_rng(seed)
    w = W.rand_weight(fmt, rng, rng, N, K)
    w["g"] = g
    return w


def pack_nibbles(nib):
    nib = nib.astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("N,K", [(16, 32), (37, 96), (100, 256), (130, 1056), (70, 2080)])
def test_small_shapes(fmt, M, N, K):
    log("gemm small", FNAME[fmt], M, N, K)
    w = weight(fmt, N, K, seed=M * 1000 + N + K, g=0.75)
    x = W.rand_bf16(np.random.default_rng(N * K + M), (M, K))
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, f"{FNAME[fmt]} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_readout_is_exact(fmt):
    # x = e_k reads back weight (n, k) exactly: pins nibble order, scale
    # indexing, the hardware E2M1/E4M3 decode (all finite E4M3 scale codes),
    # the Q4_0 offset removal and the lane-group transpose.
    N, K = 48, 1024
    rng = np.random.default_rng(17)
    nib = rng.integers(0, 16, size=(N, K))
    if fmt == W.FMT_NVFP4:
        codes_all = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
        sc = rng.choice(codes_all, size=(N, K // 16))
        sc.reshape(-1)[:len(codes_all)] = codes_all
    else:
        sc = W.to_f16_bits(np.abs(rng.normal(0, 0.02, size=(N, K // 32))))
        sc.reshape(-1)[:8] = [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x8001, 0xFBFF, 0x3C00, 0x0000]
    w = {"format": fmt, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sc, "g": 1.0}
    for k0 in range(0, K, 16):
        x = W.to_bf16_bits(np.eye(K, dtype=np.float32)[k0:k0 + 16])
        y = gemm_gpu(bv, w, x)
        y_ref, _ = oracle.gemm(w, x)
        assert np.array_equal(y, y_ref), f"k0={k0}: first diff at {np.argwhere(y != y_ref)[0]}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(8, 96, 4096), (5, 333, 3104), (16, 64, 17408)])
def test_exact_regime_bitwise(fmt, M, N, K):
    log("gemm exact regime", FNAME[fmt], M, N, K)
    rng = np.random.default_rng(M + N + K)
    x = W.to_bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    nib = rng.integers(0, 16, size=(N, K))
    if fmt == W.FMT_NVFP4:
        sc = W.to_e4m3_bits(np.exp2(rng.integers(-1, 3, size=(N, K // 16))).astype(np.float32))
    else:
        sc = W.to_f16_bits(np.exp2(rng.integers(-3, 2, size=(N, K // 32))))
    w = {"format": fmt, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sc, "g": 1.0}
    y = gemm_gpu(bv, w, x)
    y_ref, _ = oracle.gemm(w, x)
    assert np.array_equal(y, y_ref)


def packed_reference(w):
    """The packed layout, written out from its definition in mtp_verify.h."""
    N, K, fmt = w["N"], w["K"], w["format"]
    T, P = -(-N // 16), -(-K // 256)
    codes = np.zeros((T * 16, P * 128), np.uint8)
    codes[:N, :K // 2] = w["codes"]
    if fmt == W.FMT_NVFP4:
        sc = np.zeros((T * 16, P * 16), np.uint8)
        sc[:N, :K // 16] = w["scales"]
    else:
        sc = np.zeros((T * 16, P * 8), np.uint16)
        sc[:N, :K // 32] = w["scales"]
    out = np.zeros((T, P, 2304), np.uint8)
    for t in range(T):
        for p in range(P):
            blk = out[t, p]
            for l in range(64):
                r, g = l % 16, l // 16
                row = 16 * t + r
                k0 = 256 * p + 32 * g
                if fmt == W.FMT_NVFP4:
                    blk[16 * l:16 * l + 16] = codes[row, k0 // 2:k0 // 2 + 16]
                    blk[1024 + 16 * l:1024 + 16 * l + 16] = codes[row, (k0 + 128) // 2:(k0 + 128) // 2 + 16]
                    blk[2048 + 4 * l:2048 + 4 * l + 4] = [sc[row, k0 // 16], sc[row, k0 // 16 + 1],
                                                          sc[row, (k0 + 128) // 16],
                                                          sc[row, (k0 + 128) // 16 + 1]]
                else:
                    for h in range(2):
                        for q in range(4):
                            k = 256 * p + 128 * h + 32 * q + 8 * g
                            o = 1024 * h + 16 * l + 4 * q
                            blk[o:o + 4] = codes[row, k // 2:k // 2 + 4]
                    if g == 0:
                        blk[2048 + 16 * r:2048 + 16 * r + 16] = \
                            sc[row, 8 * p:8 * p + 8].view(np.uint8)
    return out.reshape(-1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(16, 256), (37, 96), (130, 1056)])
def test_pack_matches_layout_definition(fmt, N, K):
    w = weight(fmt, N, K, seed=11)
    got = host(pack_gpu(bv, w))
    assert np.array_equal(got, packed_reference(w))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(300, 2304), (2048, 4096)])
def test_rows_do_not_depend_on_m(fmt, N, K):
    # the M-row pass equals M single-row passes, bit for bit, also where the
    # row count changes how the K slices are spread over workgroups
    w = weight(fmt, N, K, seed=5)
    x = W.rand_bf16(np.random.default_rng(6), (16, K))
    y16 = gemm_gpu(bv, w, x)
    for M in (1, 2, 5, 8):
        yM = gemm_gpu(bv, w, x[:M])
        assert np.array_equal(yM, y16[:M]), M
    for m in (0, 7, 15):
        assert np.array_equal(gemm_gpu(bv, w, x[m:m + 1])[0], y16[m])


@pytest.mark.parametrize("fmt", FMTS)
def test_strides_scale_and_bf16_output(fmt):
    N, K, M = 250, 1536, 6
    w = weight(fmt, N, K, seed=8, g=0.37)
    x = W.rand_bf16(np.random.default_rng(9), (M, K))
    y, yb = gemm_gpu(bv, w, x, ldx_pad=24, ldy_pad=7, want_bf16=True)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, "strided")
    # the bf16 copy is the nearest-even rounding of the fp32 result
    expect = W.to_bf16_bits(y.astype(np.float32))
    assert np.array_equal(yb, expect)


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_Q4_0])
def test_non_finite_activations(fmt):
    # an infinity in row 0 and a NaN in row 2.  nvfp4 (whose workgroups then
    # take the bf16 path) follows IEEE products and sums: +-inf where the
    # weight is nonzero, NaN where it is zero (inf * 0).  Q4_0 gives NaN in
    # every output of such a row (its per-block offset correction subtracts
    # the infinite block sum).  The other rows stay within the usual bound.
    N, K, M = 200, 1024, 4
    w = weight(fmt, N, K, seed=14)
    rng = np.random.default_rng(15)
    xf = rng.normal(size=(M, K)).astype(np.float32)
    xf[0, 77] = np.inf
    xf[2, 300] = np.nan
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    if fmt == W.FMT_NVFP4:
        assert np.array_equal(np.isnan(y), np.isnan(y_ref)), "NaN pattern"
        assert np.array_equal(np.isposinf(y), np.isposinf(y_ref)), "+inf pattern"
        assert np.array_equal(np.isneginf(y), np.isneginf(y_ref)), "-inf pattern"
    else:
        assert np.isnan(y[0]).all()
    assert np.isnan(y[2]).all() and not np.isfinite(y[0]).any()
    assert_gemm_close(y[[1, 3]], y_ref[[1, 3]], b_ref[[1, 3]], "finite rows")


@pytest.mark.parametrize("M", [1, 8])
def test_nvfp4_activations_outside_fp16_range(M):
    # nvfp4 activations are staged as fp16 when every value fits; a value
    # beyond the fp16 range sends the workgroup through the bf16 path, and
    # magnitudes below the fp16 normal range stay within the tolerance
    N, K = 200, 1536
    w = weight(W.FMT_NVFP4, N, K, seed=12)
    rng = np.random.default_rng(13)
    xf = rng.normal(size=(M, K)).astype(np.float32)
    xf[:, 5] = 3.0e5
    xf[0, 700] = -2.5e34          # times |w| <= 2688 stays inside fp32
    xf[:, 900:940] = 1.0e-30 * rng.normal(size=(M, 40))
    xf[:, 1000:1040] = 3.0e-6 * rng.normal(size=(M, 40))
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, "wide-range activations")
    # only tiny values: fp16 path throughout
    xs = W.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32) * 1e-5)
    y = gemm_gpu(bv, w, xs)
    y_ref, b_ref = oracle.gemm(w, xs)
    assert_gemm_close(y, y_ref, b_ref, "tiny activations")


def positive_nvfp4(N, K, seed):
    """nvfp4 weights with positive codes only (E2M1 0.5 .. 6), so that the
    products of same-signed activations never cancel."""
    rng = np.random.default_rng(seed)
    nib = rng.integers(1, 8, size=(N, K))
    sc = W.to_e4m3_bits(np.exp2(rng.uniform(-4, 2, size=(N, K // 16))).astype(np.float32))
    return {"format": W.FMT_NVFP4, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sc,
            "g": 1.0}


@pytest.mark.parametrize("M", [1, 8])
def test_nvfp4_tiny_same_signed_activations(M):
    # bf16 magnitudes below 2^-17 have bits below the fp16 subnormal spacing
    # (2^-24).  Same-signed rows against positive weights add every
    # truncation error with one sign, so a lossy fp16 copy misses the bound
    # by several times; the staging must keep them exact.
    N, K = 160, 4096
    w = positive_nvfp4(N, K, seed=41)
    rng = np.random.default_rng(42)
    xf = np.empty((M, K), np.float32)
    xf[0] = 1.0078125 * 2.0 ** -18                       # 2^-18 + 2^-25
    if M > 1:
        xf[1:] = np.exp2(rng.uniform(-24, -17, size=(M - 1, K)))   # uniform in exponent
        xf[2:4] = rng.uniform(2.0 ** -24, 2.0 ** -17, size=(2, K))
        xf[4:] *= -1.0
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, "tiny same-signed activations")


def test_nvfp4_tiny_one_hot_reads_largest_weight_exactly():
    # one activation (1 + 2^-7) * 2^-20 against weight 6 * 448 = 2688 (code 7,
    # scale 0x7E): the product is exact in fp32, so the result must be too
    N, K = 32, 512
    nib = np.full((N, K), 7)
    sc = np.full((N, K // 16), 0x7E, np.uint8)
    w = {"format": W.FMT_NVFP4, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sc,
         "g": 1.0}
    xf = np.zeros((4, K), np.float32)
    for m, k in enumerate((0, 129, 300, 511)):
        xf[m, k] = (1.0 + 2.0 ** -7) * 2.0 ** -20 * (-1.0 if m % 2 else 1.0)
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, _ = oracle.gemm(w, x)
    assert np.array_equal(y, y_ref)
    assert y_ref[0, 0] == 2688.0 * (1.0 + 2.0 ** -7) * 2.0 ** -20


@pytest.mark.parametrize("scale_exp", [-40, -20, 18, 60])
@pytest.mark.parametrize("M", [1, 8])
def test_nvfp4_scaled_exact_regime_bitwise(scale_exp, M):
    # integer activations times 2^scale_exp with power-of-two weight scales:
    # every product and partial sum is exact in fp32, so the GPU must match
    # the oracle bit for bit when the activations lie outside the fp16 window
    # (below 2^-17 or from 65536 up) as well as inside it
    N, K = 96, 2048
    rng = np.random.default_rng(43 + M)
    xf = rng.integers(-4, 5, size=(M, K)).astype(np.float64) * 2.0 ** scale_exp
    x = W.to_bf16_bits(xf.astype(np.float32))
    nib = rng.integers(0, 16, size=(N, K))
    sc = W.to_e4m3_bits(np.exp2(rng.integers(-1, 3, size=(N, K // 16))).astype(np.float32))
    w = {"format": W.FMT_NVFP4, "N": N, "K": K, "codes": pack_nibbles(nib), "scales": sc,
         "g": 1.0}
    y = gemm_gpu(bv, w, x)
    y_ref, _ = oracle.gemm(w, x)
    assert np.array_equal(y, y_ref)


def test_nvfp4_subnormal_and_mixed_range_activations():
    # bf16 subnormals (below 2^-126) alone, and rows spanning more than the
    # 33 binades one fp16 scale can hold (1e4 next to 1e-7: bf16 path)
    N, K, M = 200, 1024, 4
    w = weight(W.FMT_NVFP4, N, K, seed=44)
    rng = np.random.default_rng(45)
    xf = rng.integers(-4, 5, size=(M, K)).astype(np.float32) * np.float32(2.0 ** -130)
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, "subnormal activations")
    xf = rng.normal(size=(M, K)).astype(np.float32)
    xf[:, 3] = 1.0e4
    xf[:, 10:200] = 1.0e-7 * rng.normal(size=(M, 190))
    x = W.to_bf16_bits(xf)
    y = gemm_gpu(bv, w, x)
    y_ref, b_ref = oracle.gemm(w, x)
    assert_gemm_close(y, y_ref, b_ref, "mixed-range activations")


def test_deterministic_across_calls():
    N, K, M = 5120, 17408, 8          # K split over workgroups
    assert bv.gemm_plan_info(W.FMT_Q4_0, M, N, K)["KG"] > 1
    w = weight(W.FMT_Q4_0, N, K, seed=3)
    x = W.rand_bf16(np.random.default_rng(3), (M, K))
    packed = pack_gpu(bv, w)
    ws = bv.gemm_workspace(N, K, DEV)
    xd = dev(x)
    ys = []
    for _ in range(3):                # one workspace: its counters must return to zero
        y, _ = bv.verify_gemm(W.FMT_Q4_0, xd, packed, N, K, ws=ws)
        ys.append(host(y).astype(np.float64))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    assert not host(ws)[:4 * 320].any()
    y1 = ys[0]
    y_ref, b_ref = oracle.gemm(w, x, cols=np.arange(0, N, 7))
    assert_gemm_close(y1[:, ::7], y_ref, b_ref, "q4 down")


def test_one_workspace_serves_several_shapes():
    # K-split plans of different shapes in turn on one zeroed workspace: the
    # partial sums one shape leaves behind must not act as another shape's
    # arrival counters (small T first, then a larger T, then back)
    shapes = [(W.FMT_Q4_0, 512, 17408), (W.FMT_Q4_0, 5120, 17408), (W.FMT_NVFP4, 1024, 17408),
              (W.FMT_Q4_0, 512, 17408)]
    M = 4
    for fmt, N, K in shapes:
        assert bv.gemm_plan_info(fmt, M, N, K)["KG"] > 1, (N, K)
    need = max(bv.gemm_workspace_bytes(N, K) for _, N, K in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (fmt, N, K) in enumerate(shapes):
        log("shared workspace", i, FNAME[fmt], N, K)
        w = weight(fmt, N, K, seed=50 + i)
        x = W.rand_bf16(np.random.default_rng(60 + i), (M, K))
        y, _ = bv.verify_gemm(fmt, dev(x), pack_gpu(bv, w), N, K, ws=ws)
        cols = np.arange(0, N, 5)
        y_ref, b_ref = oracle.gemm(w, x, cols=cols)
        assert_gemm_close(host(y).astype(np.float64)[:, cols], y_ref, b_ref, f"shape {i}")
    assert not host(ws)[:256 * 1024].any()


# ---------------------------------------------------------------------------
# full workload sizes, sampled columns
# ---------------------------------------------------------------------------

def sample_cols(N, n=1536, seed=0):
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(min(N, 64)), np.arange(max(0, N - 64), N),
                                     rng.integers(0, N, n)]))
    return cols


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_ffn_up_4096x14336_nvfp4(M):
    cfg = W.config1(M=8)
    log("C1 M", M)
    x = cfg["x"][:M]
    y = gemm_gpu(bv, cfg["w"], x)
    cols = sample_cols(cfg["w"]["N"], seed=M)
    y_ref, b_ref = oracle.gemm(cfg["w"], x, cols=cols)
    assert_gemm_close(y[:, cols], y_ref, b_ref, f"C1 M={M}")


def test_dense_layer_q4_0_projections():
    cfg = W.config2(M=8)
    for name, p in cfg["proj"].items():
        log("C2", name)
        for M in (2, 8):
            y = gemm_gpu(bv, p["w"], p["x"][:M])
            cols = sample_cols(p["w"]["N"], n=512, seed=M)
            y_ref, b_ref = oracle.gemm(p["w"], p["x"][:M], cols=cols)
            assert_gemm_close(y[:, cols], y_ref, b_ref, f"C2 {name} M={M}")


def test_dense_layer_fused_qkv_and_gate_up():
    cfg = W.config2(M=8, shapes=(("q", 5120, 6144), ("k", 5120, 1024), ("v", 5120, 1024),
                                  ("gate", 5120, 17408), ("up", 5120, 17408)))
    p = cfg["proj"]
    x = p["q"]["x"]
    for names in (("q", "k", "v"), ("gate", "up")):
        ws = [p[n]["w"] for n in names]
        fused = {"format": W.FMT_Q4_0, "K": 5120, "N": sum(w["N"] for w in ws), "g": 1.0,
                 "codes": np.concatenate([w["codes"] for w in ws]),
                 "scales": np.concatenate([w["scales"] for w in ws])}
        log("C2 fused", names, fused["N"])
        y = gemm_gpu(bv, fused, x)
        cols = sample_cols(fused["N"], n=1024, seed=1)
        y_ref, b_ref = oracle.gemm(fused, x, cols=cols)
        assert_gemm_close(y[:, cols], y_ref, b_ref, f"fused {names}")


def test_lm_head_5376x262144_nvfp4():
    c = W.config3_inputs()
    log("C3 gemm")
    y = gemm_gpu(bv, c["w"], c["x"])
    cols = sample_cols(c["V"], n=2048, seed=3)
    y_ref, b_ref = oracle.gemm(c["w"], c["x"], cols=cols)
    assert_gemm_close(y[:, cols], y_ref, b_ref, "C3")
