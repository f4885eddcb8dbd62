// Verify GEMM: y[M][N] = x[M][K] . W for M = 1..16 rows against 4-bit
// block-quantised weights, reading every weight byte once for all rows.
//
// "Faster Gemma 4 on MLX with multi-token prediction", sixth paragraph: the
// verify batch (2-8 tokens) is too small for large-batch matmul kernels and
// too large for matrix-vector kernels; the useful kernel reads and unpacks
// each weight block once and reuses it across the batch.  Qiita roofline
// article, §2-3: the weight bytes stay those of one token while only the
// arithmetic grows, so the pass stays bound by memory bandwidth.
//
// MI355X design (the engine is in engine.h):
//  * Weights are repacked once (mtp_pack_weights) into 2304-byte blocks of
//    16 rows x 256 K that match the matrix-core operand layout, so a wave
//    streams 1 KiB code loads and one scale load per 128-wide K step.
//  * Decoded weights are the B operand of v_mfma_f32_16x16x32_bf16 and the
//    M activation rows (staged once in LDS) the A operand: the matrix cores
//    absorb the M-fold arithmetic that would otherwise bound a vector-ALU
//    kernel at M = 8, so the cost stays that of the weight stream.
//  * nvfp4: E2M1 x E4M3 products are exact in bf16, so every weight is
//    decoded once into an MFMA operand.  Q4_0-style: d*(u-8) is not exact in
//    bf16, so one MFMA covers exactly one 32-block on the exact values 128+u
//    with the accumulator started at -136*sum(x), and the fp16 scale is
//    applied in fp32 afterwards.
//  * The slice split of K is a function of the matrix shape only and partial
//    sums are added in slice order, so results are deterministic and a row's
//    result does not depend on M or on the other rows.
#include <algorithm>
#include <type_traits>

#include "engine.h"
#include "internal.h"

namespace mtp {
namespace {

using eng::kPairBytes;
using eng::kPairK;

// ---- packing ---------------------------------------------------------------

// One wave per (matrix, tile, pair) block; lane l = 16 g + r covers row
// 16 t + r.  Rows past N and K past the matrix are written as zero codes and
// zero scales, which contribute exactly nothing.
template <int FMT>
__global__ __launch_bounds__(64) void pack_kernel(const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ scales, int N,
                                                  int K, int T, int P,
                                                  uint8_t *__restrict__ out) {
  const int64_t blk = blockIdx.x;
  const int e = (int)(blk / ((int64_t)T * P));
  const int rem = (int)(blk - (int64_t)e * T * P);
  const int t = rem / P, p = rem - t * P;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const int n = 16 * t + r;
  const bool row_ok = n < N;
  const uint8_t *crow = codes + ((int64_t)e * N + (row_ok ? n : 0)) * (K / 2);
  uint8_t *o = out + blk * kPairBytes;
  if (FMT == MTP_FMT_NVFP4) {
    const uint8_t *srow = scales + ((int64_t)e * N + (row_ok ? n : 0)) * (K / 16);
    const int k0 = kPairK * p + 32 * g, k1 = k0 + 128;
    const bool ok0 = row_ok && k0 < K, ok1 = row_ok && k1 < K;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 c0 = ok0 ? *reinterpret_cast<const u32x4 *>(crow + k0 / 2) : z;
    const u32x4 c1 = ok1 ? *reinterpret_cast<const u32x4 *>(crow + k1 / 2) : z;
    const uint32_t s0 = ok0 ? *reinterpret_cast<const uint16_t *>(srow + k0 / 16) : 0u;
    const uint32_t s1 = ok1 ? *reinterpret_cast<const uint16_t *>(srow + k1 / 16) : 0u;
    *reinterpret_cast<u32x4 *>(o + 16 * lane) = c0;
    *reinterpret_cast<u32x4 *>(o + eng::kHalfBytes + 16 * lane) = c1;
    *reinterpret_cast<uint32_t *>(o + eng::kScaleOff + 4 * lane) = s0 | (s1 << 16);
  } else {
    const uint16_t *srow =
        reinterpret_cast<const uint16_t *>(scales) + ((int64_t)e * N + (row_ok ? n : 0)) * (K / 32);
    uint32_t d[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kPairK * p + 128 * h + 32 * q + 8 * g;
        d[4 * h + q] = (row_ok && k < K) ? *reinterpret_cast<const uint32_t *>(crow + k / 2) : 0u;
      }
    *reinterpret_cast<u32x4 *>(o + 16 * lane) = u32x4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x4 *>(o + eng::kHalfBytes + 16 * lane) = u32x4{d[4], d[5], d[6], d[7]};
    const int b0 = 8 * p + 2 * g, nb = K / 32;
    const uint32_t s0 = (row_ok && b0 < nb) ? srow[b0] : 0u;
    const uint32_t s1 = (row_ok && b0 + 1 < nb) ? srow[b0 + 1] : 0u;
    *reinterpret_cast<uint32_t *>(o + eng::kScaleOff + 16 * r + 4 * g) = s0 | (s1 << 16);
  }
}

// ---- dense GEMM ------------------------------------------------------------

struct GemmArgs {
  const uint8_t *w;
  const uint16_t *x;
  int64_t ldx;
  float *y;
  int64_t ldy;
  uint16_t *yb;
  int64_t ldyb;
  float gscale;
  int M, N, K, T, P;
  int TW, J, S, ppj, KG, TG, G;
  int tg_base, tg_rem;   // TG = tg_base * G + tg_rem: tile groups per workgroup without a division
  eng::Fixup fx;
};

struct DenseTiles {
  int TW, T;
  __device__ __forceinline__ int operator()(int tg, int tw) const {
    const int t = tg * TW + tw;
    return t < T ? t : -1;
  }
};

// Thread o writes output (m, c) = divmod(o, 16 TW) of the tile group, so a
// row's columns are stored by consecutive lanes.
struct DenseEpi {
  const GemmArgs *a;
  __device__ __forceinline__ void operator()(int tg, const f32x4 *fin) const {
    const int cols = a->TW * 16, nthreads = a->TW * a->J * kWave;
    for (int o = threadIdx.x; o < a->M * cols; o += nthreads) {
      const int m = o / cols, c = o - m * cols;
      const int n = tg * cols + c;
      if (n < a->N) {
        const float v = a->gscale * eng::fin_at(fin, c >> 4, m, c & 15);
        if (a->y) a->y[(int64_t)m * a->ldy + n] = v;
        if (a->yb) a->yb[(int64_t)m * a->ldyb + n] = f32_to_bf16_rne(v);
      }
    }
  }
};

template <int FMT, int PP>
__global__ __launch_bounds__(eng::kMaxThreads) void gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  eng::Plan pl;
  pl.TW = a.TW; pl.J = a.J; pl.S = a.S; pl.ppj = a.ppj; pl.KG = a.KG;
  // grid (KG, G): the K group runs fastest in launch order
  pl.kg = blockIdx.x;
  pl.tg_first = blockIdx.y;
  pl.tg_step = a.G;
  pl.tg_count = a.tg_base + (pl.tg_first < a.tg_rem ? 1 : 0);
  const eng::XSource xs{a.x, a.ldx, nullptr, 1};
  eng::run<FMT, PP, 1, false, false>(a.w, a.P, a.K, a.M, xs, pl, DenseTiles{a.TW, a.T}, a.fx,
                                     lds, false, DenseEpi{&a});
}

// Slices of the K range: a function of the shape only (see engine.h).
// Workgroups are 8 waves (TW tiles x J slices).  Small matrices (<= 128
// tiles) spread their K over up to 8 slices of at least 2 pairs so that
// enough waves stream;
// matrices of 768..1024 tiles take 2 slices (4 tiles per workgroup fill the
// CUs in one round); the rest take 4 (2 tiles per workgroup, several rounds
// or a persistent loop).  A slice holds at most kMaxPpj pairs so that one
// slice of MTP_MAX_M rows always fits the LDS of one workgroup.
constexpr int kMaxPpj = 16;

void slices(int T, int P, int &S, int &ppj) {
  int s;
  if (T <= 128) s = std::max(1, std::min(8, P / 2));   // slices of >= 2 pairs
  else if (T >= 768 && T <= 1024) s = 2;
  else s = 4;
  s = std::min(s, P);
  s = std::max(s, (P + kMaxPpj - 1) / kMaxPpj);
  ppj = (P + s - 1) / s;
  S = (P + ppj - 1) / ppj;
}

// Workspace of a K-split plan: the arrival counters (one per tile group,
// indexed below T) in a header of at least kCounterHeader bytes, then the
// slice partials.  Matrices of up to kCounterHeader / 4 tiles all put their
// partials past the same fixed header, so the partial sums one shape leaves
// behind never lie where another shape looks for its (zero) counters.
constexpr size_t kCounterHeader = 256 * 1024;

size_t counter_bytes(int T) {
  return std::max(kCounterHeader, ((size_t)T * 4 + 255) & ~(size_t)255);
}

size_t split_ws_bytes(int T, int S) { return counter_bytes(T) + (size_t)T * S * kWave * 16; }

}  // namespace

size_t packed_weight_bytes(int N, int K) { return eng::packed_bytes(N, K); }

hipError_t launch_pack(int format, int count, int N, int K, const uint8_t *codes,
                       const void *scales, uint8_t *packed, hipStream_t stream) {
  const int T = eng::tiles_of(N), P = eng::pairs_of(K);
  const int64_t blocks = (int64_t)count * T * P;
  const uint8_t *s = static_cast<const uint8_t *>(scales);
  if (format == MTP_FMT_NVFP4)
    hipLaunchKernelGGL(pack_kernel<MTP_FMT_NVFP4>, dim3((unsigned)blocks), dim3(64), 0, stream,
                       codes, s, N, K, T, P, packed);
  else
    hipLaunchKernelGGL(pack_kernel<MTP_FMT_Q4_0>, dim3((unsigned)blocks), dim3(64), 0, stream,
                       codes, s, N, K, T, P, packed);
  return hipGetLastError();
}

size_t gemm_ws_bytes(int N, int K) {
  const int T = eng::tiles_of(N), P = eng::pairs_of(K);
  int S, ppj;
  slices(T, P, S, ppj);
  if (S == 1) return 0;
  return split_ws_bytes(T, S);
}

GemmPlan gemm_plan(int format, int M, int N, int K) {
  GemmPlan pl;
  pl.T = eng::tiles_of(N);
  pl.P = eng::pairs_of(K);
  slices(pl.T, pl.P, pl.S, pl.ppj);
  const size_t budget = 144 * 1024;
  // slices per workgroup: all of them if the staged rows fit; otherwise one
  // (the K groups then meet through the workspace)
  pl.J = std::min(pl.S, eng::kWgWaves);
  auto fits = [&](int J) {
    return eng::lds_bytes(format, M, std::min(J * pl.ppj, pl.P), eng::kWgWaves / J, J) <= budget;
  };
  if (pl.J < pl.S || !fits(pl.J)) pl.J = 1;
  while (pl.J > 1 && !fits(pl.J)) --pl.J;
  pl.KG = (pl.S + pl.J - 1) / pl.J;
  // tiles per workgroup: fill the 8 waves
  pl.TW = 1;
  while (pl.TW * 2 * pl.J <= eng::kWgWaves) pl.TW *= 2;
  pl.TG = (pl.T + pl.TW - 1) / pl.TW;
  pl.threads = pl.TW * pl.J * kWave;
  pl.lds = eng::lds_bytes(format, M, std::min(pl.J * pl.ppj, pl.P), pl.TW, pl.J);
  return finish_plan(pl);
}

constexpr int kDeepPP[] = {3, 4, 5, 6, 8};   // blocks in flight a wave, one workgroup per CU

GemmPlan finish_plan(GemmPlan pl) {
  // Workgroups resident on 256 CUs by LDS and wave slots; when every tile
  // group has its own workgroup, one round; otherwise a persistent loop whose
  // load stream runs on across the tile groups of a workgroup.  A wave's
  // positions per tile group are rounded up to whole rounds of PP blocks in
  // flight (padding positions load empty windows and skip the arithmetic).
  // One round of workgroups (one tile group each) takes kPPDeep - 1 or
  // kPPDeep, whichever pads less (the deeper on a tie): deeper bursts only
  // queue behind the activation loads.  A persistent workgroup alone on its
  // CU (its 8 waves may hold up to 256 registers each) takes the depth of
  // kDeepPP that pads least, the deeper on a tie: up to a whole slice of 8
  // blocks in flight across its tile groups.  Two workgroups on one CU take
  // kPPShallow, whose registers leave room for both.
  int per_cu = (int)(eng::kMaxLds / std::max<size_t>(pl.lds + 1024, 1));
  per_cu = std::max(1, std::min(per_cu, eng::kMaxWaves / (pl.threads / kWave)));
  const int64_t one_round = std::max<int64_t>(1, 256 / pl.KG);
  auto pad = [&](int pp) { return (pl.ppj + pp - 1) / pp * pp - pl.ppj; };
  int deep = kDeepPP[0];
  for (int pp : kDeepPP)
    if (pad(pp) <= pad(deep)) deep = pp;
  if (pl.TG <= one_round) {
    pl.G = pl.TG;
    pl.PP = pad(eng::kPPDeep - 1) < pad(eng::kPPDeep) ? eng::kPPDeep - 1 : eng::kPPDeep;
  } else {
    const int64_t cap = std::max<int64_t>(1, (int64_t)256 * per_cu / pl.KG);
    pl.G = (int)std::min<int64_t>(pl.TG, cap);
    pl.PP = per_cu == 1 ? deep : eng::kPPShallow;
  }
  pl.grid = pl.G * pl.KG;
  pl.ws_bytes = pl.KG > 1 ? split_ws_bytes(pl.T, pl.S) : 0;
  return pl;
}

hipError_t launch_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                       const uint8_t *packed, float gscale, float *y, int64_t ldy, uint16_t *yb,
                       int64_t ldyb, void *ws, const GemmPlan &pl, hipStream_t stream) {
  GemmArgs a;
  a.w = packed; a.x = x; a.ldx = ldx;
  a.y = y; a.ldy = ldy; a.yb = yb; a.ldyb = ldyb;
  a.gscale = gscale; a.M = M; a.N = N; a.K = K; a.T = pl.T; a.P = pl.P;
  a.TW = pl.TW; a.J = pl.J; a.S = pl.S; a.ppj = pl.ppj; a.KG = pl.KG; a.TG = pl.TG; a.G = pl.G;
  a.tg_base = pl.TG / pl.G; a.tg_rem = pl.TG % pl.G;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  a.fx.cnt = reinterpret_cast<uint32_t *>(w8);
  a.fx.part = reinterpret_cast<f32x4 *>(w8 ? w8 + counter_bytes(pl.T) : nullptr);
  auto go = [&](auto kernel) {
    eng::allow_large_lds(kernel);
    hipLaunchKernelGGL(kernel, dim3(pl.KG, pl.G), dim3(pl.threads), pl.lds, stream, a);
  };
  // one kernel per (format, blocks in flight: kPPShallow or one of kDeepPP)
  auto pick = [&](auto fmt_tag) {
    constexpr int F = decltype(fmt_tag)::value;
    switch (pl.PP) {
      case 2: go(gemm_kernel<F, 2>); break;
      case 3: go(gemm_kernel<F, 3>); break;
      case 4: go(gemm_kernel<F, 4>); break;
      case 5: go(gemm_kernel<F, 5>); break;
      case 6: go(gemm_kernel<F, 6>); break;
      default: go(gemm_kernel<F, 8>); break;
    }
  };
  static_assert(eng::kPPShallow == 2, "a kernel exists for the shallow depth");
  if (format == MTP_FMT_NVFP4) pick(std::integral_constant<int, MTP_FMT_NVFP4>{});
  else pick(std::integral_constant<int, MTP_FMT_Q4_0>{});
  return hipGetLastError();
}

}  // namespace mtp
