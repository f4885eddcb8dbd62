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
// MI355X design:
//  * A wave owns a tile of 16 output columns (weight rows).  Each lane streams
//    16 contiguous code bytes (32 weights) of one row per 128-wide K step with
//    one 128-bit load; the 4 lane groups of a wave cover the step.
//  * Decoded weights feed v_mfma_f32_16x16x32_bf16 as the B operand; the M
//    activation rows (zero-padded to 16) are the A operand, read from LDS.
//    The matrix cores absorb the M-fold arithmetic that would otherwise bound
//    a vector-ALU kernel at M = 8, so the cost stays that of the weight stream.
//  * nvfp4: E2M1 x E4M3 products are exact in bf16, so weights are decoded
//    once per step directly into MFMA operands.
//  * Q4_0-style: d*(u-8) is not exact in bf16, so one MFMA covers exactly one
//    32-weight block on the raw codes (128+u, exact) with the accumulator
//    started at -136*sum(x) (removing the offset), and the fp16 block scale is
//    applied afterwards in fp32.  A lane-group transpose (permlane swaps) turns
//    the coalesced per-lane block loads into the per-MFMA block layout.
//  * Activations are staged in LDS in 1024-wide chunks shared by the four
//    waves of a workgroup; weight loads run several steps ahead of the math.
//  * Long K is split across workgroups; the fp32 partials are summed in a
//    fixed order by a second kernel, so results are deterministic.
#include "gemm_core.h"
#include "internal.h"

namespace mtp {
namespace {

using core::kThreads;
using core::kWaves;
using core::kStepK;

struct GemmArgs {
  const uint8_t *codes;
  const void *scales;
  const uint16_t *x;
  int64_t ldx;
  float *y;
  int64_t ldy;
  uint16_t *yb;
  int64_t ldyb;
  float *part;
  float gscale;
  int M, N, K;
  int split_k;
  int splits;
};

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int n0 = (blockIdx.x * kWaves + wave) * 16;
  const int nrow = min(n0 + r, N - 1);  // rows past N read row N-1, never stored
  const uint8_t *crow[1] = {p.codes + (int64_t)nrow * (K / 2)};
  const void *srow[1] = {core::scale_row<FMT>(p.scales, nrow, K)};
  const int k_begin = blockIdx.y * p.split_k;
  const int k_end = min(K, k_begin + p.split_k);
  const core::XSource xs{p.x, p.ldx, nullptr};
  f32x4 acc[1];
  core::run_tiles<FMT, 1>(acc, crow, srow, xs, M, K, k_begin, k_end, lds);

  const int n = n0 + r;
  if (n < N) {
    const float v[4] = {acc[0].x, acc[0].y, acc[0].z, acc[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M) {
        if (p.splits == 1) {
          const float o = p.gscale * v[i];
          if (p.y) p.y[(int64_t)m * p.ldy + n] = o;
          if (p.yb) p.yb[(int64_t)m * p.ldyb + n] = f32_to_bf16_rne(o);
        } else {
          p.part[((int64_t)blockIdx.y * M + m) * N + n] = v[i];
        }
      }
    }
  }
}

// Sum the split-K partials in split order, scale, store.
__global__ __launch_bounds__(256) void gemm_combine(const float *part, int splits, int M, int N,
                                                    float gscale, float *y, int64_t ldy,
                                                    uint16_t *yb, int64_t ldyb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;
  float s = 0.0f;
  for (int sp = 0; sp < splits; ++sp) s += part[sp * MN + i];
  const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  const float o = gscale * s;
  if (y) y[(int64_t)m * ldy + n] = o;
  if (yb) yb[(int64_t)m * ldyb + n] = f32_to_bf16_rne(o);
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K) {
  GemmPlan plan;
  const int groups = (N + kWaves * 16 - 1) / (kWaves * 16);
  const int steps = (K + kStepK - 1) / kStepK;
  const int target_wgs = 1024;  // about four workgroups per CU
  int splits = (target_wgs + groups - 1) / groups;
  splits = max(1, min(splits, steps / 4));
  const int per = (steps + splits - 1) / splits;
  splits = (steps + per - 1) / per;
  plan.splits = splits;
  plan.split_k = per * kStepK;
  plan.ws_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  return plan;
}

hipError_t launch_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                       const uint8_t *codes, const void *scales, float gscale, float *y,
                       int64_t ldy, uint16_t *yb, int64_t ldyb, void *ws, const GemmPlan &plan,
                       hipStream_t stream) {
  GemmArgs a;
  a.codes = codes; a.scales = scales; a.x = x; a.ldx = ldx;
  a.y = y; a.ldy = ldy; a.yb = yb; a.ldyb = ldyb;
  a.part = static_cast<float *>(ws);
  a.gscale = gscale; a.M = M; a.N = N; a.K = K;
  a.split_k = plan.split_k; a.splits = plan.splits;
  const dim3 grid((N + kWaves * 16 - 1) / (kWaves * 16), plan.splits);
  const size_t shm = core::lds_bytes(M, format);
  if (format == MTP_FMT_NVFP4)
    hipLaunchKernelGGL(gemm_kernel<MTP_FMT_NVFP4>, grid, dim3(kThreads), shm, stream, a);
  else
    hipLaunchKernelGGL(gemm_kernel<MTP_FMT_Q4_0>, grid, dim3(kThreads), shm, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL(gemm_combine, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream,
                     a.part, plan.splits, M, N, gscale, y, ldy, yb, ldyb);
  return hipGetLastError();
}

}  // namespace mtp
