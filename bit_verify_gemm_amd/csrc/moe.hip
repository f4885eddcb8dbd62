// Routed-MoE verify pass with expert deduplication.
//
// Qiita roofline article, §3-2: in a verify mini-batch the candidate tokens
// can route to different experts, so the unique expert weights read grow
// with the batch ("expert scattering"), while routing correlation partly
// offsets it.  Ollama mtp.go commit log, flush message: MLX's segmented
// gather path for MoE heads needs tokens*topK/experts >= 4 to pay off; a
// verify batch (8 tokens, top-8 of 128) sits at 0.5, so here every unique
// expert is simply read once for all of its rows.
//
// Pipeline (all on the device, no host round trip):
//  1. route:   one workgroup sorts the T*topk (expert, pair) keys, lists the
//              unique experts and each expert's pairs in pair order.
//  2. gate_up: grid = (F tiles) x (unique-expert slots); a wave computes a
//              gate tile and the matching up tile for all rows of its expert
//              and writes h = bf16(silu(gate) * up) per pair.
//  3. down:    grid = (H tiles) x (slots); y[pair] = W_d[e] . h[pair].
//  4. combine: out[t] = sum over slots in slot order of w[t][s] * y[t, s].
// The grids are sized for the largest possible number of unique experts;
// slots beyond the actual count exit at once.
#include "gemm_core.h"
#include "internal.h"

namespace mtp {
namespace {

using core::kThreads;
using core::kWaves;

constexpr int kMaxPairs = 1024;
constexpr int kInvalidKey = 0x7FFFFFFF - kMaxPairs;  // above e * kMaxPairs + p for e < 2^20

struct MoeLayout {
  size_t nuniq, uexp, ustart, ucount, spair, stok, h, y, bytes;
};

MoeLayout moe_layout(int T, int H, int F, int topk) {
  const size_t P = (size_t)T * topk;
  MoeLayout L;
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  L.nuniq = take(sizeof(int32_t));
  L.uexp = take(sizeof(int32_t) * P);
  L.ustart = take(sizeof(int32_t) * P);
  L.ucount = take(sizeof(int32_t) * P);
  L.spair = take(sizeof(int32_t) * P);
  L.stok = take(sizeof(int32_t) * P);
  L.h = take(sizeof(uint16_t) * P * F);
  L.y = take(sizeof(float) * P * H);
  L.bytes = o;
  return L;
}

struct MoeArgs {
  const uint16_t *x;
  const int32_t *ids;
  const float *gw;
  const uint8_t *gu_codes;
  const void *gu_scales;
  const float *gu_global;
  const uint8_t *dn_codes;
  const void *dn_scales;
  const float *dn_global;
  float *out;
  uint16_t *h_out;
  int T, H, F, E, topk, P;
  int32_t *nuniq, *uexp, *ustart, *ucount, *spair, *stok;
  uint16_t *h;
  float *y;
};

__global__ __launch_bounds__(kMaxPairs) void moe_route(MoeArgs a) {
  __shared__ int32_t key[kMaxPairs];
  __shared__ int32_t sorted[kMaxPairs];
  __shared__ int32_t start[kMaxPairs];
  const int p = threadIdx.x;
  const int P = a.P;
  int e = -1;
  if (p < P) {
    e = a.ids[p];
    if (e < 0 || e >= a.E) e = -1;
    // distinct keys: invalid pairs sort after every valid one, in pair order
    key[p] = (e < 0) ? kInvalidKey + p : e * kMaxPairs + p;
  }
  __syncthreads();
  int rank = 0;
  if (p < P) {
    for (int q = 0; q < P; ++q) rank += key[q] < key[p];
    sorted[rank] = p;
  }
  __syncthreads();
  // a sorted position starts a new expert when its expert differs from the
  // previous one; invalid pairs sort last and start nothing
  if (p < P) {
    const int pp = sorted[p];
    const int ke = key[pp];
    const bool valid = ke < kInvalidKey;
    const bool first = valid && (p == 0 || key[sorted[p - 1]] / kMaxPairs != ke / kMaxPairs);
    start[p] = first ? 1 : 0;
    a.spair[p] = pp;
    a.stok[p] = pp / a.topk;
  }
  __syncthreads();
  if (p == 0) {
    int u = 0, prev = -1;
    for (int i = 0; i < P; ++i) {
      if (key[sorted[i]] >= kInvalidKey) break;
      if (start[i]) {
        if (prev >= 0) a.ucount[u - 1] = i - prev;
        a.uexp[u] = key[sorted[i]] / kMaxPairs;
        a.ustart[u] = i;
        prev = i;
        ++u;
      }
    }
    if (prev >= 0) {
      int end = prev;
      while (end < P && key[sorted[end]] < kInvalidKey) ++end;
      a.ucount[u - 1] = end - prev;
    }
    *a.nuniq = u;
  }
  // rows of h for invalid pairs are zero
  if (a.h_out && p < P && e < 0)
    for (int f = 0; f < a.F; ++f) a.h_out[(int64_t)p * a.F + f] = 0;
}

// silu(v) = v / (1 + exp(-v)), written so that no intermediate overflows:
// for v < 0 it is v * e / (1 + e) with e = exp(v) (gradual underflow).
__device__ __forceinline__ float silu(float v) {
  if (v >= 0.0f) return v / (1.0f + expf(-v));
  const float e = expf(v);
  return v * e / (1.0f + e);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_gate_up(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, F = a.F;
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int f0 = (blockIdx.x * kWaves + wave) * 16;
  const int frow = min(f0 + r, F - 1);
  const uint8_t *cb = a.gu_codes + (int64_t)e * (2 * F) * (H / 2);
  const int bs = (FMT == MTP_FMT_NVFP4) ? 16 : 32;
  const int ssz = (FMT == MTP_FMT_NVFP4) ? 1 : 2;
  const uint8_t *sb = static_cast<const uint8_t *>(a.gu_scales) + (int64_t)e * (2 * F) * (H / bs) * ssz;
  const uint8_t *crow[2] = {cb + (int64_t)frow * (H / 2), cb + (int64_t)(F + frow) * (H / 2)};
  const void *srow[2] = {core::scale_row<FMT>(sb, frow, H), core::scale_row<FMT>(sb, F + frow, H)};
  const float gsc = a.gu_global ? a.gu_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += 16) {
    const int mc = min(16, rows - c0);
    const core::XSource xs{a.x, H, a.stok + first + c0};
    f32x4 acc[2];
    core::run_tiles<FMT, 2>(acc, crow, srow, xs, mc, H, 0, H, lds);
    const int f = f0 + r;
    if (f < F) {
      const float gv[4] = {acc[0].x, acc[0].y, acc[0].z, acc[0].w};
      const float uv[4] = {acc[1].x, acc[1].y, acc[1].z, acc[1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < mc) {
          const float gate = gsc * gv[i], up = gsc * uv[i];
          const float act = silu(gate);
          const uint16_t hb = f32_to_bf16_rne(act * up);
          const int pair = a.spair[first + c0 + m];
          a.h[(int64_t)pair * F + f] = hb;
          if (a.h_out) a.h_out[(int64_t)pair * F + f] = hb;
        }
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_down(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, F = a.F;
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int n0 = (blockIdx.x * kWaves + wave) * 16;
  const int nrow = min(n0 + r, H - 1);
  const uint8_t *cb = a.dn_codes + (int64_t)e * H * (F / 2);
  const int bs = (FMT == MTP_FMT_NVFP4) ? 16 : 32;
  const int ssz = (FMT == MTP_FMT_NVFP4) ? 1 : 2;
  const uint8_t *sb = static_cast<const uint8_t *>(a.dn_scales) + (int64_t)e * H * (F / bs) * ssz;
  const uint8_t *crow[1] = {cb + (int64_t)nrow * (F / 2)};
  const void *srow[1] = {core::scale_row<FMT>(sb, nrow, F)};
  const float gsc = a.dn_global ? a.dn_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += 16) {
    const int mc = min(16, rows - c0);
    const core::XSource xs{a.h, F, a.spair + first + c0};
    f32x4 acc[1];
    core::run_tiles<FMT, 1>(acc, crow, srow, xs, mc, F, 0, F, lds);
    const int n = n0 + r;
    if (n < H) {
      const float v[4] = {acc[0].x, acc[0].y, acc[0].z, acc[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < mc) a.y[(int64_t)a.spair[first + c0 + m] * H + n] = gsc * v[i];
      }
    }
  }
}

__global__ __launch_bounds__(256) void moe_combine(MoeArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * a.H) return;
  const int t = (int)(i / a.H), n = (int)(i - (int64_t)t * a.H);
  float s = 0.0f;
  for (int k = 0; k < a.topk; ++k) {
    const int p = t * a.topk + k;
    const int e = a.ids[p];
    if (e >= 0 && e < a.E) s += a.gw[p] * a.y[(int64_t)p * a.H + n];
  }
  a.out[i] = s;
}

}  // namespace

size_t moe_ws_bytes(int T, int H, int F, int E, int topk) {
  (void)E;
  return moe_layout(T, H, F, topk).bytes;
}

hipError_t launch_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                      const int32_t *ids, const float *gw, const uint8_t *gu_codes,
                      const void *gu_scales, const float *gu_global, const uint8_t *dn_codes,
                      const void *dn_scales, const float *dn_global, float *out,
                      uint16_t *h_out, void *ws, hipStream_t stream) {
  const MoeLayout L = moe_layout(T, H, F, topk);
  uint8_t *w = static_cast<uint8_t *>(ws);
  MoeArgs a;
  a.x = x; a.ids = ids; a.gw = gw;
  a.gu_codes = gu_codes; a.gu_scales = gu_scales; a.gu_global = gu_global;
  a.dn_codes = dn_codes; a.dn_scales = dn_scales; a.dn_global = dn_global;
  a.out = out; a.h_out = h_out;
  a.T = T; a.H = H; a.F = F; a.E = E; a.topk = topk; a.P = T * topk;
  a.nuniq = reinterpret_cast<int32_t *>(w + L.nuniq);
  a.uexp = reinterpret_cast<int32_t *>(w + L.uexp);
  a.ustart = reinterpret_cast<int32_t *>(w + L.ustart);
  a.ucount = reinterpret_cast<int32_t *>(w + L.ucount);
  a.spair = reinterpret_cast<int32_t *>(w + L.spair);
  a.stok = reinterpret_cast<int32_t *>(w + L.stok);
  a.h = reinterpret_cast<uint16_t *>(w + L.h);
  a.y = reinterpret_cast<float *>(w + L.y);
  const int slots = (a.P < E) ? a.P : E;
  hipLaunchKernelGGL(moe_route, dim3(1), dim3(kMaxPairs), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t shm = core::lds_bytes(16, format);
  const dim3 gu_grid((F + kWaves * 16 - 1) / (kWaves * 16), slots);
  const dim3 dn_grid((H + kWaves * 16 - 1) / (kWaves * 16), slots);
  if (format == MTP_FMT_NVFP4) {
    hipLaunchKernelGGL(moe_gate_up<MTP_FMT_NVFP4>, gu_grid, dim3(kThreads), shm, stream, a);
    hipLaunchKernelGGL(moe_down<MTP_FMT_NVFP4>, dn_grid, dim3(kThreads), shm, stream, a);
  } else {
    hipLaunchKernelGGL(moe_gate_up<MTP_FMT_Q4_0>, gu_grid, dim3(kThreads), shm, stream, a);
    hipLaunchKernelGGL(moe_down<MTP_FMT_Q4_0>, dn_grid, dim3(kThreads), shm, stream, a);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t TH = (int64_t)T * H;
  hipLaunchKernelGGL(moe_combine, dim3((unsigned)((TH + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mtp
