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
//  2. gate_up: grid = (tile groups) x (unique-expert slots); a workgroup
//              streams gate tiles and the matching up tiles of its expert
//              through the engine of the dense GEMM (engine.h) for all rows
//              of that expert and writes h = bf16(silu(gate) * up) per pair.
//  3. down:    the same for y[pair] = W_d[e] . h[pair].
//  4. combine: out[t] = sum over slots in slot order of w[t][s] * y[t, s].
// The grids are sized for the largest possible number of unique experts;
// slots beyond the actual count exit at once.  The K split of each expert
// matrix depends only on its shape, so a pair's result does not depend on
// which other tokens chose the same expert.
#include <algorithm>

#include "engine.h"
#include "internal.h"

namespace mtp {
namespace {

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
  const uint8_t *gu_packed;
  const float *gu_global;
  const uint8_t *dn_packed;
  const float *dn_global;
  float *out;
  uint16_t *h_out;
  int T, H, F, E, topk, P;
  int rc;                 // rows per engine pass
  struct { int TW, J, S, ppj; } gu, dn;
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

struct GateUpTiles {
  int TWh, Fg;   // gate tiles per workgroup, gate tiles of the expert
  __device__ __forceinline__ int operator()(int tg, int tw) const {
    const int t = tg * TWh + tw / 2;
    if (t >= Fg) return -1;
    return (tw & 1) ? Fg + t : t;   // slot 2q: gate tile, slot 2q + 1: the matching up tile
  }
};

struct GateUpEpi {
  const MoeArgs *a;
  int TWh, nthreads, mc, c0, first;
  float gsc;
  __device__ __forceinline__ void operator()(int tg, const f32x4 *fin) const {
    const int cols = TWh * 16;
    for (int o = threadIdx.x; o < mc * cols; o += nthreads) {
      const int m = o / cols, c = o - m * cols;
      const int f = tg * cols + c;
      if (f < a->F) {
        const int q = c >> 4;
        const float gate = gsc * eng::fin_at(fin, 2 * q, m, c & 15);
        const float up = gsc * eng::fin_at(fin, 2 * q + 1, m, c & 15);
        const uint16_t hb = f32_to_bf16_rne(silu(gate) * up);
        const int pair = a->spair[first + c0 + m];
        a->h[(int64_t)pair * a->F + f] = hb;
        if (a->h_out) a->h_out[(int64_t)pair * a->F + f] = hb;
      }
    }
  }
};

template <int FMT>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_gate_up(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int P = eng::pairs_of(a.H);
  const uint8_t *w = a.gu_packed + (int64_t)e * eng::packed_bytes(2 * a.F, a.H);
  eng::Plan pl;
  pl.TW = a.gu.TW; pl.J = a.gu.J; pl.S = a.gu.S; pl.ppj = a.gu.ppj; pl.KG = 1; pl.kg = 0;
  pl.tg_first = blockIdx.x; pl.tg_step = gridDim.x; pl.tg_count = 1;
  const GateUpTiles tiles{pl.TW / 2, a.F / 16};
  const float gsc = a.gu_global ? a.gu_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += a.rc) {
    const int mc = min(a.rc, rows - c0);
    const eng::XSource xs{a.x, a.H, a.stok + first + c0};
    eng::run<FMT, eng::kPPShallow>(w, P, a.H, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr},
                                   lds, c0 > 0,
                                   GateUpEpi{&a, pl.TW / 2, pl.TW * pl.J * kWave, mc, c0, first, gsc});
  }
}

struct DownEpi {
  const MoeArgs *a;
  int TW, nthreads, mc, c0, first;
  float gsc;
  __device__ __forceinline__ void operator()(int tg, const f32x4 *fin) const {
    const int cols = TW * 16;
    for (int o = threadIdx.x; o < mc * cols; o += nthreads) {
      const int m = o / cols, c = o - m * cols;
      const int n = tg * cols + c;
      if (n < a->H)
        a->y[(int64_t)a->spair[first + c0 + m] * a->H + n] = gsc * eng::fin_at(fin, c >> 4, m, c & 15);
    }
  }
};

struct DownTiles {
  int TW, T;
  __device__ __forceinline__ int operator()(int tg, int tw) const {
    const int t = tg * TW + tw;
    return t < T ? t : -1;
  }
};

template <int FMT>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_down(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int P = eng::pairs_of(a.F);
  const uint8_t *w = a.dn_packed + (int64_t)e * eng::packed_bytes(a.H, a.F);
  eng::Plan pl;
  pl.TW = a.dn.TW; pl.J = a.dn.J; pl.S = a.dn.S; pl.ppj = a.dn.ppj; pl.KG = 1; pl.kg = 0;
  pl.tg_first = blockIdx.x; pl.tg_step = gridDim.x; pl.tg_count = 1;
  const DownTiles tiles{pl.TW, eng::tiles_of(a.H)};
  const float gsc = a.dn_global ? a.dn_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += a.rc) {
    const int mc = min(a.rc, rows - c0);
    const eng::XSource xs{a.h, a.F, a.spair + first + c0};
    eng::run<FMT, eng::kPPShallow>(w, P, a.F, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr},
                                   lds, c0 > 0,
                                   DownEpi{&a, pl.TW, pl.TW * pl.J * kWave, mc, c0, first, gsc});
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

// Engine shape of one expert matrix: a single workgroup covers all slices
// (S of about 8 pairs each); rc rows are staged per pass.
struct MoePlan {
  int TW, J, S, ppj, tg, threads;
  size_t lds;
};

MoePlan moe_plan(int format, int N, int K, int rc, int tw_max, bool paired) {
  MoePlan m;
  const int P = eng::pairs_of(K);
  m.S = std::max(1, std::min((P + 4) / 8, paired ? eng::kWgWaves / 2 : eng::kWgWaves));
  m.ppj = (P + m.S - 1) / m.S;
  m.S = (P + m.ppj - 1) / m.ppj;
  m.J = m.S;
  m.TW = std::max(paired ? 2 : 1, std::min(tw_max, eng::kWgWaves / m.J));
  if (paired) m.TW &= ~1;
  const int tiles = paired ? eng::tiles_of(N) / 2 : eng::tiles_of(N);
  const int per = paired ? m.TW / 2 : m.TW;
  m.tg = (tiles + per - 1) / per;
  m.threads = m.TW * m.J * kWave;
  m.lds = eng::lds_bytes(format, rc, std::min(m.J * m.ppj, P), m.TW, m.J);
  return m;
}

// Rows staged per pass: up to 16 (and T, which bounds the rows of an expert
// unless a token repeats an expert), fewer if the staged rows would not fit.
int moe_rows(int format, int T, int H, int F) {
  int rc = std::min(16, T);
  while (rc > 1 && (moe_plan(format, 2 * F, H, rc, 4, true).lds > 144 * 1024 ||
                    moe_plan(format, H, F, rc, 8, false).lds > 144 * 1024))
    --rc;
  return rc;
}

}  // namespace

bool moe_fits(int format, int T, int H, int F) {
  const int rc = moe_rows(format, T, H, F);
  return moe_plan(format, 2 * F, H, rc, 4, true).lds <= 144 * 1024 &&
         moe_plan(format, H, F, rc, 8, false).lds <= 144 * 1024;
}

size_t moe_ws_bytes(int T, int H, int F, int E, int topk) {
  (void)E;
  return moe_layout(T, H, F, topk).bytes;
}

hipError_t launch_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                      const int32_t *ids, const float *gw, const uint8_t *gu_packed,
                      const float *gu_global, const uint8_t *dn_packed, const float *dn_global,
                      float *out, uint16_t *h_out, void *ws, hipStream_t stream) {
  const MoeLayout L = moe_layout(T, H, F, topk);
  uint8_t *w = static_cast<uint8_t *>(ws);
  MoeArgs a;
  a.x = x; a.ids = ids; a.gw = gw;
  a.gu_packed = gu_packed; a.gu_global = gu_global;
  a.dn_packed = dn_packed; a.dn_global = dn_global;
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
  a.rc = moe_rows(format, T, H, F);
  const MoePlan gu = moe_plan(format, 2 * F, H, a.rc, 4, true);
  const MoePlan dn = moe_plan(format, H, F, a.rc, 8, false);
  a.gu = {gu.TW, gu.J, gu.S, gu.ppj};
  a.dn = {dn.TW, dn.J, dn.S, dn.ppj};
  const int slots = (a.P < E) ? a.P : E;
  hipLaunchKernelGGL(moe_route, dim3(1), dim3(kMaxPairs), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 gu_grid(gu.tg, slots), dn_grid(dn.tg, slots);
  if (format == MTP_FMT_NVFP4) {
    eng::allow_large_lds(moe_gate_up<MTP_FMT_NVFP4>);
    eng::allow_large_lds(moe_down<MTP_FMT_NVFP4>);
    hipLaunchKernelGGL(moe_gate_up<MTP_FMT_NVFP4>, gu_grid, dim3(gu.threads), gu.lds, stream, a);
    hipLaunchKernelGGL(moe_down<MTP_FMT_NVFP4>, dn_grid, dim3(dn.threads), dn.lds, stream, a);
  } else {
    eng::allow_large_lds(moe_gate_up<MTP_FMT_Q4_0>);
    eng::allow_large_lds(moe_down<MTP_FMT_Q4_0>);
    hipLaunchKernelGGL(moe_gate_up<MTP_FMT_Q4_0>, gu_grid, dim3(gu.threads), gu.lds, stream, a);
    hipLaunchKernelGGL(moe_down<MTP_FMT_Q4_0>, dn_grid, dim3(dn.threads), dn.lds, stream, a);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t TH = (int64_t)T * H;
  hipLaunchKernelGGL(moe_combine, dim3((unsigned)((TH + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mtp
