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
  struct { int TW, J, S, ppj, tg; } gu, dn;
  int32_t *nuniq, *uexp, *ustart, *ucount, *spair, *stok;
  uint16_t *h;
  float *y;
};

// One workgroup of roundup(P, 64) threads: thread p ranks key p, then
// position p of the sorted order knows whether it starts an expert; block
// prefix counts of those starts number the unique experts.
__global__ __launch_bounds__(kMaxPairs) void moe_route(MoeArgs a) {
  __shared__ int32_t key[kMaxPairs];
  __shared__ int32_t sorted[kMaxPairs];
  __shared__ int32_t ustart[kMaxPairs];
  __shared__ int32_t wave_starts[kMaxPairs / kWave], wave_valid[kMaxPairs / kWave];
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
  if (p < P) {
    int rank = 0;
    for (int q = 0; q < P; ++q) rank += key[q] < key[p];
    sorted[rank] = p;
  }
  __syncthreads();
  // sorted position p starts an expert when its expert differs from the one
  // before; invalid pairs sort last and start nothing
  bool first = false, valid = false;
  int ke = 0;
  if (p < P) {
    const int pp = sorted[p];
    ke = key[pp];
    valid = ke < kInvalidKey;
    first = valid && (p == 0 || key[sorted[p - 1]] / kMaxPairs != ke / kMaxPairs);
    a.spair[p] = pp;
    a.stok[p] = pp / a.topk;
  }
  const uint64_t fb = __builtin_amdgcn_ballot_w64(first);
  const uint64_t vb = __builtin_amdgcn_ballot_w64(valid);
  const int w = p / kWave, l = p % kWave;
  if (l == 0) {
    wave_starts[w] = __builtin_popcountll(fb);
    wave_valid[w] = __builtin_popcountll(vb);
  }
  __syncthreads();
  int u = __builtin_popcountll(fb & ((1ull << l) - 1ull)), nuniq = 0, nvalid = 0;
  for (int q = 0; q < (int)(blockDim.x / kWave); ++q) {
    if (q < w) u += wave_starts[q];
    nuniq += wave_starts[q];
    nvalid += wave_valid[q];   // the valid positions are a prefix of the order
  }
  if (first) {
    ustart[u] = p;
    a.uexp[u] = ke / kMaxPairs;
    a.ustart[u] = p;
  }
  __syncthreads();
  if (p < nuniq) a.ucount[p] = (p + 1 < nuniq ? ustart[p + 1] : nvalid) - ustart[p];
  if (p == 0) *a.nuniq = nuniq;
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
  int TWh, Fg;   // gate tiles per tile group, gate tiles of the expert
  __device__ __forceinline__ int operator()(int tg, int s) const {
    const int t = tg * TWh + s / 2;
    if (t >= Fg) return -1;
    return (s & 1) ? Fg + t : t;   // slot 2q: gate tile, slot 2q + 1: the matching up tile
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
  // one wave holds gate tile tg * TWh + tw in acc[0] and its up tile in acc[1]
  __device__ __forceinline__ void wave(int tg, int tw, const f32x4 *acc) const {
    const int lane = threadIdx.x & (kWave - 1);
    const int f = (tg * TWh + tw) * 16 + (lane & 15);
    if (f >= a->F) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = eng::acc_row(lane, i);
      if (m < mc) {
        const float gate = gsc * acc[0][i], up = gsc * acc[1][i];
        const uint16_t hb = f32_to_bf16_rne(silu(gate) * up);
        const int pair = a->spair[first + c0 + m];
        a->h[(int64_t)pair * a->F + f] = hb;
        if (a->h_out) a->h_out[(int64_t)pair * a->F + f] = hb;
      }
    }
  }
};

// PAIRED: one wave streams a gate tile and its up tile together (J == 1)
template <int FMT, int PP, bool PAIRED>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_gate_up(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int P = eng::pairs_of(a.H);
  const uint8_t *w = a.gu_packed + (int64_t)e * eng::packed_bytes(2 * a.F, a.H);
  eng::Plan pl;
  pl.TW = a.gu.TW; pl.J = a.gu.J; pl.S = a.gu.S; pl.ppj = a.gu.ppj; pl.KG = 1; pl.kg = 0;
  pl.tg_first = blockIdx.x; pl.tg_step = gridDim.x;
  pl.tg_count = (a.gu.tg - pl.tg_first + gridDim.x - 1) / gridDim.x;
  const int TWh = PAIRED ? pl.TW : pl.TW / 2;
  const GateUpTiles tiles{TWh, a.F / 16};
  const float gsc = a.gu_global ? a.gu_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += a.rc) {
    const int mc = min(a.rc, rows - c0);
    const eng::XSource xs{a.x, a.H, a.stok + first + c0};
    eng::run<FMT, PP, PAIRED ? 2 : 1, PAIRED>(
        w, P, a.H, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr}, lds, c0 > 0,
        GateUpEpi{&a, TWh, pl.TW * pl.J * kWave, mc, c0, first, gsc});
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
  __device__ __forceinline__ void wave(int tg, int tw, const f32x4 *acc) const {
    const int lane = threadIdx.x & (kWave - 1);
    const int n = (tg * TW + tw) * 16 + (lane & 15);
    if (n >= a->H) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = eng::acc_row(lane, i);
      if (m < mc) a->y[(int64_t)a->spair[first + c0 + m] * a->H + n] = gsc * acc[0][i];
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

// LOCAL: one slice per tile (J == 1), each wave finishes its own tile
template <int FMT, int PP, bool LOCAL>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_down(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= *a.nuniq) return;  // whole workgroup
  const int e = a.uexp[slot], first = a.ustart[slot], rows = a.ucount[slot];
  const int P = eng::pairs_of(a.F);
  const uint8_t *w = a.dn_packed + (int64_t)e * eng::packed_bytes(a.H, a.F);
  eng::Plan pl;
  pl.TW = a.dn.TW; pl.J = a.dn.J; pl.S = a.dn.S; pl.ppj = a.dn.ppj; pl.KG = 1; pl.kg = 0;
  pl.tg_first = blockIdx.x; pl.tg_step = gridDim.x;
  pl.tg_count = (a.dn.tg - pl.tg_first + gridDim.x - 1) / gridDim.x;
  const DownTiles tiles{pl.TW, eng::tiles_of(a.H)};
  const float gsc = a.dn_global ? a.dn_global[e] : 1.0f;
  for (int c0 = 0; c0 < rows; c0 += a.rc) {
    const int mc = min(a.rc, rows - c0);
    const eng::XSource xs{a.h, a.F, a.spair + first + c0};
    eng::run<FMT, PP, 1, LOCAL>(w, P, a.F, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr}, lds,
                                c0 > 0, DownEpi{&a, pl.TW, pl.TW * pl.J * kWave, mc, c0, first, gsc});
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
// (S of about 8 pairs each); rc rows are staged per pass.  G workgroups per
// expert slot share its tg tile groups, so that the grid holds about
// kWaveTarget waves: a workgroup stages its rows once for several tile
// groups when there are many slots.
constexpr int kWaveTarget = 4096;   // 16 waves per CU on 256 CUs; later workgroups wait for a slot

struct MoePlan {
  int TW, J, S, ppj, tg, G, threads;
  size_t lds;
};

MoePlan moe_plan(int format, int N, int K, int rc, int tw_max, bool paired) {
  MoePlan m;
  const int P = eng::pairs_of(K);
  m.S = std::max(1, std::min((P + 4) / 8, paired ? eng::kWgWaves / 2 : eng::kWgWaves));
  m.ppj = (P + m.S - 1) / m.S;
  m.S = (P + m.ppj - 1) / m.ppj;
  m.J = m.S;
  const int tiles = paired ? eng::tiles_of(N) / 2 : eng::tiles_of(N);
  int per;   // tiles (gate/up tile pairs) per tile group
  if (m.J == 1) {
    // one wave per tile (per gate/up pair, streamed together) finishes it alone
    m.TW = std::min(tw_max, eng::kWgWaves);
    per = m.TW;
  } else {
    // the slices of a tile meet in LDS; gate and up tiles sit in separate waves
    m.TW = std::max(paired ? 2 : 1, std::min(tw_max, eng::kWgWaves / m.J));
    if (paired) m.TW &= ~1;
    per = paired ? m.TW / 2 : m.TW;
  }
  m.tg = (tiles + per - 1) / per;
  m.threads = m.TW * m.J * kWave;
  m.lds = eng::lds_bytes(format, rc, std::min(m.J * m.ppj, P), m.TW, m.J);
  m.G = m.tg;
  return m;
}

void moe_spread(MoePlan &m, int slots) {
  const int per_slot = std::max(1, kWaveTarget / (slots * (m.threads / kWave)));
  const int rounds = (m.tg + per_slot - 1) / per_slot;   // tile groups per workgroup
  m.G = (m.tg + rounds - 1) / rounds;                     // balanced
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
  const int slots = (a.P < E) ? a.P : E;
  MoePlan gu = moe_plan(format, 2 * F, H, a.rc, 4, true);
  MoePlan dn = moe_plan(format, H, F, a.rc, 8, false);
  moe_spread(gu, slots);
  moe_spread(dn, slots);
  a.gu = {gu.TW, gu.J, gu.S, gu.ppj, gu.tg};
  a.dn = {dn.TW, dn.J, dn.S, dn.ppj, dn.tg};
  const int route_threads = (a.P + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(moe_route, dim3(1), dim3(route_threads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 gu_grid(gu.G, slots), dn_grid(dn.G, slots);
  auto go = [&](auto gate_up, auto down) {
    eng::allow_large_lds(gate_up);
    eng::allow_large_lds(down);
    hipLaunchKernelGGL(gate_up, gu_grid, dim3(gu.threads), gu.lds, stream, a);
    hipLaunchKernelGGL(down, dn_grid, dim3(dn.threads), dn.lds, stream, a);
  };
  // four blocks per wave in flight: the grid holds about one 8-wave
  // workgroup per CU
  constexpr int kD = eng::kPPDeep, kN = MTP_FMT_NVFP4, kQ = MTP_FMT_Q4_0;
  const bool pg = gu.J == 1, ld = dn.J == 1;
  if (format == kN) {
    if (pg) ld ? go(moe_gate_up<kN, kD, true>, moe_down<kN, kD, true>)
               : go(moe_gate_up<kN, kD, true>, moe_down<kN, kD, false>);
    else    ld ? go(moe_gate_up<kN, kD, false>, moe_down<kN, kD, true>)
               : go(moe_gate_up<kN, kD, false>, moe_down<kN, kD, false>);
  } else {
    if (pg) ld ? go(moe_gate_up<kQ, kD, true>, moe_down<kQ, kD, true>)
               : go(moe_gate_up<kQ, kD, true>, moe_down<kQ, kD, false>);
    else    ld ? go(moe_gate_up<kQ, kD, false>, moe_down<kQ, kD, true>)
               : go(moe_gate_up<kQ, kD, false>, moe_down<kQ, kD, false>);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t TH = (int64_t)T * H;
  hipLaunchKernelGGL(moe_combine, dim3((unsigned)((TH + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mtp
