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
// Pipeline (two kernels, all on the device, no host round trip):
//  1. gate_up: grid = (G workgroups) x (expert slots).  Every workgroup
//              first derives the routing from topk_ids itself (see route),
//              then streams gate tiles and the matching up tiles of its
//              slot's expert through the engine of the dense GEMM (engine.h)
//              for all rows of that expert and writes
//              h = bf16(silu(gate) * up) per pair.
//  2. down:    the routing gate_up published in the workspace (no second
//              ranking), then y[pair] = W_d[e] . h[pair]; each
//              (pair, 16-column tile) it finishes counts one arrival for the
//              pair's token, and the arrival that completes a token's valid
//              pairs for a tile writes out[t] = sum over slots in slot order
//              of w[t][s] * y[t, s] for those 16 columns.
// The grids are sized for the largest possible number of unique experts;
// slots beyond the actual count exit at once.  The K split of each expert
// matrix depends only on its shape, so a pair's result does not depend on
// which other tokens chose the same expert.
#include <algorithm>
#include <mutex>
#include <vector>

#include "engine.h"
#include "internal.h"

namespace mtp {
namespace {

constexpr int kMaxPairs = 1024;
constexpr int kNoExpert = 0x7FFFFFFF;   // routing key of a pair whose id is outside [0, E)

struct MoeLayout {
  size_t cnt, h, y, route, bytes;
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
  L.cnt = take(sizeof(uint32_t) * T * eng::tiles_of(H));
  L.h = take(sizeof(uint16_t) * P * F);
  L.y = take(sizeof(float) * P * H);
  L.route = take(sizeof(int32_t) * (2 * P + 3 * P));   // order, key, then (e, first, rows) per slot
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
  uint32_t *cnt;          // [token][16-column tile of H]: pairs whose y is stored
  uint16_t *h;            // [pair][F]
  float *y;               // [pair][H]
  int32_t *route;         // the routing gate_up derived: order [P], key [P], slots [P][3]
};

// The routing as one workgroup sees it (LDS).
struct Route {
  int32_t key[kMaxPairs];     // expert of pair p, kNoExpert for an id outside [0, E) or p >= P
  int32_t order[kMaxPairs];   // the pairs ranked by (key, pair)
  int32_t starts[kMaxPairs / kWave], valid[kMaxPairs / kWave];   // per 64 ranks
  int32_t part[4][kWave];     // partial ranks (up to 64 pairs, four waves)
  int32_t e, first, rows;     // the slot: expert (-1: none), ranks first .. first + rows - 1
};

// Every workgroup derives the routing from topk_ids itself (all of them get
// the same): the pairs are ranked by (expert, pair index); the unique experts
// of the valid pairs, in increasing order, are the slots, and slot s holds
// the pairs of its expert in pair order.  Invalid pairs rank last and belong
// to no slot.  Called by every thread of the workgroup.
__device__ void route(const MoeArgs &a, Route &R, int slot) {
  const int P = a.P, nt = blockDim.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  // The rank order (expert, pair) is that of the distinct combined keys
  // expert * kMaxPairs + pair (an invalid pair's expert reads as E; E <=
  // 2^20 keeps them below 2^31), so ranking takes one compare per pair; the
  // combined keys sit in R.order until every rank is known.  Keys past P (up
  // to a multiple of 16) are the largest int: they rank below no pair, so
  // the rank loop reads whole groups of 16.
  const int P16 = (P + 15) & ~15;
  for (int p = threadIdx.x; p < P16; p += nt) {
    const int e = p < P ? a.ids[p] : -1;
    const bool ok = e >= 0 && e < a.E;
    R.key[p] = ok ? e : kNoExpert;
    R.order[p] = p < P ? (ok ? e : a.E) * kMaxPairs + p : 0x7FFFFFFF;
  }
  __syncthreads();
  if (P16 <= kWave && nt >= 4 * kWave) {
    // up to 64 pairs: each of four waves counts one quarter of the keys for
    // every pair (lane = pair), then the four counts are added
    if (wave < 4) {
      const int q0 = wave * (P16 / 4);
      int r = 0;
      if (lane < P) {
        const int ck = R.order[lane];
        for (int j = 0; j < P16 / 4; ++j) r += R.order[q0 + j] < ck ? 1 : 0;
      }
      R.part[wave][lane] = r;
    }
    __syncthreads();   // every combined key is read
    if (threadIdx.x < P) {
      const int p = threadIdx.x;
      R.order[R.part[0][p] + R.part[1][p] + R.part[2][p] + R.part[3][p]] = p;
    }
    __syncthreads();
  } else {
    constexpr int kMaxPerThread = kMaxPairs / kWave;   // workgroups have >= 64 threads
    int rank[kMaxPerThread];
#pragma unroll
    for (int u = 0; u < kMaxPerThread; ++u) {
      const int p = threadIdx.x + u * nt;
      rank[u] = 0;
      if (p < P) {
        const int ck = R.order[p];
        for (int q0 = 0; q0 < P16; q0 += 16) {
          int kq[16];   // all 16 loads in flight before the compares
#pragma unroll
          for (int j = 0; j < 16; ++j) kq[j] = R.order[q0 + j];
#pragma unroll
          for (int j = 0; j < 16; ++j) rank[u] += kq[j] < ck ? 1 : 0;
        }
      }
    }
    __syncthreads();   // every combined key is read
#pragma unroll
    for (int u = 0; u < kMaxPerThread; ++u) {
      const int p = threadIdx.x + u * nt;
      if (p < P) R.order[rank[u]] = p;
    }
    __syncthreads();
  }
  // rank i starts a slot when its pair is valid and its expert differs from
  // that of rank i - 1; chunk c covers ranks 64c .. 64c + 63
  const int nch = (P + kWave - 1) / kWave;
  auto chunk = [&](int c, uint64_t &vb) -> uint64_t {
    const int i = c * kWave + lane;
    bool st = false, vd = false;
    if (i < P) {
      const int k = R.key[R.order[i]];
      vd = k != kNoExpert;
      st = vd && (i == 0 || R.key[R.order[i - 1]] != k);
    }
    vb = __ballot(vd);
    return __ballot(st);
  };
  if (nch > 1) {   // (one chunk: the search below takes its counts itself)
    for (int c = wave; c < nch; c += nt / kWave) {
      uint64_t vb;
      const uint64_t sb = chunk(c, vb);
      if (lane == 0) {
        R.starts[c] = __popcll(sb);
        R.valid[c] = __popcll(vb);
      }
    }
    __syncthreads();
  }
  if (wave == 0) {
    // the rank of start number `slot` and of the next start (or the number
    // of valid pairs: they rank first)
    int before = 0, nvalid = 0, first = -1, end = -1;
    for (int c = 0; c < nch; ++c) {
      uint64_t vb = 0, sb = 0;
      if (nch == 1) sb = chunk(0, vb);
      const int sc = nch == 1 ? __popcll(sb) : R.starts[c];
      nvalid += nch == 1 ? __popcll(vb) : R.valid[c];
      if (slot < before + sc && slot + 1 >= before) {   // start `slot` or `slot + 1` is here
        if (nch > 1) sb = chunk(c, vb);
        // the start number of this lane's rank: starts below it in the chunk
        const int num = before + __popcll(sb & ((1ull << lane) - 1ull));
        const bool st = (sb >> lane) & 1ull;
        const uint64_t h0 = __ballot(st && num == slot), h1 = __ballot(st && num == slot + 1);
        if (h0) first = c * kWave + __ffsll((long long)h0) - 1;
        if (h1) end = c * kWave + __ffsll((long long)h1) - 1;
      }
      before += sc;
    }
    if (end < 0) end = nvalid;
    if (lane == 0) {
      R.first = first;
      R.rows = first < 0 ? 0 : end - first;
      R.e = first < 0 ? -1 : R.key[R.order[first]];
    }
  }
  __syncthreads();
}

// Set-up of one call, spread over the workgroups of the gate_up kernel (the
// down kernel runs after it): clears the arrival counters and out (tokens
// with no valid pair never complete an arrival and keep the zeros), and
// writes zero rows of h_out for invalid pairs.  Workgroup b of nb takes its
// share of each.
__device__ void clear_call_state(const MoeArgs &a, const Route &R) {
  const int nb = gridDim.x * gridDim.y, b = blockIdx.y * gridDim.x + blockIdx.x;
  auto share = [&](int n, auto &&f) {
    const int per = (n + nb - 1) / nb, i1 = min(n, (b + 1) * per);
    for (int i = b * per + (int)threadIdx.x; i < i1; i += blockDim.x) f(i);
  };
  share(a.T * eng::tiles_of(a.H), [&](int i) {
    __hip_atomic_store(a.cnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  share(a.T * a.H, [&](int i) { a.out[i] = 0.0f; });
  if (a.h_out)
    for (int p = b; p < a.P; p += nb)
      if (R.key[p] == kNoExpert)
        for (int f = threadIdx.x; f < a.F; f += blockDim.x) a.h_out[(int64_t)p * a.F + f] = 0;
}

// The routing for the down kernel (which runs after this one): workgroup
// (0, 0) writes the ranked pairs and their keys, the first workgroup of
// each slot its (expert, first rank, rows).
__device__ void publish_route(const MoeArgs &a, const Route &R) {
  if (blockIdx.x != 0) return;
  if (blockIdx.y == 0)
    for (int p = threadIdx.x; p < a.P; p += blockDim.x) {
      a.route[p] = R.order[p];
      a.route[a.P + p] = R.key[p];
    }
  if (threadIdx.x == 0) {
    int32_t *sl = a.route + 2 * a.P + 3 * blockIdx.y;
    sl[0] = R.e;
    sl[1] = R.first;
    sl[2] = R.rows;
  }
}

// The down kernel's view of the routing, read from what gate_up published.
__device__ void load_route(const MoeArgs &a, Route &R, int slot) {
  for (int p = threadIdx.x; p < a.P; p += blockDim.x) {
    R.order[p] = a.route[p];
    R.key[p] = a.route[a.P + p];
  }
  if (threadIdx.x == 0) {
    const int32_t *sl = a.route + 2 * a.P + 3 * slot;
    R.e = sl[0];
    R.first = sl[1];
    R.rows = sl[2];
  }
  __syncthreads();
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
  int TWh, nthreads, mc;
  const int32_t *pairs;   // pair of each row of this pass (LDS)
  float gsc;
  __device__ __forceinline__ void put(int m, int f, float gate, float up) const {
    const uint16_t hb = f32_to_bf16_rne(silu(gate) * up);
    const int pair = pairs[m];
    a->h[(int64_t)pair * a->F + f] = hb;
    if (a->h_out) a->h_out[(int64_t)pair * a->F + f] = hb;
  }
  __device__ __forceinline__ void operator()(int tg, const f32x4 *fin) const {
    const int cols = TWh * 16;
    for (int o = threadIdx.x; o < mc * cols; o += nthreads) {
      const int m = o / cols, c = o - m * cols;
      const int f = tg * cols + c;
      if (f < a->F) {
        const int q = c >> 4;
        put(m, f, gsc * eng::fin_at(fin, 2 * q, m, c & 15),
            gsc * eng::fin_at(fin, 2 * q + 1, m, c & 15));
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
      if (m < mc) put(m, f, gsc * acc[0][i], gsc * acc[1][i]);
    }
  }
};

// PAIRED: one wave streams a gate tile and its up tile together (J == 1)
template <int FMT, int PP, bool PAIRED>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_gate_up(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ Route R;
  route(a, R, blockIdx.y);
  clear_call_state(a, R);
  publish_route(a, R);
  const int e = __builtin_amdgcn_readfirstlane(R.e);
  if (e < 0) return;  // a slot past the unique experts (whole workgroup)
  const int first = __builtin_amdgcn_readfirstlane(R.first);
  const int rows = __builtin_amdgcn_readfirstlane(R.rows);
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
    const int32_t *pairs = R.order + first + c0;
    const eng::XSource xs{a.x, a.H, pairs, a.topk};   // row of pair p: token p / topk
    eng::run<FMT, PP, PAIRED ? 2 : 1, PAIRED, true>(
        w, P, a.H, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr}, lds, c0 > 0,
        GateUpEpi{&a, TWh, pl.TW * pl.J * kWave, mc, pairs, gsc});
  }
}

// y rows are stored at agent scope: another workgroup (on another XCD) may
// add them into out.
struct DownEpi {
  const MoeArgs *a;
  int TW, nthreads, mc;
  const int32_t *pairs;
  float gsc;
  __device__ __forceinline__ void put(int m, int n, float v) const {
    __hip_atomic_store(a->y + (int64_t)pairs[m] * a->H + n, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void operator()(int tg, const f32x4 *fin) const {
    const int cols = TW * 16;
    for (int o = threadIdx.x; o < mc * cols; o += nthreads) {
      const int m = o / cols, c = o - m * cols;
      const int n = tg * cols + c;
      if (n < a->H) put(m, n, gsc * eng::fin_at(fin, c >> 4, m, c & 15));
    }
  }
  __device__ __forceinline__ void wave(int tg, int tw, const f32x4 *acc) const {
    const int lane = threadIdx.x & (kWave - 1);
    const int n = (tg * TW + tw) * 16 + (lane & 15);
    if (n >= a->H) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = eng::acc_row(lane, i);
      if (m < mc) put(m, n, gsc * acc[0][i]);
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

// After the down passes of a workgroup (every thread calls it): once all of
// its y stores are complete, each (row, tile) it produced counts one arrival
// for the row's token and tile; the arrival that completes the token's
// valid pairs writes out[t] for the tile's 16 columns, adding the token's
// slots in slot order.
__device__ void arrive_and_combine(const MoeArgs &a, const Route &R, const eng::Plan &pl,
                                   int first, int rows) {
  __shared__ int done_n;
  __shared__ int done[eng::kMaxThreads];
  __builtin_amdgcn_s_waitcnt(0);   // this thread's y stores are complete
  __syncthreads();                 // ... and every thread's
  const int ntiles = eng::tiles_of(a.H);
  const int per = pl.tg_count * pl.TW;   // tile positions of this workgroup
  const int combos = per * rows;
  for (int base = 0; base < combos; base += blockDim.x) {
    if (threadIdx.x == 0) done_n = 0;
    __syncthreads();
    const int c = base + threadIdx.x;
    if (c < combos) {
      const int m = c / per, s = c - m * per;
      const int tile = (pl.tg_first + (s / pl.TW) * pl.tg_step) * pl.TW + s % pl.TW;
      if (tile < ntiles) {
        const int t = R.order[first + m] / a.topk;
        uint32_t need = 0;
        for (int k = 0; k < a.topk; ++k) need += R.key[t * a.topk + k] != kNoExpert ? 1u : 0u;
        const uint32_t old = __hip_atomic_fetch_add(a.cnt + (int64_t)t * ntiles + tile, 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1u == need) done[atomicAdd(&done_n, 1)] = t * ntiles + tile;
      }
    }
    __syncthreads();
    const int nd = done_n;
    for (int i = threadIdx.x; i < nd * 16; i += blockDim.x) {
      const int d = done[i >> 4], t = d / ntiles;
      const int n = (d - t * ntiles) * 16 + (i & 15);
      float s = 0.0f;
      for (int k0 = 0; k0 < a.topk; k0 += 8) {
        // eight slots' loads in flight at once (an invalid slot's y is read
        // but not used), then the sum in slot order
        float yv[8], wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int p = t * a.topk + min(k0 + j, a.topk - 1);
          yv[j] = __hip_atomic_load(a.y + (int64_t)p * a.H + n, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
          wv[j] = a.gw[p];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < a.topk && R.key[t * a.topk + k0 + j] != kNoExpert) s += wv[j] * yv[j];
      }
      a.out[(int64_t)t * a.H + n] = s;
    }
    __syncthreads();
  }
}

// LOCAL: one slice per tile (J == 1), each wave finishes its own tile
template <int FMT, int PP, bool LOCAL>
__global__ __launch_bounds__(eng::kMaxThreads) void moe_down(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ Route R;
  load_route(a, R, blockIdx.y);
  const int e = __builtin_amdgcn_readfirstlane(R.e);
  if (e < 0) return;  // a slot past the unique experts (whole workgroup)
  const int first = __builtin_amdgcn_readfirstlane(R.first);
  const int rows = __builtin_amdgcn_readfirstlane(R.rows);
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
    const int32_t *pairs = R.order + first + c0;
    const eng::XSource xs{a.h, a.F, pairs, 1};
    eng::run<FMT, PP, 1, LOCAL, true>(w, P, a.F, mc, xs, pl, tiles, eng::Fixup{nullptr, nullptr},
                                      lds, c0 > 0,
                                      DownEpi{&a, pl.TW, pl.TW * pl.J * kWave, mc, pairs, gsc});
  }
  arrive_and_combine(a, R, pl, first, rows);
}

// Engine shape of one expert matrix: a single workgroup covers all slices
// (S of about 8 pairs each); rc rows are staged per pass.  Workgroups have
// at most kMoeTiles waves of tiles, so that several share a CU (the kernels
// hold more than 128 registers per lane, three waves per SIMD).  G
// workgroups per expert slot share its tg tile groups, as many as the GPU
// holds at once: a workgroup streams several tile groups (staging its rows
// once) only when all slots' workgroups would not fit in one round.
constexpr int kMoeTiles = 4;

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

// resident: workgroups of the kernel the whole GPU holds at once
void moe_spread(MoePlan &m, int slots, int resident) {
  const int per_slot = std::max(1, resident / slots);
  const int rounds = (m.tg + per_slot - 1) / per_slot;   // tile groups per workgroup
  m.G = (m.tg + rounds - 1) / rounds;                     // balanced
}

// Workgroups of `kernel` (threads, dynamic LDS) resident on the current
// device at once: per-CU occupancy from the runtime times the CU count.
template <typename Kernel>
int resident_workgroups(Kernel *kernel, int threads, size_t lds) {
  struct Entry { const void *k; int threads; size_t lds; int dev, n; };
  static std::mutex mu;
  static std::vector<Entry> seen;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const void *k = reinterpret_cast<const void *>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry &e : seen)
    if (e.k == k && e.threads == threads && e.lds == lds && e.dev == dev) return e.n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 1;
  (void)hipGetLastError();
  seen.push_back(Entry{k, threads, lds, dev, per_cu * cus});
  return per_cu * cus;
}

// Rows staged per pass: up to 16 (and T, which bounds the rows of an expert
// unless a token repeats an expert), fewer if the staged rows would not fit.
int moe_rows(int format, int T, int H, int F) {
  int rc = std::min(16, T);
  while (rc > 1 && (moe_plan(format, 2 * F, H, rc, kMoeTiles, true).lds > 144 * 1024 ||
                    moe_plan(format, H, F, rc, kMoeTiles, false).lds > 144 * 1024))
    --rc;
  return rc;
}

}  // namespace

bool moe_fits(int format, int T, int H, int F) {
  const int rc = moe_rows(format, T, H, F);
  return moe_plan(format, 2 * F, H, rc, kMoeTiles, true).lds <= 144 * 1024 &&
         moe_plan(format, H, F, rc, kMoeTiles, false).lds <= 144 * 1024;
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
  a.cnt = reinterpret_cast<uint32_t *>(w + L.cnt);
  a.h = reinterpret_cast<uint16_t *>(w + L.h);
  a.y = reinterpret_cast<float *>(w + L.y);
  a.route = reinterpret_cast<int32_t *>(w + L.route);
  a.rc = moe_rows(format, T, H, F);
  const int slots = (a.P < E) ? a.P : E;
  MoePlan gu = moe_plan(format, 2 * F, H, a.rc, kMoeTiles, true);
  MoePlan dn = moe_plan(format, H, F, a.rc, kMoeTiles, false);
  // the engine splits a workgroup's waves into (tile, slice) by shifts
  if ((gu.TW & (gu.TW - 1)) || (dn.TW & (dn.TW - 1))) return hipErrorInvalidValue;
  a.gu = {gu.TW, gu.J, gu.S, gu.ppj, gu.tg};
  a.dn = {dn.TW, dn.J, dn.S, dn.ppj, dn.tg};
  auto go = [&](auto gate_up, auto down) {
    eng::allow_large_lds(gate_up);
    eng::allow_large_lds(down);
    moe_spread(gu, slots, resident_workgroups(gate_up, gu.threads, gu.lds));
    moe_spread(dn, slots, resident_workgroups(down, dn.threads, dn.lds));
    hipLaunchKernelGGL(gate_up, dim3(gu.G, slots), dim3(gu.threads), gu.lds, stream, a);
    hipLaunchKernelGGL(down, dim3(dn.G, slots), dim3(dn.threads), dn.lds, stream, a);
  };
  // four blocks per wave in flight
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
  return hipGetLastError();
}

}  // namespace mtp
