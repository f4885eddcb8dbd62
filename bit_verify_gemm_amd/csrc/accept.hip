// Acceptance step of the verify pass: greedy prefix match and Leviathan/Chen
// rejection sampling with residual correction, plus the rollback index.
//
// Gemini Nano summary, analysis §3, and Qiita roofline article, §2-4: greedy
// verification keeps the longest prefix that agrees with the target and
// always commits one more (correction) token.  MTPLX blog post, "Why it is
// interesting on a Mac specifically": rejection sampling with residual
// correction preserves the target's output at temperature 0.6, top_p 0.95.
// Ollama mtp.go commit log: the sampler pipeline is temperature/softmax ->
// top-p -> normalise -> categorical, target distributions are reused for
// acceptance, bonus and residual draws, and at temperature 0 acceptance is
// argmax matching.  Ollama news item, fifth paragraph: a rollback point lets
// a rejection rewind to the last accepted token without a return to the CPU.
//
// Everything runs on the device.  Probability mass is computed in fp64 and
// summed as exact 128-bit fixed-point integers (resolution 2^-100), so sums
// are independent of thread order and the outputs are a deterministic
// function of the inputs.  The top-p nucleus is found by a 4-pass radix
// select over the order-preserving 32-bit key of each logit, with per-digit
// mass histograms; ties at the cut are broken by index.
#include <algorithm>
#include <mutex>

#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

namespace mtp {
namespace {

typedef unsigned long long u64;

constexpr int kBlock = 256;
constexpr int kMaxBlocksPerRow = 128;
constexpr int kBins = 256;
constexpr int kBatch = 8;   // row entries each thread loads at once (all in flight)

// Entries base + t + i * kBlock (i < kBatch) of row zr for thread t, or
// `fill` past j1: all loads are issued before any value is used.
__device__ __forceinline__ void load_batch(const float *zr, int base, int j1, float fill,
                                           float (&v)[kBatch]) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int j = base + (int)threadIdx.x + i * kBlock;
    v[i] = j < j1 ? zr[j] : fill;
  }
}

int blocks_per_row(int V) {
  int nb = (V + 2047) / 2048;
  return nb < 1 ? 1 : (nb > kMaxBlocksPerRow ? kMaxBlocksPerRow : nb);
}

// The final draw spreads its one row over more blocks (one entry per thread
// up to kMaxDrawBlocks blocks).
constexpr int kMaxDrawBlocks = 2048;
int draw_blocks(int V) {
  int nb = (V + kBlock - 1) / kBlock;
  return nb < 1 ? 1 : (nb > kMaxDrawBlocks ? kMaxDrawBlocks : nb);
}

// ---- 128-bit fixed point (value * 2^100) -----------------------------------

struct Fx {
  u64 lo, hi;
};

__device__ __forceinline__ Fx fx_zero() { return Fx{0ull, 0ull}; }

// floor(v * 2^100) for 0 <= v < 2^27 (values below 2^-100 become 0).
__device__ __forceinline__ Fx to_fx(double v) {
  Fx r = fx_zero();
  if (!(v > 0.0)) return r;
  const u64 bits = (u64)__double_as_longlong(v);
  const int ex = (int)((bits >> 52) & 0x7FF);
  if (ex == 0) return r;
  const u64 mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int sh = ex - 975;  // v * 2^100 = mant * 2^(ex - 1075 + 100)
  if (sh >= 64) {
    r.hi = mant << (sh - 64);
  } else if (sh > 0) {
    r.lo = mant << sh;
    r.hi = mant >> (64 - sh);
  } else if (sh == 0) {
    r.lo = mant;
  } else if (sh > -64) {
    r.lo = mant >> (-sh);
  }
  return r;
}

__device__ __forceinline__ void fx_add(Fx &a, const Fx &b) {
  const u64 lo = a.lo + b.lo;
  a.hi += b.hi + (lo < a.lo ? 1ull : 0ull);
  a.lo = lo;
}

__device__ __forceinline__ Fx fx_sum(Fx a, const Fx &b) {
  fx_add(a, b);
  return a;
}

__device__ __forceinline__ bool fx_ge(const Fx &a, const Fx &b) {
  return a.hi > b.hi || (a.hi == b.hi && a.lo >= b.lo);
}

__device__ __forceinline__ bool fx_gt(const Fx &a, const Fx &b) {
  return a.hi > b.hi || (a.hi == b.hi && a.lo > b.lo);
}

__device__ __forceinline__ bool fx_nonzero(const Fx &a) { return (a.lo | a.hi) != 0ull; }

__device__ __forceinline__ double fx_to_double(const Fx &a) {
  return ldexp((double)a.hi, -36) + ldexp((double)a.lo, -100);
}

// Sums shared by the blocks of a kernel are kept as three 64-bit limbs,
// L0 += bits 0..31, L1 += bits 32..63, L2 += bits 64..127 of each
// contribution, so that the atomic adds need no carry (and no returned
// value); a limb of at most 2^20 contributions cannot overflow.
__device__ __forceinline__ void fx_atomic_add3(u64 *p, Fx v) {
  if (v.lo & 0xFFFFFFFFull) atomicAdd(p, v.lo & 0xFFFFFFFFull);
  if (v.lo >> 32) atomicAdd(p + 1, v.lo >> 32);
  if (v.hi) atomicAdd(p + 2, v.hi);
}

__device__ __forceinline__ Fx fx_from3(u64 l0, u64 l1, u64 l2) {
  Fx r;
  r.lo = l0 + (l1 << 32);
  r.hi = l2 + (l1 >> 32) + (r.lo < l0 ? 1ull : 0ull);
  return r;
}

__device__ __forceinline__ Fx fx_load3(const u64 *p) { return fx_from3(p[0], p[1], p[2]); }

// DPP moves: lane i reads a lane of its own row of 16 within the same
// instruction.  dpp0: a shift or broadcast (row_shr:n reads lane i - n,
// row_bcast:15 and :31 the last lane of the row before, resp. of row 1;
// lanes without a source, and rows outside row_mask, read 0).  dppp: a
// permutation within each row.
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118,
              kDppBcast15 = 0x142, kDppBcast31 = 0x143, kDppSwap1 = 0xB1, kDppSwap2 = 0x4E,
              kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, row_mask, 0xF, false);
}
template <int ctrl>
__device__ __forceinline__ uint32_t dppp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, ctrl, 0xF, 0xF, false);
}

// Inclusive sum over the lanes of the wave.
__device__ __forceinline__ int dpp_incl(int x) {
  x += (int)dpp0<kDppShr1>((uint32_t)x);
  x += (int)dpp0<kDppShr2>((uint32_t)x);
  x += (int)dpp0<kDppShr4>((uint32_t)x);
  x += (int)dpp0<kDppShr8>((uint32_t)x);
  x += (int)dpp0<kDppBcast15, 0xA>((uint32_t)x);
  x += (int)dpp0<kDppBcast31, 0xC>((uint32_t)x);
  return x;
}

// Wave-wide extrema (the same value in every lane).
__device__ __forceinline__ uint32_t dpp_umax(uint32_t x) {
  x = max(x, dppp<kDppSwap1>(x));
  x = max(x, dppp<kDppSwap2>(x));
  x = max(x, dppp<kDppHalfMirror>(x));
  x = max(x, dppp<kDppMirror>(x));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(r0, r1), max(r2, r3));   // unsigned: keys use all 32 bits
}
__device__ __forceinline__ uint32_t dpp_umin(uint32_t x) {
  x = min(x, dppp<kDppSwap1>(x));
  x = min(x, dppp<kDppSwap2>(x));
  x = min(x, dppp<kDppHalfMirror>(x));
  x = min(x, dppp<kDppMirror>(x));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return min(min(r0, r1), min(r2, r3));
}

template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ Fx dpp0_fx(const Fx &a) {
  Fx r;
  r.lo = (u64)dpp0<ctrl, row_mask>((uint32_t)a.lo) |
         ((u64)dpp0<ctrl, row_mask>((uint32_t)(a.lo >> 32)) << 32);
  r.hi = (u64)dpp0<ctrl, row_mask>((uint32_t)a.hi) |
         ((u64)dpp0<ctrl, row_mask>((uint32_t)(a.hi >> 32)) << 32);
  return r;
}

// Inclusive exact sum over the lanes of the wave.
__device__ __forceinline__ Fx dpp_fx_incl(Fx x) {
  fx_add(x, dpp0_fx<kDppShr1>(x));
  fx_add(x, dpp0_fx<kDppShr2>(x));
  fx_add(x, dpp0_fx<kDppShr4>(x));
  fx_add(x, dpp0_fx<kDppShr8>(x));
  fx_add(x, dpp0_fx<kDppBcast15, 0xA>(x));
  fx_add(x, dpp0_fx<kDppBcast31, 0xC>(x));
  return x;
}

__device__ __forceinline__ Fx fx_readlane(const Fx &a, int l) {
  Fx r;
  r.lo = (u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a.lo, l) |
         ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a.lo >> 32), l) << 32);
  r.hi = (u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a.hi, l) |
         ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a.hi >> 32), l) << 32);
  return r;
}
__device__ __forceinline__ double dbl_readlane(double v, int l) {
  const u64 b = (u64)__double_as_longlong(v);
  const u64 r = (u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l) |
                ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l) << 32);
  return __longlong_as_double((long long)r);
}

// Exact wave-wide sum (integer adds commute), in every lane.  Whole waves
// call it.
__device__ __forceinline__ Fx fx_wave_sum(Fx a) { return fx_readlane(dpp_fx_incl(a), kWave - 1); }

// Signed wave-wide extrema, in every lane.  Whole waves call them.
__device__ __forceinline__ int dpp_imin(int x) {
  x = min(x, (int)dppp<kDppSwap1>((uint32_t)x));
  x = min(x, (int)dppp<kDppSwap2>((uint32_t)x));
  x = min(x, (int)dppp<kDppHalfMirror>((uint32_t)x));
  x = min(x, (int)dppp<kDppMirror>((uint32_t)x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int dpp_imax(int x) {
  x = max(x, (int)dppp<kDppSwap1>((uint32_t)x));
  x = max(x, (int)dppp<kDppSwap2>((uint32_t)x));
  x = max(x, (int)dppp<kDppHalfMirror>((uint32_t)x));
  x = max(x, (int)dppp<kDppMirror>((uint32_t)x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ float dpp_fmax(float x) {
  x = fmaxf(x, __uint_as_float(dppp<kDppSwap1>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dppp<kDppSwap2>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dppp<kDppHalfMirror>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dppp<kDppMirror>(__float_as_uint(x))));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// An fp64 DPP shift (as dpp0, each half moved alike).
template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ double dpp0_d(double v) {
  const u64 b = (u64)__double_as_longlong(v);
  return __longlong_as_double((long long)((u64)dpp0<ctrl, row_mask>((uint32_t)b) |
                                          ((u64)dpp0<ctrl, row_mask>((uint32_t)(b >> 32)) << 32)));
}

// Inclusive fp64 sum over the lanes of the wave (a fixed order of additions).
__device__ __forceinline__ double dpp_dincl(double x) {
  x += dpp0_d<kDppShr1>(x);
  x += dpp0_d<kDppShr2>(x);
  x += dpp0_d<kDppShr4>(x);
  x += dpp0_d<kDppShr8>(x);
  x += dpp0_d<kDppBcast15, 0xA>(x);
  x += dpp0_d<kDppBcast31, 0xC>(x);
  return x;
}

// Block-wide sum; result valid in every thread.  `red` holds kBlock/kWave Fx.
__device__ Fx fx_block_sum(Fx a, Fx *red) {
  a = fx_wave_sum(a);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = a;
  __syncthreads();
  Fx s = fx_zero();
  for (int i = 0; i < kBlock / kWave; ++i) fx_add(s, red[i]);
  return s;
}

// Order-preserving key: a < b as floats  <=>  key(a) < key(b).
__device__ __forceinline__ uint32_t fkey(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- workspace layout -------------------------------------------------------

struct RowState {
  float zmax;
  uint32_t kappa;   // key of the last nucleus value (all keys >= kappa)
  int32_t cutoff;   // entries with key == kappa and index <= cutoff are inside
  int32_t all;      // bit 0: the nucleus is the whole row; bit 1 (rej_one): the
                    // row's resolving workgroup drew the row's token itself
  double mass;      // nucleus mass S' (sum of e over the nucleus)
};

// Radix-select state after s passes: the selected key prefix (top 8s bits)
// and the mass of the entries strictly above it.
struct SelState {
  u64 above_lo, above_hi;
  uint32_t prefix;
  int32_t pad;
};

// Inputs of the acceptance test of one draft: p'(x) and q(x).
struct AccIn {
  double px, qx;
};

constexpr int kMaxRows = 64;

// Per draw block: residual sum (lo, hi), e sum (lo, hi), and the first index
// whose residual, resp. e, is positive in fp64 (kNone: none).
constexpr int kBlkWords = 6;
constexpr int kNone = 0x7FFFFFFF;

struct Layout {
  size_t hdr, maxp, zmax, hist, total, sel, rows, acc, blk, gpart, ahist, above, ccount, acount,
      asec,
      cand, wsum, bytes;
};

// The one-launch rejection kernel (rej_one): workgroups of kOneThreads, each
// holding up to kOneChunk entries of one row in LDS; used when every row fits
// in at most kMaxOneBlocks workgroups altogether (all resident at once, one
// per compute unit).
constexpr int kOneThreads = 1024;
constexpr int kOneChunk = 8192;
constexpr int kMaxOneBlocks = 256;
constexpr int kXBins = 1024;          // approximate mass bins of the cut search
// Workspace header (offset 0, the same for every shape): one 4 KiB page per
// row and one for the call, so that the words workgroups wait on lie apart.
// Row page: arrival counters of the mass pass and the candidate step (a
// third word is kept zero); the row's tagged candidate-bin and state words;
// its workgroups' tagged chunk maxima.  Call page: the count of workgroups
// whose draw sums are in, an error word, the generation number of the last
// call.  Zero
// before first use; every call of the one-launch kernel leaves the counters
// zero and advances the generation number (the tagged words need no reset).
constexpr int kPageWords = 512;
constexpr int kRowCnt = 0, kRowCand = 1, kRowDraw = 2, kRowBins = 64, kRowState = 128,
              kRowSlots = 256;
constexpr int kCallRows = 0, kCallErr = 1, kCallGen = 2;
constexpr int kRowPick = 192;   // rej_one: the row's tagged token when its resolver drew it
// rej_one: a workgroup hands its entries above the candidate bins to the
// row's resolver when it has at most kAboveCap of them
constexpr int kAboveCap = 256;
// rej_one's exchange area after the pages: kXW tagged words per workgroup
// (row * G + g): its chunk maximum, its approximate mass, the key of its
// (kTopK + 1)-th largest entry and its kTopK largest entries (key, index).
constexpr int kTopK = 2;
constexpr int kXW = 3 + 2 * kTopK;
static_assert(kTopK >= 2, "word 5 holds a workgroup's second key");
constexpr int kXchg = (kMaxRows + 1) * kPageWords;
constexpr int kHdrWords = kXchg + kMaxOneBlocks * kXW;
static_assert(kRowSlots + kMaxOneBlocks <= kPageWords, "slots fit the row page");

// LDS of rej_one for chunks of C entries: logits, e values, approximate bins.
__host__ __device__ constexpr int one_e_offset(int C) { return (4 * C + 15) & ~15; }
__host__ __device__ constexpr int one_b_offset(int C) { return one_e_offset(C) + 8 * C; }
__host__ __device__ constexpr int one_lds_bytes(int C) { return one_b_offset(C) + 2 * C; }
// Dynamic LDS of rej_one: the chunk, or (in the workgroup that resolves a
// row's cut, once it no longer needs its chunk) one_cand_room candidates as
// (key << 32 | index, e) pairs.
constexpr int kCandLdsBytes = 96 * 1024;
__host__ __device__ constexpr int one_dyn_bytes(int C) {
  return one_lds_bytes(C) > kCandLdsBytes ? one_lds_bytes(C) : kCandLdsBytes;
}
__host__ __device__ constexpr int one_cand_room(int C) { return one_dyn_bytes(C) / 16; }

// Workgroups per row of rej_one, or 0 where it does not apply: enough to
// spread the rows over the compute units (at least 1024 entries each), with
// at most kOneChunk entries each.
int one_blocks_per_row(int M, int V) {
  int G = std::max((V + kOneChunk - 1) / kOneChunk, std::min(kMaxOneBlocks / M, (V + 1023) / 1024));
  if (G < 1) G = 1;
  const int C = (V + G - 1) / G;
  G = (V + C - 1) / C;   // no empty chunk
  if (C > kOneChunk || (int64_t)M * G > kMaxOneBlocks) return 0;
  return G;
}

// Room for rej_one's per-call regions at any row count up to M (so that a
// workspace sized for M rows serves every smaller M): candidate entries,
// workgroups and rows.
struct OneRoom {
  size_t cand, blocks, rows;
};

OneRoom one_room(int M, int V) {
  OneRoom r{0, 0, 0};
  for (int m = 1; m <= M; ++m) {
    const int G = one_blocks_per_row(m, V);
    if (!G) continue;
    r.cand = std::max(r.cand, (size_t)m * G * (size_t)((V + G - 1) / G));
    r.blocks = std::max(r.blocks, (size_t)m * G);
    r.rows = (size_t)m;
  }
  return r;
}

Layout layout(int M, int V) {
  const size_t nb = (size_t)blocks_per_row(V);
  const OneRoom one = one_room(M, V);
  Layout L;
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  L.hdr = take(sizeof(u64) * kHdrWords);
  L.maxp = take(sizeof(float) * M * nb);
  L.zmax = take(sizeof(float) * M);
  L.hist = take(sizeof(u64) * 4 * kBins * 4 * M);
  L.total = take(sizeof(u64) * 3 * M);
  L.sel = take(sizeof(SelState) * 4 * M);
  L.rows = take(sizeof(RowState) * M);
  L.acc = take(sizeof(AccIn) * M);
  L.blk = take(sizeof(u64) * kBlkWords * (size_t)std::max(draw_blocks(V), kMaxOneBlocks));
  L.gpart = take(sizeof(float) * 2 * M * nb);
  L.ahist = take(sizeof(double) * kXBins * one.rows);
  L.above = take(sizeof(u64) * 3 * M);
  L.ccount = take(sizeof(int32_t) * one.blocks);
  L.acount = take(sizeof(int32_t) * one.blocks);
  L.asec = take(sizeof(u64) * kAboveCap * one.blocks);
  L.cand = take(sizeof(u64) * one.cand);
  L.wsum = take(one.blocks ? sizeof(u64) * 4 * kMaxOneBlocks * (kOneThreads / kWave) : 0);
  L.bytes = o;
  return L;
}

struct RejArgs {
  const float *z;
  int64_t ldl;
  const float *q;
  int64_t ldq;
  const int32_t *drafts;
  const float *u;
  double T;
  double top_p;
  int M, V, nb, chunk;
  int nbd, chunkd;  // blocks of the final draw and entries per draw block
  int64_t base_len;
  int32_t *tokens;
  int32_t *counts;
  int64_t *rollback;
  float *maxp;      // [row][block] partial maxima
  float *zmax;      // [row]
  u64 *hist;        // [pass][row][bin][L0, L1, L2, count]
  u64 *total;       // [row][L0, L1, L2]
  SelState *sel;    // [pass][row]: state after `pass` selections (pass >= 1)
  RowState *rows;
  AccIn *acc;       // [row]: inputs of draft row's acceptance test
  u64 *blk;         // [block][res lo, res hi, e lo, e hi, first res > 0, first e > 0]
  u64 *hdr;         // rej_one: counters (see kHdrWords)
  double *ahist;    // rej_one: [row][kXBins] approximate mass histogram
  u64 *above;       // rej_one: [row][L0, L1, L2] exact mass above the candidate bins
  int32_t *ccount;  // rej_one: [row][workgroup] candidates
  int32_t *acount;  // rej_one: [row][workgroup] entries above the candidate bins, -1: > kAboveCap
  u64 *asec;        // rej_one: [row][workgroup][kAboveCap] those entries (key << 32 | index)
  u64 *cand;        // rej_one: [row][workgroup][C] candidates (key << 32 | index)
  u64 *wsum;        // rej_one: [res lo, res hi, e lo, e hi][row][workgroup][wave] draw range sums
  int G, C;         // rej_one: workgroups per row, entries per workgroup
};

__device__ __forceinline__ u64 *hist_at(const RejArgs &p, int pass, int row) {
  return p.hist + ((size_t)(pass * p.M + row) * kBins) * 4;
}

// Histogram of one row (global, limbs) into LDS as (mass lo, mass hi, count)
// per bin.
__device__ void hist_to_lds(const u64 *g, u64 *h) {
  for (int b = threadIdx.x; b < kBins; b += kBlock) {
    const u64 *s = g + 4 * b;
    const Fx m = fx_load3(s);
    h[3 * b] = m.lo;
    h[3 * b + 1] = m.hi;
    h[3 * b + 2] = s[3];
  }
}

__device__ __forceinline__ Fx fx_sub(Fx a, const Fx &b) {
  const u64 lo = a.lo - b.lo;
  a.hi = a.hi - b.hi - (a.lo < b.lo ? 1ull : 0ull);
  a.lo = lo;
  return a;
}

// ---- greedy -------------------------------------------------------------------

// Better candidate: a number beats NaN, larger beats smaller, lower index
// breaks ties.
__device__ __forceinline__ bool better(float v, int j, float bv, int bj) {
  if (isnan(v)) return false;
  if (isnan(bv)) return true;
  return v > bv || (v == bv && j < bj);
}

__device__ __forceinline__ void wave_best(float &bv, int &bj) {
  for (int m = kWave / 2; m > 0; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oj = __shfl_xor(bj, m);
    if (better(ov, oj, bv, bj)) { bv = ov; bj = oj; }
  }
}

__global__ __launch_bounds__(kBlock) void greedy_partial(const float *z, int64_t ldl, int V,
                                                         int nb, int chunk, float *pv, int *pj) {
  const int b = blockIdx.x, row = blockIdx.y;
  const float *zr = z + (int64_t)row * ldl;
  const int j0 = b * chunk, j1 = min(V, j0 + chunk);
  float bv = __int_as_float(0x7FC00000);
  int bj = 0x7FFFFFFF;
  for (int base = j0; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(zr, base, j1, __int_as_float(0x7FC00000), v);   // NaN never wins
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = base + (int)threadIdx.x + i * kBlock;
      if (better(v[i], j, bv, bj)) { bv = v[i]; bj = j; }
    }
  }
  wave_best(bv, bj);
  __shared__ float sv[kBlock / kWave];
  __shared__ int sj[kBlock / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) { sv[threadIdx.x / kWave] = bv; sj[threadIdx.x / kWave] = bj; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBlock / kWave; ++w)
      if (better(sv[w], sj[w], bv, bj)) { bv = sv[w]; bj = sj[w]; }
    pv[row * nb + b] = bv;
    pj[row * nb + b] = bj;
  }
}

// Row argmax from the block partials (one wave per row, 16 waves), then
// the prefix match, tokens, counts and rollback.  A wave loads both of its
// lanes' partials (nb <= 128) before comparing them.
constexpr int kFinalThreads = 1024;
static_assert(kMaxBlocksPerRow <= 2 * kWave, "two partials per lane");
__global__ __launch_bounds__(kFinalThreads) void greedy_final(const float *pv, const int *pj,
                                                              int M, int nb,
                                                              const int32_t *drafts,
                                                              int64_t base_len, int32_t *tokens,
                                                              int32_t *counts, int64_t *rollback) {
  __shared__ int g[64];
  __shared__ int d[64];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (threadIdx.x < M - 1) d[threadIdx.x] = drafts[threadIdx.x];   // issued with the partials' loads
  for (int row = wave; row < M; row += kFinalThreads / kWave) {
    const int b0 = lane, b1 = lane + kWave;
    const float v0 = b0 < nb ? pv[row * nb + b0] : __int_as_float(0x7FC00000);
    const int j0 = b0 < nb ? pj[row * nb + b0] : 0x7FFFFFFF;
    const float v1 = b1 < nb ? pv[row * nb + b1] : __int_as_float(0x7FC00000);
    const int j1 = b1 < nb ? pj[row * nb + b1] : 0x7FFFFFFF;
    float bv = v0;
    int bj = j0;
    if (better(v1, j1, bv, bj)) { bv = v1; bj = j1; }
    wave_best(bv, bj);
    if (lane == 0) g[row] = (bj == 0x7FFFFFFF) ? 0 : bj;  // all-NaN row: index 0
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < M - 1 && d[a] == g[a]) ++a;
    for (int i = 0; i < M; ++i) tokens[i] = (i <= a) ? g[i] : -1;
    counts[0] = a;
    counts[1] = a + 1;
    *rollback = base_len + a + 1;
  }
}

// ---- rejection sampling ----------------------------------------------------

__device__ __forceinline__ double e_of(float z, float zmax, double T) {
  return exp(((double)z - (double)zmax) / T);
}

// e_of(z) when its fixed-point value can be non-zero, else 0: below
// (z - zmax) / T = -70.5, e < 2.4e-31 < 2^-100 and floor(e * 2^100) is 0, so
// the exponential is skipped.  Every sum of the row is the same either way.
__device__ __forceinline__ double e_or_zero(float z, float zmax, double T) {
  const double x = ((double)z - (double)zmax) / T;
  return x < -70.5 ? 0.0 : exp(x);
}

// Nucleus threshold in fixed point: top_p * S (at least one unit, so that
// top_p <= 0 keeps exactly the first entry).
__device__ __forceinline__ Fx threshold(const RejArgs &p, double S) {
  Fx t = to_fx(p.top_p > 0.0 ? p.top_p * S : 0.0);
  if (!fx_nonzero(t)) t.lo = 1ull;
  return t;
}

// One radix-select step, run by all lanes of one wave over a 256-bin
// histogram in LDS (h[3b] mass lo, h[3b+1] mass hi, h[3b+2] count).  Walking
// from the top bin down, the chosen bin is the first whose inclusion brings
// the mass to `thr`; if rounding never gets there, the lowest occupied bin.
// `above` enters as the mass above the histogram's range and leaves as the
// mass strictly above the chosen bin.  Lane L covers bins 255-4L .. 252-4L.
__device__ __forceinline__ int select_bin_wave(const u64 *h, const Fx &thr, Fx &above) {
  const int lane = threadIdx.x & (kWave - 1);
  Fx m[4];
  u64 c[4];
  Fx lsum = fx_zero();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = kBins - 1 - 4 * lane - i;
    m[i] = Fx{h[3 * b], h[3 * b + 1]};
    c[i] = h[3 * b + 2];
    fx_add(lsum, m[i]);
  }
  Fx incl = dpp_fx_incl(lsum);
  Fx cum = fx_sum(above, fx_sub(incl, lsum));   // mass of all higher bins
  int found = -1, last = -1;
  Fx found_above = fx_zero(), last_above = fx_zero();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (c[i]) {
      const Fx next = fx_sum(cum, m[i]);
      if (found < 0 && fx_ge(next, thr)) { found = kBins - 1 - 4 * lane - i; found_above = cum; }
      last = kBins - 1 - 4 * lane - i;
      last_above = cum;
      cum = next;
    }
  }
  const u64 hit = __ballot(found >= 0);
  if (hit) {
    const int src = __ffsll((long long)hit) - 1;
    above = fx_readlane(found_above, src);
    return __shfl(found, src);
  }
  const u64 occ = __ballot(last >= 0);
  if (!occ) return -1;
  const int src = 63 - __clzll((long long)occ);
  above = fx_readlane(last_above, src);
  return __shfl(last, src);
}

// Row maxima (partial) and zeroing of this call's accumulators.
__global__ __launch_bounds__(kBlock) void rej_rowmax(RejArgs p) {
  const int b = blockIdx.x, row = blockIdx.y;
  const float *zr = p.z + (int64_t)row * p.ldl;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float m = -__builtin_inff();
  for (int base = j0; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(zr, base, j1, -__builtin_inff(), v);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) m = fmaxf(m, v[i]);
  }
  for (int s = kWave / 2; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  __shared__ float sm[kBlock / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) sm[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBlock / kWave; ++w) m = fmaxf(m, sm[w]);
    p.maxp[row * p.nb + b] = m;
  }
  // zero this row's histograms (4 passes) and total, spread over the row's blocks
  const int words = 4 * kBins * 4;
  for (int i = b * kBlock + threadIdx.x; i < words; i += p.nb * kBlock) {
    const int pass = i / (kBins * 4), w = i - pass * kBins * 4;
    hist_at(p, pass, row)[w] = 0ull;
  }
  if (b == 0 && threadIdx.x < 3) p.total[3 * row + threadIdx.x] = 0ull;
}

// Index of the t-th (1-based) entry of row `zr` with key == kappa, scanning in
// index order with the whole block.  Returns V-1 if there are fewer.
__device__ int find_tth_tie(const float *zr, int V, uint32_t kappa, int t) {
  __shared__ int cnt[kBlock];
  const int per = (V + kBlock - 1) / kBlock;
  const int j0 = threadIdx.x * per, j1 = min(V, j0 + per);
  int c = 0;
  for (int j = j0; j < j1; ++j) c += (fkey(zr[j]) == kappa);
  cnt[threadIdx.x] = c;
  __syncthreads();
  __shared__ int found;
  if (threadIdx.x == 0) {
    found = V - 1;
    int acc = 0;
    for (int i = 0; i < kBlock; ++i) {
      if (acc + cnt[i] >= t) {
        int need = t - acc;
        const int a0 = i * per, a1 = min(V, a0 + per);
        for (int j = a0; j < a1; ++j)
          if (fkey(zr[j]) == kappa && --need == 0) { found = j; break; }
        break;
      }
      acc += cnt[i];
    }
  }
  __syncthreads();
  const int r = found;
  __syncthreads();
  return r;
}

__device__ __forceinline__ bool in_nucleus(const RowState &rs, float z, int j) {
  if (rs.all & 1) return true;
  const uint32_t k = fkey(z);
  return k > rs.kappa || (k == rs.kappa && j <= rs.cutoff);
}

// One block per row, after the last radix pass: the last selection step
// fixes the nucleus (kappa and the tie cut), then the inputs of the row's
// acceptance test are taken.  Every load that does not depend on the
// selection (the draft's own entries, the state of the earlier steps, the
// histogram) is issued up front.
__global__ __launch_bounds__(kBlock) void rej_select(RejArgs p) {
  __shared__ u64 hbuf[kBins * 3];
  __shared__ RowState s_rs;
  __shared__ uint32_t s_kappa;
  __shared__ u64 s_t, s_n;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const float zmax = p.zmax[row];
  int x = -1;
  float zx = 0.0f;
  double qx = 0.0;
  if (threadIdx.x == 0 && row < p.M - 1) {
    x = p.drafts[row];
    if (x >= 0 && x < p.V) {
      zx = p.z[(int64_t)row * p.ldl + x];
      qx = (double)p.q[(int64_t)row * p.ldq + x];
    } else {
      x = -1;
    }
  }
  const double S = fx_to_double(fx_load3(p.total + 3 * row));
  if (p.top_p >= 1.0) {
    if (threadIdx.x == 0) s_rs = RowState{zmax, 0u, p.V, 1, S};
    __syncthreads();
  } else {
    const SelState st = p.sel[3 * p.M + row];
    hist_to_lds(hist_at(p, 3, row), hbuf);
    __syncthreads();
    if (wave == 0) {
      Fx above = Fx{st.above_lo, st.above_hi};
      const uint32_t prefix = st.prefix;
      const Fx thr = threshold(p, S);
      const int bin = select_bin_wave(hbuf, thr, above);
      const uint32_t kappa = (prefix << 8) | (uint32_t)(bin < 0 ? 0 : bin);
      if (lane == 0) {
        const u64 n = hbuf[3 * (kappa & 0xFF) + 2];
        const double ek = e_of(key_to_float(kappa), zmax, p.T);
        const double above_d = fx_to_double(above);
        const double tt = ceil((fx_to_double(thr) - above_d) / ek);
        const u64 t = (tt < 1.0) ? 1ull : (tt >= (double)n ? n : (u64)tt);
        s_kappa = kappa;
        s_t = t;
        s_n = n;
        s_rs = RowState{zmax, kappa, p.V, 0, above_d + (double)t * ek};
      }
    }
    __syncthreads();
    if (s_t < s_n) {   // ties at the cut: the first t of them in index order are inside
      const int cut = find_tth_tie(p.z + (int64_t)row * p.ldl, p.V, s_kappa, (int)s_t);
      if (threadIdx.x == 0) s_rs.cutoff = cut;
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    const RowState rs = s_rs;
    p.rows[row] = rs;
    if (row < p.M - 1) {
      double px = 0.0;
      if (x >= 0 && in_nucleus(rs, zx, x)) px = e_of(zx, rs.zmax, p.T) / rs.mass;
      p.acc[row] = AccIn{px, x >= 0 ? qx : 0.0};
    }
  }
}

// Radix pass `pass` (0..3).  Pass 0 reduces the row maximum and sums the
// row's total mass; pass s >= 1 first takes selection step s on histogram
// s-1 (every block computes the same result, block 0 records it for the
// next pass).  Then the pass histograms, by key digit, the mass of the
// entries that match the selected prefix and have non-zero mass.  The
// block's first entries are loaded before the selection step, so that their
// latency overlaps it.
__global__ __launch_bounds__(kBlock) void rej_pass(RejArgs p, int pass, int with_hist) {
  __shared__ u64 sh[kBins * 3];
  __shared__ u64 hprev[kBins * 3];
  __shared__ Fx red[kBlock / kWave];
  __shared__ float s_zmax;
  __shared__ uint32_t s_prefix;
  const int b = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const float *zr = p.z + (int64_t)row * p.ldl;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float v0[kBatch];
  load_batch(zr, j0, j1, -__builtin_inff(), v0);   // -inf: no mass
  for (int i = threadIdx.x; i < kBins * 3; i += kBlock) sh[i] = 0ull;
  if (pass == 0) {
    if (wave == 0) {
      float m = -__builtin_inff();
      for (int k = lane; k < p.nb; k += kWave) m = fmaxf(m, p.maxp[row * p.nb + k]);
      for (int s = kWave / 2; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
      if (lane == 0) {
        s_zmax = m;
        s_prefix = 0;
        if (b == 0) p.zmax[row] = m;
      }
    }
  } else {
    const float zm = p.zmax[row];
    const double S = fx_to_double(fx_load3(p.total + 3 * row));
    SelState st = SelState{0ull, 0ull, 0u, 0};
    if (pass > 1) st = p.sel[(pass - 1) * p.M + row];
    hist_to_lds(hist_at(p, pass - 1, row), hprev);
    __syncthreads();
    if (wave == 0) {
      Fx above = Fx{st.above_lo, st.above_hi};
      const int bin = select_bin_wave(hprev, threshold(p, S), above);
      const uint32_t prefix = (st.prefix << 8) | (uint32_t)(bin < 0 ? 0 : bin);
      if (lane == 0) {
        s_prefix = prefix;
        s_zmax = zm;
        if (b == 0) p.sel[pass * p.M + row] = SelState{above.lo, above.hi, prefix, 0};
      }
    }
  }
  __syncthreads();
  const float zmax = s_zmax;
  const uint32_t prefix = s_prefix;
  const int shift = 24 - 8 * pass;
  Fx tot = fx_zero();
  auto take = [&](const float (&v)[kBatch]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float zj = v[i];
      const uint32_t key = fkey(zj);
      if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
      const Fx e = to_fx(e_or_zero(zj, zmax, p.T));
      if (!fx_nonzero(e)) continue;     // below the fixed-point resolution: no mass
      if (pass == 0) fx_add(tot, e);
      if (with_hist) {
        const int d = (key >> shift) & 0xFF;
        u64 *bin = sh + 3 * d;
        if (e.lo) {
          const u64 old = atomicAdd(bin, e.lo);
          atomicAdd(bin + 1, e.hi + ((old + e.lo < old) ? 1ull : 0ull));
        } else {
          atomicAdd(bin + 1, e.hi);
        }
        atomicAdd(bin + 2, 1ull);
      }
    }
  };
  take(v0);
  for (int base = j0 + kBatch * kBlock; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(zr, base, j1, -__builtin_inff(), v);
    take(v);
  }
  if (pass == 0) {
    tot = fx_block_sum(tot, red);
    if (threadIdx.x == 0) fx_atomic_add3(p.total + 3 * row, tot);
  }
  if (with_hist) {
    __syncthreads();
    u64 *gh = hist_at(p, pass, row);
    for (int d = threadIdx.x; d < kBins; d += kBlock) {
      if (sh[3 * d + 2]) {
        fx_atomic_add3(gh + 4 * d, Fx{sh[3 * d], sh[3 * d + 1]});
        atomicAdd(gh + 4 * d + 3, sh[3 * d + 2]);
      }
    }
  }
}

// Accepted drafts: the first row i < M-1 with u_i * q_i(x_i) >= p'_i(x_i)
// stops the run (evaluated by every wave; wave-uniform result).
__device__ __forceinline__ int accepted_run(const RejArgs &p) {
  const int lane = threadIdx.x & (kWave - 1);
  bool reject = false;
  if (lane < p.M - 1) {
    const AccIn in = p.acc[lane];
    reject = !((double)p.u[lane] * in.qx < in.px);
  }
  const u64 rej = __ballot(reject);
  return rej ? __ffsll((long long)rej) - 1 : p.M - 1;
}

// Weights of the final draw for entry j of row `row`, in fixed point, and
// whether each is positive in fp64 (pe: e > 0, pres: e / mass - q > 0).  The
// fixed-point weights drop values below 2^-100; the flags do not, so that a
// draw whose target is below that resolution (u = 0 picks the first positive
// weight) still follows the fp64 weights.  (rs.mass >= 1, the row maximum's
// own weight.)
__device__ __forceinline__ void draw_weights(const RejArgs &p, const RowState &rs, int row,
                                             bool residual, int j, Fx &wres, Fx &we, bool &pres,
                                             bool &pe) {
  const float zj = p.z[(int64_t)row * p.ldl + j];
  double e = 0.0, x = 0.0;
  pe = false;
  const bool in = in_nucleus(rs, zj, j);
  if (in) {
    x = ((double)zj - (double)rs.zmax) / p.T;
    e = x < -70.5 ? 0.0 : exp(x);            // as e_or_zero
    pe = x > -744.0 || exp(x) > 0.0;         // exp(-744) ~ 1e-323 is still positive
  }
  we = to_fx(e);
  pres = false;
  if (residual) {
    const double qj = (double)p.q[(int64_t)row * p.ldq + j];
    const double d = e / rs.mass - qj;
    wres = to_fx(d > 0.0 ? d : 0.0);
    pres = d > 0.0;
    // e skipped below 2^-100: positive residual only where q is smaller still
    if (in && e == 0.0 && qj < 0x1p-100) pres = exp(x) / rs.mass - qj > 0.0;
  } else {
    wres = fx_zero();
  }
}

// The same weight in fp64, as the definition reads (no skipped exponential):
// e inside the nucleus, or max(0, e / mass - q).
__device__ __forceinline__ double draw_weight_f64(const RejArgs &p, const RowState &rs, int row,
                                                  bool residual, int j) {
  const float zj = p.z[(int64_t)row * p.ldl + j];
  const double e = in_nucleus(rs, zj, j) ? exp(((double)zj - (double)rs.zmax) / p.T) : 0.0;
  if (!residual) return e;
  const double d = e / rs.mass - (double)p.q[(int64_t)row * p.ldq + j];
  return d > 0.0 ? d : 0.0;
}

// A draw whose target u * W lies below the fixed-point resolution, in fp64
// and index order as the definition reads: W = w_0 + .. + w_{V-1} summed in
// order, then the smallest j whose running sum exceeds u * W (the last
// positive weight if rounding passes the end).  The block computes 256
// weights at a time; thread 0 adds them in order.  Slow (a sequential pass
// over the row), but reached only by u = 0-like targets that the first
// positive index does not settle, or by residuals whose every positive
// weight is below 2^-100.
template <int NT>
__device__ __forceinline__ int draw_f64_sequential(const RejArgs &p, const RowState &rs, int row,
                                                   bool residual, double u) {
  __shared__ double sw[NT];
  __shared__ double s_t;
  __shared__ int s_found, s_last;
  double W = 0.0;
  int last = -1;
  for (int base = 0; base < p.V; base += NT) {
    const int j = base + (int)threadIdx.x;
    sw[threadIdx.x] = j < p.V ? draw_weight_f64(p, rs, row, residual, j) : 0.0;
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < NT && base + i < p.V; ++i) {
        W += sw[i];
        if (sw[i] > 0.0) last = base + i;
      }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    s_t = u * W;
    s_found = -1;
    s_last = last;
  }
  __syncthreads();
  double cum = 0.0;
  for (int base = 0; base < p.V; base += NT) {
    const int j = base + (int)threadIdx.x;
    sw[threadIdx.x] = j < p.V ? draw_weight_f64(p, rs, row, residual, j) : 0.0;
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < NT && base + i < p.V; ++i) {
        cum += sw[i];
        if (cum > s_t) {
          s_found = base + i;
          break;
        }
      }
    __syncthreads();
    if (s_found >= 0) break;
  }
  const int r = s_found >= 0 ? s_found : (s_last >= 0 ? s_last : p.V - 1);
  __syncthreads();
  return r;
}

// Exclusive 128-bit prefix sums over the threads of the block (thread order);
// also returns the block total.  `wsum` holds kBlock/kWave Fx.
__device__ Fx fx_block_exclusive(Fx v, Fx *wsum, Fx &total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  Fx incl = dpp_fx_incl(v);
  __syncthreads();
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  Fx before = fx_zero();
  total = fx_zero();
  for (int w = 0; w < kBlock / kWave; ++w) {
    if (w < wave) fx_add(before, wsum[w]);
    fx_add(total, wsum[w]);
  }
  return fx_sum(before, fx_sub(incl, v));
}

// The final draw, in two kernels: rej_draw_sums has every block sum its chunk
// of the draw weights of the row of the final draw (row a of the first
// rejection, or the last row for the bonus); rej_draw_pick (one block)
// picks the smallest j with prefix weight > u * total (index order), or the
// last j with a positive weight if rounding passes the end, and writes the
// committed run.  It finds the chunk of the crossing from the chunk sums (a
// block-wide prefix, then the first crossing by atomic minimum), then the
// entry inside it.  (The kernel boundary, not an arrival counter, orders the
// chunk sums before the pick: one counter shared by thousands of blocks
// serialises their arrivals.)
__global__ __launch_bounds__(kBlock) void rej_draw_sums(RejArgs p) {
  __shared__ Fx wsum[kBlock / kWave];
  __shared__ int s_fr, s_fe;
  const int a = accepted_run(p);
  const int residual = a < p.M - 1;
  const RowState rs = p.rows[a];
  const int b = blockIdx.x;
  const int j0 = b * p.chunkd, j1 = min(p.V, j0 + p.chunkd);
  if (threadIdx.x == 0) {
    s_fr = kNone;
    s_fe = kNone;
  }
  __syncthreads();
  Fx sr = fx_zero(), se = fx_zero();
  int fr = kNone, fe = kNone;   // this thread's first positive entries (j rises)
  for (int j = j0 + threadIdx.x; j < j1; j += kBlock) {
    Fx wr, we;
    bool pr, pe;
    draw_weights(p, rs, a, residual != 0, j, wr, we, pr, pe);
    fx_add(sr, wr);
    fx_add(se, we);
    if (pr && fr == kNone) fr = j;
    if (pe && fe == kNone) fe = j;
  }
  if (fr != kNone) atomicMin(&s_fr, fr);
  if (fe != kNone) atomicMin(&s_fe, fe);
  sr = fx_block_sum(sr, wsum);   // (its barriers also order the minima above)
  se = fx_block_sum(se, wsum);
  if (threadIdx.x == 0) {
    u64 *o = p.blk + kBlkWords * b;
    o[0] = sr.lo;
    o[1] = sr.hi;
    o[2] = se.lo;
    o[3] = se.hi;
    o[4] = (u64)s_fr;
    o[5] = (u64)s_fe;
  }
}

__global__ __launch_bounds__(kBlock) void rej_draw_pick(RejArgs p) {
  __shared__ Fx wsum[kBlock / kWave];
  __shared__ int s_blk, s_lastnz, s_pick, s_fr, s_fe;
  __shared__ Fx s_before;
  __shared__ RowState s_rows[kMaxRows];
  // thread t holds chunks k0 .. k1-1 (in order); their sums and every row's
  // nucleus are loaded before the accepted run is known (none depends on it)
  constexpr int kPer = kMaxDrawBlocks / kBlock;
  const int per = (p.nbd + kBlock - 1) / kBlock;
  const int k0 = min(p.nbd, (int)threadIdx.x * per), k1 = min(p.nbd, k0 + per);
  Fx cr[kPer], ce[kPer];
  int fr = kNone, fe = kNone;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cr[i] = ce[i] = fx_zero();
    if (k0 + i < k1) {
      const u64 *o = p.blk + kBlkWords * (k0 + i);
      cr[i] = Fx{o[0], o[1]};
      ce[i] = Fx{o[2], o[3]};
      fr = min(fr, (int)o[4]);
      fe = min(fe, (int)o[5]);
    }
  }
  if (threadIdx.x < p.M) s_rows[threadIdx.x] = p.rows[threadIdx.x];
  if (threadIdx.x == 0) {
    s_fr = kNone;
    s_fe = kNone;
  }
  const int a = accepted_run(p);
  const int residual = a < p.M - 1;
  __syncthreads();
  if (fr != kNone) atomicMin(&s_fr, fr);
  if (fe != kNone) atomicMin(&s_fe, fe);
  const RowState rs = s_rows[a];
  Fx lres = fx_zero(), le = fx_zero();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    fx_add(lres, cr[i]);
    fx_add(le, ce[i]);
  }
  const Fx tres = fx_block_sum(lres, wsum);   // (its barriers also order the minima)
  const Fx te = fx_block_sum(le, wsum);
  // the residual is used when any of its fp64 weights is positive (its sum
  // in fp64 is then positive), even if all of them are below 2^-100
  const bool use_res = residual && s_fr != kNone;
  const double u = (double)p.u[p.M - 1];
  const Fx target = to_fx(u * fx_to_double(use_res ? tres : te));
  if (!fx_nonzero(target)) {
    // below the fixed-point resolution: u = 0 takes the first positive weight
    // (the first index whose running sum exceeds 0); any other target is
    // settled in fp64 by the sequential definition
    int pick;
    if (u == 0.0) {
      const int f = use_res ? s_fr : s_fe;
      pick = f != kNone ? f : p.V - 1;
    } else {
      pick = draw_f64_sequential<kBlock>(p, rs, a, use_res, u);
    }
    if (threadIdx.x < p.M) {
      const int i = threadIdx.x;
      p.tokens[i] = (i < a) ? p.drafts[i] : (i == a ? pick : -1);
    }
    if (threadIdx.x == 0) {
      p.counts[0] = a;
      p.counts[1] = a + 1;
      *p.rollback = p.base_len + a + 1;
    }
    return;
  }
  Fx total_unused;
  Fx cum = fx_block_exclusive(use_res ? lres : le, wsum, total_unused);
  if (threadIdx.x == 0) {
    s_blk = 0x7FFFFFFF;
    s_lastnz = -1;
    s_pick = -1;
  }
  __syncthreads();
  int found = -1, lastnz = -1;
  Fx found_before = fx_zero();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const Fx s = use_res ? cr[i] : ce[i];
    const Fx next = fx_sum(cum, s);
    if (k0 + i < k1) {
      if (found < 0 && fx_gt(next, target)) { found = k0 + i; found_before = cum; }
      if (fx_nonzero(s)) lastnz = k0 + i;
    }
    cum = next;
  }
  // prefix sums only grow: the first crossing chunk is the least one found
  if (found >= 0) atomicMin(&s_blk, found);
  if (lastnz >= 0) atomicMax(&s_lastnz, lastnz);
  __syncthreads();
  if (found >= 0 && found == s_blk) s_before = found_before;
  __syncthreads();
  const bool exact = s_blk != 0x7FFFFFFF;
  // exact: the crossing lies in chunk s_blk; otherwise rounding passed the
  // end and the pick is the last positive entry of the last positive chunk
  const int blk = exact ? s_blk : s_lastnz;
  if (blk >= 0) {
    const int j0 = blk * p.chunkd, j1 = min(p.V, j0 + p.chunkd);
    for (int base = j0; base < j1; base += kBlock) {
      // thread t holds entry base + t
      const int jt = base + (int)threadIdx.x;
      Fx wr = fx_zero(), we = fx_zero();
      bool pr, pe;
      if (jt < j1) draw_weights(p, rs, a, residual != 0, jt, wr, we, pr, pe);
      const Fx w = use_res ? wr : we;
      Fx total;
      const Fx before = fx_sum(s_before, fx_block_exclusive(w, wsum, total));
      if (exact) {
        // the entry whose weight crosses the target is the pick
        if (!fx_gt(before, target) && fx_gt(fx_sum(before, w), target)) s_pick = jt;
      } else if (fx_nonzero(w)) {
        atomicMax(&s_pick, jt);
      }
      __syncthreads();
      if (threadIdx.x == 0) s_before = fx_sum(s_before, total);
      __syncthreads();
    }
  }
  __syncthreads();
  const int pick = s_pick < 0 ? p.V - 1 : s_pick;   // no positive weight at all: the last id
  if (threadIdx.x < p.M) {
    const int i = threadIdx.x;
    p.tokens[i] = (i < a) ? p.drafts[i] : (i == a ? pick : -1);
  }
  if (threadIdx.x == 0) {
    p.counts[0] = a;
    p.counts[1] = a + 1;
    *p.rollback = p.base_len + a + 1;
  }
}

constexpr int kSSortMax = 2048;   // entries the one-launch resolvers sort at most

// Place in an LDS list for the lanes with `flag` (one atomic per wave on the
// list's count; order within the list unspecified).  Whole waves call it.
__device__ __forceinline__ int wave_append(bool flag, int *count) {
  const int lane = threadIdx.x & (kWave - 1);
  const u64 b = __ballot(flag);
  int base = 0;
  if (lane == 0 && b) base = atomicAdd(count, __popcll(b));
  base = __builtin_amdgcn_readfirstlane(base);   // every lane is active here
  return base + __popcll(b & ((1ull << lane) - 1ull));
}

// Sorts the n (<= kSSortMax) distinct non-zero values of a (LDS, room for
// kSSortMax) in descending order and returns where they are: in b (room for
// n) for n <= 256, ranked by counting (1024 / n2 lanes a value, four loads
// in flight a lane), else in a by a bitonic network.  The whole workgroup
// calls it.
__device__ __forceinline__ const u64 *sort_desc(u64 *a, u64 *b, int n) {
  const int tid = threadIdx.x;
  int n2 = 16;
  while (n2 < n) n2 <<= 1;
  __syncthreads();
  if (n2 <= 256) {
    const int P = kOneThreads / n2, e = tid / P, part = tid - e * P;
    const u64 mine = e < n ? a[e] : 0ull;
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    if (e < n) {
      int k = part;
      for (; k + 3 * P < n; k += 4 * P) {
        const u64 x0 = a[k], x1 = a[k + P], x2 = a[k + 2 * P], x3 = a[k + 3 * P];
        r0 += x0 > mine ? 1 : 0;
        r1 += x1 > mine ? 1 : 0;
        r2 += x2 > mine ? 1 : 0;
        r3 += x3 > mine ? 1 : 0;
      }
      for (; k < n; k += P) r0 += a[k] > mine ? 1 : 0;
    }
    int rank = (r0 + r1) + (r2 + r3);
    for (int s = P / 2; s > 0; s >>= 1) rank += __shfl_xor(rank, s);
    if (e < n && part == 0) b[rank] = mine;
    __syncthreads();
    return b;
  }
  for (int i = n + tid; i < n2; i += kOneThreads) a[i] = 0ull;
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      if (tid < n2 / 2) {
        const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1)), l = i | j;
        const u64 x = a[i], y = a[l];
        if ((i & k) == 0 ? x < y : x > y) {
          a[i] = y;
          a[l] = x;
        }
      }
    }
  }
  __syncthreads();
  return a;
}

// ---- rejection acceptance in one launch --------------------------------------
//
// The steps of the kernels above in one launch of G workgroups per row.  Each
// workgroup holds a chunk of up to kOneChunk entries of its row in LDS, with
// the entries' e values, for the whole call.  Rows never wait for each
// other, and a workgroup waits only on words of its own row in the
// workspace header:
//   (1) the row maximum: each workgroup publishes its chunk maximum in a
//       slot tagged with the call's generation number and waits until every
//       slot of its row carries this call's tag; with top_p < 1 it also hands
//       over its chunk's approximate mass and largest entries (exchange
//       words, see rej_top_settle);
//   (2a) with top_p < 1, wave 0 of every workgroup judges the row's exchange
//       words while the other waves start step 2: when they settle the cut,
//       workgroup 0 draws the row's token in one wave, publishes it with the
//       row's state and arrives for the whole row, and steps 2 to 4 are
//       skipped;
//   (2) the mass pass: the exact row total and an approximate fp64 mass
//       histogram over kXBins bins of x = (z - zmax) / T are summed over the
//       row.  x is a monotone function of z, so each bin is an interval of
//       keys, and these bins spread a row far more evenly than the leading
//       bits of its keys (the histogram's LDS atomics rarely collide).  The
//       last workgroup of the row to arrive derives, from the fp64 prefix
//       sums and a bound on their rounding, the range of bins that must hold
//       the nucleus cut, and publishes it in a tagged word;
//   (3) each workgroup adds the exact mass of its entries above that range
//       and writes its entries inside it (the candidates, in index order) to
//       its own segment of the workspace; the last to arrive resolves the cut
//       alone (an exact pass over fine bins of x, then an exact sort of the
//       fine bin that holds the cut), then publishes the row's state and
//       acceptance input behind a tagged word;
//   (4) every workgroup sums its chunk's draw weights for its own row before
//       the accepted run is known (the residual for a draft row, p' for
//       every row), per wave over contiguous ranges;
//   (5) the last workgroup of the last row to finish derives the accepted
//       run a from every row's acceptance input and picks the token from row
//       a's workgroup and range sums (or takes the token row a drew itself,
//       in one wave), then resets the counters and advances the generation
//       number.
// Every decision is taken on exact fixed-point sums, as in the kernels above,
// so the outputs are theirs.  A wait that runs past its bound sets the error
// word and goes on (no wave is left spinning).

constexpr int kSpinLimit = 1 << 21;
constexpr int kOneWaves = kOneThreads / kWave;
constexpr int kKPer = kOneChunk / kOneThreads;    // chunk entries per thread
constexpr int kResPer = 8;                        // candidate loads each thread keeps in flight
constexpr double kXScale = (double)kXBins / 70.5;
constexpr int kSortMax = kXBins / 4;              // entries of a fine bin sorted directly
static_assert(kXBins == kOneThreads, "one approximate bin per thread");
static_assert(kKPer * kOneThreads == kOneChunk, "whole entries per thread");
static_assert(kKPer * kOneWaves == 2 * kWave, "two compaction counts per lane");

// Draw ranges: each wave of a workgroup of the drawing row covers one_range(C)
// consecutive entries of the chunk; a thread of the picking workgroup holds
// at most kMaxRangesPerThread range sums.
__host__ __device__ constexpr int one_range(int C) { return (C + kOneWaves - 1) / kOneWaves; }
constexpr int kRanges = kMaxOneBlocks * kOneWaves;
constexpr int kMaxRangesPerThread = kRanges / kOneThreads;
static_assert(one_range(kOneChunk) <= kKPer * kWave, "a wave's range fits its registers");
static_assert(one_range(kOneChunk) <= kOneThreads, "a range fits one entry per thread");

__device__ __forceinline__ int wave_min(int v) { return dpp_imin(v); }
__device__ __forceinline__ int wave_max(int v) { return dpp_imax(v); }

// Approximate bin of an entry with non-zero fixed-point mass (x in [-70.5, 0]).
__device__ __forceinline__ int xbin(double x) {
  const int b = (int)(-x * kXScale);
  return b < kXBins - 1 ? b : kXBins - 1;
}

__device__ __forceinline__ u64 ld_ag(const u64 *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(u64 *p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agi(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agi(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agd(const double *p) {
  return __longlong_as_double((long long)ld_ag(reinterpret_cast<const u64 *>(p)));
}

// Data crossing workgroups is only ever written by agent-scope atomic
// stores and read-modify-writes and read by agent-scope atomic loads, which
// all act at the coherence point beyond the per-XCD caches; so ordering needs
// no cache-wide fences (an agent-scope acquire or release would write back
// or invalidate the whole L2), only completion: every thread waits for its
// own writes (s_waitcnt) before the arrival that publishes them is counted,
// and a reader issues its loads only after it has seen that arrival.

// The calling lane waits until slot s carries tag in its high word and
// returns it (bounded: past kSpinLimit polls the error word is set and the
// wait ends).
__device__ __forceinline__ u64 wait_slot(const u64 *s, uint32_t tag, u64 *err) {
  u64 v = ld_ag(s);
  int it = 0;
  while ((uint32_t)(v >> 32) != tag) {
    if (++it > kSpinLimit) {
      st_ag(err, 1ull);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    v = ld_ag(s);
  }
  return v;
}

// Workgroup-wide exact sum (all kOneThreads threads); valid in every thread.
__device__ Fx fx_sum_one(Fx a, Fx *red) {
  a = fx_wave_sum(a);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = a;
  __syncthreads();
  Fx s = fx_zero();
  for (int i = 0; i < kOneWaves; ++i) fx_add(s, red[i]);
  return s;
}

// Exclusive exact prefix over the threads (thread order) and the total.
__device__ __forceinline__ Fx fx_excl_one(Fx v, Fx *red, Fx &total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const Fx incl = dpp_fx_incl(v);
  __syncthreads();
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  Fx before = fx_zero();
  total = fx_zero();
  for (int w = 0; w < kOneWaves; ++w) {
    if (w < wave) fx_add(before, red[w]);
    fx_add(total, red[w]);
  }
  return fx_sum(before, fx_sub(incl, v));
}

// Inclusive fp64 prefix over the threads in one fixed order of additions (so
// every workgroup that runs it on the same values gets the same sums).
__device__ double dscan_one(double v, double *dred) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const double incl = dpp_dincl(v);
  __syncthreads();
  if (lane == kWave - 1) dred[wave] = incl;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += dred[w];
  return before + incl;
}

// Workgroup-wide count of `flag` and the exclusive count before this thread.
__device__ int count_one(bool flag, int &before, int *wcnt) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const u64 b = __ballot(flag);
  __syncthreads();
  if (lane == 0) wcnt[wave] = __popcll(b);
  __syncthreads();
  int tot = 0, pre = 0;
  for (int w = 0; w < kOneWaves; ++w) {
    if (w < wave) pre += wcnt[w];
    tot += wcnt[w];
  }
  before = pre + __popcll(b & ((1ull << lane) - 1ull));
  return tot;
}

// Adds mass e (non-zero) with one count to LDS bin d (lo with carry, hi).
__device__ __forceinline__ void hist_add(u64 *sh, int d, const Fx &e) {
  u64 *bin = sh + 3 * d;
  if (e.lo) {
    const u64 old = atomicAdd(bin, e.lo);
    atomicAdd(bin + 1, e.hi + ((old + e.lo < old) ? 1ull : 0ull));
  } else {
    atomicAdd(bin + 1, e.hi);
  }
  atomicAdd(bin + 2, 1ull);
}

// The draw weights of entry j (as draw_weights) from its logit zj and draft
// probability qj at hand; e_all is its e_or_zero value when have_e, else it
// is computed here (inside the nucleus only).  The exponential is taken at
// most twice: e itself, and exp(x) again only where e is not positive (the
// flags then need the unskipped value).
__device__ __forceinline__ void draw_weights_v(const RowState &rs, double T, bool residual, int j,
                                               float zj, double qj, bool have_e, double e_all,
                                               Fx &wres, Fx &we, bool &pres, bool &pe) {
  const bool in = in_nucleus(rs, zj, j);
  double e = 0.0, x = 0.0, ex = 0.0;
  if (in) {
    x = ((double)zj - (double)rs.zmax) / T;
    if (!have_e) e_all = x < -70.5 ? 0.0 : exp(x);
    e = e_all;
    ex = e > 0.0 ? e : exp(x);
  }
  pe = in && (e > 0.0 || x > -744.0 || ex > 0.0);
  we = to_fx(e);
  pres = false;
  wres = fx_zero();
  if (residual) {
    const double d = e / rs.mass - qj;
    wres = to_fx(d > 0.0 ? d : 0.0);
    pres = d > 0.0;
    if (in && e == 0.0 && qj < 0x1p-100) pres = ex / rs.mass - qj > 0.0;
  }
}

// A row's state in six tagged words of its page (tag << 32 | 32 bits):
// kappa, cutoff, all, the two halves of mass, and zmax.  Each word carries
// the tag, so a reader that sees all six tags has the whole state in one
// round trip, whatever order the stores landed in.
constexpr int kStateWords = 6;

__device__ __forceinline__ void publish_state(u64 *rp, uint32_t tag, const RowState &rs) {
  const u64 mb = (u64)__double_as_longlong(rs.mass);
  const uint32_t v[kStateWords] = {rs.kappa, (uint32_t)rs.cutoff, (uint32_t)rs.all, (uint32_t)mb,
                                   (uint32_t)(mb >> 32), __float_as_uint(rs.zmax)};
  for (int i = 0; i < kStateWords; ++i) st_ag(rp + kRowState + i, ((u64)tag << 32) | v[i]);
}

__device__ __forceinline__ RowState row_state_of(const u64 *w) {
  RowState rs;
  __builtin_memcpy(&rs, w, sizeof(rs));
  return rs;
}

// Called by a whole wave: lanes 0..5 wait for their word; the state is
// returned in every lane.
__device__ __forceinline__ RowState wait_state(const u64 *rp, uint32_t tag, u64 *err) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t w = lane < kStateWords ? (uint32_t)wait_slot(rp + kRowState + lane, tag, err) : 0u;
  RowState rs;
  rs.zmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)w, 5));
  rs.kappa = (uint32_t)__builtin_amdgcn_readlane((int)w, 0);
  rs.cutoff = __builtin_amdgcn_readlane((int)w, 1);
  rs.all = __builtin_amdgcn_readlane((int)w, 2);
  const u64 mb = (u64)(uint32_t)__builtin_amdgcn_readlane((int)w, 3) |
                 ((u64)(uint32_t)__builtin_amdgcn_readlane((int)w, 4) << 32);
  rs.mass = __longlong_as_double((long long)mb);
  return rs;
}

// Acceptance input of a draft row: p'(x) under nucleus rs and q(x), for a
// draft x whose logit zx and draft probability qx are at hand (valid: x in
// [0, V)).
__device__ __forceinline__ void publish_acc(const RejArgs &p, int row, const RowState &rs, int x,
                                            bool valid, float zx, float qx) {
  double px = 0.0, qd = 0.0;
  if (valid) {
    if (in_nucleus(rs, zx, x)) px = e_of(zx, rs.zmax, p.T) / rs.mass;
    qd = (double)qx;
  }
  u64 *o = reinterpret_cast<u64 *>(p.acc + row);
  st_ag(o, (u64)__double_as_longlong(px));
  st_ag(o + 1, (u64)__double_as_longlong(qd));
}

// Loads the draft of row `row` (< M-1), its logit and draft probability.
__device__ __forceinline__ void load_draft(const RejArgs &p, int row, int &x, bool &valid,
                                           float &zx, float &qx) {
  x = p.drafts[row];
  valid = x >= 0 && x < p.V;
  zx = valid ? p.z[(int64_t)row * p.ldl + x] : 0.0f;
  qx = valid ? p.q[(int64_t)row * p.ldq + x] : 0.0f;
}

// The token of a row whose nucleus is at hand, as the picker of rej_one
// draws it when the accepted run stops at the row: the residual
// max(0, p' - q) for a draft row (p' if that is all zero), else p', in index
// order, with u_{M-1}.  srt holds the N <= kOneThreads nucleus entries in
// index order as (~index << 32 | slot); at(slot, z, q) gives an entry's
// logit and the draft's q at it.  The whole workgroup calls it; every thread
// gets the token.
template <typename At>
__device__ __forceinline__ int rej_nucleus_draw(const RejArgs &p, const RowState &rs, int row, const u64 *srt,
                                int N, const At &at, Fx *red) {
  __shared__ int s_fr, s_fe, s_pick, s_lastw;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const bool residual = row < p.M - 1;
  if (tid == 0) {
    s_fr = kNone;
    s_fe = kNone;
    s_pick = -1;
    s_lastw = -1;
  }
  __syncthreads();
  int jt = -1;
  Fx wr = fx_zero(), we = fx_zero();
  bool pr = false, pe = false;
  if (tid < N) {
    const u64 v = srt[tid];
    jt = (int)(0xFFFFFFFFu - (uint32_t)(v >> 32));
    float zt, qt;
    at((int)(uint32_t)v, zt, qt);
    draw_weights_v(rs, p.T, residual, jt, zt, (double)qt, false, 0.0, wr, we, pr, pe);
  }
  {   // the first index with a positive fp64 residual, resp. p'
    const int fr = wave_min(pr ? jt : kNone), fe = wave_min(pe ? jt : kNone);
    if (lane == 0) {
      if (fr != kNone) atomicMin(&s_fr, fr);
      if (fe != kNone) atomicMin(&s_fe, fe);
    }
  }
  __syncthreads();
  const bool use_res = residual && s_fr != kNone;
  const Fx w = use_res ? wr : we;
  Fx tot;
  const Fx bef = fx_excl_one(w, red, tot);   // (its barriers also publish s_fr, s_fe)
  const double u = (double)p.u[p.M - 1];
  const Fx target = to_fx(u * fx_to_double(tot));
  if (!fx_nonzero(target)) {
    if (u == 0.0) {
      const int f = use_res ? s_fr : s_fe;
      return f != kNone ? f : p.V - 1;
    }
    return draw_f64_sequential<kOneThreads>(p, rs, row, use_res, u);
  }
  if (tid < N && !fx_gt(bef, target) && fx_gt(fx_sum(bef, w), target)) s_pick = jt;
  const int lw = wave_max(tid < N && fx_nonzero(w) ? jt : -1);
  if (lane == 0 && lw >= 0) atomicMax(&s_lastw, lw);
  __syncthreads();
  return s_pick >= 0 ? s_pick : (s_lastw >= 0 ? s_lastw : p.V - 1);
}

// ---- rej_one: rows whose cut the top entries settle ------------------------
//
// Steps (1) and (2a) of rej_one.  Every workgroup of a row with top_p < 1
// hands over, with its chunk maximum, an approximate mass of its chunk, its
// kTopK largest entries and its (kTopK + 1)-th key; every workgroup of the
// row then reads all of them and takes the same decision, on the same words
// in the same order.  A workgroup hands over all of its entries above its
// own r-th key (r <= kTopK), so the entries above the largest of the
// workgroups' r-th keys are a prefix of the row in nucleus order (a top
// set).  Sa, the sum of the chunks' approximate masses, differs from the
// exact mass S of step 2 (fixed point, below V 2^-100 lost) by a relative
// error below 2^-14: its terms are fp32 exponentials of arguments below 2^8
// in magnitude (one ulp each, plus the argument's three roundings), summed
// eight at a time in fp32 and in fp64 beyond.  So the threshold lies between
// the thresholds of Sa (1 -+ 2^-9) -+ V 2^-98, and the cut is settled when,
// over a top set in nucleus order, the first group of equal keys whose exact
// prefix reaches the upper threshold is the first to reach the lower one,
// and the count of its ties inside is the same under both.  The row's state
// then is the one steps 2 and 3 would find.

constexpr double kLog2e = 1.4426950408889634;

// (key << 32 | index) -> a value that descends in nucleus order (key
// descending, index ascending)
__device__ __forceinline__ u64 order_key(u64 e) {
  return (e & 0xFFFFFFFF00000000ull) | (0xFFFFFFFFull - (e & 0xFFFFFFFFull));
}

__device__ __forceinline__ uint32_t lane_push(int to, uint32_t v) {   // v to lane `to`
  return (uint32_t)__builtin_amdgcn_ds_permute(to * 4, (int)v);
}

// Run by one whole wave.  xw: the row's exchange words (payloads), workgroup
// b's at xw + b * kXW; lst: kWave entries of LDS scratch.  Returns the row
// maximum in zmax and whether the cut is settled; if so, the row's state in
// rs and, in lanes < n (the nucleus, in nucleus order), the entries (key << 32
// | index), their e (as step 2 computes it) and, when want_q, the draft's q.
// The top sets tried grow: entries above the largest of the workgroups' r-th
// keys for r = 1, ..., kTopK (a workgroup handed over all of its entries
// above its own r-th key, its (kTopK + 1)-th in word 2, so each is a prefix of
// the row), until one holds a group that reaches the lower threshold.
__device__ __forceinline__ bool rej_top_settle(const RejArgs &p, int row, int G, const uint32_t *xw,
                                               u64 *lst, bool want_q, float &zmax, RowState &rs,
                                               u64 &ent, double &ee, float &qe, int &n) {
  const int lane = threadIdx.x & (kWave - 1);
  const double T = p.T;
  const float L2 = (float)(kLog2e / T);
  uint32_t best = fkey(-__builtin_inff());
  for (int b = lane; b < G; b += kWave) best = max(best, xw[b * kXW]);
  best = dpp_umax(best);
  zmax = key_to_float(best);
  double sa = 0.0;   // (the chunks' masses scaled by fp32 exponentials too)
  for (int b = lane; b < G; b += kWave) {
    const float sg = __uint_as_float(xw[b * kXW + 1]);
    if (sg > 0.0f)
      sa += (double)sg * (double)__builtin_amdgcn_exp2f((key_to_float(xw[b * kXW]) - zmax) * L2);
  }
  sa = dbl_readlane(dpp_dincl(sa), kWave - 1);
  n = 0;
  if (!(fabsf(zmax) <= 3.4e38f) || !(sa >= 0.5 && sa <= 1e300)) return false;
  const double slo = fmax(0.0, sa * (1.0 - 0x1p-9) - (double)p.V * 0x1p-98);
  const double shi = sa * (1.0 + 0x1p-9) + (double)p.V * 0x1p-98;
  const Fx thl = threshold(p, slo), thh = threshold(p, shi);
  auto fx_int = [](int k) { return Fx{0ull, (u64)k << 36}; };   // k in fixed point (1 = 2^100)
  if (fx_gt(thl, fx_int(G * kTopK))) return false;   // (every e is at most 1)
  {
    // the common case first: the row maximum alone reaches the upper
    // threshold (its e is exactly 1) and no other entry ties with it (it is
    // the only handed-over entry with its key, and every workgroup's second
    // key lies below it); then the nucleus is that entry, as the general
    // steps below would find
    uint32_t k2 = 0u;
    for (int b = lane; b < G; b += kWave) k2 = max(k2, xw[b * kXW + 5]);
    k2 = dpp_umax(k2);
    int at = -1, cnt = 0;
    for (int c0 = 0; c0 < G * kTopK; c0 += kWave) {
      const int c = c0 + lane, b = c / kTopK, i = c - b * kTopK;
      const bool f = c < G * kTopK && xw[b * kXW + 3 + 2 * i] == best;
      const u64 bal = __ballot(f);
      if (bal && at < 0) at = __builtin_amdgcn_readlane(c < G * kTopK ? (int)xw[b * kXW + 4 + 2 * i] : 0,
                                                        __ffsll((long long)bal) - 1);
      cnt += __popcll(bal);
    }
    if (k2 < best && cnt == 1 && !fx_gt(thh, fx_int(1)) && (uint32_t)at < (uint32_t)p.V) {
      rs = RowState{zmax, best, p.V, 0, 1.0};
      n = 1;
      ent = ((u64)best << 32) | (uint32_t)at;
      ee = 1.0;
      qe = want_q && lane == 0 ? p.q[(int64_t)row * p.ldq + at] : 0.0f;
      return true;
    }
  }
#pragma unroll 1
  for (int r = 1; r <= kTopK; ++r) {
    const int wk = r == kTopK ? 2 : 3 + 2 * r;
    uint32_t ks = 0u;
    for (int b = lane; b < G; b += kWave) ks = max(ks, xw[b * kXW + wk]);
    ks = dpp_umax(ks);
    int nt = 0;
    for (int c0 = 0; c0 < G * kTopK; c0 += kWave) {
      const int c = c0 + lane;
      bool f = false;
      u64 e = 0ull;
      if (c < G * kTopK) {
        const int b = c / kTopK, i = c - b * kTopK;
        const uint32_t key = xw[b * kXW + 3 + 2 * i];
        f = key > ks;
        e = ((u64)key << 32) | xw[b * kXW + 4 + 2 * i];
      }
      const u64 bal = __ballot(f);
      const int pos = nt + __popcll(bal & ((1ull << lane) - 1ull));
      if (f && pos < kWave) lst[pos] = e;
      nt += __popcll(bal);
    }
    if (nt > kWave) return false;
    if (nt == 0 || fx_gt(thl, fx_int(nt))) continue;   // (every e is at most 1)
    __builtin_amdgcn_wave_barrier();
    const bool val = lane < nt;
    const u64 te = val ? lst[lane] : 0ull;
    if (__ballot(val && (uint32_t)te >= (uint32_t)p.V)) return false;   // (never: indices of the row)
    float tq = 0.0f;
    if (want_q && val) tq = p.q[(int64_t)row * p.ldq + (int)(uint32_t)te];   // (used at the end)
    // nucleus order: each entry's rank, then entry r to lane r
    const u64 ok = order_key(te);
    int rank = val ? 0 : lane;
    for (int k = 0; k < nt; ++k) {
      const u64 o = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(ok >> 32), k) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)ok, k);
      rank += (val && o > ok) ? 1 : 0;
    }
    const uint32_t skey = lane_push(rank, (uint32_t)(te >> 32));
    const uint32_t sidx = lane_push(rank, (uint32_t)te);
    // exact prefix masses (e as step 2 computes it) and the cut group
    const double e = val ? e_or_zero(key_to_float(skey), zmax, T) : 0.0;
    const Fx f = to_fx(e);
    const Fx incl = dpp_fx_incl(f);
    const uint32_t nkey =
        (uint32_t)__builtin_amdgcn_ds_bpermute(((lane + 1) & (kWave - 1)) * 4, (int)skey);
    const bool gend = val && (lane == nt - 1 || nkey != skey);
    const u64 hh = __ballot(gend && fx_ge(incl, thh)), hl = __ballot(gend && fx_ge(incl, thl));
    if (!hl) continue;   // the cut lies beyond this set
    if (!hh || __ffsll((long long)hh) != __ffsll((long long)hl)) return false;
    const int gl = __ffsll((long long)hh) - 1;   // the cut group's last entry
    const uint32_t kappa = (uint32_t)__builtin_amdgcn_readlane((int)skey, gl);
    const int gs = __ffsll((long long)__ballot(val && skey == kappa)) - 1;   // its first
    const double above_d = fx_to_double(fx_readlane(fx_sub(incl, f), gs));
    const int nk = gl - gs + 1;
    const double ek = dbl_readlane(e, gs);   // (e_of at kappa: its x is above -70.5)
    auto ties_in = [&](const Fx &th) {   // as steps 2 and 3 count them
      const double tt = ceil((fx_to_double(th) - above_d) / ek);
      return tt < 1.0 ? 1 : (tt >= (double)nk ? nk : (int)tt);
    };
    const int t = nk == 1 ? 1 : ties_in(thl);
    if (nk > 1 && t != ties_in(thh)) return false;
    const int cutoff = t < nk ? __builtin_amdgcn_readlane((int)sidx, gs + t - 1) : p.V;
    rs = RowState{zmax, kappa, cutoff, 0, above_d + (double)t * ek};
    n = gs + t;
    ent = ((u64)skey << 32) | sidx;
    ee = e;
    qe = __uint_as_float(lane_push(rank, __float_as_uint(tq)));
    return true;
  }
  return false;
}

// rej_nucleus_draw by one wave, for n <= kWave nucleus entries held by lanes
// < n (key << 32 | index, e as step 2 computes it, draft q) in any order.  Returns the token, or -2
// when u > 0 and the target falls below the fixed-point resolution (the
// fp64 sequence over the row then decides); use_res as it drew.
__device__ __forceinline__ int wave_nucleus_draw(const RejArgs &p, const RowState &rs, int row,
                                                 u64 ent, double ee, float qe, int n, double u,
                                                 bool &use_res) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool residual = row < p.M - 1, val = lane < n;
  const int j = val ? (int)(uint32_t)ent : kNone;
  int jt = j;
  float zt = key_to_float((uint32_t)(ent >> 32)), qt = qe;
  double et = ee;
  if (n > 1) {   // index order
    int rank = val ? 0 : lane;
    for (int k = 0; k < n; ++k) rank += (val && __builtin_amdgcn_readlane(j, k) < j) ? 1 : 0;
    jt = (int)lane_push(rank, (uint32_t)j);
    zt = key_to_float(lane_push(rank, (uint32_t)(ent >> 32)));
    qt = __uint_as_float(lane_push(rank, __float_as_uint(qe)));
    const u64 eb = (u64)__double_as_longlong(ee);
    et = __longlong_as_double((long long)(((u64)lane_push(rank, (uint32_t)(eb >> 32)) << 32) |
                                          lane_push(rank, (uint32_t)eb)));
  }
  Fx wr = fx_zero(), we = fx_zero();
  bool pr = false, pe = false;
  if (val) draw_weights_v(rs, p.T, residual, jt, zt, (double)qt, true, et, wr, we, pr, pe);
  const int fr = wave_min(pr ? jt : kNone), fe = wave_min(pe ? jt : kNone);
  use_res = residual && fr != kNone;
  const Fx w = use_res ? wr : we;
  const Fx incl = dpp_fx_incl(w);
  const Fx target = to_fx(u * fx_to_double(fx_readlane(incl, kWave - 1)));
  if (!fx_nonzero(target)) {
    if (u == 0.0) {
      const int f = use_res ? fr : fe;
      return f != kNone ? f : p.V - 1;
    }
    return -2;
  }
  const u64 hit = __ballot(val && !fx_gt(fx_sub(incl, w), target) && fx_gt(incl, target));
  if (hit) return __builtin_amdgcn_readlane(jt, __ffsll((long long)hit) - 1);
  const int lw = wave_max(val && fx_nonzero(w) ? jt : -1);
  return lw >= 0 ? lw : p.V - 1;
}

// Step 5 of rej_one by one wave (of the last workgroup to arrive) when the
// accepted run ends at a row that drew its own token: every row's acceptance
// input, state word `all` and token word are loaded at once, then the run a
// (the first rejected draft, else M - 1) and row a's token give the outputs,
// and the counters are reset for the next call.  Returns false, writing
// nothing, when row a's token is left to the workgroup's draw.
__device__ __forceinline__ bool rej_pick_drawn(const RejArgs &p, uint32_t tag, u64 gen, u64 *err) {
  const int lane = threadIdx.x & (kWave - 1), M = p.M;
  u64 ax = 0ull, aq = 0ull, ws = 0ull, wp = 0ull;
  float ul = 0.0f;
  if (lane < M - 1) {
    const u64 *o = reinterpret_cast<const u64 *>(p.acc + lane);
    ax = ld_ag(o);
    aq = ld_ag(o + 1);
    ul = p.u[lane];
  }
  if (lane < M) {
    const u64 *r = p.hdr + (size_t)lane * kPageWords;
    ws = ld_ag(r + kRowState + 2);
    wp = ld_ag(r + kRowPick);
  }
  const double px = __longlong_as_double((long long)ax), qx = __longlong_as_double((long long)aq);
  const u64 rej = __ballot(lane < M - 1 && !((double)ul * qx < px));
  const int a = rej ? __ffsll((long long)rej) - 1 : M - 1;
  auto lane_u64 = [&](u64 v) {
    return ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), a) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, a);
  };
  u64 wsa = lane_u64(ws);
  if ((uint32_t)(wsa >> 32) != tag) wsa = wait_slot(p.hdr + (size_t)a * kPageWords + kRowState + 2, tag, err);
  if (!((uint32_t)wsa & 2u)) return false;
  u64 wpa = lane_u64(wp);
  if ((uint32_t)(wpa >> 32) != tag) wpa = wait_slot(p.hdr + (size_t)a * kPageWords + kRowPick, tag, err);
  const int pick = (int)(uint32_t)wpa;
  if (lane < M) p.tokens[lane] = lane < a ? p.drafts[lane] : (lane == a ? pick : -1);
  if (lane == 0) {
    p.counts[0] = a;
    p.counts[1] = a + 1;
    *p.rollback = p.base_len + a + 1;
  }
  // every other workgroup is done with the counters: reset them, advance the generation
  if (lane < M) {
    u64 *r = p.hdr + (size_t)lane * kPageWords;
    st_ag(r + kRowCnt, 0ull);
    st_ag(r + kRowCand, 0ull);
    st_ag(r + kRowDraw, 0ull);
  }
  if (lane == 0) {
    u64 *cp = p.hdr + (size_t)kMaxRows * kPageWords;
    st_ag(cp + kCallRows, 0ull);
    st_ag(cp + kCallGen, gen);
  }
  return true;
}

__global__ __launch_bounds__(kOneThreads) void rej_one(RejArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  const int C = p.C;
  float *zc = reinterpret_cast<float *>(dyn);                          // [C] logits
  double *ec = reinterpret_cast<double *>(dyn + one_e_offset(C));      // [C] e_or_zero
  uint16_t *bc = reinterpret_cast<uint16_t *>(dyn + one_b_offset(C));  // [C] bin or 0xFFFF
  __shared__ u64 hx[3 * kXBins];   // exact bin masses, three carry-free limbs (fx_atomic_add3)
  __shared__ u64 sh[kBins * 3];
  __shared__ Fx red[kOneWaves], wred[kOneWaves];
  __shared__ double dred[kOneWaves];
  __shared__ int wcnt[kOneWaves];
  __shared__ int koff[kKPer * kOneWaves + 1], koffa[kKPer * kOneWaves + 1];
  __shared__ int segoff[kMaxOneBlocks], aoff[kMaxOneBlocks];
  __shared__ float s_f[kOneWaves];
  __shared__ u64 s_gen, s_abv_lo, s_abv_hi, s_nk;
  __shared__ u64 s_w[6];
  __shared__ float s_zmax, s_zx, s_qx;
  __shared__ uint32_t s_kmin, s_kmax, s_prefix;
  __shared__ int s_blo, s_bhi, s_last, s_flag, s_nc, s_cut, s_a, s_x;
  __shared__ int s_pick, s_blk, s_lastnz, s_fr, s_fe;
  __shared__ int s_an, s_drew, s_lastw, s_nc2;
  __shared__ int s_fast, s_next;
  __shared__ double s_sw[kOneWaves];
  __shared__ u64 s_tk[kOneWaves * (kTopK + 1)], s_lst[kWave];
  __shared__ Fx s_before;
  const int G = p.G, row = blockIdx.x / G, g = blockIdx.x - row * G;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int j0 = g * C, n = min(C, p.V - j0);
  u64 *const rp = p.hdr + (size_t)row * kPageWords;            // this row's page
  u64 *const cp = p.hdr + (size_t)kMaxRows * kPageWords;       // the call's page
  u64 *const err = cp + kCallErr;
  const bool nucleus = !(p.top_p >= 1.0);
  const double T = p.T;
  bool chunk_lost = false;   // this workgroup's LDS holds candidates, not its chunk

  // (1) the chunk into LDS and its maximum; this row's sums are cleared
  // (shared out over the row's workgroups) before the maximum is published.
  // With top_p < 1 each workgroup then also hands over its chunk's
  // approximate mass and top entries, read and judged in step 2a.
  if (tid == 0) {
    s_gen = ld_ag(cp + kCallGen) + 1ull;
    s_drew = 0;
    s_fast = 0;
  }
  const float *zr = p.z + (int64_t)row * p.ldl + j0;
  u64 *const xg = p.hdr + kXchg + (size_t)row * G * kXW;   // the row's exchange words
  {
    float v[kKPer];
#pragma unroll
    for (int k = 0; k < kKPer; ++k) {
      const int i = k * kOneThreads + tid;
      v[k] = i < n ? zr[i] : -__builtin_inff();
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kKPer; ++k) {
      const int i = k * kOneThreads + tid;
      if (i < n) zc[i] = v[k];
      m = fmaxf(m, v[k]);
    }
    if (nucleus)
      for (int w = g * kOneThreads + tid; w < kXBins; w += G * kOneThreads)
        st_ag(reinterpret_cast<u64 *>(p.ahist + (size_t)row * kXBins) + w, 0ull);
    if (g == 0 && tid < 3) {
      st_ag(p.total + 3 * row + tid, 0ull);
      st_ag(p.above + 3 * row + tid, 0ull);
    }
    const float mt = m;   // this thread's maximum
    m = dpp_fmax(m);
    if (lane == 0) s_f[wave] = m;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t tag = (uint32_t)s_gen;
    const float mg = dpp_fmax(lane < kOneWaves ? s_f[lane] : -__builtin_inff());
    if (wave == 0) {   // this chunk's maximum out, the row's in
      if (lane == 0)
        st_ag(nucleus ? xg + (size_t)g * kXW : rp + kRowSlots + g, ((u64)tag << 32) | fkey(mg));
      const u64 *sl = nucleus ? xg : rp + kRowSlots;
      const int st = nucleus ? kXW : 1;
      uint32_t best = fkey(-__builtin_inff());
      for (int q = lane; q < G; q += kWave) {
        u64 w = ld_ag(sl + (size_t)q * st);
        if ((uint32_t)(w >> 32) != tag) w = wait_slot(sl + (size_t)q * st, tag, err);
        best = max(best, (uint32_t)w);
      }
      best = dpp_umax(best);
      if (lane == 0) s_zmax = key_to_float(best);
    }
    if (nucleus) {
      // each wave's mass relative to the chunk maximum (fp32
      // exponentials) and its kTopK + 1 largest keys with multiplicity (the
      // winning lane of a round takes its next largest); then wave 0 merges
      // them into this chunk's words
      const float L2 = (float)(kLog2e / T);
      float sw = 0.0f;
      if (mg > -__builtin_inff()) {
#pragma unroll
        for (int k = 0; k < kKPer; ++k) sw += __builtin_amdgcn_exp2f((v[k] - mg) * L2);
      }
      const double swd = dbl_readlane(dpp_dincl((double)sw), kWave - 1);
      // only a wave with at most kTopK wave maxima above its own can hold
      // one of the chunk's kTopK + 1 largest entries: the others' entries lie
      // below the chunk's (kTopK + 1)-th key and are left out
      const bool part =
          __popcll(__ballot(lane < kOneWaves && s_f[lane & (kOneWaves - 1)] > m)) <= kTopK;
      uint32_t kk[kKPer];
#pragma unroll
      for (int k = 0; k < kKPer; ++k) kk[k] = fkey(v[k]);
      uint32_t bv = fkey(mt);
      int bk = 0;
#pragma unroll
      for (int k = kKPer - 1; k >= 0; --k) bk = kk[k] == bv ? k : bk;
      uint32_t taken = 0u;
      if (!part && lane <= kTopK) s_tk[wave * (kTopK + 1) + lane] = 0ull;
#pragma unroll 1
      for (int r = 0; part && r <= kTopK; ++r) {
        const uint32_t wm = dpp_umax(bv);
        const int wl = __ffsll((long long)__ballot(bv == wm)) - 1;
        const int wi = __builtin_amdgcn_readlane(j0 + bk * kOneThreads + tid, wl);
        if (lane == 0) s_tk[wave * (kTopK + 1) + r] = ((u64)wm << 32) | (uint32_t)wi;
        if (r < kTopK && lane == wl) {   // the winner's next largest
          taken |= 1u << bk;
          bv = 0u;   // (every key of a number is above 0)
#pragma unroll
          for (int k = 0; k < kKPer; ++k) {
            if (!((taken >> k) & 1u) && kk[k] > bv) {
              bv = kk[k];
              bk = k;
            }
          }
        }
      }
      if (lane == 0) s_sw[wave] = swd;
      __syncthreads();
      if (wave == 0) {
        // this chunk's words 1..: its approximate mass relative to its
        // maximum, the (kTopK + 1)-th key, the kTopK largest entries
        const double sg = dbl_readlane(dpp_dincl(lane < kOneWaves ? s_sw[lane] : 0.0), kWave - 1);
        constexpr int kCand = kOneWaves * (kTopK + 1);
        static_assert(kCand <= 2 * kWave, "two wave candidates a lane");
        u64 c0 = lane < kCand ? s_tk[lane] : 0ull;
        u64 c1 = lane + kWave < kCand ? s_tk[lane + kWave] : 0ull;
        uint32_t pl = lane == 1 ? __float_as_uint((float)sg) : 0u;
#pragma unroll 1
        for (int r = 0; r <= kTopK; ++r) {
          const bool hi = (uint32_t)(c1 >> 32) > (uint32_t)(c0 >> 32);
          const uint32_t cv = (uint32_t)((hi ? c1 : c0) >> 32);
          const uint32_t wm = dpp_umax(cv);
          const int wl = __ffsll((long long)__ballot(cv == wm)) - 1;
          const uint32_t wi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(hi ? c1 : c0), wl);
          if (lane == wl) {
            if (hi) c1 = 0ull;
            else c0 = 0ull;
          }
          if (r < kTopK) {
            if (lane == 3 + 2 * r) pl = wm;
            if (lane == 4 + 2 * r) pl = wi;
          } else if (lane == 2) {
            pl = wm;
          }
        }
        if (lane >= 1 && lane < kXW) st_ag(xg + (size_t)g * kXW + lane, ((u64)tag << 32) | pl);
      }
    }
    __syncthreads();
  }
  const uint32_t tag = (uint32_t)s_gen;
  const float zmax = s_zmax;

  // (2) e of every entry (kept in LDS), the row's exact mass and, with
  // top_p < 1, the chunk's exact mass per bin of x (kept for step 3) and the
  // row's approximate histogram.  With top_p < 1 and room for the row's
  // exchange words (in sh, or past the chunk when they do not fit there),
  // wave 0 takes no exponentials: it loads those words and judges them (2a)
  // meanwhile, and the other waves stop early when the cut is settled.
  if (nucleus)
    for (int i = tid; i < 3 * kXBins; i += kOneThreads) hx[i] = 0ull;
  uint32_t *const xw =
      !nucleus ? nullptr
      : G * kXW <= kBins * 3 * 2 ? reinterpret_cast<uint32_t *>(sh)
      : ((one_lds_bytes(C) + 15) & ~15) + G * kXW * 4 <= one_dyn_bytes(C)
          ? reinterpret_cast<uint32_t *>(dyn + ((one_lds_bytes(C) + 15) & ~15))
          : nullptr;
  const bool solo = xw != nullptr;
  volatile int *const fast_flag = &s_fast;
  if (tid == 0) s_next = 0;
  __syncthreads();
  Fx tot = fx_zero();
  // the exponentials: with wave 0 judging, the waves take kWave entries at a
  // time from a shared count (wave 0 joins when the row is not settled) and
  // stop once it is; else thread t takes entries t, t + kOneThreads, ...
  auto e_pass = [&](int i) {
    const double x = ((double)zc[i] - (double)zmax) / T;
    const double e = x < -70.5 ? 0.0 : exp(x);     // as e_or_zero
    ec[i] = e;
    const Fx f = to_fx(e);
    uint16_t b = 0xFFFF;
    if (fx_nonzero(f)) {
      fx_add(tot, f);
      b = (uint16_t)xbin(x);
      if (nucleus) {
        u64 *h = hx + 3 * b;
        if (f.lo & 0xFFFFFFFFull) atomicAdd(h, f.lo & 0xFFFFFFFFull);
        if (f.lo >> 32) atomicAdd(h + 1, f.lo >> 32);
        if (f.hi) atomicAdd(h + 2, f.hi);
      }
    }
    bc[i] = b;
  };
  auto shared_pass = [&]() {
    for (;;) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_next, kWave);
      base = __builtin_amdgcn_readfirstlane(base);
      if (base >= n || *fast_flag) break;   // (a settled row leaves these sums unused)
      if (base + lane < n) e_pass(base + lane);
    }
  };
  if (solo && wave == 0) {
    // (2a) do the top entries settle the cut?  Every workgroup of the row
    // judges the same words alike; if so, workgroup 0 draws the row's token,
    // publishes it with the row's state and arrives for the whole row, and
    // the others leave.  (Wave 0 issues first on its SIMD meanwhile: its
    // chain is serial, the exponentials are not.)
    __builtin_amdgcn_s_setprio(3);
    const bool draw = g == 0, draft_row = row < p.M - 1;
    double u_last = 0.0;
    int dx = -1;
    bool dvalid = false;
    float dzx = 0.0f, dqx = 0.0f;
    if (draw) {   // (loaded first, used last)
      u_last = (double)p.u[p.M - 1];
      if (draft_row) load_draft(p, row, dx, dvalid, dzx, dqx);
    }
    constexpr int kWB = 8;   // loads in flight a lane
    for (int i0 = 0; i0 < G * kXW; i0 += kWB * kWave) {
      u64 w[kWB];
#pragma unroll
      for (int r = 0; r < kWB; ++r) {
        const int i = i0 + r * kWave + lane;
        w[r] = i < G * kXW ? ld_ag(xg + i) : 0ull;
      }
#pragma unroll
      for (int r = 0; r < kWB; ++r) {
        const int i = i0 + r * kWave + lane;
        if (i < G * kXW) {
          u64 v = w[r];
          if ((uint32_t)(v >> 32) != tag) v = wait_slot(xg + i, tag, err);
          xw[i] = (uint32_t)v;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    float zm;
    RowState rs0;
    u64 ent = 0ull;
    double ee = 0.0;
    float qe = 0.0f;
    int nn = 0;
    const bool settled =
        rej_top_settle(p, row, G, xw, s_lst, draw && draft_row, zm, rs0, ent, ee, qe, nn);
    if (lane == 0 && settled) *fast_flag = 1;   // (the other waves stop)
    if (!settled) {
      __builtin_amdgcn_s_setprio(0);
      shared_pass();
    }
    if (settled && draw) {
      bool use_res = false;
      const int pick = wave_nucleus_draw(p, rs0, row, ent, ee, qe, nn, u_last, use_res);
      u64 before = 0ull;
      if (lane == 0) {
        if (draft_row) publish_acc(p, row, rs0, dx, dvalid, dzx, dqx);
        __builtin_memcpy(s_w, &rs0, sizeof(rs0));
        s_fr = use_res ? 1 : 0;
        s_pick = pick;
        if (pick != -2) {   // (else the fp64 sequence below, by the whole workgroup)
          RowState rs = rs0;
          rs.all = 2;
          publish_state(rp, tag, rs);
          st_ag(rp + kRowPick, ((u64)tag << 32) | (uint32_t)pick);
          __builtin_amdgcn_s_waitcnt(0);   // acceptance input, state and token before the count
          before = __hip_atomic_fetch_add(cp + kCallRows, (u64)G, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (pick != -2) {
        before = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(before >> 32), 0) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)before, 0);
        // the last to arrive: step 5 here, unless row a's token needs the workgroup
        const bool last = before + (u64)G == (u64)p.M * G;
        const bool done = last && rej_pick_drawn(p, tag, s_gen, err);
        if (lane == 0) {
          s_flag = last && !done;
          s_drew = 1;
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  } else if (solo) {
    shared_pass();
  } else {
    for (int i = tid; i < n; i += kOneThreads) e_pass(i);
  }
  tot = fx_sum_one(tot, red);     // (its barriers also complete the histogram and publish 2a)
  if (s_fast) {   // (uniform)
    if (g != 0) return;
    if (!s_drew) {   // the token below the fixed-point resolution with u > 0
      const RowState rs0 = row_state_of(s_w);
      const int pick =
          draw_f64_sequential<kOneThreads>(p, rs0, row, s_fr != 0, (double)p.u[p.M - 1]);
      if (tid == 0) {
        RowState rs = rs0;
        rs.all = 2;
        publish_state(rp, tag, rs);
        st_ag(rp + kRowPick, ((u64)tag << 32) | (uint32_t)pick);
        __builtin_amdgcn_s_waitcnt(0);
        s_flag = __hip_atomic_fetch_add(cp + kCallRows, (u64)G, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) + (u64)G == (u64)p.M * G;
        s_drew = 1;
      }
      __syncthreads();
    }
  } else {
    if (tid == 0 && fx_nonzero(tot)) fx_atomic_add3(p.total + 3 * row, tot);
    if (nucleus) {
      const Fx m = fx_load3(hx + 3 * tid);
      if (fx_nonzero(m)) unsafeAtomicAdd(p.ahist + (size_t)row * kXBins + tid, fx_to_double(m));
    }
  }
  if (!s_drew) {   // (uniform: a row drawn in step 2a goes to step 5)
    // arrival; the last workgroup of the row reads the row's sums
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_flag = __hip_atomic_fetch_add(rp + kRowCnt, 1ull, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == (u64)(G - 1);
    __syncthreads();
    const bool last2 = s_flag;

    if (!nucleus) {
      // the whole row is the nucleus: the last workgroup publishes the row's
      // state (its mass) and the acceptance input
      if (last2 && tid == 0) {
        const u64 *tr = p.total + 3 * row;
        const Fx S = fx_from3(ld_ag(tr), ld_ag(tr + 1), ld_ag(tr + 2));
        const RowState rs = RowState{zmax, 0u, p.V, 1, fx_to_double(S)};
        if (row < p.M - 1) {
          int x;
          bool valid;
          float zx, qx;
          load_draft(p, row, x, valid, zx, qx);
          publish_acc(p, row, rs, x, valid, zx, qx);
        }
        __builtin_amdgcn_s_waitcnt(0);   // the acceptance input before the state
        publish_state(rp, tag, rs);
      }
    } else {
      // (2b) the range [blo, bhi] of approximate bins that holds the cut, found
      // by the last workgroup of the row and published in a tagged word.  The
      // fp64 sums carry a relative error below (C + G + 32) * 2^-53 (the
      // longest chain of additions behind any of them: within a chunk, over
      // the chunks, the prefix), and fixed point drops below V * 2^-100; E
      // bounds both with room to spare.  No bin before blo reaches the
      // threshold, bin bhi does (or bhi is the last occupied bin).
      if (last2) {
        if (tid == 0) {
          const u64 *tr = p.total + 3 * row;
          for (int w = 0; w < 3; ++w) s_w[w] = ld_ag(tr + w);
          s_blo = kXBins;
          s_bhi = kXBins;
          s_last = -1;
        }
        const double v = ld_agd(p.ahist + (size_t)row * kXBins + tid);
        const double cum = dscan_one(v, dred);    // (its barriers publish s_w)
        const double Sd = fx_to_double(fx_from3(s_w[0], s_w[1], s_w[2]));
        const double thr_d = fx_to_double(threshold(p, Sd));
        const double E = (double)(C + G + 64) * 0x1p-51 * (Sd + 1.0) + (double)p.V * 0x1p-98;
        {   // first thread of each condition, last occupied bin: one LDS atomic per wave
          const u64 b0 = __ballot(cum >= thr_d - E), b1 = __ballot(cum >= thr_d + E);
          const u64 b2 = __ballot(v > 0.0);
          if (lane == 0) {
            if (b0) atomicMin(&s_blo, wave * kWave + __ffsll((long long)b0) - 1);
            if (b1) atomicMin(&s_bhi, wave * kWave + __ffsll((long long)b1) - 1);
            if (b2) atomicMax(&s_last, wave * kWave + 63 - __clzll((long long)b2));
          }
        }
        __syncthreads();
        if (tid == 0) {
          s_blo = min(s_blo, s_last);
          s_bhi = min(s_bhi, s_last);
          st_ag(rp + kRowBins,
                ((u64)tag << 32) | ((u64)(s_blo + 1) << 16) | (u64)(s_bhi + 1));
        }
      } else if (tid == 0) {
        const u64 w = wait_slot(rp + kRowBins, tag, err);
        s_blo = (int)((w >> 16) & 0xFFFF) - 1;
        s_bhi = (int)(w & 0xFFFF) - 1;
      }
      __syncthreads();
      const int blo = s_blo, bhi = s_bhi;

      // (3) the exact mass above the range (the chunk's bins before blo, one a
      // thread), and the candidates in index order (entry k * kOneThreads + t
      // is thread t's k-th)
      // Entries above the range (in the nucleus whatever the cut) also go to
      // the workspace when there are at most kAboveCap of them, so that a
      // resolver whose nucleus is small can draw the row's token alone.
      {
        Fx ab = tid < blo ? fx_load3(hx + 3 * tid) : fx_zero();
        u64 bal[kKPer], abl[kKPer];
#pragma unroll
        for (int k = 0; k < kKPer; ++k) {
          const int i = k * kOneThreads + tid;
          const int b = i < n ? (int)bc[i] : 0xFFFF;
          bal[k] = __ballot(b >= blo && b <= bhi);
          abl[k] = __ballot(b < blo);
          if (lane == 0) {
            koff[k * kOneWaves + wave] = __popcll(bal[k]);
            koffa[k * kOneWaves + wave] = __popcll(abl[k]);
          }
        }
        ab = fx_sum_one(ab, red);     // (its barriers also publish koff and koffa)
        if (tid == 0 && fx_nonzero(ab)) fx_atomic_add3(p.above + 3 * row, ab);
        if (wave < 2) {
          int *ko = wave == 0 ? koff : koffa;
          const int c0 = ko[2 * lane], c1 = ko[2 * lane + 1];
          const int incl = dpp_incl(c0 + c1);
          const int before = incl - c0 - c1;
          ko[2 * lane] = before;
          ko[2 * lane + 1] = before + c0;
          if (lane == kWave - 1) ko[kKPer * kOneWaves] = incl;
        }
        __syncthreads();
        u64 *seg = p.cand + (size_t)(row * G + g) * C;
#pragma unroll
        for (int k = 0; k < kKPer; ++k) {
          if ((bal[k] >> lane) & 1ull) {
            const int i = k * kOneThreads + tid;
            const int pos = koff[k * kOneWaves + wave] + __popcll(bal[k] & ((1ull << lane) - 1ull));
            st_ag(seg + pos, ((u64)fkey(zc[i]) << 32) | (uint32_t)(j0 + i));
          }
        }
        const int na = koffa[kKPer * kOneWaves];
        if (na <= kAboveCap) {
          u64 *aseg = p.asec + (size_t)(row * G + g) * kAboveCap;
#pragma unroll
          for (int k = 0; k < kKPer; ++k) {
            if ((abl[k] >> lane) & 1ull) {
              const int i = k * kOneThreads + tid;
              const int pos = koffa[k * kOneWaves + wave] + __popcll(abl[k] & ((1ull << lane) - 1ull));
              st_ag(aseg + pos, ((u64)fkey(zc[i]) << 32) | (uint32_t)(j0 + i));
            }
          }
        }
        if (tid == 0) {
          st_agi(p.ccount + row * G + g, koff[kKPer * kOneWaves]);
          st_agi(p.acount + row * G + g, na <= kAboveCap ? na : -1);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        s_flag = __hip_atomic_fetch_add(rp + kRowCand, 1ull, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (u64)(G - 1);
      __syncthreads();

      chunk_lost = s_flag;
      if (s_flag) {
        // (3b) the last workgroup of the row resolves the cut.  Independent
        // loads first: segment sizes (wave 0), the row's sums (thread 64),
        // the draft (thread 128).
        if (wave == 0) {
          // candidates, and entries above the range (-1: not handed over), a
          // workgroup at a time
          int c[4], ca[4], loc = 0, loca = 0;
          bool over = false;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = 4 * lane + r;
            c[r] = q < G ? ld_agi(p.ccount + row * G + q) : 0;
            ca[r] = q < G ? ld_agi(p.acount + row * G + q) : 0;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            loc += c[r];
            over = over || ca[r] < 0;
            loca += max(ca[r], 0);
          }
          int incl = dpp_incl(loc), incla = dpp_incl(loca);
          int o = incl - loc, oa = incla - loca;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            segoff[4 * lane + r] = o;
            aoff[4 * lane + r] = oa;
            o += c[r];
            oa += max(ca[r], 0);
          }
          const bool any_over = __ballot(over) != 0ull;
          if (lane == kWave - 1) {
            s_nc = incl;
            s_an = any_over ? -1 : incla;
          }
        } else if (tid == 64) {
          const u64 *abr = p.above + 3 * row, *tr = p.total + 3 * row;
          for (int w = 0; w < 3; ++w) {
            s_w[w] = ld_ag(abr + w);
            s_w[3 + w] = ld_ag(tr + w);
          }
        } else if (tid == 128 && row < p.M - 1) {
          int x;
          bool valid;
          float zx, qx;
          load_draft(p, row, x, valid, zx, qx);
          s_x = valid ? x : -1;
          s_zx = zx;
          s_qx = qx;
        }
        __syncthreads();
        const int nc = s_nc;
        const Fx A = fx_from3(s_w[0], s_w[1], s_w[2]);
        const double Sd = fx_to_double(fx_from3(s_w[3], s_w[4], s_w[5]));
        const Fx thr = threshold(p, Sd);
        const double thr_d = fx_to_double(thr);
        auto seg_of = [&](int c) {   // the last segment starting at or before c
          int lo = 0, hi = G - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (segoff[mid] <= c) lo = mid; else hi = mid - 1;
          }
          return lo;
        };
        auto cand_load = [&](int c) {
          const int q = seg_of(c);
          return ld_ag(p.cand + (size_t)(row * G + q) * C + (c - segoff[q]));
        };
        auto e_of_key = [&](u64 v) {   // e of a candidate, as step (2) computed it
          return e_of(key_to_float((uint32_t)(v >> 32)), zmax, T);
        };
        // the candidates into LDS, over this workgroup's chunk (reloaded from
        // the logits if this row draws); any beyond the room stay in the
        // workspace and are loaded again where needed
        const int room = one_cand_room(C), nl = min(nc, room);
        u64 *lk = reinterpret_cast<u64 *>(dyn);
        double *le = reinterpret_cast<double *>(dyn + (size_t)room * 8);
        for (int base = 0; base < nl; base += kResPer * kOneThreads) {
          int sq[kResPer];
          u64 v[kResPer];
#pragma unroll
          for (int k = 0; k < kResPer; ++k) {
            const int c = base + k * kOneThreads + tid;
            sq[k] = c < nl ? seg_of(c) : 0;
          }
#pragma unroll
          for (int k = 0; k < kResPer; ++k) {
            const int c = base + k * kOneThreads + tid;
            v[k] = c < nl ? ld_ag(p.cand + (size_t)(row * G + sq[k]) * C + (c - segoff[sq[k]]))
                          : 0ull;
          }
#pragma unroll
          for (int k = 0; k < kResPer; ++k) {
            const int c = base + k * kOneThreads + tid;
            if (c < nl) {
              lk[c] = v[k];
              le[c] = e_of_key(v[k]);
            }
          }
        }
        __syncthreads();
        // What a small nucleus would draw from, fetched while the cut is
        // resolved (none of it depends on the cut): with every workgroup's
        // entries above the range handed over and room for them and all the
        // candidates in one workgroup (pre), the entries above the range and,
        // for a draft row, the draft's q at every candidate; held in registers
        // until the draw (the q at the entries above follows in step 3e)
        const bool pre = s_an >= 0 && s_an + nc <= kOneThreads;
        const bool draft_row = row < p.M - 1;
        u64 pv = 0ull;
        float pqc = 0.0f;
        if (pre) {
          if (tid < s_an) {
            int lo = 0, hi = G - 1;   // the last workgroup whose entries start at or before tid
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (aoff[mid] <= tid) lo = mid;
              else hi = mid - 1;
            }
            pv = ld_ag(p.asec + (size_t)(row * G + lo) * kAboveCap + (tid - aoff[lo]));
          }
          if (draft_row && tid < nc) pqc = p.q[(int64_t)row * p.ldq + (int)(uint32_t)lk[tid]];
        }
        auto each = [&](auto &&f) {   // every candidate once
          for (int c = tid; c < nl; c += kOneThreads) f(lk[c], le[c]);
          for (int c = room + tid; c < nc; c += kOneThreads) {
            const u64 v = cand_load(c);
            f(v, e_of_key(v));
          }
        };
        // (3c) one exact pass over fine bins of x: fb(z) = (t - blo) * 256 /
        // (bhi - blo + 1) with t = -x * kXScale (x as step (2) computes it) is a
        // monotone function of z like the bins themselves, so the selection
        // over fine bins is exact, and it spreads the candidates evenly (few
        // LDS atomics collide).  Digit 255 - fb puts larger logits in higher
        // bins, as select_bin_wave expects.
        const double S2 = 256.0 / (double)(bhi - blo + 1);
        auto fbin = [&](u64 v) {
          const double x = ((double)key_to_float((uint32_t)(v >> 32)) - (double)zmax) / T;
          const int b = (int)((-x * kXScale - (double)blo) * S2);
          return 255 - (b < 0 ? 0 : (b > 255 ? 255 : b));
        };
        // (few candidates skip it: they are all sorted directly)
        const bool few = nc <= kWave;
        if (!few) {
          for (int i = tid; i < kBins * 3; i += kOneThreads) sh[i] = 0ull;
          __syncthreads();
          each([&](u64 v, double e) { hist_add(sh, fbin(v), to_fx(e)); });
          __syncthreads();
          if (wave == 0) {
            Fx a2 = A;
            int bin = select_bin_wave(sh, thr, a2);
            if (bin < 0) bin = 0;
            if (lane == 0) {
              s_prefix = (uint32_t)bin;
              s_abv_lo = a2.lo;
              s_abv_hi = a2.hi;
              s_nk = sh[3 * bin + 2];
              s_nc = 0;
            }
          }
          __syncthreads();
        }
        const int fsel = few ? 0 : (int)s_prefix, n2 = few ? nc : (int)s_nk;
        Fx above = few ? A : Fx{s_abv_lo, s_abv_hi};
        uint32_t kappa = 0u;
        u64 nk = 0ull;
        int cut_pos = -1;   // where the cut group starts among the sorted entries
        // the fine bin's entries, gathered and sorted by (key descending, index
        // ascending) in the LDS of the step (2) bin masses, when they fit
        u64 *gk = hx, *sk = gk + kSortMax;   // (hx is free once step 3 has read it)
        double *ge = reinterpret_cast<double *>(hx + 2 * kSortMax), *se2 = ge + kSortMax;
        const bool small = n2 <= kSortMax;
        // one wave sorts up to kWave entries (from the candidates themselves
        // when they are few, else from the gathered fine bin) and finds the cut
        // group in them with wave-level scans
        auto wave_cut = [&](const u64 *srck, const double *srce) {
          if (wave == 0) {
            auto skey = [](u64 v) {
              return (v & 0xFFFFFFFF00000000ull) | (0xFFFFFFFFull - (v & 0xFFFFFFFFull));
            };
            const bool valid = lane < n2;
            const u64 v0 = valid ? srck[lane] : 0ull;
            const double e0 = valid ? srce[lane] : 0.0;
            const u64 mine = skey(v0);
            int rank = 0;
            for (int j = 0; j < n2; ++j) rank += skey(srck[j]) > mine;
            if (valid) {
              sk[rank] = v0;
              se2[rank] = e0;
            }
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            const u64 v = valid ? sk[lane] : 0ull;
            const Fx f = valid ? to_fx(se2[lane]) : fx_zero();
            Fx incl = dpp_fx_incl(f);
            const Fx excl = fx_sum(above, fx_sub(incl, f));
            const uint32_t key = (uint32_t)(v >> 32);
            const bool gend = valid && (lane == n2 - 1 || (uint32_t)(sk[lane + 1] >> 32) != key);
            const u64 hit = __ballot(gend && fx_ge(fx_sum(excl, f), thr));
            const int gl = hit ? __ffsll((long long)hit) - 1 : n2 - 1;
            const uint32_t kap = (uint32_t)__builtin_amdgcn_readlane((int)key, gl);
            const u64 first = __ballot(valid && key == kap);
            const int gs = __ffsll((long long)first) - 1;
            const Fx ab = fx_readlane(excl, gs);
            if (lane == 0) {
              s_prefix = kap;
              s_abv_lo = ab.lo;
              s_abv_hi = ab.hi;
              s_nk = (u64)(gl - gs + 1);
              s_cut = gs;
            }
          }
          __syncthreads();
          kappa = s_prefix;
          above = Fx{s_abv_lo, s_abv_hi};
          nk = s_nk;
          cut_pos = s_cut;
        };
        if (nc > 0 && few) {
          wave_cut(lk, le);
        } else if (nc > 0 && small) {
          each([&](u64 v, double e) {
            if (fbin(v) == fsel) {
              const int pos = atomicAdd(&s_nc, 1);
              gk[pos] = v;
              ge[pos] = e;
            }
          });
          __syncthreads();
          if (n2 <= kWave) {
            wave_cut(gk, ge);
          } else {
          // rank = entries before this one in the order; the sort key
          // (key << 32 | ~index) is distinct and descends in that order
          auto skey = [](u64 v) {
            return (v & 0xFFFFFFFF00000000ull) | (0xFFFFFFFFull - (v & 0xFFFFFFFFull));
          };
          if (tid < n2) {
            const u64 mine = skey(gk[tid]);
            int rank = 0;
            for (int j = 0; j < n2; ++j) rank += skey(gk[j]) > mine;
            sk[rank] = gk[tid];
            se2[rank] = ge[tid];
          }
          __syncthreads();
          // exclusive prefix in the order; the cut is the first key whose group
          // reaches the threshold (else the last group)
          const u64 v = tid < n2 ? sk[tid] : 0ull;
          const Fx f = tid < n2 ? to_fx(se2[tid]) : fx_zero();
          Fx tot_unused;
          const Fx excl = fx_sum(above, fx_excl_one(f, red, tot_unused));
          const uint32_t key = (uint32_t)(v >> 32);
          const bool gend = tid < n2 && (tid == n2 - 1 || (uint32_t)(sk[tid + 1] >> 32) != key);
          if (tid == 0) {
            s_blk = 0x7FFFFFFF;
            s_lastnz = 0x7FFFFFFF;
          }
          __syncthreads();
          {
            const u64 hit = __ballot(gend && fx_ge(fx_sum(excl, f), thr));
            if (lane == 0 && hit) atomicMin(&s_blk, wave * kWave + __ffsll((long long)hit) - 1);
          }
          __syncthreads();
          const int gl = s_blk != 0x7FFFFFFF ? s_blk : n2 - 1;   // the cut group's last entry
          kappa = (uint32_t)(sk[gl] >> 32);
          {
            const u64 first = __ballot(tid < n2 && key == kappa);
            if (lane == 0 && first)
              atomicMin(&s_lastnz, wave * kWave + __ffsll((long long)first) - 1);
          }
          __syncthreads();
          const int gs = s_lastnz;   // the cut group's first entry
          if (tid == gs) {
            s_abv_lo = excl.lo;
            s_abv_hi = excl.hi;
          }
          __syncthreads();
          above = Fx{s_abv_lo, s_abv_hi};
          nk = (u64)(gl - gs + 1);
          cut_pos = gs;
          }
        } else if (nc > 0) {
          // a large fine bin (many equal or nearly equal logits): radix passes
          // over the keys of its entries
          uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
          each([&](u64 v, double) {
            if (fbin(v) != fsel) return;
            const uint32_t k = (uint32_t)(v >> 32);
            kmn = min(kmn, k);
            kmx = max(kmx, k);
          });
          for (int s2 = kWave / 2; s2 > 0; s2 >>= 1) {
            kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, s2));
            kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, s2));
          }
          if (tid == 0) {
            s_kmin = 0xFFFFFFFFu;
            s_kmax = 0u;
          }
          __syncthreads();
          if (lane == 0) {
            atomicMin(&s_kmin, kmn);
            atomicMax(&s_kmax, kmx);
          }
          __syncthreads();
          kmn = s_kmin;
          kmx = s_kmax;
          int lo_bit = kmn == kmx ? 0 : 32 - __clz((int)(kmn ^ kmx));
          uint32_t prefix = lo_bit == 32 ? 0u : (kmn >> lo_bit);
          nk = (u64)n2;
          while (lo_bit > 0) {
            const int db = min(8, lo_bit), shift = lo_bit - db;
            for (int i = tid; i < kBins * 3; i += kOneThreads) sh[i] = 0ull;
            __syncthreads();
            each([&](u64 v, double e) {
              const uint32_t k = (uint32_t)(v >> 32);
              if (fbin(v) != fsel || (lo_bit < 32 && (k >> lo_bit) != prefix)) return;
              hist_add(sh, (int)((k >> shift) & ((1u << db) - 1u)), to_fx(e));
            });
            __syncthreads();
            if (wave == 0) {
              Fx a2 = above;
              int bin = select_bin_wave(sh, thr, a2);
              if (bin < 0) bin = 0;
              if (lane == 0) {
                s_prefix = (prefix << db) | (uint32_t)bin;
                s_abv_lo = a2.lo;
                s_abv_hi = a2.hi;
                s_nk = sh[3 * bin + 2];
              }
            }
            __syncthreads();
            prefix = s_prefix;
            above = Fx{s_abv_lo, s_abv_hi};
            nk = s_nk;
            lo_bit = shift;
            __syncthreads();
          }
          kappa = prefix;
        }
        const double ek = e_of(key_to_float(kappa), zmax, T);
        const double above_d = fx_to_double(above);
        const double tt = ceil((thr_d - above_d) / ek);
        const u64 t = (tt < 1.0) ? 1ull : (tt >= (double)nk ? nk : (u64)tt);
        int cutoff = p.V;
        if (t < nk && cut_pos >= 0) {
          // the group is sorted by index: its t-th entry is the last inside
          cutoff = (int)(uint32_t)sk[cut_pos + (int)t - 1];
        } else if (t < nk) {
          // ties at the cut: the first t in index order (the candidates' order)
          // are inside
          if (tid == 0) s_cut = p.V;
          int seen = 0;
          auto round = [&](bool valid, u64 v) {
            const bool f = valid && (uint32_t)(v >> 32) == kappa;
            int pre;
            const int tot_r = count_one(f, pre, wcnt);
            if (f && (u64)(seen + pre + 1) == t) s_cut = (int)(uint32_t)v;
            seen += tot_r;
            return (u64)seen >= t;
          };
          bool done = false;
          for (int base = 0; !done && base < nc; base += kOneThreads) {
            const int c = base + tid;
            done = round(c < nc, c < nl ? lk[c] : (c < nc ? cand_load(c) : 0ull));
          }
          __syncthreads();
          cutoff = s_cut;
        }
        // (3e) a small nucleus (pre: at most kOneThreads entries in the
        // nucleus, all of them at hand): this workgroup draws the row's token
        // itself (the draw row a would make, as the picker below does it) and
        // the row's other workgroups leave as soon as they see the state
        const RowState rs0 = RowState{zmax, kappa, cutoff, 0, above_d + (double)t * ek};
        const bool tiny = pre;
        float pqa = 0.0f;
        if (tiny && draft_row && tid < s_an) pqa = p.q[(int64_t)row * p.ldq + (int)(uint32_t)pv];
        if (tid == 0) {
          RowState rs = rs0;
          if (tiny) rs.all = 2;
          if (row < p.M - 1) publish_acc(p, row, rs0, s_x, s_x >= 0, s_zx, s_qx);
          __builtin_amdgcn_s_waitcnt(0);   // the acceptance input before the state
          publish_state(rp, tag, rs);
        }
        if (tiny) {
          // the nucleus in index order: entries keyed (~index << 32 | slot),
          // slot i < kOneThreads the i-th entry above the range, kOneThreads + c
          // candidate c
          u64 *nuc = hx;   // (free: the fine-bin sort is done)
          u64 *abv = reinterpret_cast<u64 *>(dyn + 16384);   // (the candidates use
          float *qa = reinterpret_cast<float *>(dyn + 8192);  // at most 8 KiB of lk)
          float *qc = qa + kOneThreads;
          const int na = s_an;
          if (tid < na) {
            abv[tid] = pv;
            qa[tid] = pqa;
            nuc[tid] = ((u64)(0xFFFFFFFFu - (uint32_t)pv) << 32) | (uint32_t)tid;
          }
          if (tid < nc) qc[tid] = pqc;
          if (tid == 0) s_nc2 = na;
          __syncthreads();
          {   // the candidates inside the cut (nc <= kOneThreads - na: one round)
            const int c = tid;
            const u64 v = c < nc ? lk[c] : 0ull;
            const bool f =
                c < nc && in_nucleus(rs0, key_to_float((uint32_t)(v >> 32)), (int)(uint32_t)v);
            const int at = wave_append(f, &s_nc2);
            if (f && at < kOneThreads)
              nuc[at] = ((u64)(0xFFFFFFFFu - (uint32_t)v) << 32) | (uint32_t)(kOneThreads + c);
          }
          __syncthreads();
          const int N = min(s_nc2, kOneThreads);
          const u64 *srt = sort_desc(nuc, hx + 2 * kOneThreads, N);
          const int pick = rej_nucleus_draw(
              p, rs0, row, srt, N,
              [&](int sl, float &zt, float &qt) {
                const bool ab = sl < kOneThreads;
                const u64 e0 = ab ? abv[sl] : lk[sl - kOneThreads];
                zt = key_to_float((uint32_t)(e0 >> 32));
                qt = draft_row ? (ab ? qa[sl] : qc[sl - kOneThreads]) : 0.0f;
              },
              red);
          // the row's token, then the arrivals of all of its workgroups at once
          if (tid == 0) {
            st_ag(rp + kRowPick, ((u64)tag << 32) | (uint32_t)pick);
            __builtin_amdgcn_s_waitcnt(0);
            s_flag = __hip_atomic_fetch_add(cp + kCallRows, (u64)G, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + (u64)G == (u64)p.M * G;
            s_drew = 1;
          }
          __syncthreads();
        }
      }
    }
  }

  // (4) the draw weights of this row, before the accepted run is known:
  // the residual max(0, p' - q) for a draft row (drawn if its draft is the
  // first rejected), p' itself (drawn by the last row, or where a residual
  // is all zero).  Wave w sums a contiguous range of the chunk (entries w*L
  // .. w*L+L-1).  Then the arrivals are counted per row and over the rows;
  // the very last workgroup derives the accepted run a and picks the token
  // from row a's range sums.
  {
    const bool residual = row < p.M - 1;
    const int L = one_range(C), rb = wave * L;
    if (!s_drew) {   // (uniform; a resolver that drew its row has arrived already)
    float qv[kKPer], zv[kKPer];   // (loaded before the wait, which they do not need)
#pragma unroll
    for (int r = 0; r < kKPer; ++r) {
      const int i = rb + r * kWave + lane;
      const bool ok = r * kWave + lane < L && i < n;
      qv[r] = (ok && residual) ? p.q[(int64_t)row * p.ldq + j0 + i] : 0.0f;
      zv[r] = (ok && chunk_lost) ? zr[i] : 0.0f;
    }
    if (wave == 0) {
      const RowState rs0 = wait_state(rp, tag, err);
      if (lane == 0) {
        __builtin_memcpy(s_w, &rs0, sizeof(rs0));
        s_fr = kNone;
        s_fe = kNone;
      }
    }
    __syncthreads();
    const RowState rs = row_state_of(s_w);
    if (rs.all & 2) return;   // this row's resolver drew its token: nothing to sum
    Fx sr = fx_zero(), se = fx_zero();
    int fr = kNone, fe = kNone;
#pragma unroll
    for (int r = 0; r < kKPer; ++r) {
      const int i = rb + r * kWave + lane;
      if (r * kWave + lane < L && i < n) {
        Fx wr, we;
        bool pr, pe;
        draw_weights_v(rs, T, residual, j0 + i, chunk_lost ? zv[r] : zc[i], (double)qv[r],
                       !chunk_lost, chunk_lost ? 0.0 : ec[i], wr, we, pr, pe);
        fx_add(sr, wr);
        fx_add(se, we);
        if (pr && fr == kNone) fr = j0 + i;
        if (pe && fe == kNone) fe = j0 + i;
      }
    }
    sr = fx_wave_sum(sr);
    se = fx_wave_sum(se);
    fr = wave_min(fr);
    fe = wave_min(fe);
    if (lane == 0) {
      u64 *o = p.wsum + (size_t)blockIdx.x * kOneWaves + wave;
      st_ag(o, sr.lo);
      st_ag(o + kRanges, sr.hi);
      st_ag(o + 2 * kRanges, se.lo);
      st_ag(o + 3 * kRanges, se.hi);
      red[wave] = sr;
      wred[wave] = se;
      if (fr != kNone) atomicMin(&s_fr, fr);
      if (fe != kNone) atomicMin(&s_fe, fe);
    }
    __syncthreads();
    if (wave == 0) {   // the workgroup's sums (lanes 0..15 hold the waves')
      Fx br = lane < kOneWaves ? red[lane] : fx_zero();
      Fx be = lane < kOneWaves ? wred[lane] : fx_zero();
      br = fx_wave_sum(br);
      be = fx_wave_sum(be);
      if (lane == 0) {
        u64 *o = p.blk + kBlkWords * blockIdx.x;
        st_ag(o, br.lo);
        st_ag(o + 1, br.hi);
        st_ag(o + 2, be.lo);
        st_ag(o + 3, be.hi);
        st_ag(o + 4, (u64)s_fr);
        st_ag(o + 5, (u64)s_fe);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)   // one count over the call's workgroups
      s_flag = __hip_atomic_fetch_add(cp + kCallRows, 1ull, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == (u64)(p.M * G - 1);
    __syncthreads();
    }
    if (s_flag) {
      // (5) the last workgroup of the call: the accepted run, then the draw
      // from row a (every row's state, acceptance input and sums are in).
      // Wave 0 finds the workgroup and the range of the crossing from the
      // workgroup and range sums (wave-level scans, no block barriers); then
      // the whole workgroup scans that range.
      if (wave == 0) {
        bool reject = false;
        if (lane < p.M - 1) {
          const u64 *o = reinterpret_cast<const u64 *>(p.acc + lane);
          const double px = __longlong_as_double((long long)ld_ag(o));
          const double qx = __longlong_as_double((long long)ld_ag(o + 1));
          reject = !((double)p.u[lane] * qx < px);
        }
        const u64 rej = __ballot(reject);
        const int a = rej ? __ffsll((long long)rej) - 1 : p.M - 1;
        const bool residual = a < p.M - 1;
        bool drawn;
        {   // row a's state (its words are all in: every row arrived after them)
          const RowState rsa = wait_state(p.hdr + (size_t)a * kPageWords, tag, err);
          if (lane == 0) __builtin_memcpy(s_w + 3, &rsa, sizeof(rsa));
          drawn = (rsa.all & 2) != 0;
        }
        if (drawn) {   // row a's resolver drew its token (it stored it before arriving)
          const u64 wp = wait_slot(p.hdr + (size_t)a * kPageWords + kRowPick, tag, err);
          if (lane == 0) {
            s_a = a;
            s_flag = 1;
            s_pick = (int)(uint32_t)wp;
          }
        } else {
        Fx br[kMaxOneBlocks / kWave], be[kMaxOneBlocks / kWave];
        int bfr = kNone, bfe = kNone;
#pragma unroll
        for (int c = 0; c < kMaxOneBlocks / kWave; ++c) {
          const int q = c * kWave + lane;
          br[c] = be[c] = fx_zero();
          if (c * kWave >= G) continue;
          if (q < G) {
            const u64 *o = p.blk + kBlkWords * (a * G + q);
            br[c] = Fx{ld_ag(o), ld_ag(o + 1)};
            be[c] = Fx{ld_ag(o + 2), ld_ag(o + 3)};
            bfr = min(bfr, (int)ld_ag(o + 4));
            bfe = min(bfe, (int)ld_ag(o + 5));
          }
        }
        Fx lr = fx_zero(), le = fx_zero();
#pragma unroll
        for (int c = 0; c < kMaxOneBlocks / kWave; ++c) {
          fx_add(lr, br[c]);
          fx_add(le, be[c]);
        }
        const Fx tres = fx_wave_sum(lr), te = fx_wave_sum(le);
        bfr = wave_min(bfr);
        bfe = wave_min(bfe);
        const bool use_res = residual && bfr != kNone;
        const double u = (double)p.u[p.M - 1];
        const Fx target = to_fx(u * fx_to_double(use_res ? tres : te));
        int mode = 0, pick = -1, blk = -1, rng = -1;   // mode 0: range rng holds the pick
        Fx before = fx_zero();
        if (!fx_nonzero(target)) {
          // below the fixed-point resolution (see rej_draw_pick): u = 0 takes
          // the first positive weight, any other target the fp64 sequence
          if (u == 0.0) {
            const int f = use_res ? bfr : bfe;
            mode = 1;
            pick = f != kNone ? f : p.V - 1;
          } else {
            mode = 2;
          }
        } else {
          // the workgroup of the crossing (workgroups in index order: c-major)
          Fx cum = fx_zero();
          bool exact = false;
          int lastnz = -1;
#pragma unroll
          for (int c = 0; c < kMaxOneBlocks / kWave; ++c) {
            if (c * kWave >= G) break;   // (uniform)
            const int q = c * kWave + lane;
            const Fx w = use_res ? br[c] : be[c];
            Fx incl = dpp_fx_incl(w);
            const Fx bef = fx_sum(cum, fx_sub(incl, w));
            const u64 hit = __ballot(!exact && q < G && !fx_gt(bef, target) &&
                                     fx_gt(fx_sum(bef, w), target));
            if (hit) {
              const int l = __ffsll((long long)hit) - 1;
              exact = true;
              blk = c * kWave + l;
              before = fx_readlane(bef, l);
            }
            const u64 nz = __ballot(q < G && fx_nonzero(w));
            if (nz) lastnz = c * kWave + 63 - __clzll((long long)nz);
            fx_add(cum, fx_readlane(incl, kWave - 1));
          }
          if (!exact) {
            blk = lastnz;
            before = fx_zero();
          }
          if (blk >= 0) {
            // the range of the crossing inside workgroup blk (lane w < 16 holds
            // range w), or its last positive range
            const size_t rq = ((size_t)a * G + blk) * kOneWaves + lane;
            Fx w = fx_zero();
            if (lane < kOneWaves) {
              const u64 *o = p.wsum + rq + (use_res ? 0 : 2 * kRanges);
              w = Fx{ld_ag(o), ld_ag(o + kRanges)};
            }
            Fx incl = dpp_fx_incl(w);
            const Fx bef = fx_sum(before, fx_sub(incl, w));
            if (exact) {
              const u64 hit = __ballot(lane < kOneWaves && !fx_gt(bef, target) &&
                                       fx_gt(fx_sum(bef, w), target));
              const int l = hit ? __ffsll((long long)hit) - 1 : 0;
              rng = l;
              before = fx_readlane(bef, l);
            } else {
              const u64 nz = __ballot(lane < kOneWaves && fx_nonzero(w));
              rng = nz ? 63 - __clzll((long long)nz) : 0;
            }
            mode = exact ? 0 : 3;
          } else {
            mode = 1;
            pick = p.V - 1;   // no positive weight at all: the last id
          }
        }
        if (lane == 0) {
          s_a = a;
          s_flag = mode;
          s_pick = pick;
          s_blk = blk;
          s_lastnz = rng;
          s_before = before;
          s_fr = use_res ? 1 : 0;
          s_abv_lo = target.lo;
          s_abv_hi = target.hi;
        }
        }
      }
      __syncthreads();
      const int a = s_a, mode = s_flag;
      const bool residual = a < p.M - 1, use_res = s_fr != 0;
      const RowState rs = row_state_of(s_w + 3);
      int pick = s_pick;
      if (mode == 2) {
        pick = draw_f64_sequential<kOneThreads>(p, rs, a, use_res, (double)p.u[p.M - 1]);
      } else if (mode == 0 || mode == 3) {
        // the range's entries, thread t holding entry t: exact, the entry whose
        // weight crosses the target; else the last positive one
        const Fx target = Fx{s_abv_lo, s_abv_hi};
        const int gb = s_blk, s0 = s_lastnz * L;
        const int len = max(0, min(L, min(C, p.V - gb * C) - s0));
        const int jt = gb * C + s0 + tid;
        Fx w = fx_zero();
        if (tid < len) {
          const float zt = p.z[(int64_t)a * p.ldl + jt];
          const float qt = residual ? p.q[(int64_t)a * p.ldq + jt] : 0.0f;
          Fx wr, we;
          bool pr, pe;
          draw_weights_v(rs, T, residual, jt, zt, (double)qt, false, 0.0, wr, we, pr, pe);
          w = use_res ? wr : we;
        }
        if (tid == 0) s_pick = -1;
        Fx tot2;
        Fx bef = fx_excl_one(w, red, tot2);   // (its barriers also publish s_pick)
        if (mode == 0) bef = fx_sum(s_before, bef);
        int lastw = -1;
        if (tid < len) {
          if (mode == 0) {
            if (!fx_gt(bef, target) && fx_gt(fx_sum(bef, w), target)) s_pick = jt;   // one entry
          } else if (fx_nonzero(w)) {
            lastw = jt;
          }
        }
        lastw = wave_max(lastw);
        if (lane == 0 && lastw >= 0) atomicMax(&s_pick, lastw);
        __syncthreads();
        pick = s_pick < 0 ? p.V - 1 : s_pick;
      }
      if (tid < p.M) p.tokens[tid] = (tid < a) ? p.drafts[tid] : (tid == a ? pick : -1);
      if (tid == 0) {
        p.counts[0] = a;
        p.counts[1] = a + 1;
        *p.rollback = p.base_len + a + 1;
      }
      // (6) every other workgroup has left: the counters are reset and the
      // generation advances for the next call
      if (tid < p.M) {
        u64 *r = p.hdr + (size_t)tid * kPageWords;
        st_ag(r + kRowCnt, 0ull);
        st_ag(r + kRowCand, 0ull);
        st_ag(r + kRowDraw, 0ull);
      }
      if (tid == 0) {
        st_ag(cp + kCallRows, 0ull);
        st_ag(cp + kCallGen, s_gen);
      }
    }
  }

}

// ---- sampled acceptance: the full sampler pipeline, sparse top-k path -------
//
// Ollama mtp.go commit log, the MLX sampler rework: penalties -> top-k ->
// temperature/softmax -> top-p -> min-p -> normalize -> categorical, the
// common top-k path keeping sparse per-row ids and probabilities that sampled
// MTP reuses for acceptance, bonus and residual draws.  Rows are the B*M
// (sequence, position) pairs.  Kernels: samp_prep (penalised copy of each
// row, clears the count histograms), four samp_count radix passes (counts of
// the order-preserving keys: the top-k cut is the K-th largest key, ties by
// index), samp_compact_count / samp_compact_write (the K kept entries of each
// row in index order, placed by per-block counts, no atomics), samp_row (one
// workgroup per row: sort, softmax in fp64, top-p and min-p cuts on exact
// fixed-point prefix sums, the row's acceptance inputs) and samp_draw (one
// workgroup per sequence: the accepted run and the residual or bonus draw).

constexpr int kMaxTopK = 1024;
constexpr int kRowThreads = 1024;
constexpr int kMaxPenaltyWindow = 4096;

struct SampArgs {
  const float *z;
  int64_t ldl;
  float *zp;                 // penalised rows [rows][V], or nullptr (no penalties)
  const int32_t *htok;       // history [B][ldh]
  const int32_t *hlen;       // [B]
  int64_t ldh;
  const int32_t *drafts;     // [B][M-1]
  const float *q;            // dense [B*(M-1)][ldq], or nullptr
  int64_t ldq;
  const int32_t *qi;         // sparse [B*(M-1)][Kq]
  const float *qp;
  int Kq;
  const float *u;            // [B][M]
  const int64_t *base_len;   // [B] or nullptr
  double T, top_p, min_p;
  float rp, pp, fq;          // repeat, presence, frequency penalties
  int last_n;
  int B, M, V, K, nb, chunk;
  int32_t *tokens;
  int32_t *counts;
  int64_t *rollback;
  int32_t *out_ids;          // optional [rows][K]
  float *out_probs;
  uint32_t *hcnt;            // [4][rows][kBins]
  SelState *sel;             // [4][rows]: state after `pass` selections; [0]: the cut
  uint32_t *bcnt;            // [rows][nb][2]: entries above the cut key, ties at it
  int32_t *lid;              // [rows][K] kept entries in index order
  float *lz;
  int32_t *sid;              // [rows][K] the row's support in index order
  double *sp;                //   p'
  double *se;                //   e
  int32_t *nkept;            // [rows]
  AccIn *acc;                // [rows]
  // samp_one
  uint32_t *rowcnt;          // [rows] arrivals (workspace head, zero between calls)
  uint32_t *seqcnt;          // [B] rows done
  u64 *info;                 // [rows][G] (smallest candidate key << 32) | candidate count
  u64 *cand;                 // [rows][G][C] candidates (key << 32 | index), index order
  u64 *res;                  // [rows] (draft rejected << 31) | token this row would draw
  int G, C, pen, lkc;        // lkc: log2 of the candidate slots read in the first round
};

__device__ __forceinline__ const float *samp_src(const SampArgs &p, int row) {
  return p.zp ? p.zp + (int64_t)row * p.V : p.z + (int64_t)row * p.ldl;
}

__device__ __forceinline__ int64_t samp_src_ld(const SampArgs &p) { return p.zp ? p.V : p.ldl; }

// Penalised logit: fp32, every operation rounded on its own.
__device__ __forceinline__ float penalise(float x, int c, const SampArgs &p) {
  if (p.rp != 1.0f) x = x > 0.0f ? __fdiv_rn(x, p.rp) : __fmul_rn(x, p.rp);
  x = __fsub_rn(x, __fmul_rn((float)c, p.fq));
  return __fsub_rn(x, p.pp);
}

// grid (nb, rows).  Clears this call's count histograms; with penalties,
// writes the penalised copy of the row: the window (the last last_n tokens
// of history ++ drafts before the row) is scanned once per block and its
// tokens inside the block's range kept in LDS, so each entry counts its
// occurrences there.
__global__ __launch_bounds__(kBlock) void samp_prep(SampArgs p) {
  __shared__ int32_t lt[kMaxPenaltyWindow];
  __shared__ int nl;
  const int b = blockIdx.x, row = blockIdx.y, seq = row / p.M, pos = row - seq * p.M;
  const int rows = p.B * p.M;
  for (int i = b * kBlock + threadIdx.x; i < 4 * kBins; i += p.nb * kBlock)
    p.hcnt[(size_t)(i / kBins) * rows * kBins + (size_t)row * kBins + (i % kBins)] = 0u;
  if (!p.zp) return;
  const float *zr = p.z + (int64_t)row * p.ldl;
  float *out = p.zp + (int64_t)row * p.V;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float v0[kBatch];
  load_batch(zr, j0, j1, 0.0f, v0);
  if (threadIdx.x == 0) nl = 0;
  __syncthreads();
  const int Lh = p.htok ? max(0, min(p.hlen[seq], (int)p.ldh)) : 0;
  const int total = Lh + pos, w0 = max(0, total - p.last_n);
  for (int c = w0 + (int)threadIdx.x; c < total; c += kBlock) {
    const int t = c < Lh ? p.htok[(int64_t)seq * p.ldh + c]
                         : p.drafts[(int64_t)seq * (p.M - 1) + (c - Lh)];
    if (t >= j0 && t < j1) lt[atomicAdd(&nl, 1)] = t;
  }
  __syncthreads();
  const int n = nl;
  auto put = [&](const float (&v)[kBatch], int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = base + (int)threadIdx.x + i * kBlock;
      if (j < j1) {
        int c = 0;
        for (int k = 0; k < n; ++k) c += lt[k] == j ? 1 : 0;
        out[j] = c ? penalise(v[i], c, p) : v[i];
      }
    }
  };
  put(v0, j0);
  for (int base = j0 + kBatch * kBlock; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(zr, base, j1, 0.0f, v);
    put(v, base);
  }
}

// The cut state after `pass` selection steps of a row: every block of a pass
// takes the step itself from the previous pass's counts (count-weighted
// select_bin_wave: the bin where the count from the top reaches K).
__device__ void samp_select(const SampArgs &p, int pass, int row, u64 *h, uint32_t &prefix,
                            Fx &above) {
  const int rows = p.B * p.M;
  const uint32_t *g = p.hcnt + ((size_t)(pass - 1) * rows + row) * kBins;
  SelState st = SelState{0ull, 0ull, 0u, 0};
  if (pass > 1) st = p.sel[(size_t)(pass - 1) * rows + row];
  for (int d = threadIdx.x; d < kBins; d += blockDim.x) {
    const uint32_t c = g[d];
    h[3 * d] = c;
    h[3 * d + 1] = 0ull;
    h[3 * d + 2] = c;
  }
  __syncthreads();
  __shared__ uint32_t s_prefix;
  __shared__ u64 s_alo, s_ahi;
  if (threadIdx.x < kWave) {
    Fx ab = Fx{st.above_lo, st.above_hi};
    const int bin = select_bin_wave(h, Fx{(u64)p.K, 0ull}, ab);
    if (threadIdx.x == 0) {
      s_prefix = (st.prefix << 8) | (uint32_t)(bin < 0 ? 0 : bin);
      s_alo = ab.lo;
      s_ahi = ab.hi;
    }
  }
  __syncthreads();
  prefix = s_prefix;
  above = Fx{s_alo, s_ahi};
}

// Radix pass `pass` over the keys of the kept-entry candidates: counts by
// key digit of the entries matching the selected prefix.
__global__ __launch_bounds__(kBlock) void samp_count(SampArgs p, int pass) {
  __shared__ uint32_t sh[kBins];
  __shared__ u64 hbuf[kBins * 3];
  const int b = blockIdx.x, row = blockIdx.y, rows = p.B * p.M;
  const float *src = samp_src(p, row);
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float v0[kBatch];
  load_batch(src, j0, j1, 0.0f, v0);
  for (int i = threadIdx.x; i < kBins; i += kBlock) sh[i] = 0u;
  uint32_t prefix = 0;
  Fx above = fx_zero();
  if (pass > 0) {
    samp_select(p, pass, row, hbuf, prefix, above);
    if (b == 0 && threadIdx.x == 0)
      p.sel[(size_t)pass * rows + row] = SelState{above.lo, above.hi, prefix, 0};
  } else {
    __syncthreads();
  }
  const int shift = 24 - 8 * pass;
  auto take = [&](const float (&v)[kBatch], int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = base + (int)threadIdx.x + i * kBlock;
      const uint32_t key = fkey(v[i]);
      if (j < j1 && (pass == 0 || (key >> (shift + 8)) == prefix))
        atomicAdd(&sh[(key >> shift) & 0xFF], 1u);
    }
  };
  take(v0, j0);
  for (int base = j0 + kBatch * kBlock; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(src, base, j1, 0.0f, v);
    take(v, base);
  }
  __syncthreads();
  uint32_t *g = p.hcnt + ((size_t)pass * rows + row) * kBins;
  for (int d = threadIdx.x; d < kBins; d += kBlock)
    if (sh[d]) atomicAdd(g + d, sh[d]);
}

// Last selection step (every block), then the block's counts of entries
// above the cut key and of ties at it.
__global__ __launch_bounds__(kBlock) void samp_compact_count(SampArgs p) {
  __shared__ u64 hbuf[kBins * 3];
  __shared__ uint32_t s_a, s_e;
  const int b = blockIdx.x, row = blockIdx.y;
  const float *src = samp_src(p, row);
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float v0[kBatch];
  load_batch(src, j0, j1, 0.0f, v0);
  if (threadIdx.x == 0) s_a = s_e = 0u;
  uint32_t kappa;
  Fx above;
  samp_select(p, 4, row, hbuf, kappa, above);
  if (b == 0 && threadIdx.x == 0)   // the cut: key kappa, the first t ties by index are kept
    p.sel[row] = SelState{above.lo, above.hi, kappa, (int32_t)((u64)p.K - above.lo)};
  uint32_t na = 0, ne = 0;
  auto take = [&](const float (&v)[kBatch], int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = base + (int)threadIdx.x + i * kBlock;
      const uint32_t key = fkey(v[i]);
      if (j < j1) {
        na += key > kappa ? 1u : 0u;
        ne += key == kappa ? 1u : 0u;
      }
    }
  };
  take(v0, j0);
  for (int base = j0 + kBatch * kBlock; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(src, base, j1, 0.0f, v);
    take(v, base);
  }
  if (na) atomicAdd(&s_a, na);
  if (ne) atomicAdd(&s_e, ne);
  __syncthreads();
  if (threadIdx.x == 0) {
    p.bcnt[((size_t)row * p.nb + b) * 2] = s_a;
    p.bcnt[((size_t)row * p.nb + b) * 2 + 1] = s_e;
  }
}

// Exclusive count of `flag` over the threads of a kBlock block (thread
// order); the block total in `total`.
__device__ __forceinline__ uint32_t block_excl_count(bool flag, uint32_t *wtot, uint32_t &total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const u64 m = __ballot(flag);
  const uint32_t in_wave = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) wtot[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0;
  total = 0;
  for (int w = 0; w < kBlock / kWave; ++w) {
    if (w < wave) before += wtot[w];
    total += wtot[w];
  }
  return before + in_wave;
}

// The kept entries of the row, in index order: a block's place follows from
// the counts of the blocks before it (the first t ties by index are kept).
__global__ __launch_bounds__(kBlock) void samp_compact_write(SampArgs p) {
  __shared__ uint32_t s_off, s_tb;
  __shared__ bool s_none;
  __shared__ uint32_t wtot[kBlock / kWave];
  const int b = blockIdx.x, row = blockIdx.y;
  const float *src = samp_src(p, row);
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float v0[kBatch];
  load_batch(src, j0, j1, 0.0f, v0);
  const SelState cut = p.sel[row];
  const uint32_t kappa = cut.prefix, t = (uint32_t)cut.pad;
  if (threadIdx.x < kWave) {
    // ties before this block, and the kept entries before it
    uint32_t ties = 0, kept = 0;
    for (int k = threadIdx.x; k < b; k += kWave) {
      const uint32_t a = p.bcnt[((size_t)row * p.nb + k) * 2];
      const uint32_t e = p.bcnt[((size_t)row * p.nb + k) * 2 + 1];
      ties += e;
      kept += a;
    }
    for (int m = kWave / 2; m > 0; m >>= 1) {
      ties += __shfl_xor(ties, m);
      kept += __shfl_xor(kept, m);
    }
    if (threadIdx.x == 0) {
      s_tb = ties;
      s_off = kept + min(ties, t);   // ties before the block are kept in index order up to t
      // nothing to place: no entry above the cut and no tie still kept
      const uint32_t a = p.bcnt[((size_t)row * p.nb + b) * 2];
      const uint32_t e = p.bcnt[((size_t)row * p.nb + b) * 2 + 1];
      s_none = a == 0u && (e == 0u || ties >= t);
    }
  }
  __syncthreads();
  if (s_none) return;
  uint32_t tb = s_tb, off = s_off;
  int32_t *lid = p.lid + (size_t)row * p.K;
  float *lz = p.lz + (size_t)row * p.K;
  auto put = [&](const float (&v)[kBatch], int base) {
    for (int i = 0; i < kBatch; ++i) {
      const int j = base + (int)threadIdx.x + i * kBlock;
      const uint32_t key = fkey(v[i]);
      const bool tie = j < j1 && key == kappa;
      uint32_t ntie;
      const uint32_t trank = tb + block_excl_count(tie, wtot, ntie);
      const bool keep = j < j1 && (key > kappa || (tie && trank < t));
      uint32_t nkeep;
      const uint32_t at = off + block_excl_count(keep, wtot, nkeep);
      if (keep && at < (uint32_t)p.K) {   // (always: the counts place exactly K entries)
        lid[at] = j;
        lz[at] = v[i];
      }
      tb += ntie;
      off += nkeep;
    }
  };
  put(v0, j0);
  for (int base = j0 + kBatch * kBlock; base < j1; base += kBatch * kBlock) {
    float v[kBatch];
    load_batch(src, base, j1, 0.0f, v);
    put(v, base);
  }
}

// ---- per-row pipeline (one workgroup of kRowThreads per row) ----------------

constexpr int kRowWaves = kRowThreads / kWave;

// Exclusive 128-bit prefix over the threads of the workgroup (thread order).
__device__ Fx fx_row_exclusive(Fx v, Fx *wsum, Fx &total) {
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const Fx incl = dpp_fx_incl(v);
  __syncthreads();
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  Fx before = fx_zero();
  total = fx_zero();
  for (int w = 0; w < nw; ++w) {
    if (w < wave) fx_add(before, wsum[w]);
    fx_add(total, wsum[w]);
  }
  return fx_sum(before, fx_sub(incl, v));
}

// Bitonic sort of n2 (a power of two, at most the workgroup size) (key, id)
// pairs in LDS, thread i owning slot i; `before(a, b)` orders them.  Slots n .. pow2 - 1 must hold entries
// that order last.
template <typename Before>
__device__ void bitonic(float *key, int32_t *id, int n2, Before before) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      const int i = threadIdx.x, l = i ^ j;
      if (i < n2 && l > i) {
        const bool up = (i & k) == 0;
        const float ki = key[i], kl = key[l];
        const int32_t ii = id[i], il = id[l];
        const bool swap = up ? before(kl, il, ki, ii) : before(ki, ii, kl, il);
        if (swap) {
          key[i] = kl; key[l] = ki;
          id[i] = il; id[l] = ii;
        }
      }
    }
  }
  __syncthreads();
}

// q of draft row r (r = seq * (M-1) + pos) at id x; sparse lists take their
// first listing of x (staged in LDS: qid/qpr, Kq entries).
__device__ __forceinline__ double samp_q(const SampArgs &p, int r, int x, const int32_t *qid,
                                         const float *qpr) {
  if (p.q) return (double)p.q[(int64_t)r * p.ldq + x];
  for (int k = 0; k < p.Kq; ++k)
    if (qid[k] == x) return (double)qpr[k];
  return 0.0;
}

__global__ __launch_bounds__(kRowThreads) void samp_row(SampArgs p) {
  __shared__ float skey[kMaxTopK];
  __shared__ int32_t sid[kMaxTopK];
  __shared__ Fx wsum[kRowWaves];
  __shared__ int32_t qid[kMaxTopK];
  __shared__ float qpr[kMaxTopK];
  __shared__ int s_cp, s_cm;
  __shared__ double s_px;
  __shared__ int s_qk;
  const int row = blockIdx.x, seq = row / p.M, pos = row - seq * p.M;
  const int j = threadIdx.x, K = p.K, nt = blockDim.x;
  const bool draft_row = pos < p.M - 1;
  const int r = seq * (p.M - 1) + pos;
  // the draft and its dense q are loaded first (they do not depend on the
  // cuts); a sparse list is staged with the entries
  int x = -1;
  double qx_dense = 0.0;
  if (draft_row) {
    x = p.drafts[(int64_t)r];
    if (p.q && j == 0 && x >= 0 && x < p.V) qx_dense = (double)p.q[(int64_t)r * p.ldq + x];
  }
  if (draft_row && !p.q)
    for (int k = j; k < p.Kq; k += nt) {
      qid[k] = p.qi[(int64_t)r * p.Kq + k];
      qpr[k] = p.qp[(int64_t)r * p.Kq + k];
    }
  int n2 = 1;
  while (n2 < K) n2 <<= 1;
  if (j < n2) {
    skey[j] = j < K ? p.lz[(size_t)row * K + j] : -__builtin_inff();
    sid[j] = j < K ? p.lid[(size_t)row * K + j] : 0x7FFFFFFF;
  }
  if (j == 0) {
    s_cp = K;
    s_cm = K;
    s_px = 0.0;
    s_qk = 0x7FFFFFFF;
  }
  // order of probability: value descending, index ascending (padding last)
  bitonic(skey, sid, n2, [](float ka, int32_t ia, float kb, int32_t ib) {
    return ka > kb || (ka == kb && ia < ib);
  });
  double e = 0.0;
  Fx fe = fx_zero();
  if (j < K) {
    e = p.T == 0.0 ? (j == 0 ? 1.0 : 0.0) : exp(((double)skey[j] - (double)skey[0]) / p.T);
    fe = to_fx(e);
  }
  Fx S;
  const Fx before = fx_row_exclusive(fe, wsum, S);
  const Fx cum = fx_sum(before, fe);
  // top-p: the first entry whose cumulative mass reaches top_p * S
  if (p.T == 0.0) {
    if (j == 0) s_cp = 1;
  } else if (p.top_p < 1.0) {
    Fx thr = to_fx(p.top_p > 0.0 ? p.top_p * fx_to_double(S) : 0.0);
    if (!fx_nonzero(thr)) thr.lo = 1ull;
    if (j < K && fx_ge(cum, thr) && !fx_ge(before, thr)) s_cp = j + 1;
  }
  // min-p: the first entry (after the first) with e below min_p
  if (p.min_p > 0.0 && j >= 1 && j < K && e < p.min_p) atomicMin(&s_cm, j);
  __syncthreads();
  const int kept = min(s_cp, s_cm);
  // mass of the kept prefix (exact), then p' = e / mass
  __shared__ Fx s_mass;
  if (j == kept - 1) s_mass = cum;
  __syncthreads();
  const double mass = fx_to_double(s_mass);
  const bool in = j < kept;
  const double pj = in ? e / mass : 0.0;
  if (p.out_ids) {
    if (j < K) {   // the support: kept entries whose p' is positive in fp64
      const bool sup = in && pj > 0.0;
      p.out_ids[(size_t)row * K + j] = sup ? sid[j] : -1;
      p.out_probs[(size_t)row * K + j] = sup ? (float)pj : 0.0f;
    }
  }
  // acceptance inputs of the row's draft
  if (draft_row) {
    if (in && sid[j] == x) s_px = pj;
    if (!p.q)
      for (int k = j; k < p.Kq; k += nt)
        if (qid[k] == x) atomicMin(&s_qk, k);
  }
  // the support in index order for the draws: e and p' by id
  __shared__ double se_s[kMaxTopK], sp_s[kMaxTopK];
  __syncthreads();
  if (j < kept) {
    se_s[j] = e;
    sp_s[j] = pj;
    skey[j] = (float)j;   // remembers the slot of each id through the sort
  }
  int m2 = 1;
  while (m2 < kept) m2 <<= 1;
  if (j >= kept && j < m2) {
    sid[j] = 0x7FFFFFFF;
    skey[j] = 0.0f;
  }
  bitonic(skey, sid, m2, [](float, int32_t ia, float, int32_t ib) { return ia < ib; });
  if (j < kept) {
    const int s = (int)skey[j];
    p.sid[(size_t)row * K + j] = sid[j];
    p.se[(size_t)row * K + j] = se_s[s];
    p.sp[(size_t)row * K + j] = sp_s[s];
  }
  if (j == 0) {
    p.nkept[row] = kept;
    if (draft_row) {
      double qx = 0.0;
      if (x >= 0 && x < p.V) qx = p.q ? qx_dense : (s_qk != 0x7FFFFFFF ? (double)qpr[s_qk] : 0.0);
      p.acc[row] = AccIn{(x >= 0 && x < p.V) ? s_px : 0.0, qx};
    }
  }
}

// One workgroup per sequence: the accepted run a (first draft with
// u_i * q_i(x_i) >= p'_i(x_i)), then the draw from the residual
// max(0, p'_a - q_a) over row a's support (from p'_a if it is all zero), or
// the bonus from p'_{M-1}, in index order: the smallest id whose cumulative
// weight exceeds u_{M-1} times the total (the last positive if rounding
// passes the end).
__global__ __launch_bounds__(kRowThreads) void samp_draw(SampArgs p) {
  __shared__ Fx wsum[kRowWaves];
  __shared__ int32_t qid[kMaxTopK];
  __shared__ float qpr[kMaxTopK];
  __shared__ int s_a, s_pick, s_last;
  const int seq = blockIdx.x, j = threadIdx.x, nt = blockDim.x;
  // the drafts (committed as they are up to the run) do not depend on it
  const int32_t dj = j < p.M - 1 ? p.drafts[(int64_t)seq * (p.M - 1) + j] : -1;
  if (j < kWave) {
    bool reject = false;
    if (j < p.M - 1) {
      const AccIn in = p.acc[seq * p.M + j];
      reject = !((double)p.u[(int64_t)seq * p.M + j] * in.qx < in.px);
    }
    const u64 rej = __ballot(reject);
    if (j == 0) {
      s_a = rej ? __ffsll((long long)rej) - 1 : p.M - 1;
      s_pick = 0x7FFFFFFF;
      s_last = -1;
    }
  }
  __syncthreads();
  const int a = s_a, row = seq * p.M + a;
  const bool residual = a < p.M - 1;
  const int r = seq * (p.M - 1) + a;
  if (residual && !p.q)
    for (int k = j; k < p.Kq; k += nt) {
      qid[k] = p.qi[(int64_t)r * p.Kq + k];
      qpr[k] = p.qp[(int64_t)r * p.Kq + k];
    }
  __syncthreads();
  const int n = p.nkept[row];
  int32_t id = -1;
  Fx wr = fx_zero(), we = fx_zero();
  double dres = 0.0, dp = 0.0;   // fp64 residual and p'
  if (j < n) {
    id = p.sid[(size_t)row * p.K + j];
    we = to_fx(p.se[(size_t)row * p.K + j]);
    dp = p.sp[(size_t)row * p.K + j];
    if (residual) {
      const double d = dp - samp_q(p, r, id, qid, qpr);
      dres = d > 0.0 ? d : 0.0;
      wr = to_fx(dres);
    }
  }
  // first support slot (id order) with a positive fp64 residual, resp. p'
  __shared__ int s_fr, s_fp;
  if (j == 0) {
    s_fr = 0x7FFFFFFF;
    s_fp = 0x7FFFFFFF;
  }
  __syncthreads();
  if (dres > 0.0) atomicMin(&s_fr, j);
  if (dp > 0.0) atomicMin(&s_fp, j);
  Fx tres;
  fx_row_exclusive(wr, wsum, tres);   // (its barriers also order the minima)
  // the residual is used when any of its fp64 weights is positive, even if
  // all of them are below the fixed-point resolution
  const bool use_res = residual && s_fr != 0x7FFFFFFF;
  const Fx w = use_res ? wr : we;
  Fx W;
  const Fx before = fx_row_exclusive(w, wsum, W);
  const double u = (double)p.u[(int64_t)seq * p.M + p.M - 1];
  const Fx target = to_fx(u * fx_to_double(W));
  if (!fx_nonzero(target)) {
    // below 2^-100: u = 0 takes the first positive weight (the first slot
    // whose running sum exceeds 0); another target follows the fp64
    // definition in index order (the residual, or p' itself), summed by one
    // thread over the support
    if (j == 0) {
      const int f = use_res ? s_fr : s_fp;
      int slot = f;
      if (u != 0.0) {
        auto wgt = [&](int k) {
          const double pk = p.sp[(size_t)row * p.K + k];
          if (!use_res) return pk;
          const double d = pk - samp_q(p, r, p.sid[(size_t)row * p.K + k], qid, qpr);
          return d > 0.0 ? d : 0.0;
        };
        double Wd = 0.0;
        int last = -1;
        for (int k = 0; k < n; ++k) {
          const double wk = wgt(k);
          Wd += wk;
          if (wk > 0.0) last = k;
        }
        const double t = u * Wd;
        double cum = 0.0;
        slot = last;
        for (int k = 0; k < n; ++k) {
          cum += wgt(k);
          if (cum > t) {
            slot = k;
            break;
          }
        }
      }
      s_pick = (slot >= 0 && slot < n) ? p.sid[(size_t)row * p.K + slot] : p.V - 1;
    }
  } else if (j < n) {
    const Fx cum = fx_sum(before, w);
    if (fx_gt(cum, target) && !fx_gt(before, target)) s_pick = id;
    if (fx_nonzero(w)) atomicMax(&s_last, j);
  }
  __syncthreads();
  if (j == 0 && s_pick == 0x7FFFFFFF)   // rounding passed the end
    s_pick = s_last >= 0 ? p.sid[(size_t)row * p.K + s_last] : p.V - 1;
  __syncthreads();
  if (j < p.M) {
    const int32_t tok = j < a ? dj : (j == a ? s_pick : -1);
    p.tokens[(int64_t)seq * p.M + j] = tok;
  }
  if (j == 0) {
    p.counts[2 * seq] = a;
    p.counts[2 * seq + 1] = a + 1;
    p.rollback[seq] = (p.base_len ? p.base_len[seq] : 0) + a + 1;
  }
}

// ---- sampled acceptance in one launch ----------------------------------------
//
// The pipeline above in one launch of G workgroups per row, with no
// workgroup ever waiting for another.  Each workgroup penalises its chunk
// of up to kOneChunk entries in registers, bins it by d = chunk max - z
// (sbin), and takes as candidates its entries in the bins up to the first
// whose count from the top reaches K: a superset of the chunk's own top K.
// It writes them in index order to its own segment of the workspace,
// publishes their number and smallest key (0 when the chunk holds fewer
// than K entries, all of them candidates), and arrives on the row's
// counter.  The last workgroup of the row to arrive resolves the row alone:
//   - kappa = the largest published key.  The workgroup that published it
//     holds at least K entries with keys >= kappa, and every workgroup's
//     entries with keys >= kappa are among its candidates, so the set S of
//     candidates with keys >= kappa holds the row's top K;
//   - a histogram of S over bins of d = row max - z finds the bin where the
//     count from the top reaches K; the entries of S up to that bin are
//     sorted (key descending, index ascending) and the first K are the
//     row's top K in the order of probability.  When that bin is too full
//     to sort (heavy ties) a radix select finds the K-th key instead, and
//     the ties at it are taken in index order;
//   - softmax, top-p and min-p on exact fixed-point prefix sums, p', the
//     row's acceptance input, and the draw the row would make if the
//     accepted run stopped at it (the residual for a draft row, the bonus
//     for the last), in index order over its support, as samp_row and
//     samp_draw do;
//   - the row's verdict and token go to the workspace; the last row of the
//     sequence to finish derives the accepted run and writes the outputs.
// The resolver's steps are short chains on one workgroup, so each runs on
// as few waves as its data needs (the others wait at the next barrier),
// and wave-wide sums and extrema move data between lanes with DPP rather
// than through LDS.  Data crossing workgroups follows the rules of rej_one
// (agent-scope atomic stores and loads, each writer's stores complete
// before it arrives).  The counters live in the workspace head; each call
// leaves them zero.

constexpr int kSHB = 2048;              // bins of d: exponent and 5 mantissa bits
constexpr int kSBinBase = 3072;         // bin 0 takes every d below 2^-31
constexpr int kSRoom = 8192;            // entries of S the resolver keeps in LDS
constexpr int kSMaxG = 256;
constexpr int kSMaxRows = 4096;
constexpr int kSMaxSeqs = 1024;
constexpr int kSCandBudget = 16384;     // expected candidates per row the launch rule allows
constexpr int kSSlotPer = 8;            // first-round candidate slots per resolver thread
constexpr int kSOffL = 0;                           // u64 [kSRoom]: S (first the penalty window)
constexpr int kSOffSort = kSOffL + 8 * kSRoom;      // u64 [kSSortMax]: entries to sort
constexpr int kSOffE = kSOffSort + 8 * kSSortMax;   // fp64 [kMaxTopK]: e by rank
constexpr int kSOffP = kSOffE + 8 * kMaxTopK;       //   p' by rank
constexpr int kSOffQ = kSOffP + 8 * kMaxTopK;       //   q(id) by rank
constexpr int kSOffId = kSOffQ + 8 * kMaxTopK;      // int32 [kMaxTopK]: id by rank
constexpr int kSOffQid = kSOffId + 4 * kMaxTopK;    // the sparse draft list
constexpr int kSOffQpr = kSOffQid + 4 * kMaxTopK;
constexpr int kSDyn = kSOffQpr + 4 * kMaxTopK;
static_assert(4 * kMaxPenaltyWindow <= 8 * kSRoom, "the penalty window fits where S goes");
static_assert(kSHB == 32 * kWave, "32 bins per lane of one wave");
static_assert(kSSortMax == 2 * kOneThreads, "one compare-exchange per thread and step");
static_assert(kMaxTopK <= kOneThreads && kMaxTopK <= kSSortMax, "one kept entry per thread");
static_assert(kSMaxG <= 4 * kWave, "four segments per lane");
static_assert(kWave == 64, "the accepted run takes one lane per row");

// Bin of z below zmax (a key >= z's): the exponent and leading 5 mantissa
// bits of d = zmax - z, shifted and clamped, so bins are about 3% of d wide.
// d is monotone in z, so each bin is an interval of keys.
__device__ __forceinline__ int sbin(float zmax, float z) {
  const int b = (int)(__float_as_uint(zmax - z) >> 18) - kSBinBase;
  return b < 0 ? 0 : (b < kSHB ? b : kSHB - 1);
}

// Exclusive exact prefix of v over the threads of the first W waves (thread
// order; the other threads must pass zero) and their total.  The whole
// workgroup calls it.
__device__ Fx fx_excl_w(Fx v, Fx *red, Fx &total, int W) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  Fx incl = v;
  if (wave < W) incl = dpp_fx_incl(v);
  __syncthreads();
  if (wave < W && lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  Fx before = fx_zero();
  total = fx_zero();
  for (int w = 0; w < W; ++w) {
    if (w < wave) fx_add(before, red[w]);
    fx_add(total, red[w]);
  }
  return fx_sum(before, fx_sub(incl, v));
}

// One wave: the first bin of h[0 .. kSHB) where the count from bin 0 reaches
// K, the count before it and its own (the same in every lane); bin -1 when
// the total stays below K.
__device__ void first_bin_reaching(const uint32_t *h, int K, int &bin, int &before, int &cnt) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint4 *h4 = reinterpret_cast<const uint4 *>(h + 32 * lane);
  int s = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 c = h4[q];
    s += (int)(c.x + c.y + c.z + c.w);
  }
  const int incl = dpp_incl(s);
  const u64 b = __ballot(incl - s < K && incl >= K);
  bin = -1;
  before = 0;
  cnt = 0;
  if (!b) return;
  const int L = __ffsll((long long)b) - 1;
  const int base = __builtin_amdgcn_readlane(incl - s, L);
  const int hv = lane < 32 ? (int)h[32 * L + lane] : 0;
  const int inc2 = base + dpp_incl(hv);
  const u64 b2 = __ballot(lane < 32 && inc2 >= K && inc2 - hv < K);
  const int l2 = __ffsll((long long)b2) - 1;
  bin = 32 * L + l2;
  before = __builtin_amdgcn_readlane(inc2 - hv, l2);
  cnt = __builtin_amdgcn_readlane(hv, l2);
}

__device__ __forceinline__ uint32_t add_ag32(uint32_t *c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_ag32(uint32_t *c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 of the last row of a sequence to finish: the accepted run a (the
// first rejected draft row, else M-1) and the sequence's outputs.
__device__ void samp_commit(const SampArgs &p, int seq) {
  const int i = threadIdx.x & (kWave - 1);
  const u64 rw = i < p.M ? ld_ag(p.res + (size_t)seq * p.M + i) : 0ull;
  const u64 rej = __ballot(i < p.M - 1 && ((rw >> 31) & 1ull));
  const int a = rej ? __ffsll((long long)rej) - 1 : p.M - 1;
  const int tok = __shfl((int)(rw & 0x7FFFFFFFull), a);
  if (i < p.M)
    p.tokens[(int64_t)seq * p.M + i] =
        i < a ? p.drafts[(int64_t)seq * (p.M - 1) + i] : (i == a ? tok : -1);
  if (i == 0) {
    p.counts[2 * seq] = a;
    p.counts[2 * seq + 1] = a + 1;
    p.rollback[seq] = (p.base_len ? p.base_len[seq] : 0) + a + 1;
    clear_ag32(p.seqcnt + seq);
  }
}

// Steps (3)-(5) for K <= 64 on wave 0 alone (the other waves have left):
// lane j holds rank j; every prefix is a DPP scan, every cut, first and
// last a ballot, the index order a count over readlane, and the weights
// reach index order through LDS within the wave, so no workgroup barrier
// is needed.  Same decisions, in the same arithmetic, as the general path.
__device__ void samp_small(const SampArgs &p, const u64 *top, int row, int seq, int pos,
                           double qx_dense, const int32_t *qid, const float *qpr, double ub,
                           unsigned char *scratch) {
  const int lane = threadIdx.x & (kWave - 1), K = p.K;
  const double T = p.T;
  const bool draft_row = pos < p.M - 1;
  const int r = seq * (p.M - 1) + pos;
  const int x = draft_row ? p.drafts[r] : -1;
  const bool xvalid = x >= 0 && x < p.V;
  const bool act = lane < K;
  int idj = -1;
  double e = 0.0;
  float qpre = 0.0f;
  if (act) {
    const float z0 = key_to_float((uint32_t)(top[0] >> 32));
    const u64 w = top[lane];
    idj = (int)(0xFFFFFFFFu - (uint32_t)w);
    if (draft_row && p.q && idj >= 0 && idj < p.V) qpre = p.q[(int64_t)r * p.ldq + idj];
    e = T == 0.0 ? (lane == 0 ? 1.0 : 0.0)
                 : exp(((double)key_to_float((uint32_t)(w >> 32)) - (double)z0) / T);
  }
  // softmax mass, top-p and min-p cuts, p'
  const Fx fe = to_fx(e);
  const Fx incl = dpp_fx_incl(fe);
  const Fx before = fx_sub(incl, fe);
  int cp = K;
  if (T == 0.0) {
    cp = 1;
  } else if (p.top_p < 1.0) {
    Fx thr = to_fx(p.top_p > 0.0 ? p.top_p * fx_to_double(fx_readlane(incl, kWave - 1)) : 0.0);
    if (!fx_nonzero(thr)) thr.lo = 1ull;
    const u64 b = __ballot(act && fx_ge(incl, thr) && !fx_ge(before, thr));
    if (b) cp = __ffsll((long long)b);
  }
  int cm = K;
  if (p.min_p > 0.0) {
    const u64 b = __ballot(act && lane >= 1 && e < p.min_p);
    if (b) cm = __ffsll((long long)b) - 1;
  }
  const int kept = min(cp, cm);
  const bool in = lane < kept;
  const double pj = in ? e / fx_to_double(fx_readlane(incl, kept - 1)) : 0.0;
  if (p.out_ids && act) {   // the support: kept entries whose p' is positive in fp64
    const bool sup = in && pj > 0.0;
    p.out_ids[(size_t)row * K + lane] = sup ? idj : -1;
    p.out_probs[(size_t)row * K + lane] = sup ? (float)pj : 0.0f;
  }
  // the acceptance input of the row's draft
  double px = 0.0, qx = 0.0;
  if (draft_row && xvalid) {
    const u64 bx = __ballot(in && idj == x);
    if (bx) px = dbl_readlane(pj, __ffsll((long long)bx) - 1);
    if (p.q) {
      qx = qx_dense;
    } else {
      for (int k0 = 0; k0 < p.Kq; k0 += kWave) {
        const u64 bq = __ballot(k0 + lane < p.Kq && qid[k0 + lane] == x);
        if (bq) {
          qx = (double)qpr[k0 + __ffsll((long long)bq) - 1];
          break;
        }
      }
    }
  }
  // the draw this row would make: weights at rank order, then index order
  const bool residual = draft_row;
  double qj = 0.0;
  if (residual && in) {
    if (p.q) {
      qj = (double)qpre;
    } else {
      for (int k = 0; k < p.Kq; ++k)
        if (qid[k] == idj) {
          qj = (double)qpr[k];
          break;
        }
    }
  }
  double dres = 0.0;
  Fx wr = fx_zero();
  if (residual && in) {
    const double d = pj - qj;
    dres = d > 0.0 ? d : 0.0;
    wr = to_fx(dres);
  }
  // the residual is used when any of its fp64 weights is positive, even if
  // all of them are below the fixed-point resolution
  const bool use_res = residual && __ballot(in && dres > 0.0) != 0ull;
  const Fx w = use_res ? wr : (in ? fe : fx_zero());
  int rid = 0;   // place in index order among the kept ids (distinct)
  for (int k = 0; k < kept; ++k) rid += __builtin_amdgcn_readlane(idj, k) < idj ? 1 : 0;
  Fx *wS = reinterpret_cast<Fx *>(scratch);
  int32_t *idS = reinterpret_cast<int32_t *>(scratch + sizeof(Fx) * kWave);
  double *pS = reinterpret_cast<double *>(scratch + (sizeof(Fx) + 4) * kWave);
  double *qS = reinterpret_cast<double *>(scratch + (sizeof(Fx) + 12) * kWave);
  if (in) {
    wS[rid] = w;
    idS[rid] = idj;
    pS[rid] = pj;
    qS[rid] = qj;
  }
  __builtin_amdgcn_wave_barrier();
  const bool sv = lane < kept;   // lane s now holds index-order slot s
  const Fx ws = sv ? wS[lane] : fx_zero();
  const int ids = sv ? idS[lane] : -1;
  const double dps = sv ? pS[lane] : 0.0;
  double dress = 0.0;
  if (residual && sv) {
    const double d = dps - qS[lane];
    dress = d > 0.0 ? d : 0.0;
  }
  const u64 bfr = __ballot(dress > 0.0), bfp = __ballot(dps > 0.0);
  const Fx wincl = dpp_fx_incl(ws);
  const Fx bef = fx_sub(wincl, ws);
  const Fx target = to_fx(ub * fx_to_double(fx_readlane(wincl, kWave - 1)));
  int pick;
  if (!fx_nonzero(target)) {
    // below 2^-100: u = 0 takes the first positive weight; another target
    // follows the fp64 definition in index order (every lane alike)
    int slot = use_res ? (bfr ? __ffsll((long long)bfr) - 1 : kNone)
                       : (bfp ? __ffsll((long long)bfp) - 1 : kNone);
    if (ub != 0.0) {
      auto wgt = [&](int k) {
        if (!use_res) return pS[k];
        const double d = pS[k] - qS[k];
        return d > 0.0 ? d : 0.0;
      };
      double Wd = 0.0;
      int last = -1;
      for (int k = 0; k < kept; ++k) {
        const double wk = wgt(k);
        Wd += wk;
        if (wk > 0.0) last = k;
      }
      const double tt = ub * Wd;
      double cm2 = 0.0;
      slot = last;
      for (int k = 0; k < kept; ++k) {
        cm2 += wgt(k);
        if (cm2 > tt) {
          slot = k;
          break;
        }
      }
    }
    pick = (slot >= 0 && slot < kept) ? idS[slot] : p.V - 1;
  } else {
    const u64 bp = __ballot(sv && fx_gt(wincl, target) && !fx_gt(bef, target));
    if (bp) {
      pick = __builtin_amdgcn_readlane(ids, __ffsll((long long)bp) - 1);
    } else {   // rounding passed the end: the last positive weight
      const u64 bl = __ballot(sv && fx_nonzero(ws));
      pick = bl ? __builtin_amdgcn_readlane(ids, 63 - __clzll((long long)bl)) : p.V - 1;
    }
  }
  // the row's verdict and token; the last row of the sequence commits it
  bool reject = false;
  if (draft_row) reject = !((double)p.u[(int64_t)seq * p.M + pos] * qx < px);
  int last = 0;
  if (lane == 0) {
    st_ag(p.res + row, ((u64)(reject ? 1u : 0u) << 31) | (u64)(uint32_t)pick);
    __builtin_amdgcn_s_waitcnt(0);
    last = add_ag32(p.seqcnt + seq) == (uint32_t)(p.M - 1) ? 1 : 0;
  }
  if (__builtin_amdgcn_readfirstlane(last)) samp_commit(p, seq);
}

// grid (rows * G), kOneThreads threads, kSDyn bytes of dynamic LDS.
__global__ __launch_bounds__(kOneThreads) void samp_one(SampArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  __shared__ __attribute__((aligned(16))) uint32_t hs[kSHB];
  __shared__ int koff[kKPer * kOneWaves + 1];
  __shared__ int wcnt[kOneWaves];
  __shared__ uint32_t wkey[kOneWaves];
  __shared__ Fx red[kOneWaves];
  __shared__ int segoff[kSMaxG + 1], segcnt[kSMaxG], remoff[kSMaxG + 1];
  __shared__ Fx s_mass;
  __shared__ double s_px, s_qx;
  __shared__ uint32_t s_kmax, s_kap;
  __shared__ int s_nl, s_bst, s_A, s_n2, s_last, s_ns, s_m, s_dig, s_abv;
  __shared__ int s_cp, s_cm, s_qk, s_fr, s_fp, s_pick, s_lastw;
  const int G = p.G, C = p.C, row = blockIdx.x / G, g = blockIdx.x - row * G;
  const int seq = row / p.M, pos = row - seq * p.M;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int j0 = g * C, n = min(C, p.V - j0), K = p.K;

  // (1) the chunk, penalised in registers: entry k * kOneThreads + t is
  // thread t's k-th
  const float *zr = p.z + (int64_t)row * p.ldl + j0;
  float v[kKPer];
#pragma unroll
  for (int k = 0; k < kKPer; ++k) {
    const int i = k * kOneThreads + tid;
    v[k] = i < n ? zr[i] : 0.0f;
  }
  for (int i = tid; i < kSHB; i += kOneThreads) hs[i] = 0u;
  if (p.pen) {
    // the window's tokens inside the chunk, then each entry's count
    int32_t *lt = reinterpret_cast<int32_t *>(dyn + kSOffL);
    if (tid == 0) s_nl = 0;
    __syncthreads();
    const int Lh = p.htok ? max(0, min(p.hlen[seq], (int)p.ldh)) : 0;
    const int total = Lh + pos, w0 = max(0, total - p.last_n);
    for (int c = w0 + tid; c < total; c += kOneThreads) {
      const int t = c < Lh ? p.htok[(int64_t)seq * p.ldh + c]
                           : p.drafts[(int64_t)seq * (p.M - 1) + (c - Lh)];
      if (t >= j0 && t < j0 + n) lt[atomicAdd(&s_nl, 1)] = t;
    }
    __syncthreads();
    const int nl = s_nl;
#pragma unroll
    for (int k = 0; k < kKPer; ++k) {
      const int i = k * kOneThreads + tid;
      int c = 0;
      for (int q = 0; q < nl; ++q) c += lt[q] == j0 + i ? 1 : 0;
      if (c && i < n) v[k] = penalise(v[k], c, p);
    }
  }
  // the chunk maximum by key (+0 above -0), then the count histogram and
  // (wave 0) the first bin where the count from the top reaches K
  uint32_t km = 0u;
#pragma unroll
  for (int k = 0; k < kKPer; ++k)
    if (k * kOneThreads + tid < n) km = max(km, fkey(v[k]));
  km = dpp_umax(km);
  if (lane == 0) wkey[wave] = km;
  __syncthreads();
  km = 0u;
  for (int w = 0; w < kOneWaves; ++w) km = max(km, wkey[w]);
  const float mg = key_to_float(km);
  int bk[kKPer];
#pragma unroll
  for (int k = 0; k < kKPer; ++k) {
    bk[k] = kSHB;
    if (k * kOneThreads + tid < n) {
      bk[k] = sbin(mg, v[k]);
      atomicAdd(&hs[bk[k]], 1u);
    }
  }
  __syncthreads();
  if (wave == 0) {
    int bin, before, cnt;
    first_bin_reaching(hs, K, bin, before, cnt);
    if (lane == 0) s_bst = bin;
  }
  __syncthreads();
  const int bst0 = s_bst;   // -1: the chunk holds fewer than K entries, all candidates
  // the candidates, in index order, and their smallest key
  {
    u64 bal[kKPer];
    uint32_t kmn = 0xFFFFFFFFu;
#pragma unroll
    for (int k = 0; k < kKPer; ++k) {
      const bool c = k * kOneThreads + tid < n && (bst0 < 0 || bk[k] <= bst0);
      bal[k] = __ballot(c);
      if (lane == 0) koff[k * kOneWaves + wave] = __popcll(bal[k]);
      if (c) kmn = min(kmn, fkey(v[k]));
    }
    kmn = dpp_umin(kmn);
    if (lane == 0) wkey[wave] = kmn;
    __syncthreads();
    if (wave == 0) {
      const int c0 = koff[2 * lane], c1 = koff[2 * lane + 1];
      const int incl = dpp_incl(c0 + c1);
      const int before = incl - c0 - c1;
      koff[2 * lane] = before;
      koff[2 * lane + 1] = before + c0;
      if (lane == kWave - 1) koff[kKPer * kOneWaves] = incl;
    }
    __syncthreads();
    u64 *seg = p.cand + (size_t)(row * G + g) * C;
#pragma unroll
    for (int k = 0; k < kKPer; ++k) {
      if ((bal[k] >> lane) & 1ull) {
        const int i = k * kOneThreads + tid;
        const int at = koff[k * kOneWaves + wave] + __popcll(bal[k] & ((1ull << lane) - 1ull));
        st_ag(seg + at, ((u64)fkey(v[k]) << 32) | (uint32_t)(j0 + i));
      }
    }
    if (tid == 0) {
      uint32_t kg = 0u;
      if (bst0 >= 0) {
        kg = 0xFFFFFFFFu;
        for (int w = 0; w < kOneWaves; ++w) kg = min(kg, wkey[w]);
      }
      st_ag(p.info + row * G + g, ((u64)kg << 32) | (u64)(uint32_t)koff[kKPer * kOneWaves]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = add_ag32(p.rowcnt + row) == (uint32_t)(G - 1);
  __syncthreads();
  if (!s_last) return;

  // (2) the last workgroup of the row resolves it.  One round of loads:
  // the first Kc slots of every segment (valid or not: Kc is a power of two
  // <= C, so they stay inside the segment), the segments' words (wave 0),
  // the draft and its dense q (last wave), the sparse draft list.
  if (tid == 0) clear_ag32(p.rowcnt + row);
  const bool draft_row = pos < p.M - 1;
  const int r = seq * (p.M - 1) + pos;
  const double T = p.T;
  const int W = (K + kWave - 1) / kWave;   // waves of the per-rank steps
  const int lk = p.lkc, Kc = 1 << lk, nslot = G << lk;
  u64 vs[kSSlotPer];
#pragma unroll
  for (int t = 0; t < kSSlotPer; ++t) {
    const int sl = t * kOneThreads + tid;
    vs[t] = sl < nslot ? ld_ag(p.cand + (size_t)(row * G + (sl >> lk)) * C + (sl & (Kc - 1)))
                       : 0ull;
  }
  int32_t *qid = reinterpret_cast<int32_t *>(dyn + kSOffQid);
  float *qpr = reinterpret_cast<float *>(dyn + kSOffQpr);
  if (draft_row && !p.q)
    for (int k = tid; k < p.Kq; k += kOneThreads) {
      qid[k] = p.qi[(int64_t)r * p.Kq + k];
      qpr[k] = p.qp[(int64_t)r * p.Kq + k];
    }
  if (tid == kOneThreads - kWave) {
    const int x = draft_row ? p.drafts[r] : -1;
    s_qx = (draft_row && p.q && x >= 0 && x < p.V) ? (double)p.q[(int64_t)r * p.ldq + x] : 0.0;
  }
  const int x = draft_row ? p.drafts[r] : -1;
  const bool xvalid = x >= 0 && x < p.V;
  const double ub = (double)p.u[(int64_t)seq * p.M + p.M - 1];
  if (wave == 0) {
    // counts, offsets, kappa; counts past Kc are left for a second round
    int c[4], ex[4], s = 0, e = 0;
    uint32_t kap = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sg = 4 * lane + q;
      c[q] = 0;
      if (sg < G) {
        const u64 w = ld_ag(p.info + row * G + sg);
        c[q] = (int)(uint32_t)w;
        kap = max(kap, (uint32_t)(w >> 32));
      }
      ex[q] = max(0, c[q] - Kc);
      s += c[q];
      e += ex[q];
    }
    const int incl = dpp_incl(s), einc = dpp_incl(e);
    int before = incl - s, ebefore = einc - e;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sg = 4 * lane + q;
      if (sg < G) {
        segoff[sg] = before;
        segcnt[sg] = c[q];
        remoff[sg] = ebefore;
      }
      before += c[q];
      ebefore += ex[q];
    }
    if (lane == kWave - 1) {
      segoff[G] = incl;
      remoff[G] = einc;
    }
    kap = dpp_umax(kap);
    if (lane == 0) {
      s_kap = kap;
      s_ns = 0;
      s_kmax = 0u;
    }
  }
  __syncthreads();
  const int nc = segoff[G], nrem = remoff[G];
  const uint32_t kap = s_kap;
  // candidate i of the row (index order): segment by binary search
  auto cand_at = [&](int i) -> u64 {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (segoff[mid] <= i) lo = mid;
      else hi = mid;
    }
    return ld_ag(p.cand + (size_t)(row * G + lo) * C + (i - segoff[lo]));
  };
  // f(i, w) for every candidate in rounds of kOneThreads * kResPer (loads
  // in flight), the same number of calls in every thread (i >= nc: padding)
  auto for_cands = [&](auto &&f) {
    for (int base = 0; base < nc; base += kOneThreads * kResPer) {
      u64 vv[kResPer];
#pragma unroll
      for (int t = 0; t < kResPer; ++t) {
        const int i = base + t * kOneThreads + tid;
        vv[t] = i < nc ? cand_at(i) : 0ull;
      }
#pragma unroll
      for (int t = 0; t < kResPer; ++t) f(base + t * kOneThreads + tid, vv[t]);
    }
  };
  // S into LDS (while it fits) and the row maximum: the loaded slots, then
  // the candidates past Kc
  u64 *Ls = reinterpret_cast<u64 *>(dyn + kSOffL);
  {
    uint32_t kmx = 0u;
    auto take = [&](bool valid, u64 w) {
      const uint32_t key = (uint32_t)(w >> 32);
      const bool f = valid && key >= kap;
      const int at = wave_append(f, &s_ns);
      if (f) {
        if (at < kSRoom) Ls[at] = w;
        kmx = max(kmx, key);
      }
    };
#pragma unroll
    for (int t = 0; t < kSSlotPer; ++t) {
      if (t * kOneThreads >= nslot) break;   // (uniform)
      const int sl = t * kOneThreads + tid;
      take(sl < nslot && (sl & (Kc - 1)) < segcnt[min(sl >> lk, G - 1)], vs[t]);
    }
    for (int base = 0; base < nrem; base += kOneThreads * kResPer) {
      u64 vv[kResPer];
#pragma unroll
      for (int t = 0; t < kResPer; ++t) {
        const int i = base + t * kOneThreads + tid;
        vv[t] = 0ull;
        if (i < nrem) {
          int lo = 0, hi = G;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (remoff[mid] <= i) lo = mid;
            else hi = mid;
          }
          vv[t] = ld_ag(p.cand + (size_t)(row * G + lo) * C + Kc + (i - remoff[lo]));
        }
      }
#pragma unroll
      for (int t = 0; t < kResPer; ++t) take(base + t * kOneThreads + tid < nrem, vv[t]);
    }
    kmx = dpp_umax(kmx);
    if (lane == 0) atomicMax(&s_kmax, kmx);
  }
  for (int i = tid; i < kSHB; i += kOneThreads) hs[i] = 0u;
  __syncthreads();
  const int ns = s_ns;
  const bool inl = ns <= kSRoom;
  const float zmax = key_to_float(s_kmax);
  // histogram of S by d = zmax - z; (wave 0) the bin where the count reaches K
  if (inl) {
    for (int i = tid; i < ns; i += kOneThreads)
      atomicAdd(&hs[sbin(zmax, key_to_float((uint32_t)(Ls[i] >> 32)))], 1u);
  } else {
    for_cands([&](int i, u64 w) {
      const uint32_t key = (uint32_t)(w >> 32);
      if (i < nc && key >= kap) atomicAdd(&hs[sbin(zmax, key_to_float(key))], 1u);
    });
  }
  __syncthreads();
  if (wave == 0) {
    int bin, before, cnt;
    first_bin_reaching(hs, K, bin, before, cnt);
    if (lane == 0) {
      s_bst = bin;
      s_A = before;
      s_n2 = bin < 0 ? 0x7FFFFFFF : cnt;
      s_m = 0;
    }
  }
  __syncthreads();
  const int bst = s_bst;
  u64 *Sa = reinterpret_cast<u64 *>(dyn + kSOffSort);
  // an entry to sort, keyed (key << 32 | ~index): descending order is key
  // descending, index ascending
  auto put = [&](bool f, u64 w) {
    const int at = wave_append(f, &s_m);
    if (f && at < kSSortMax)
      Sa[at] = (w & 0xFFFFFFFF00000000ull) | (0xFFFFFFFFull - (w & 0xFFFFFFFFull));
  };
  if ((int64_t)s_A + s_n2 <= kSSortMax) {
    // S up to the bin of the cut
    if (inl) {
      for (int base = 0; base < ns; base += kOneThreads) {
        const int i = base + tid;
        const u64 w = i < ns ? Ls[i] : 0ull;
        put(i < ns && sbin(zmax, key_to_float((uint32_t)(w >> 32))) <= bst, w);
      }
    } else {
      for_cands([&](int i, u64 w) {
        const uint32_t key = (uint32_t)(w >> 32);
        put(i < nc && key >= kap && sbin(zmax, key_to_float(key)) <= bst, w);
      });
    }
  } else {
    // radix select of the K-th key of S, 8 bits a pass; then the entries
    // above it and the first ties at it in index order
    uint32_t prefix = 0u;
    int above = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kBins; i += kOneThreads) hs[i] = 0u;
      if (tid == 0) {
        s_dig = 0;
        s_abv = above;
      }
      __syncthreads();
      for_cands([&](int i, u64 w) {
        const uint32_t key = (uint32_t)(w >> 32);
        if (i < nc && key >= kap && (pass == 0 || (key >> (shift + 8)) == prefix))
          atomicAdd(&hs[(key >> shift) & 0xFFu], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        int c[4], s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = (int)hs[255 - 4 * lane - q];
          s += c[q];
        }
        const int incl = dpp_incl(s);
        int acc = above + incl - s;
        if (acc < K && acc + s >= K) {
          for (int q = 0; q < 4; ++q) {
            if (acc + c[q] >= K) {
              s_dig = 255 - 4 * lane - q;
              s_abv = acc;
              break;
            }
            acc += c[q];
          }
        }
      }
      __syncthreads();
      prefix = (prefix << 8) | (uint32_t)s_dig;
      above = s_abv;
      __syncthreads();
    }
    const uint32_t kst = prefix;
    const int t = K - above;
    int seen = 0;
    for_cands([&](int i, u64 w) {
      const uint32_t key = (uint32_t)(w >> 32);
      const bool tie = i < nc && key == kst;
      int pre;
      const int nt = count_one(tie, pre, wcnt);
      put((i < nc && key > kst) || (tie && seen + pre < t), w);
      seen += nt;
    });
  }
  __syncthreads();
  const u64 *top = sort_desc(Sa, Ls, min(s_m, kSSortMax));
  if (K <= kWave) {   // one wave from here on
    if (wave == 0) samp_small(p, top, row, seq, pos, s_qx, qid, qpr, ub, dyn + kSOffE);
    return;
  }

  // (3) the row's target over its top K (thread j of the first W waves
  // holds rank j): e, the top-p and min-p cuts, p'; as samp_row
  const int j = tid;
  double *eR = reinterpret_cast<double *>(dyn + kSOffE);
  double *pR = reinterpret_cast<double *>(dyn + kSOffP);
  double *qR = reinterpret_cast<double *>(dyn + kSOffQ);
  int32_t *idR = reinterpret_cast<int32_t *>(dyn + kSOffId);
  int idj = -1;
  double e = 0.0;
  float qpre = 0.0f;   // the draft's dense q at this rank's id, loaded early
  Fx fe = fx_zero();
  if (j < K) {
    const float z0 = key_to_float((uint32_t)(top[0] >> 32));
    const u64 w = top[j];
    idj = (int)(0xFFFFFFFFu - (uint32_t)w);
    if (draft_row && p.q && idj >= 0 && idj < p.V) qpre = p.q[(int64_t)r * p.ldq + idj];
    e = T == 0.0 ? (j == 0 ? 1.0 : 0.0)
                 : exp(((double)key_to_float((uint32_t)(w >> 32)) - (double)z0) / T);
    fe = to_fx(e);
  }
  if (tid == 0) {
    s_cp = K;
    s_cm = K;
    s_px = 0.0;
    s_qk = kNone;
    s_fr = kNone;
    s_fp = kNone;
    s_pick = kNone;
    s_lastw = -1;
  }
  Fx Ssum;
  const Fx before = fx_excl_w(fe, red, Ssum, W);
  const Fx cum = fx_sum(before, fe);
  if (T == 0.0) {
    if (j == 0) s_cp = 1;
  } else if (p.top_p < 1.0 && j < K) {
    Fx thr = to_fx(p.top_p > 0.0 ? p.top_p * fx_to_double(Ssum) : 0.0);
    if (!fx_nonzero(thr)) thr.lo = 1ull;
    if (fx_ge(cum, thr) && !fx_ge(before, thr)) s_cp = j + 1;
  }
  if (p.min_p > 0.0 && wave < W) {
    const u64 b = __ballot(j >= 1 && j < K && e < p.min_p);
    if (lane == 0 && b) atomicMin(&s_cm, wave * kWave + __ffsll((long long)b) - 1);
  }
  __syncthreads();
  const int kept = min(s_cp, s_cm);
  if (j == kept - 1) s_mass = cum;
  __syncthreads();
  const bool in = j < kept;
  const double pj = in ? e / fx_to_double(s_mass) : 0.0;
  if (p.out_ids && j < K) {   // the support: kept entries whose p' is positive in fp64
    const bool sup = in && pj > 0.0;
    p.out_ids[(size_t)row * K + j] = sup ? idj : -1;
    p.out_probs[(size_t)row * K + j] = sup ? (float)pj : 0.0f;
  }
  if (draft_row) {
    if (in && idj == x) s_px = pj;
    if (!p.q)
      for (int k = tid; k < p.Kq; k += kOneThreads)
        if (qid[k] == x) atomicMin(&s_qk, k);
  }
  // (4) the draw this row would make, in index order over its support: the
  // residual max(0, p' - q) for a draft row (p' if that is all zero), else
  // p'; as samp_draw
  const bool residual = draft_row;
  if (in) {
    double qj = 0.0;
    if (residual) {
      if (p.q) {
        qj = (double)qpre;
      } else {
        for (int k = 0; k < p.Kq; ++k)
          if (qid[k] == idj) {
            qj = (double)qpr[k];
            break;
          }
      }
    }
    eR[j] = e;
    pR[j] = pj;
    qR[j] = qj;
    idR[j] = idj;
    Sa[j] = ((u64)(0xFFFFFFFFu - (uint32_t)idj) << 32) | (uint32_t)j;
  }
  const u64 *byid = sort_desc(Sa, Ls, kept);
  const int s = tid;
  int ids = -1;
  double dres = 0.0, dp = 0.0;
  Fx wr = fx_zero(), we = fx_zero();
  if (s < kept) {
    const int jj = (int)(uint32_t)byid[s];
    ids = idR[jj];
    dp = pR[jj];
    we = to_fx(eR[jj]);
    if (residual) {
      const double d = dp - qR[jj];
      dres = d > 0.0 ? d : 0.0;
      wr = to_fx(dres);
    }
  }
  if (wave < W) {
    const u64 b0 = __ballot(dres > 0.0), b1 = __ballot(dp > 0.0);
    if (lane == 0) {
      if (b0) atomicMin(&s_fr, wave * kWave + __ffsll((long long)b0) - 1);
      if (b1) atomicMin(&s_fp, wave * kWave + __ffsll((long long)b1) - 1);
    }
  }
  __syncthreads();
  // the residual is used when any of its fp64 weights is positive, even if
  // all of them are below the fixed-point resolution
  const bool use_res = residual && s_fr != kNone;
  const Fx w = use_res ? wr : we;
  Fx Wt;
  const Fx bef = fx_excl_w(w, red, Wt, W);
  const Fx target = to_fx(ub * fx_to_double(Wt));
  if (!fx_nonzero(target)) {
    // below 2^-100: u = 0 takes the first positive weight; another target
    // follows the fp64 definition in index order, summed by one thread
    if (tid == 0) {
      int slot = use_res ? s_fr : s_fp;
      if (ub != 0.0) {
        auto wgt = [&](int k) {
          const int jj = (int)(uint32_t)byid[k];
          if (!use_res) return pR[jj];
          const double d = pR[jj] - qR[jj];
          return d > 0.0 ? d : 0.0;
        };
        double Wd = 0.0;
        int last = -1;
        for (int k = 0; k < kept; ++k) {
          const double wk = wgt(k);
          Wd += wk;
          if (wk > 0.0) last = k;
        }
        const double tt = ub * Wd;
        double cm = 0.0;
        slot = last;
        for (int k = 0; k < kept; ++k) {
          cm += wgt(k);
          if (cm > tt) {
            slot = k;
            break;
          }
        }
      }
      s_pick = (slot >= 0 && slot < kept) ? idR[(int)(uint32_t)byid[slot]] : p.V - 1;
    }
  } else if (wave < W) {
    if (s < kept && fx_gt(fx_sum(bef, w), target) && !fx_gt(bef, target)) s_pick = ids;
    const u64 b = __ballot(s < kept && fx_nonzero(w));
    if (lane == 0 && b) atomicMax(&s_lastw, wave * kWave + 63 - __clzll((long long)b));
  }
  __syncthreads();
  // (5) the row's verdict and token; the last row of the sequence to finish
  // writes the sequence's outputs
  if (tid == 0) {
    int pick = s_pick;
    if (pick == kNone)   // rounding passed the end: the last positive weight
      pick = s_lastw >= 0 ? idR[(int)(uint32_t)byid[s_lastw]] : p.V - 1;
    bool reject = false;
    if (draft_row) {
      double qx = 0.0;
      if (xvalid) qx = p.q ? s_qx : (s_qk != kNone ? (double)qpr[s_qk] : 0.0);
      const double px = xvalid ? s_px : 0.0;
      reject = !((double)p.u[(int64_t)seq * p.M + pos] * qx < px);
    }
    st_ag(p.res + row, ((u64)(reject ? 1u : 0u) << 31) | (u64)(uint32_t)pick);
    __builtin_amdgcn_s_waitcnt(0);
    s_last = add_ag32(p.seqcnt + seq) == (uint32_t)(p.M - 1);
  }
  __syncthreads();
  if (s_last && wave == 0) samp_commit(p, seq);
}

}  // namespace

size_t accept_ws_bytes(int M, int V) { return layout(M, V).bytes; }

namespace {

// The two greedy kernels on the per-block partial maxima pv/pj (M x nb each).
hipError_t launch_greedy_parts(const float *logits, int M, int V, int64_t ldl,
                               const int32_t *drafts, int64_t base_len, int32_t *tokens,
                               int32_t *counts, int64_t *rollback, float *pv, int *pj,
                               hipStream_t stream) {
  const int nb = blocks_per_row(V);
  const int chunk = (V + nb - 1) / nb;
  hipLaunchKernelGGL(greedy_partial, dim3(nb, M), dim3(kBlock), 0, stream, logits, ldl, V, nb,
                     chunk, pv, pj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_final, dim3(1), dim3(kFinalThreads), 0, stream, pv, pj, M, nb, drafts,
                     base_len, tokens, counts, rollback);
  return hipGetLastError();
}

// ---- greedy acceptance without a caller workspace ----------------------------
//
// For callers that cannot allocate (graph capture, fixed serving loops): the
// partial maxima live in this file-scope device array, one copy per GPU, kept
// until the process ends; every call on a GPU overwrites its copy before
// reading it, so nothing needs clearing, and calls that overlap on one GPU
// race on it.  In host code the array's name stands for a host-side shadow,
// not a device address: its device address is looked up once per device
// (with that device current) and only that address reaches the kernels.
constexpr size_t kStaticScratchBytes = 2 * sizeof(float) * kMaxRows * kMaxBlocksPerRow;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void *addr[kMaxDevices];
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_accept_greedy(const float *logits, int M, int V, int64_t ldl,
                                const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                int32_t *counts, int64_t *rollback, void *ws, hipStream_t stream) {
  const Layout L = layout(M, V);
  const int nb = blocks_per_row(V);
  uint8_t *w = static_cast<uint8_t *>(ws);
  float *pv = reinterpret_cast<float *>(w + L.gpart);
  int *pj = reinterpret_cast<int *>(pv + (size_t)M * nb);
  return launch_greedy_parts(logits, M, V, ldl, drafts, base_len, tokens, counts, rollback, pv,
                             pj, stream);
}

size_t greedy_static_bytes(int M, int V) { return 2 * sizeof(float) * (size_t)M * blocks_per_row(V); }

size_t greedy_static_max_bytes() { return kStaticScratchBytes; }

hipError_t launch_accept_greedy_static(const float *logits, int M, int V, int64_t ldl,
                                       const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                       int32_t *counts, int64_t *rollback, hipStream_t stream) {
  if (greedy_static_bytes(M, V) > kStaticScratchBytes) return hipErrorInvalidValue;
  void *p = nullptr;
  const hipError_t e = scratch_address(&p);
  if (e != hipSuccess) return e;
  float *pv = static_cast<float *>(p);
  int *pj = reinterpret_cast<int *>(pv + (size_t)M * blocks_per_row(V));
  return launch_greedy_parts(logits, M, V, ldl, drafts, base_len, tokens, counts, rollback, pv,
                             pj, stream);
}

hipError_t launch_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                                   const float *q, int64_t ldq, const int32_t *drafts,
                                   const float *u, float temperature, float top_p,
                                   int64_t base_len, int32_t *tokens, int32_t *counts,
                                   int64_t *rollback, void *ws, hipStream_t stream) {
  const Layout L = layout(M, V);
  uint8_t *w = static_cast<uint8_t *>(ws);
  RejArgs p;
  p.z = logits; p.ldl = ldl; p.q = q; p.ldq = ldq; p.drafts = drafts; p.u = u;
  p.T = (double)temperature; p.top_p = (double)top_p;
  p.M = M; p.V = V; p.nb = blocks_per_row(V); p.chunk = (V + p.nb - 1) / p.nb;
  p.nbd = draw_blocks(V); p.chunkd = (V + p.nbd - 1) / p.nbd;
  p.base_len = base_len; p.tokens = tokens; p.counts = counts; p.rollback = rollback;
  p.maxp = reinterpret_cast<float *>(w + L.maxp);
  p.zmax = reinterpret_cast<float *>(w + L.zmax);
  p.hist = reinterpret_cast<u64 *>(w + L.hist);
  p.total = reinterpret_cast<u64 *>(w + L.total);
  p.sel = reinterpret_cast<SelState *>(w + L.sel);
  p.rows = reinterpret_cast<RowState *>(w + L.rows);
  p.acc = reinterpret_cast<AccIn *>(w + L.acc);
  p.blk = reinterpret_cast<u64 *>(w + L.blk);
  p.hdr = reinterpret_cast<u64 *>(w + L.hdr);
  p.ahist = reinterpret_cast<double *>(w + L.ahist);
  p.above = reinterpret_cast<u64 *>(w + L.above);
  p.ccount = reinterpret_cast<int32_t *>(w + L.ccount);
  p.acount = reinterpret_cast<int32_t *>(w + L.acount);
  p.asec = reinterpret_cast<u64 *>(w + L.asec);
  p.cand = reinterpret_cast<u64 *>(w + L.cand);
  p.wsum = reinterpret_cast<u64 *>(w + L.wsum);
  p.G = one_blocks_per_row(M, V);
  p.C = p.G ? (V + p.G - 1) / p.G : 0;
  if (p.G > 0) {
    // one launch: every row's chunks resident in LDS, the steps separated by
    // per-row meeting points (rej_one)
    static std::once_flag lds_once;
    std::call_once(lds_once, [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(rej_one),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                one_dyn_bytes(kOneChunk));
      (void)hipGetLastError();   // a refusal shows up as the launch's own error
    });
    hipLaunchKernelGGL(rej_one, dim3(M * p.G), dim3(kOneThreads), (size_t)one_dyn_bytes(p.C),
                       stream, p);
    return hipGetLastError();
  }
  const dim3 rows_grid(p.nb, M);
  hipLaunchKernelGGL(rej_rowmax, rows_grid, dim3(kBlock), 0, stream, p);
  const int with_hist = (p.top_p < 1.0) ? 1 : 0;
  const int passes = with_hist ? 4 : 1;
  for (int pass = 0; pass < passes; ++pass)
    hipLaunchKernelGGL(rej_pass, rows_grid, dim3(kBlock), 0, stream, p, pass, with_hist);
  hipLaunchKernelGGL(rej_select, dim3(M), dim3(kBlock), 0, stream, p);
  hipLaunchKernelGGL(rej_draw_sums, dim3(p.nbd), dim3(kBlock), 0, stream, p);
  hipLaunchKernelGGL(rej_draw_pick, dim3(1), dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

// ---- sampled acceptance: host side -------------------------------------------

namespace {

struct SampLayout {
  int G, C;   // samp_one's workgroups per row and chunk (G == 0: the chained kernels)
  size_t zp, hcnt, sel, bcnt, lid, lz, sid, sp, se, nkept, acc, info, cand, res, bytes;
};

// Workgroups per row of samp_one, or 0 for the chained kernels: the rows
// spread over the compute units as for rej_one (chunks of at most
// kOneChunk entries), while the rows' expected candidates (about K + 16 a
// workgroup) stay within kSCandBudget and the counters fit the head.
int samp_one_blocks(int B, int M, int V, int K) {
  const int64_t rows = (int64_t)B * M;
  if (rows > kSMaxRows || B > kSMaxSeqs || M > kWave) return 0;
  int G = std::max((V + kOneChunk - 1) / kOneChunk,
                   std::min(std::max(1, kMaxOneBlocks / (int)rows), (V + 1023) / 1024));
  const int C = (V + G - 1) / G;
  G = (V + C - 1) / C;   // no empty chunk
  if (G > kSMaxG || (int64_t)G * (K + 16) > kSCandBudget) return 0;
  return G;
}

// Head (offset 0, the same for every shape): samp_one's row and sequence
// counters, zero before first use and after every call.  The per-call
// regions of samp_one and of the chained kernels follow it (one or the
// other).
constexpr size_t kSHeadBytes = sizeof(uint32_t) * (kSMaxRows + kSMaxSeqs);
static_assert(kSHeadBytes % 256 == 0, "regions stay 256-byte aligned");

SampLayout samp_layout(int B, int M, int V, int top_k, bool penalties) {
  const size_t rows = (size_t)B * M, K = (size_t)std::min(top_k, V);
  const size_t nb = (size_t)blocks_per_row(V);
  SampLayout L{};
  L.G = samp_one_blocks(B, M, V, (int)K);
  L.C = L.G ? (V + L.G - 1) / L.G : 0;
  size_t o = kSHeadBytes;
  auto take = [&](size_t n) {
    size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  if (L.G) {
    L.info = take(sizeof(u64) * rows * L.G);
    L.cand = take(sizeof(u64) * rows * L.G * L.C);
    L.res = take(sizeof(u64) * rows);
  } else {
    L.zp = take(penalties ? sizeof(float) * rows * V : 0);
    L.hcnt = take(sizeof(uint32_t) * 4 * rows * kBins);
    L.sel = take(sizeof(SelState) * 4 * rows);
    L.bcnt = take(sizeof(uint32_t) * 2 * rows * nb);
    L.lid = take(sizeof(int32_t) * rows * K);
    L.lz = take(sizeof(float) * rows * K);
    L.sid = take(sizeof(int32_t) * rows * K);
    L.sp = take(sizeof(double) * rows * K);
    L.se = take(sizeof(double) * rows * K);
    L.nkept = take(sizeof(int32_t) * rows);
    L.acc = take(sizeof(AccIn) * rows);
  }
  L.bytes = o;
  return L;
}

}  // namespace

size_t sampled_ws_bytes(int B, int M, int V, int top_k, bool penalties) {
  return samp_layout(B, M, V, top_k, penalties).bytes;
}

hipError_t launch_accept_sampled(const SampledCall &c, void *ws, hipStream_t stream) {
  const bool pen = c.penalty_last_n > 0 &&
                   (c.repeat_penalty != 1.0f || c.presence_penalty != 0.0f ||
                    c.frequency_penalty != 0.0f);
  const SampLayout L = samp_layout(c.B, c.M, c.V, c.top_k, pen);
  uint8_t *w = static_cast<uint8_t *>(ws);
  SampArgs p;
  p.z = c.logits; p.ldl = c.ldl;
  p.zp = pen ? reinterpret_cast<float *>(w + L.zp) : nullptr;
  p.htok = c.history; p.hlen = c.history_len; p.ldh = c.ldh;
  p.drafts = c.drafts;
  p.q = c.q; p.ldq = c.ldq; p.qi = c.q_ids; p.qp = c.q_probs; p.Kq = c.Kq;
  p.u = c.uniforms; p.base_len = c.base_len;
  p.T = (double)c.temperature; p.top_p = (double)c.top_p; p.min_p = (double)c.min_p;
  p.rp = c.repeat_penalty; p.pp = c.presence_penalty; p.fq = c.frequency_penalty;
  p.last_n = c.penalty_last_n;
  p.B = c.B; p.M = c.M; p.V = c.V; p.K = std::min(c.top_k, c.V);
  p.nb = blocks_per_row(c.V); p.chunk = (c.V + p.nb - 1) / p.nb;
  p.tokens = c.tokens; p.counts = c.counts; p.rollback = c.rollback;
  p.out_ids = c.out_ids; p.out_probs = c.out_probs;
  const int rows = c.B * c.M;
  if (L.G) {
    p.G = L.G;
    p.C = L.C;
    p.pen = pen ? 1 : 0;
    p.zp = nullptr;
    p.rowcnt = reinterpret_cast<uint32_t *>(w);
    p.seqcnt = p.rowcnt + kSMaxRows;
    p.info = reinterpret_cast<u64 *>(w + L.info);
    p.cand = reinterpret_cast<u64 *>(w + L.cand);
    p.res = reinterpret_cast<u64 *>(w + L.res);
    // first-round slots per segment: a power of two, at most C, all G
    // segments' slots within kSSlotPer loads a thread, room for K and more
    int kc = 1, lkc = 0;
    while (kc * 2 <= L.C && (int64_t)L.G * kc * 2 <= kSSlotPer * kOneThreads &&
           kc < p.K + 64) {
      kc *= 2;
      ++lkc;
    }
    p.lkc = lkc;
    static std::once_flag samp_once;
    std::call_once(samp_once, [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(samp_one),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kSDyn);
    });
    hipLaunchKernelGGL(samp_one, dim3(rows * L.G), dim3(kOneThreads), kSDyn, stream, p);
    return hipGetLastError();
  }
  p.hcnt = reinterpret_cast<uint32_t *>(w + L.hcnt);
  p.sel = reinterpret_cast<SelState *>(w + L.sel);
  p.bcnt = reinterpret_cast<uint32_t *>(w + L.bcnt);
  p.lid = reinterpret_cast<int32_t *>(w + L.lid);
  p.lz = reinterpret_cast<float *>(w + L.lz);
  p.sid = reinterpret_cast<int32_t *>(w + L.sid);
  p.sp = reinterpret_cast<double *>(w + L.sp);
  p.se = reinterpret_cast<double *>(w + L.se);
  p.nkept = reinterpret_cast<int32_t *>(w + L.nkept);
  p.acc = reinterpret_cast<AccIn *>(w + L.acc);
  const dim3 grid(p.nb, rows);
  hipLaunchKernelGGL(samp_prep, grid, dim3(kBlock), 0, stream, p);
  for (int pass = 0; pass < 4; ++pass)
    hipLaunchKernelGGL(samp_count, grid, dim3(kBlock), 0, stream, p, pass);
  hipLaunchKernelGGL(samp_compact_count, grid, dim3(kBlock), 0, stream, p);
  hipLaunchKernelGGL(samp_compact_write, grid, dim3(kBlock), 0, stream, p);
  // one thread per kept entry (a power of two, at least a wave)
  int nt = kWave;
  while (nt < p.K) nt <<= 1;
  hipLaunchKernelGGL(samp_row, dim3(rows), dim3(nt), 0, stream, p);
  hipLaunchKernelGGL(samp_draw, dim3(c.B), dim3(nt), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mtp
