// The streaming engine of the verify GEMM (gfx950, wave64), shared by the
// dense and the MoE kernels.
//
// Weights are read in the packed layout produced by mtp_pack_weights (see
// mtp_verify.h): one 2304-byte block per (16-row tile, 256-wide K pair)
// holds the codes of two 128-wide K steps (64 lanes x 16 B each) followed by
// all of their block scales.  Every load a wave issues is 1 KiB (codes) or
// 256 B (scales) of contiguous memory, and one tile's K range is one
// contiguous run of blocks.
//
// Work split.  The K range of a matrix is cut into S slices of ppj pairs; the
// slices, and the order in which their partial sums are added (slice 0 first),
// depend only on the matrix shape, never on the row count, so a row's result
// does not depend on which other rows share the pass.  A workgroup has
// TW x J waves: TW tiles, each with J consecutive slices (one per wave); KG
// workgroups cover the S slices of a tile group.  A workgroup stages the
// activation rows of its K range in LDS once (the x loads are issued before
// the weight prefetch so they return first), then every wave streams its
// (tile, slice) blocks with PP blocks of loads in flight, decodes each
// weight once and feeds the matrix cores for all rows at once.  A workgroup
// may process several tile groups in turn; its load stream runs on across
// tile-group boundaries.  The J slices of a tile meet in LDS; with KG > 1 the
// slice partials go to the workspace and the last workgroup of the tile group
// to arrive adds all S of them in slice order.  With one slice per tile in
// the workgroup (J == 1, KG == 1) a wave may instead finish its own tiles
// (LOCAL), with no LDS round trip or barrier between tile groups, and may
// then stream two tiles at once (NT == 2) so that one wave holds e.g. the
// matching gate and up columns of a gated MLP.
#pragma once

#include "../../include/mtp_verify.h"
#include "device.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace mtp {
namespace eng {

constexpr int kPairK = 256;
constexpr int kPairBytes = 2304;
constexpr int kHalfBytes = 1024;
constexpr int kScaleOff = 2048;
constexpr int kSlotBytes = 512;   // one pair of one activation row in LDS (256 bf16)
constexpr int kPPShallow = 2;     // blocks in flight per wave: workgroups with many tile groups
constexpr int kPPDeep = 4;        // ... one tile group per workgroup (one 8-wave workgroup per CU)
constexpr int kMaxWaves = 16;         // waves of all workgroups on one CU (<= 128 VGPRs)
constexpr int kWgWaves = 8;           // compute waves of one workgroup at most
constexpr int kMaxThreads = kWgWaves * kWave;
constexpr int kXU = 12;           // activation staging rounds in flight at once
constexpr int kMaxLds = 160 * 1024;

__host__ __device__ inline int tiles_of(int N) { return (N + 15) / 16; }
__host__ __device__ inline int pairs_of(int K) { return (K + kPairK - 1) / kPairK; }
__host__ __device__ inline size_t packed_bytes(int N, int K) {
  return (size_t)tiles_of(N) * pairs_of(K) * kPairBytes;
}

// LDS layout of a workgroup: M staged rows of np pairs plus a zero slot each,
// the Q4_0 accumulator starts, and one wave-sized slot per wave for the slice
// partials (the first TW slots then hold the summed tiles).
__host__ __device__ inline int row_bytes(int np) { return (np + 1) * kSlotBytes + 16; }
__host__ __device__ inline int cinit_floats(int format, int np) {
  return format == MTP_FMT_Q4_0 ? (np + 1) * 8 * 16 : 0;
}
__host__ __device__ inline size_t lds_bytes(int format, int M, int np, int TW, int J) {
  return (size_t)M * row_bytes(np) + (size_t)cinit_floats(format, np) * 4 +
         (size_t)(TW * J) * kWave * 16;
}

// Lets `kernel` use more than 64 KiB of dynamic LDS (once per kernel: the
// kernels that were set up are remembered by address).
template <typename Kernel>
inline void allow_large_lds(Kernel *kernel) {
  static std::mutex mu;
  static std::vector<const void *> done;
  const void *k = reinterpret_cast<const void *>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  if (std::find(done.begin(), done.end(), k) != done.end()) return;
  (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds - 1024);
  (void)hipGetLastError();   // a refusal shows up as the launch's own error
  done.push_back(k);
}

// Activation rows: row m is base + (idx[m] / div) * ld (idx == nullptr: m).
// idx may point to global memory or LDS.
struct XSource {
  const uint16_t *base;
  int64_t ld;
  const int32_t *idx;
  int div;
  __device__ __forceinline__ const uint16_t *row(int m) const {
    return base + (int64_t)(idx ? idx[m] / div : m) * ld;
  }
};

// How one workgroup walks the matrix.
struct Plan {
  int TW, J;       // tiles per workgroup, slices per tile in the workgroup
  int S, ppj;      // slices of the K range and pairs per slice
  int KG, kg;      // workgroups per tile group and this one's K group
  int tg_first, tg_step, tg_count;  // tile groups of this workgroup
};

// Cross-workgroup partial sums (KG > 1): part[(tile * S + slice) * 64 + lane]
// and one arrival counter per tile group, zero between calls.
struct Fixup {
  f32x4 *part;
  uint32_t *cnt;
};

// One wave's share of one block: 2 x 16 code bytes + the scales.
template <int FMT> struct Blk;
template <> struct Blk<MTP_FMT_NVFP4> {
  u32x4 c0, c1;
  uint32_t s;   // E4M3 bytes: step 0 (k0, k0+16), step 1 (k1, k1+16)
};
template <> struct Blk<MTP_FMT_Q4_0> {
  u32x4 c0, c1;
  u32x4 s;      // the 8 fp16 scales of the lane's row for this pair
};

// Weights are read through a buffer window per block: a window of one
// block's bytes, or an empty window whose loads return zeros without a memory
// access (blocks past a slice or past the matrix).  The loads are streaming
// (non-temporal): weights are read once per pass and must not displace the
// activations and partial sums in the caches.
using Window = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit untyped data, gfx9 family
constexpr int kLoadNT = 2;               // cache policy: non-temporal
constexpr uint32_t kXWindow = 0x80000000u;  // activation window bytes (offsets past it read 0)

__device__ __forceinline__ Window block_window(const uint8_t *p, bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p), 0, valid ? kPairBytes : 0,
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 win_load16(Window w, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w, off, 0, kLoadNT));
}

__device__ __forceinline__ void load_blk(Blk<MTP_FMT_NVFP4> &b, Window w, int lane) {
  b.c0 = win_load16(w, 16 * lane);
  b.c1 = win_load16(w, kHalfBytes + 16 * lane);
  b.s = __builtin_amdgcn_raw_buffer_load_b32(w, kScaleOff + 4 * lane, 0, kLoadNT);
}

__device__ __forceinline__ void load_blk(Blk<MTP_FMT_Q4_0> &b, Window w, int lane) {
  b.c0 = win_load16(w, 16 * lane);
  b.c1 = win_load16(w, kHalfBytes + 16 * lane);
  b.s = win_load16(w, kScaleOff + 16 * (lane & 15));
}

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// nvfp4.  Lane (r, g) holds, for step h, the codes of k = 128h + 32g .. +31
// of its row; code dword j meets the activation slots 128h + 32g + 8j .. +7,
// which the same lane supplies for activation row r in MFMA j of the step.
__device__ __forceinline__ f32x4 compute_blk(f32x4 acc, const Blk<MTP_FMT_NVFP4> &b,
                                             const uint8_t *xl, const float *) {
  const float s0 = e4m3_to_f32<0>(b.s), s1 = e4m3_to_f32<1>(b.s);
  const float s2 = e4m3_to_f32<2>(b.s), s3 = e4m3_to_f32<3>(b.s);
  const u32x4 *xa = reinterpret_cast<const u32x4 *>(xl);
  const u32x4 *xb = reinterpret_cast<const u32x4 *>(xl + 256);
  acc = mfma_16x16x32(xa[0], nvfp4_decode8(b.c0.x, s0), acc);
  acc = mfma_16x16x32(xa[1], nvfp4_decode8(b.c0.y, s0), acc);
  acc = mfma_16x16x32(xa[2], nvfp4_decode8(b.c0.z, s1), acc);
  acc = mfma_16x16x32(xa[3], nvfp4_decode8(b.c0.w, s1), acc);
  acc = mfma_16x16x32(xb[0], nvfp4_decode8(b.c1.x, s2), acc);
  acc = mfma_16x16x32(xb[1], nvfp4_decode8(b.c1.y, s2), acc);
  acc = mfma_16x16x32(xb[2], nvfp4_decode8(b.c1.z, s3), acc);
  acc = mfma_16x16x32(xb[3], nvfp4_decode8(b.c1.w, s3), acc);
  return acc;
}

// The same on fp16 activations (staged as fp16), with an fp16 decode.
__device__ __forceinline__ f32x4 compute_blk_f16(f32x4 acc, const Blk<MTP_FMT_NVFP4> &b,
                                                 const uint8_t *xl) {
  const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.s, 1.0f, false);
  const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.s, 1.0f, true);
  const f16x2 h0 = {s01.x, s01.x}, h1 = {s01.y, s01.y}, h2 = {s23.x, s23.x}, h3 = {s23.y, s23.y};
  const u32x4 *xa = reinterpret_cast<const u32x4 *>(xl);
  const u32x4 *xb = reinterpret_cast<const u32x4 *>(xl + 256);
  acc = mfma_16x16x32_f16(xa[0], nvfp4_decode8_f16(b.c0.x, h0), acc);
  acc = mfma_16x16x32_f16(xa[1], nvfp4_decode8_f16(b.c0.y, h0), acc);
  acc = mfma_16x16x32_f16(xa[2], nvfp4_decode8_f16(b.c0.z, h1), acc);
  acc = mfma_16x16x32_f16(xa[3], nvfp4_decode8_f16(b.c0.w, h1), acc);
  acc = mfma_16x16x32_f16(xb[0], nvfp4_decode8_f16(b.c1.x, h2), acc);
  acc = mfma_16x16x32_f16(xb[1], nvfp4_decode8_f16(b.c1.y, h2), acc);
  acc = mfma_16x16x32_f16(xb[2], nvfp4_decode8_f16(b.c1.z, h3), acc);
  acc = mfma_16x16x32_f16(xb[3], nvfp4_decode8_f16(b.c1.w, h3), acc);
  return acc;
}

// (Q4_0 has no fp16 path; this declaration only satisfies the discarded branch.)
template <typename B>
__device__ f32x4 compute_blk_f16(f32x4 acc, const B &b, const uint8_t *xl);

// Q4_0.  One MFMA per 32-block: lane (r, g) supplies slots 8g .. 8g+7 of
// block q of the pair (code dword q % 4 of step q / 4), activations staged in
// the matching (0,4,1,5,2,6,3,7) order.  The accumulator starts at
// -136 * sum(x) of the block, which turns the exact operands 128 + u into
// u - 8; the fp16 block scale is applied in fp32 afterwards.
__device__ __forceinline__ f32x4 q4_block(f32x4 acc, uint32_t codes, float d, const uint8_t *xl,
                                          const float *ci) {
  const u32x4 a = *reinterpret_cast<const u32x4 *>(xl);
  const f32x4 c0 = *reinterpret_cast<const f32x4 *>(ci);
  const f32x4 p = mfma_16x16x32(a, q4_decode8_offset128(codes), c0);
  acc.x = __builtin_fmaf(d, p.x, acc.x);
  acc.y = __builtin_fmaf(d, p.y, acc.y);
  acc.z = __builtin_fmaf(d, p.z, acc.z);
  acc.w = __builtin_fmaf(d, p.w, acc.w);
  return acc;
}

__device__ __forceinline__ f32x4 compute_blk(f32x4 acc, const Blk<MTP_FMT_Q4_0> &b,
                                             const uint8_t *xl, const float *ci) {
  // scheduling fences between block pairs bound the LDS operands held at once
  acc = q4_block(acc, b.c0.x, half_lo(b.s.x), xl + 0, ci + 0);
  acc = q4_block(acc, b.c0.y, half_hi(b.s.x), xl + 64, ci + 16);
  __builtin_amdgcn_sched_barrier(0);
  acc = q4_block(acc, b.c0.z, half_lo(b.s.y), xl + 128, ci + 32);
  acc = q4_block(acc, b.c0.w, half_hi(b.s.y), xl + 192, ci + 48);
  __builtin_amdgcn_sched_barrier(0);
  acc = q4_block(acc, b.c1.x, half_lo(b.s.z), xl + 256, ci + 64);
  acc = q4_block(acc, b.c1.y, half_hi(b.s.z), xl + 320, ci + 80);
  __builtin_amdgcn_sched_barrier(0);
  acc = q4_block(acc, b.c1.z, half_lo(b.s.w), xl + 384, ci + 96);
  acc = q4_block(acc, b.c1.w, half_hi(b.s.w), xl + 448, ci + 112);
  return acc;
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// Byte offset of lane group g's activation fragment inside a pair slot.
template <int FMT>
__device__ __forceinline__ int x_lane_offset(int g) {
  return (FMT == MTP_FMT_NVFP4) ? 64 * g : 16 * g;
}

// Partial sums cross workgroups (and XCDs) through agent-scope accesses,
// which bypass the per-XCD caches.
__device__ __forceinline__ void agent_store(f32x4 *p, f32x4 v) {
  float *f = reinterpret_cast<float *>(p);
  __hip_atomic_store(f + 0, v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(f + 1, v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(f + 2, v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(f + 3, v.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 agent_load(const f32x4 *p) {
  const float *f = reinterpret_cast<const float *>(p);
  f32x4 v;
  v.x = __hip_atomic_load(f + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.y = __hip_atomic_load(f + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.z = __hip_atomic_load(f + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.w = __hip_atomic_load(f + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// Element (activation row m, column c) of slot tw of the summed tiles.
__device__ __forceinline__ float fin_at(const f32x4 *fin, int tw, int m, int c) {
  return reinterpret_cast<const float *>(fin)[(tw * kWave + (m >> 2) * 16 + c) * 4 + (m & 3)];
}

// Element i (0..3) of a wave's accumulator belongs to activation row
// 4 * (lane / 16) + i and column lane % 16 of the tile.
__device__ __forceinline__ int acc_row(int lane, int i) { return 4 * (lane >> 4) + i; }

// Runs the engine over the tile groups of `pl`.
//   w, T, P   packed matrix with T tiles of P pairs; K its reduction length
//   M, xs     1..16 activation rows
//   tile_of   tile_of(tg, s) -> tile index of slot s of tile group tg, or
//             -1 for a slot past the matrix (nothing is read for it)
//   NT        tiles per wave: wave (tw, j) streams slots NT*tw .. NT*tw+NT-1
//             of each tile group, block by block in turn, into NT sums
//   LOCAL     each wave hands its own sums to epi.wave(tg, tw, acc) (acc:
//             NT accumulators, see acc_row) with no LDS or barrier; needs
//             J == 1 and KG == 1.  Otherwise (NT == 1):
//   epi       epi(tg, fin) is called by every thread of the workgroup once a
//             tile group's sums are final (only by the last-arriving
//             workgroup when KG > 1); fin_at(fin, tw, m, c) is row m of
//             column c (0..15) of slot tw.
// Every thread of the workgroup calls run with the same arguments;
// sync_entry must be true when the workgroup ran the engine before (its LDS
// may still be in use).

template <int FMT, int PP, int NT, bool LOCAL, bool GATHER, typename TileOf, typename Epi>
__device__ __forceinline__ void run(const uint8_t *w, int P, int K, int M, const XSource &xs,
                                    const Plan &pl, const TileOf &tile_of, const Fixup &fx,
                                    uint8_t *lds, bool sync_entry, Epi &&epi) {
  const int nthreads = pl.TW * pl.J * kWave;
  // wave-uniform values are pinned to scalar registers so that branches on
  // them stay scalar branches (no exec-masked both-ways execution)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4, r = lane & 15;
  // TW is a power of two (every caller's plan)
  const int tw = wave & (pl.TW - 1), j = wave >> __builtin_ctz(pl.TW);
  const int pa = pl.kg * pl.J * pl.ppj;               // first pair of the workgroup
  const int np = min(pl.J * pl.ppj, P - pa);          // pairs staged
  const int rowb = row_bytes(np);
  float *cinit = reinterpret_cast<float *>(lds + (size_t)M * rowb);
  f32x4 *red = reinterpret_cast<f32x4 *>(cinit + cinit_floats(FMT, np));
  f32x4 *fin = red;   // slot tw is read only by wave (tw, 0) before it holds the sum
  __shared__ uint32_t last_flag;
  __shared__ uint32_t wave_ovf[kWgWaves];

  // this wave's slice: pairs [pa + js, pa + js + n), n may be 0
  const int js = min(np, j * pl.ppj);
  const int n = min(np, js + pl.ppj) - js;
  static_assert(NT == 1 || (NT == 2 && LOCAL), "two tiles per wave need the wave-local finish");
  static_assert(PP % NT == 0, "a prefetch slot always feeds the same tile");
  // iterations per tile group: whole rounds of PP (the ring slot of a stream
  // position is its index mod PP); positions past the tile's blocks load
  // empty windows and skip the arithmetic
  const int nr = (pl.ppj * NT + PP - 1) / PP * PP;
  const int slice = pl.kg * pl.J + j;

  // load stream: position si of tile group su is block si / NT of the slice
  // of the wave's tile si % NT; positions past the slice, past the matrix or
  // past the last tile group get empty windows
  // (the NT tile ids are two plain scalars, not an array: a select between
  // array elements becomes an indexed private-memory load, whose wait then
  // drains every weight load in flight)
  int su = 0, si = 0;
  int stile0 = -1, stile1 = -1;
  auto tiles_at = [&](int u) {
    const int tg = pl.tg_first + u * pl.tg_step;
    stile0 = __builtin_amdgcn_readfirstlane(tile_of(tg, NT * tw));
    stile1 = NT == 1 ? stile0 : __builtin_amdgcn_readfirstlane(tile_of(tg, NT * tw + NT - 1));
  };
  tiles_at(0);
  auto next_block = [&]() -> Window {
    const int t = (NT == 1 || si % NT == 0) ? stile0 : stile1;
    const int pi = si / NT;
    const bool valid = pi < n && t >= 0;
    const int64_t blk = valid ? ((int64_t)t * P + pa + js + pi) : 0;
    const Window win = block_window(w + blk * kPairBytes, valid);
    if (++si == nr) {
      if (su + 1 < pl.tg_count) {
        si = 0;
        ++su;
        tiles_at(su);
      } else {
        si = nr;   // stays past the slice
      }
    }
    return win;
  };

  if (sync_entry) __syncthreads();  // LDS may still be read by a previous call's epilogue

  // Activations are staged as fp16 for nvfp4 and as bf16 in MFMA slot order
  // for Q4_0.  The fp16 copy is exact when every nonzero staged magnitude
  // lies in [2^-17, 65280] (see bf16x8_to_f16x8).  Otherwise the workgroup
  // restages its activations times a power of two 2^s that brings its
  // largest magnitude just below 2^16, and scales its sums back by 2^-s
  // (every product and partial sum then carries the factor exactly, so the
  // result is that of the unscaled products); if even then a nonzero value
  // would fall below 2^-17, or a value is not finite, it stages bf16 and
  // takes the bf16 path.
  uint32_t xmag = 0, xmnz = 0xFFFFFFFFu;
  auto encode = [&](u32x4 v) -> u32x4 {
    if constexpr (FMT == MTP_FMT_Q4_0) return interleave_halves(v);
    else return bf16x8_to_f16x8(v, xmag, xmnz);
  };

  // 1) activation loads, 2) the first weight block, 3) activation stores to
  // LDS (waiting for the activation loads only), 4) the rest of the
  // prefetch: the activation bytes do not queue behind the weight stream, and
  // the weight stream starts before the staging ends.  (More blocks before
  // the stores only stall the stores behind a full memory queue: with two,
  // three or four the M = 8 launch measured 0.15-0.5 us slower, with none
  // 0.7 us slower.)
  // Vector i = u * nthreads + tid of the staged rows is (m, v) = divmod(i,
  // vpr); (m, v) advance incrementally so that no division sits between the
  // loads.  Only the rounds that hold staged vectors load (xr, the same for
  // every wave); up to kXU rounds are in flight at once, so one memory
  // latency stages every shape but the largest.  Inside a round every load
  // reads a valid address (row 0 / the first staged vector when out of range)
  // so no branch splits them.
  // Q4_0 also needs the accumulator starts -136 * (sum of each 32-block of a
  // row): the four vectors of a block sit in the four lanes of an aligned
  // lane quad (vpr and nthreads are multiples of 4), which add their sums
  // across the quad; rows >= M are never stored, and the zero slot gets 0.
  const int vpr = np * 32;                  // 16-byte vectors per staged row
  const int k0 = pa * kPairK;
  const int rstep = nthreads / vpr, vstep = nthreads - rstep * vpr;
  const int xr = __builtin_amdgcn_readfirstlane((M * vpr + nthreads - 1) / nthreads);
  int xm = threadIdx.x / vpr, xvi = threadIdx.x - xm * vpr;
  // The walk keeps, per thread, (m, v) and the vector's byte offsets: in x
  // (dense rows, from xs.base) and in LDS.  A round advances them by fixed steps with one wrap check,
  // and only rounds below xr run at all.  Rows are read through a buffer
  // window whose loads past its range return zeros, so a vector past K or
  // past the last row needs no separate masking.  Gathered rows (GATHER:
  // xs.idx lists them) take their index from a table that every wave loads
  // once (lane m holds row m's), so no index load sits between the loads of
  // the staging; their byte offsets stay below 2^31 (the callers' row lists
  // index at most 1024 rows of under 2^16 vectors).
  const uint32_t ld2 = (uint32_t)xs.ld * 2u;
  const uint32_t gstep = (uint32_t)rstep * ld2 + (uint32_t)vstep * 16u;
  const uint32_t gwrap = ld2 - (uint32_t)vpr * 16u;           // (mod 2^32)
  const int lstep = rstep * rowb + vstep * 16, lwrap = rowb - vpr * 16;
  const int vk = min(vpr, (K - k0) / 8);                        // vectors of a row inside K
  uint32_t goff = (uint32_t)xm * ld2 + (uint32_t)(k0 + 8 * xvi) * 2u;
  int loff = xm * rowb + xvi * 16;
  int grow = 0;
  if constexpr (GATHER) {
    // (one lane shuffle takes the wait for the table here, in straight-line
    // code: a first use inside the conditional rounds below would wait for
    // every load in flight at each of them)
    grow = __shfl(xs.idx[lane < M ? lane : M - 1] / xs.div, lane);
  }
  const Window xwin = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(xs.base), 0,
                                                        (int)kXWindow, kRsrcWord3);
  auto step = [&]() {   // (selects, not a branch: lanes wrap at different rounds)
    xvi += vstep;
    const bool wrap = xvi >= vpr;
    xvi -= wrap ? vpr : 0;
    xm += rstep + (wrap ? 1 : 0);
    goff += gstep + (wrap ? gwrap : 0u);
    loff += lstep + (wrap ? lwrap : 0);
  };
  auto load_x = [&]() -> u32x4 {
    const bool ok = xm < M && xvi < vk;
    uint32_t off = goff;
    if constexpr (GATHER)
      off = (uint32_t)__shfl(grow, ok ? xm : 0) * ld2 + (uint32_t)(k0 + 8 * xvi) * 2u;
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(xwin, ok ? off : kXWindow, 0, 0));
  };
  // one staged vector: LDS store (rows < M; loff < 0 otherwise) and, for
  // Q4_0, its block sum (c: the accumulator-start index of its block)
  auto stage = [&](u32x4 v, int lo, int c) {
    const u32x4 val = encode(v);
    if (lo >= 0) *reinterpret_cast<u32x4 *>(lds + lo) = val;
    if constexpr (FMT == MTP_FMT_Q4_0) {
      float s = (bf16_to_f32(v.x) + bf16_to_f32(v.x >> 16)) +
                (bf16_to_f32(v.y) + bf16_to_f32(v.y >> 16));
      s += (bf16_to_f32(v.z) + bf16_to_f32(v.z >> 16)) +
           (bf16_to_f32(v.w) + bf16_to_f32(v.w >> 16));
      s += quad_xor1(s);
      s += quad_xor2(s);
      if ((lane & 3) == 0 && lo >= 0) cinit[c] = -136.0f * s;
    }
  };
  // straight-line code for the first kXU rounds (no loop around the loads, so
  // the waits before the stores count only the activation loads)
  u32x4 xv[kXU];
  int xl[kXU], xc[kXU];
#pragma unroll
  for (int u = 0; u < kXU; ++u) {
    if (u < xr) {
      xv[u] = load_x();
      xl[u] = xm < M ? loff : -1;
      xc[u] = (xvi >> 2) * 16 + xm;
      step();
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kEarly = 1;
  Blk<FMT> buf[PP];
#pragma unroll
  for (int i = 0; i < kEarly; ++i) load_blk(buf[i], next_block(), lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < kXU; ++u)
    if (u < xr) stage(xv[u], xl[u], xc[u]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = kEarly; i < PP; ++i) load_blk(buf[i], next_block(), lane);
  __builtin_amdgcn_sched_barrier(0);
  // rounds beyond kXU (only very long staged rows)
  for (int u = kXU; u < xr; ++u) {
    const u32x4 v = load_x();
    stage(v, xm < M ? loff : -1, (xvi >> 2) * 16 + xm);
    step();
  }
  {
    const bool any = __builtin_amdgcn_ballot_w64(f16_unsafe(xmag, xmnz)) != 0ull;
    if (lane == 0) wave_ovf[wave] = any ? 1u : 0u;
  }
  for (int i = threadIdx.x; i < M * 32; i += nthreads) {   // zero slot of every row
    const int m = i >> 5, v = i & 31;
    *reinterpret_cast<u32x4 *>(lds + (size_t)m * rowb + np * kSlotBytes + v * 16) =
        u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (FMT == MTP_FMT_Q4_0)
    for (int i = threadIdx.x; i < 128; i += nthreads) cinit[np * 128 + i] = 0.0f;
  __syncthreads();

  // sum the slices of the tile group and hand it to the epilogue
  auto finish_group = [&](int tg, f32x4 acc) {
    if (pl.KG == 1) {
      // add the J slices of each tile in slice order
      red[wave * kWave + lane] = acc;
      __syncthreads();
      if (j == 0) {
        f32x4 t = red[tw * kWave + lane];
        for (int q = 1; q < pl.J; ++q) t += red[(q * pl.TW + tw) * kWave + lane];
        fin[tw * kWave + lane] = t;
      }
      __syncthreads();
      epi(tg, fin);
    } else {
      const int tile = tile_of(tg, tw);
      if (tile >= 0 && slice < pl.S)
        agent_store(fx.part + ((int64_t)tile * pl.S + slice) * kWave + lane, acc);
      __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are complete
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(fx.cnt + tg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t last = old == (uint32_t)(pl.KG - 1);
        if (last) __hip_atomic_store(fx.cnt + tg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = last;
      }
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(last_flag)) {
        if (j == 0 && tile >= 0) {
          const f32x4 *src = fx.part + (int64_t)tile * pl.S * kWave + lane;
          f32x4 t = agent_load(src);
          for (int q = 1; q < pl.S; ++q) t += agent_load(src + q * kWave);
          fin[tw * kWave + lane] = t;
        }
        __syncthreads();
        epi(tg, fin);
      }
    }
  };

  uint32_t x_ovf = 0;
  if (FMT == MTP_FMT_NVFP4)
    for (int q = 0; q < nthreads / kWave; ++q) x_ovf |= wave_ovf[q];
  bool use_f16 = FMT == MTP_FMT_NVFP4;
  float xinv = 1.0f;   // 2^-s: takes the staging scale back out of the sums
  if (FMT == MTP_FMT_NVFP4 && __builtin_amdgcn_readfirstlane(x_ovf)) {
    // workgroup extremes: the largest magnitude pattern and the smallest
    // nonzero one minus 1 (0xFFFF: all zero)
    uint32_t hi = max(xmag & 0xFFFFu, xmag >> 16), lo = min(xmnz & 0xFFFFu, xmnz >> 16);
    for (int off = kWave / 2; off > 0; off >>= 1) {
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    }
    __shared__ uint32_t wave_ext[kWgWaves];
    if (lane == 0) wave_ext[wave] = hi | (lo << 16);
    __syncthreads();
    hi = 0u;
    lo = 0xFFFFu;
    for (int q = 0; q < nthreads / kWave; ++q) {
      hi = max(hi, wave_ext[q] & 0xFFFFu);
      lo = min(lo, wave_ext[q] >> 16);
    }
    // s puts the largest magnitude in [2^15, 2^16); 2^s and 2^-s stay normal
    int s = 0;
    bool scaled = false;
    if (hi < 0x7F80u) {
      s = min(126, 15 - bf16_exponent(hi));
      scaled = lo == 0xFFFFu || bf16_exponent(lo + 1u) + s >= -17;
    }
    use_f16 = scaled;
    const float sc = __builtin_ldexpf(1.0f, s);
    xinv = __builtin_ldexpf(1.0f, -s);
    for (int i = threadIdx.x; i < M * vpr; i += nthreads) {
      const int m = i / vpr, v = i - m * vpr;
      const int k = k0 + v * 8;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (k < K) val = *reinterpret_cast<const u32x4 *>(xs.row(m) + k);
      *reinterpret_cast<u32x4 *>(lds + m * rowb + v * 16) =
          scaled ? bf16x8_to_f16x8_scaled(val, sc) : val;
    }
    __syncthreads();
  }

  const uint8_t *xrow = lds + (size_t)(r % M) * rowb + x_lane_offset<FMT>(g);
  const float *crow = cinit + 4 * g;
  auto tile_groups = [&](auto f16_tag) {
    constexpr bool kF16 = decltype(f16_tag)::value;
    for (int u = 0; u < pl.tg_count; ++u) {
      const int tg = pl.tg_first + u * pl.tg_step;
      f32x4 acc[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int b0 = 0; b0 < nr; b0 += PP) {
#pragma unroll
        for (int i = 0; i < PP; ++i) {
          // the branch holds no memory loads, so the waits before each
          // block still count the loads of the blocks behind it
          const int pi = (b0 + i) / NT;
          if (pi < n) {
            const int slot = js + pi;
            f32x4 &a = acc[i % NT];
            if constexpr (kF16) a = compute_blk_f16(a, buf[i], xrow + slot * kSlotBytes);
            else a = compute_blk(a, buf[i], xrow + slot * kSlotBytes, crow + slot * 128);
          }
          load_blk(buf[i], next_block(), lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (kF16) {
#pragma unroll
        for (int q = 0; q < NT; ++q) acc[q] *= xinv;
      }
      if constexpr (LOCAL) epi.wave(tg, tw, acc);
      else finish_group(tg, acc[0]);
    }
  };
  if constexpr (FMT == MTP_FMT_NVFP4) {
    if (use_f16) {
      tile_groups(BoolTag<true>{});
    } else {
      tile_groups(BoolTag<false>{});
      // the stream's trailing loads are never consumed; retire them here so
      // that no later code has to assume they are still outstanding
      __builtin_amdgcn_s_waitcnt(0);
    }
  } else {
    tile_groups(BoolTag<false>{});
  }
}

}  // namespace eng
}  // namespace mtp
