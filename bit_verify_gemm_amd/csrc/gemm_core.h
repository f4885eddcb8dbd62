// Tile engine of the verify GEMM, shared by the dense and the MoE kernels.
//
// A workgroup of 4 waves stages up to 16 activation rows in LDS, 1024
// reduction elements at a time; each wave streams NT weight rows per lane
// (NT tiles of 16 output columns), decodes them once per 128-wide K step and
// multiplies them with all staged rows on the matrix cores.
//
// Layouts (see mtp_verify.h): codes [N][K/2] with element k in byte k/2 (low
// nibble for even k); nvfp4 scales E4M3 [N][K/16]; Q4_0 scales fp16 [N][K/32].
#pragma once

#include "../../include/mtp_verify.h"
#include "device.h"

namespace mtp {
namespace core {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStepK = 128;
constexpr int kChunkK = 1024;
constexpr int kChunkSteps = kChunkK / kStepK;
constexpr int kRowBytes = kChunkK * 2 + 16;  // padded LDS row (bank spread)
constexpr int kCinitBytes = (kChunkK / 32) * 16 * 4;
constexpr int kPF = 4;                       // weight prefetch depth (steps)

inline size_t lds_bytes(int M, int format) {
  return (size_t)(M + 1) * kRowBytes + (format == MTP_FMT_Q4_0 ? kCinitBytes : 0);
}

// Activation rows: row m is base + idx[m] * ld (idx == nullptr: m).
struct XSource {
  const uint16_t *base;
  int64_t ld;
  const int32_t *idx;
  __device__ __forceinline__ const uint16_t *row(int m) const {
    return base + (int64_t)(idx ? idx[m] : m) * ld;
  }
};

// Weight matrix rows of one format.
template <int FMT>
__device__ __forceinline__ const void *scale_row(const void *scales, int64_t n, int K) {
  return (FMT == MTP_FMT_NVFP4)
             ? static_cast<const void *>(static_cast<const uint8_t *>(scales) + n * (K / 16))
             : static_cast<const void *>(static_cast<const uint16_t *>(scales) + n * (K / 32));
}

// One lane's share of one 128-wide K step: 16 code bytes plus the scales.
template <int FMT> struct Step;
template <> struct Step<MTP_FMT_NVFP4> {
  u32x4 c;
  uint32_t s;  // two E4M3 bytes: blocks of k .. k+15 and k+16 .. k+31
};
template <> struct Step<MTP_FMT_Q4_0> {
  u32x4 c;
  u32x2 s;     // four fp16 scales: the step's four 32-blocks
};

__device__ __forceinline__ void load_step(Step<MTP_FMT_NVFP4> &d, const uint8_t *crow,
                                          const void *srow, int kb, int k_end, int g, bool) {
  const int kl = kb + 32 * g;
  if (kl < k_end) {
    d.c = *reinterpret_cast<const u32x4 *>(crow + kl / 2);
    d.s = *reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(srow) + kl / 16);
  } else {
    d.c = u32x4{0u, 0u, 0u, 0u};
    d.s = 0u;
  }
}

__device__ __forceinline__ void load_step(Step<MTP_FMT_Q4_0> &d, const uint8_t *crow,
                                          const void *srow, int kb, int k_end, int g,
                                          bool full_rows) {
  const int kl = kb + 32 * g;
  d.c = (kl < k_end) ? *reinterpret_cast<const u32x4 *>(crow + kl / 2) : u32x4{0u, 0u, 0u, 0u};
  const uint16_t *s16 = static_cast<const uint16_t *>(srow) + kb / 32;
  if (full_rows) {
    d.s = *reinterpret_cast<const u32x2 *>(s16);
  } else {
    uint32_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = (kb + 32 * t < k_end) ? (uint32_t)s16[t] : 0u;
    d.s = u32x2{s[0] | (s[1] << 16), s[2] | (s[3] << 16)};
  }
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// nvfp4: lane (r, g) covers k = kb + 32g .. +31 of its row; dword j of its
// codes meets the x slots kb + 32g + 8j .. +7 of MFMA j.
__device__ __forceinline__ f32x4 compute_step(f32x4 acc, const Step<MTP_FMT_NVFP4> &d,
                                              const uint8_t *xl, const float *, int g) {
  const uint8_t *xa = xl + 64 * g;
  const u32x4 a0 = *reinterpret_cast<const u32x4 *>(xa);
  const u32x4 a1 = *reinterpret_cast<const u32x4 *>(xa + 16);
  const u32x4 a2 = *reinterpret_cast<const u32x4 *>(xa + 32);
  const u32x4 a3 = *reinterpret_cast<const u32x4 *>(xa + 48);
  const float s0 = e4m3_to_f32<0>(d.s), s1 = e4m3_to_f32<1>(d.s);
  acc = mfma_16x16x32(a0, nvfp4_decode8(d.c.x, s0), acc);
  acc = mfma_16x16x32(a1, nvfp4_decode8(d.c.y, s0), acc);
  acc = mfma_16x16x32(a2, nvfp4_decode8(d.c.z, s1), acc);
  acc = mfma_16x16x32(a3, nvfp4_decode8(d.c.w, s1), acc);
  return acc;
}

// Q4_0: MFMA t covers the step's block t; lane group g supplies its slots
// 8g .. 8g+7 (x staged in LDS in the matching (0,4,1,5,2,6,3,7) order).
__device__ __forceinline__ f32x4 compute_step(f32x4 acc, const Step<MTP_FMT_Q4_0> &d,
                                              const uint8_t *xl, const float *cinit, int g) {
  uint32_t f[4] = {d.c.x, d.c.y, d.c.z, d.c.w};
  transpose_lane_groups(f[0], f[1], f[2], f[3]);
  const float sc[4] = {half_bits_to_f32(d.s.x), half_bits_to_f32(d.s.x >> 16),
                       half_bits_to_f32(d.s.y), half_bits_to_f32(d.s.y >> 16)};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(xl + 64 * t + 16 * g);
    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cinit + 16 * t + 4 * g);
    const f32x4 p = mfma_16x16x32(a, q4_decode8_offset128(f[t]), c0);
    acc.x = __builtin_fmaf(sc[t], p.x, acc.x);
    acc.y = __builtin_fmaf(sc[t], p.y, acc.y);
    acc.z = __builtin_fmaf(sc[t], p.z, acc.z);
    acc.w = __builtin_fmaf(sc[t], p.w, acc.w);
  }
  return acc;
}

// Copy x rows m < M, columns kc0 .. kc0+kChunkK (zero past K), into LDS; for
// Q4_0 also interleave each group of 8 into slot order and compute the
// per-block accumulator starts -136 * sum(x).
template <int FMT>
__device__ __forceinline__ void stage_chunk(const XSource &xs, int M, int K, uint8_t *lds,
                                            float *cinit, int kc0) {
  constexpr int kVec = kChunkK / 8;
  for (int i = threadIdx.x; i < M * kVec; i += kThreads) {
    const int m = i / kVec, v = i - m * kVec;
    const int k = kc0 + v * 8;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (k < K) val = *reinterpret_cast<const u32x4 *>(xs.row(m) + k);
    if (FMT == MTP_FMT_Q4_0) val = interleave_halves(val);
    *reinterpret_cast<u32x4 *>(lds + m * kRowBytes + v * 16) = val;
  }
  if (FMT == MTP_FMT_Q4_0) {
    __syncthreads();
    for (int i = threadIdx.x; i < (kChunkK / 32) * 16; i += kThreads) {
      const int b = i >> 4, m = i & 15;
      float s = 0.0f;
      if (m < M) {
        const uint16_t *xr = reinterpret_cast<const uint16_t *>(lds + m * kRowBytes) + b * 32;
        for (int j = 0; j < 32; ++j) s += bf16_to_f32(xr[j]);
      }
      cinit[i] = -136.0f * s;
    }
  }
}

// Accumulate x[0..M) . W over k in [k_begin, k_end) for NT weight rows per
// lane.  On return acc[t] holds, for lane (r = lane % 16, g = lane / 16),
// rows m = 4g .. 4g+3 of output column r of tile t.  Every thread of the
// workgroup must call this with the same M, K and K-range (it synchronises).
template <int FMT, int NT>
__device__ __forceinline__ void run_tiles(f32x4 (&acc)[NT], const uint8_t *const (&crow)[NT],
                                          const void *const (&srow)[NT], const XSource &xs,
                                          int M, int K, int k_begin, int k_end, uint8_t *lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = (k_end - k_begin + kStepK - 1) / kStepK;
  const bool full_rows = (K % kStepK) == 0;
  float *cinit = reinterpret_cast<float *>(lds + (M + 1) * kRowBytes);
  const uint8_t *xlane = lds + ((r < M) ? r : M) * kRowBytes;

  __syncthreads();  // LDS may still be in use by a previous call
  for (int i = threadIdx.x; i < kRowBytes / 16; i += kThreads)
    *reinterpret_cast<u32x4 *>(lds + M * kRowBytes + i * 16) = u32x4{0u, 0u, 0u, 0u};

  Step<FMT> buf[NT][kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i)
    if (i < nsteps)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        load_step(buf[t][i], crow[t], srow[t], k_begin + i * kStepK, k_end, g, full_rows);

#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s0 = 0; s0 < nsteps; s0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      const int st = s0 + i;
      if (st < nsteps) {
        const int kk = (st % kChunkSteps) * kStepK;
        if (kk == 0) {
          __syncthreads();
          stage_chunk<FMT>(xs, M, K, lds, cinit, k_begin + st * kStepK);
          __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const Step<FMT> cur = buf[t][i];
          if (st + kPF < nsteps)
            load_step(buf[t][i], crow[t], srow[t], k_begin + (st + kPF) * kStepK, k_end, g,
                      full_rows);
          acc[t] = compute_step(acc[t], cur, xlane + kk * 2, cinit + (kk / 32) * 16, g);
        }
      }
    }
  }
}

}  // namespace core
}  // namespace mtp
