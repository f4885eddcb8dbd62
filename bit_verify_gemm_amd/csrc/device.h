// Device-side building blocks shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// D = A(16x32) * B(32x16) + C on the matrix cores.  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, eight consecutive reduction slots
// 8*(l/16) .. 8*(l/16)+7 each; it receives D[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The same product on fp16 operands (same lane layout).
__device__ __forceinline__ f32x4 mfma_16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float((h & 0xFFFFu) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values whose low 16 bits are zero -> packed bf16 pair (exact).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// E4M3 ("FN", bias 7) byte `sel` of `v` -> fp32 (hardware conversion).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, SEL);
}

// Eight E2M1 codes (one dword, element i in nibble i) times an fp32 scale
// -> eight bf16 values in element order.  E2M1 x E4M3 products carry at most
// six significant bits, so every result is exact in bf16.
__device__ __forceinline__ u32x4 nvfp4_decode8(uint32_t codes, float scale) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  u32x4 r;
  r.x = pack_hi16(p0.x * scale, p0.y * scale);
  r.y = pack_hi16(p1.x * scale, p1.y * scale);
  r.z = pack_hi16(p2.x * scale, p2.y * scale);
  r.w = pack_hi16(p3.x * scale, p3.y * scale);
  return r;
}

// Eight E2M1 codes times an E4M3 scale held as fp16 in both halves of `s2`
// -> eight fp16 values in element order.  The products carry at most six
// significant bits and lie in [2^-10, 2688], so every result is exact in
// fp16; the hardware decode and one packed multiply per two weights make
// this half the vector work of the bf16 form.
__device__ __forceinline__ u32x4 nvfp4_decode8_f16(uint32_t codes, f16x2 s2) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2);
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2);
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2);
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2);
  return r;
}

// Eight bf16 values -> eight fp16 values (conversion toward zero).  Exact for
// zeros and for every bf16 value of magnitude in [2^-17, 65280]: a bf16 value
// has 8 significant bits, so from 2^-17 up its lowest bit is at least 2^-24,
// the spacing of fp16 subnormals.  Per 16-bit half, `mag` keeps the largest
// bf16 magnitude pattern seen and `mnz` the smallest of (magnitude pattern -
// 1) mod 2^16, so a zero leaves it at 0xFFFF (packed unsigned maximum,
// subtract and minimum: three instructions per two values);
// f16_unsafe(mag, mnz) then tells whether any value was not finite, reached
// 65536 or was nonzero below 2^-17.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v, uint32_t &mag, uint32_t &mnz) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, mag);
  u16x2 n = __builtin_bit_cast(u16x2, mnz);
  const u16x2 one = {1, 1};
  u32x4 r;
#define MTP_CVT_DWORD(c)                                                                     \
  {                                                                                          \
    const u16x2 a = __builtin_bit_cast(u16x2, v.c & 0x7FFF7FFFu);                            \
    m = __builtin_elementwise_max(m, a);                                                     \
    n = __builtin_elementwise_min(n, a - one);                                               \
    r.c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v.c << 16), \
                                                                 __uint_as_float(v.c & 0xFFFF0000u))); \
  }
  MTP_CVT_DWORD(x) MTP_CVT_DWORD(y) MTP_CVT_DWORD(z) MTP_CVT_DWORD(w)
#undef MTP_CVT_DWORD
  mag = __builtin_bit_cast(uint32_t, m);
  mnz = __builtin_bit_cast(uint32_t, n);
  return r;
}

// Whether the patterns kept by bf16x8_to_f16x8 show, in either half, a
// magnitude of 65536 (0x4780) or more, an infinity or NaN, or a nonzero
// magnitude below 2^-17 (0x3700).
__device__ __forceinline__ bool f16_unsafe(uint32_t mag, uint32_t mnz) {
  return (mag & 0xFFFFu) >= 0x4780u || (mag >> 16) >= 0x4780u || (mnz & 0xFFFFu) < 0x36FFu ||
         (mnz >> 16) < 0x36FFu;
}

// Binary exponent e of a nonzero finite bf16 magnitude pattern p:
// 2^e <= value < 2^(e+1) (subnormals included).
__device__ __forceinline__ int bf16_exponent(uint32_t p) {
  return p >= 0x80u ? (int)(p >> 7) - 127 : (31 - __builtin_clz(p)) - 133;
}

// Eight bf16 values times 2^s (a power of two given as fp32 `sc`) -> eight
// fp16 values, exact whenever every nonzero |x| * 2^s lies in [2^-17, 2^16)
// (the product is exact in fp32 and has at most 8 significant bits).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(u32x4 v, float sc) {
  u32x4 r;
#define MTP_CVT_DWORD(c)                                                                   \
  r.c = __builtin_bit_cast(uint32_t,                                                       \
                           __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v.c << 16) * sc,     \
                                                      __uint_as_float(v.c & 0xFFFF0000u) * sc));
  MTP_CVT_DWORD(x) MTP_CVT_DWORD(y) MTP_CVT_DWORD(z) MTP_CVT_DWORD(w)
#undef MTP_CVT_DWORD
  return r;
}

// Eight offset-binary int4 codes u (element i in nibble i) -> eight bf16
// values 128 + u, in the slot order (0,4,1,5,2,6,3,7).  128 + u is exact in
// bf16; the caller removes the offset through the accumulator's start value.
__device__ __forceinline__ u32x4 q4_decode8_offset128(uint32_t c) {
  const uint32_t mag = 0x43004300u, lo = 0x000F000Fu;
  u32x4 r;
  r.x = (c & lo) | mag;
  r.y = ((c >> 4) & lo) | mag;
  r.z = ((c >> 8) & lo) | mag;
  r.w = ((c >> 12) & lo) | mag;
  return r;
}

// Eight bf16 values in element order -> slot order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ u32x4 interleave_halves(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // h0 | h4 << 16
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // h1 | h5 << 16
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // h2 | h6 << 16
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // h3 | h7 << 16
  return r;
}

// Value of lane (l ^ 1), resp. (l ^ 2), within each aligned quad of lanes.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// 4x4 transpose of dwords across the four 16-lane groups of a wave: on entry
// lane (r, g) holds a[j] = element (g, j); on exit it holds element (j, g).
__device__ __forceinline__ void transpose_lane_groups(uint32_t &a0, uint32_t &a1, uint32_t &a2,
                                                      uint32_t &a3) {
  auto s02 = __builtin_amdgcn_permlane32_swap(a0, a2, false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(a1, a3, false, false);
  a0 = s02[0]; a2 = s02[1]; a1 = s13[0]; a3 = s13[1];
  auto s01 = __builtin_amdgcn_permlane16_swap(a0, a1, false, false);
  auto s23 = __builtin_amdgcn_permlane16_swap(a2, a3, false, false);
  a0 = s01[0]; a1 = s01[1]; a2 = s23[0]; a3 = s23[1];
}

}  // namespace mtp
