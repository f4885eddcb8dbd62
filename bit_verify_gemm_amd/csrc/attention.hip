// Multi-row verify attention over a shared KV prefix.
//
// Qiita roofline article, §2-3: at long context the KV reads also take
// bandwidth, but the candidates of one verify pass look at the same prefix,
// so a single KV read serves all of them, as with the weights.  Here the M
// verify rows of a sequence, and the G query heads that share each KV head,
// make R = M*G query rows per KV head; every workgroup streams one chunk of
// one KV head's positions through LDS once and applies it to all R rows on
// the matrix cores.
//
// Row r of KV head kh is query position i = r / G (absolute position L + i)
// of query head kh*G + r % G; it sees keys 0 .. L + i (causal among the
// verify rows, whose K and V are already in the cache).
//
// Per 32-position step a wave (16 query rows) computes S^T = K Q^T
// (positions x rows) with K from LDS and Q^T held in registers, updates the
// running row maxima and sums (online softmax, fp32), and adds
// O^T += V^T P^T with V^T from LDS and P^T (two bf16 parts) taken straight from the
// S^T accumulator: the reduction slots of the second product are the
// positions 4g..4g+3 and 16+4g..16+4g+3 that lane group g already holds, so
// no transpose is needed.  Chunks of the KV range run in separate
// workgroups; vattn_combine merges their (max, sum, O) in chunk order.
#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace mtp {
namespace {

constexpr int kSub = 32;          // positions per step
constexpr int kMaxRowWaves = 8;   // query rows per KV head up to 128
constexpr int kMinWaves = 4;      // waves per workgroup at least (the staging is spread over them)

using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit untyped data, gfx9 family

struct AttnArgs {
  const uint16_t *q;      // [M][Hq][D]
  const uint16_t *k;      // [Hkv][ldk][D]
  const uint16_t *v;
  int64_t ldk;
  int M, Hq, Hkv, G, L, R;
  float scale;
  int nch, ch;            // chunks per KV head and positions per chunk
  float *part;            // [Hkv][nch][R16][D] unnormalised partial outputs
  float *ml;              // [Hkv][nch][R16][2] running max and sum
  float *out;             // [M][Hq][D]
};

template <int D>
struct alignas(16) Lds {
  static constexpr int kRow = D + 8;        // K row stride (elements): 16 bytes of padding
  static constexpr int vRow = kSub + 4;     // V^T row stride (elements)
  uint16_t k[kSub * kRow];
  uint16_t vt[D * vRow];
};

__device__ __forceinline__ float wave_max16(float x) {   // over the 4 lane groups of a column
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D>
__global__ __launch_bounds__(kMaxRowWaves * kWave) void vattn_partial(AttnArgs a) {
  constexpr int kChunks = kSub * D / 8;                  // 16-byte pieces of K (and of V) per step
  __shared__ Lds<D> s;
  const int c = blockIdx.x, kh = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nt = blockDim.x, n = lane & 15, g = lane >> 4;
  const int r = wave * 16 + n;                           // this lane's query row
  const bool row_ok = r < a.R;
  const int qi = row_ok ? r / a.G : 0, h = kh * a.G + (row_ok ? r % a.G : 0);
  const int limit = a.L + qi;                            // last key position the row sees
  const int total = a.L + a.M;                           // keys in the cache
  const int c0 = c * a.ch, c1 = min(total, c0 + a.ch);

  // K and V of this head through buffer windows: positions past the cache
  // read as zeros
  const uint32_t bytes = (uint32_t)((int64_t)total * D * 2);
  const Rsrc kw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.k + (int64_t)kh * a.ldk * D), 0, (int)bytes, kRsrcWord3);
  const Rsrc vw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.v + (int64_t)kh * a.ldk * D), 0, (int)bytes, kRsrcWord3);

  // Q^T: reduction slots 32ks + 8g .. +8 of row r
  u32x4 qb[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qb[ks] = u32x4{0u, 0u, 0u, 0u};
    if (row_ok)
      qb[ks] = *reinterpret_cast<const u32x4 *>(a.q + ((int64_t)qi * a.Hq + h) * D + 32 * ks + 8 * g);
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -__builtin_inff(), l = 0.0f;

  // register staging of one step (a workgroup has at least kMinWaves
  // waves): K in 16-byte pieces (p = t, t + nt, ...) stored as they are;
  // V in blocks of 4 positions x 4 columns (four 8-byte loads), transposed
  // in registers so that each column's 4 positions go to LDS in one 8-byte
  // store
  constexpr int kPer = (kChunks + kMinWaves * kWave - 1) / (kMinWaves * kWave);
  constexpr int kVBlocks = (kSub / 4) * (D / 4);
  constexpr int kVPer = (kVBlocks + kMinWaves * kWave - 1) / (kMinWaves * kWave);
  u32x4 kr[kPer];
  u32x2 vr[kVPer][4];
  auto load_step = [&](int base) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = (int)threadIdx.x + u * nt;
      if (pc < kChunks) {
        const int pos = base + pc / (D / 8), d0 = (pc % (D / 8)) * 8;
        const int off = pos < c1 ? (pos * D + d0) * 2 : (int)bytes;   // past the chunk: zeros
        kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kw, off, 0, 0));
      }
    }
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int b = (int)threadIdx.x + u * nt;
      if (b < kVBlocks) {
        const int p0 = base + 4 * (b / (D / 4)), d0 = 4 * (b % (D / 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = p0 + r < c1 ? ((p0 + r) * D + d0) * 2 : (int)bytes;
          vr[u][r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vw, off, 0, 0));
        }
      }
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = (int)threadIdx.x + u * nt;
      if (pc < kChunks) {
        const int p = pc / (D / 8), d0 = (pc % (D / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&s.k[p * Lds<D>::kRow + d0]) = kr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int b = (int)threadIdx.x + u * nt;
      if (b < kVBlocks) {
        const int p = 4 * (b / (D / 4)), d0 = 4 * (b % (D / 4));
        // vr[u][r] = columns d0..d0+3 of position p + r (.x: d0, d0+1; .y: d0+2, d0+3);
        // column d0 + c takes the halves c of the four positions
        const uint32_t lo = 0x05040100u, hi = 0x07060302u;   // low / high halves of two words
        const u32x2 c0 = {__builtin_amdgcn_perm(vr[u][1].x, vr[u][0].x, lo),
                          __builtin_amdgcn_perm(vr[u][3].x, vr[u][2].x, lo)};
        const u32x2 c1v = {__builtin_amdgcn_perm(vr[u][1].x, vr[u][0].x, hi),
                           __builtin_amdgcn_perm(vr[u][3].x, vr[u][2].x, hi)};
        const u32x2 c2 = {__builtin_amdgcn_perm(vr[u][1].y, vr[u][0].y, lo),
                          __builtin_amdgcn_perm(vr[u][3].y, vr[u][2].y, lo)};
        const u32x2 c3 = {__builtin_amdgcn_perm(vr[u][1].y, vr[u][0].y, hi),
                          __builtin_amdgcn_perm(vr[u][3].y, vr[u][2].y, hi)};
        *reinterpret_cast<u32x2 *>(&s.vt[(d0 + 0) * Lds<D>::vRow + p]) = c0;
        *reinterpret_cast<u32x2 *>(&s.vt[(d0 + 1) * Lds<D>::vRow + p]) = c1v;
        *reinterpret_cast<u32x2 *>(&s.vt[(d0 + 2) * Lds<D>::vRow + p]) = c2;
        *reinterpret_cast<u32x2 *>(&s.vt[(d0 + 3) * Lds<D>::vRow + p]) = c3;
      }
    }
  };

  load_step(c0);
  for (int base = c0; base < c1; base += kSub) {
    __syncthreads();                 // the previous step's reads of LDS are done
    store_step();
    __syncthreads();
    if (base + kSub < c1) load_step(base + kSub);   // in flight during this step
    if (wave * 16 >= a.R) continue;                 // a staging-only wave (uniform)
    // S^T: two 16-position tiles
    f32x4 s0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 a0 = *reinterpret_cast<const u32x4 *>(&s.k[n * Lds<D>::kRow + 32 * ks + 8 * g]);
      const u32x4 a1 =
          *reinterpret_cast<const u32x4 *>(&s.k[(16 + n) * Lds<D>::kRow + 32 * ks + 8 * g]);
      s0 = mfma_16x16x32(a0, qb[ks], s0);
      s1 = mfma_16x16x32(a1, qb[ks], s1);
    }
    // scores of this lane: positions base + 4g + i (tile 0) and base + 16 + 4g + i
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p0 = base + 4 * g + i, p1 = base + 16 + 4 * g + i;
      x[i] = (p0 <= limit && p0 < c1) ? s0[i] * a.scale : -__builtin_inff();
      x[4 + i] = (p1 <= limit && p1 < c1) ? s1[i] * a.scale : -__builtin_inff();
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    mx = wave_max16(mx);
    const float mn = fmaxf(m, mx);
    float pv[8], ps = 0.0f;
    if (mn == -__builtin_inff()) {   // nothing seen yet by this row
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __expf(x[i] - mn);
        ps += pv[i];
      }
      const float alpha = __expf(m - mn);   // 0 when m is -inf
      l = l * alpha + wave_sum16(ps);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
      m = mn;
    }
    // P as two bf16 parts, ph = bf16(p) and pl = bf16(p - ph) (the
    // difference is exact in fp32): ph + pl holds p to 16 significant bits
    // (relative error below 2^-17), and both products with V are exact in
    // the fp32 accumulation of the MFMA
    uint16_t ph[8], pl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ph[i] = f32_to_bf16_rne(pv[i]);
      pl[i] = f32_to_bf16_rne(pv[i] - __uint_as_float((uint32_t)ph[i] << 16));
    }
    auto pack = [](const uint16_t *h) {
      return u32x4{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                   (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16)};
    };
    const u32x4 pbh = pack(ph), pbl = pack(pl);
    // O^T += V^T P^T: V^T rows d = 16dt + n, slots = the same eight positions
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint16_t *vrow = &s.vt[(16 * dt + n) * Lds<D>::vRow];
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + 4 * g);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16 + 4 * g);
      const u32x4 vt = u32x4{lo.x, lo.y, hi.x, hi.y};
      o[dt] = mfma_16x16x32(vt, pbh, o[dt]);
      o[dt] = mfma_16x16x32(vt, pbl, o[dt]);
    }
  }
  // partials of this chunk: lane (n, g) holds d = 16dt + 4g + i of row r
  const int R16 = (a.R + 15) / 16 * 16;
  const size_t slot = ((size_t)kh * a.nch + c) * R16 + r;
  if (r < R16) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<f32x4 *>(a.part + slot * D + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      a.ml[2 * slot] = m;
      a.ml[2 * slot + 1] = l;
    }
  }
}

// One workgroup of 1024 threads per (query row, KV head) merges the chunks:
// out = sum_c O_c e^(m_c - m) / sum_c l_c e^(m_c - m).  The chunk weights
// are computed once into LDS; 1024 / D groups of threads each add every
// (1024/D)-th chunk of a column with eight loads in flight, and the group
// sums are added in a fixed order.
constexpr int kMaxChunks = 512;

template <int D>
__global__ __launch_bounds__(1024) void vattn_combine(AttnArgs a) {
  constexpr int kCG = 1024 / D;   // chunk groups
  __shared__ float wc[kMaxChunks];
  __shared__ float red[1024 / kWave];
  __shared__ float s_mx, s_l;
  const int r = blockIdx.x, kh = blockIdx.y, t = threadIdx.x, d = t % D;
  const int lane = t & (kWave - 1), wave = t / kWave, nw = 1024 / kWave;
  const int R16 = (a.R + 15) / 16 * 16;
  const size_t base = (size_t)kh * a.nch * R16 + r;   // slot of chunk c: base + c * R16
  // row maximum over the chunks
  float mx = -__builtin_inff();
  for (int c = t; c < a.nch; c += 1024) {
    const float mc = a.ml[2 * (base + (size_t)c * R16)];
    wc[c] = mc;
    mx = fmaxf(mx, mc);
  }
  for (int s = kWave / 2; s > 0; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (t == 0) {
    float m = red[0];
    for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
    s_mx = m;
  }
  __syncthreads();
  const float m = s_mx;
  // chunk weights and each chunk's weighted sum, then the normaliser in
  // chunk order
  __shared__ float lc[kMaxChunks];
  for (int c = t; c < a.nch; c += 1024) {
    const float mc = wc[c];
    const float w = mc == -__builtin_inff() ? 0.0f : __expf(mc - m);
    wc[c] = w;
    lc[c] = a.ml[2 * (base + (size_t)c * R16) + 1] * w;
  }
  __syncthreads();
  if (t == 0) {
    float l = 0.0f;
    for (int c = 0; c < a.nch; ++c) l += lc[c];
    s_l = l;
  }
  // thread (cg, d) adds chunks cg, cg + kCG, ... of column d (eight loads in
  // flight), then the kCG sums are added in cg order
  const int cg = threadIdx.x / D;
  float acc = 0.0f;
  const float *col = a.part + base * D + d;
  int c = cg;
  for (; c + 7 * kCG < a.nch; c += 8 * kCG) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[(size_t)(c + u * kCG) * R16 * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u] * wc[c + u * kCG];
  }
  for (; c < a.nch; c += kCG) acc += col[(size_t)c * R16 * D] * wc[c];
  __shared__ float part_sum[kCG][D];
  part_sum[cg][d] = acc;
  __syncthreads();
  if (cg != 0) return;
  acc = part_sum[0][d];
  for (int k = 1; k < kCG; ++k) acc += part_sum[k][d];
  const int qi = r / a.G, h = kh * a.G + r % a.G;
  a.out[((int64_t)qi * a.Hq + h) * D + d] = acc / s_l;
}

struct AttnPlan {
  int nch, ch, R16;
  size_t part, ml, bytes;
};

AttnPlan attn_plan(int M, int Hq, int Hkv, int D, int L) {
  AttnPlan p;
  const int total = L + M, G = Hq / Hkv, R = M * G;
  p.R16 = (R + 15) / 16 * 16;
  // about four workgroups per CU, chunks of at least 64 positions
  int nch = (1024 + Hkv - 1) / Hkv;
  nch = std::max(1, std::min(std::min(nch, kMaxChunks), (total + 63) / 64));
  p.ch = ((total + nch - 1) / nch + kSub - 1) / kSub * kSub;
  p.nch = (total + p.ch - 1) / p.ch;
  const size_t slots = (size_t)Hkv * p.nch * p.R16;
  p.part = 0;
  p.ml = (sizeof(float) * slots * D + 255) & ~(size_t)255;
  p.bytes = p.ml + ((sizeof(float) * 2 * slots + 255) & ~(size_t)255);
  return p;
}

}  // namespace

size_t attention_ws_bytes(int M, int Hq, int Hkv, int D, int L) {
  return attn_plan(M, Hq, Hkv, D, L).bytes;
}

hipError_t launch_verify_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   int64_t ldk, int M, int Hq, int Hkv, int D, int L, float scale,
                                   float *out, void *ws, hipStream_t stream) {
  const AttnPlan pl = attn_plan(M, Hq, Hkv, D, L);
  uint8_t *w = static_cast<uint8_t *>(ws);
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.ldk = ldk;
  a.M = M; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.L = L; a.R = M * a.G;
  a.scale = scale; a.nch = pl.nch; a.ch = pl.ch;
  a.part = reinterpret_cast<float *>(w + pl.part);
  a.ml = reinterpret_cast<float *>(w + pl.ml);
  a.out = out;
  const dim3 grid(pl.nch, Hkv), block(std::max(kMinWaves, pl.R16 / 16) * kWave);
  const dim3 cgrid(a.R, Hkv);
  switch (D) {
    case 64:
      hipLaunchKernelGGL(vattn_partial<64>, grid, block, 0, stream, a);
      hipLaunchKernelGGL(vattn_combine<64>, cgrid, dim3(1024), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(vattn_partial<128>, grid, block, 0, stream, a);
      hipLaunchKernelGGL(vattn_combine<128>, cgrid, dim3(1024), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(vattn_partial<256>, grid, block, 0, stream, a);
      hipLaunchKernelGGL(vattn_combine<256>, cgrid, dim3(1024), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace mtp
