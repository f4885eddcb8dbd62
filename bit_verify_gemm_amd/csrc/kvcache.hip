// KV-cache rollback with lazy snapshots.
//
// Ollama mtp.go commit log, the snapshot rework: a cache snapshots itself
// as a verify write crosses each offset, and the runner commits the batch by
// restoring to the accepted count.  A KV or rotating capture points into the
// live buffer and takes a copy only when a write would destroy something it
// still needs, so rejecting a draft costs nothing.
//
// Here the only destructive write is a rotating cache's: writing position
// p >= cap into row p mod cap overwrites position p - cap.  kv_append copies
// exactly those rows out (into the M-row snapshot of each head) before it
// writes the verify rows; kv_restore puts them back for the rejected
// positions.  A linear cache never overwrites a live row, so its snapshot is
// the base length alone and its restore launches nothing.
//
// Both kernels take the per-sequence base length and rollback index from
// device memory (the accept calls write the latter), so a verify step and
// its commit need no host round trip.  One workgroup per (layer, sequence,
// KV head); every thread moves one 16-byte piece of K or of V per round, so
// a D = 128, M = 8 head is one round of 256 threads.
#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

namespace mtp {
namespace {

constexpr int kKvThreads = 256;

struct KvArgs {
  uint16_t *k, *v;              // caches [NL][B][Hkv][cap][D]
  const uint16_t *kn, *vn;      // new rows, ld_new elements apart
  uint16_t *sk, *sv;            // snapshots [NL][B][Hkv][M][D]
  const int64_t *base, *roll;   // [B]
  int32_t *err;
  int64_t cap, ld_new;
  int B, Hkv, D, M, ring;
};

__device__ __forceinline__ void raise_err(int32_t *err) {
  if (err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kKvThreads) void kv_append_kernel(KvArgs a) {
  const int u = blockIdx.x;                 // (l * B + b) * Hkv + h
  const int lb = u / a.Hkv, h = u - lb * a.Hkv, b = lb % a.B;
  const int vpr = a.D >> 3;                 // 16-byte pieces per row
  const int per = a.M * vpr;                // pieces per tensor
  const size_t head_row = (size_t)u * (size_t)a.cap;
  const int64_t base = a.base[b];
  // ring row of position base (one division per workgroup); row m follows
  const int64_t row0 = a.ring && base >= 0 ? base % a.cap : base;
  for (int i = threadIdx.x; i < 2 * per; i += kKvThreads) {
    const int t = i >= per;                 // 0: K, 1: V
    const int j = i - t * per, m = j / vpr, c = j - m * vpr;
    // the new piece does not depend on the base length: its load goes out
    // together with base_len's
    const uint16_t *src = (t ? a.vn : a.kn) + ((size_t)lb * a.M + m) * a.ld_new + (size_t)h * a.D;
    const u32x4 nv = reinterpret_cast<const u32x4 *>(src)[c];
    const int64_t p = base + m;
    if (p < 0 || (!a.ring && p >= a.cap)) {
      raise_err(a.err);
      continue;
    }
    int64_t row = row0 + m;                  // m < M <= cap: at most one wrap
    if (a.ring && row >= a.cap) row -= a.cap;
    u32x4 *dst = reinterpret_cast<u32x4 *>((t ? a.v : a.k) + (head_row + row) * a.D) + c;
    if (a.ring && p >= a.cap) {
      // The row still holds position p - cap: keep it for a rollback.
      const u32x4 old = *dst;
      u32x4 *snap = reinterpret_cast<u32x4 *>((t ? a.sv : a.sk) + ((size_t)u * a.M + m) * a.D);
      snap[c] = old;
    }
    *dst = nv;
  }
}

__device__ __forceinline__ u32x4 snap_piece(const KvArgs &a, int u, int per, int vpr, int i) {
  const int t = i >= per;
  const int j = i - t * per, m = j / vpr, c = j - m * vpr;
  return reinterpret_cast<const u32x4 *>((t ? a.sv : a.sk) + ((size_t)u * a.M + m) * a.D)[c];
}

__global__ __launch_bounds__(kKvThreads) void kv_restore_kernel(KvArgs a) {
  const int u = blockIdx.x;
  const int b = (u / a.Hkv) % a.B;
  const int vpr = a.D >> 3;
  const int per = a.M * vpr;
  // Every thread's first snapshot piece is loaded, kept or not, before the
  // base length and rollback are read, so that the two latencies overlap.
  const u32x4 first = snap_piece(a, u, per, vpr, min((int)threadIdx.x, 2 * per - 1));
  const int64_t base = a.base[b];
  int64_t r = a.roll[b];
  if (r < base || r > base + a.M) {
    if (threadIdx.x == 0) raise_err(a.err);
    r = r < base ? base : base + a.M;
  }
  const size_t head_row = (size_t)u * (size_t)a.cap;
  const int64_t row0 = base >= 0 ? base % a.cap : 0;
  for (int i = threadIdx.x; i < 2 * per; i += kKvThreads) {
    const int t = i >= per;
    const int j = i - t * per, m = j / vpr, c = j - m * vpr;
    const int64_t p = base + m;
    // rows below the rollback stay; a row below cap overwrote nothing (and
    // a negative position was never written)
    if (p < r || p < a.cap) continue;
    const u32x4 old = i == (int)threadIdx.x ? first : snap_piece(a, u, per, vpr, i);
    int64_t row = row0 + m;
    if (row >= a.cap) row -= a.cap;
    reinterpret_cast<u32x4 *>((t ? a.v : a.k) + (head_row + row) * a.D)[c] = old;
  }
}

}  // namespace

hipError_t launch_kv_append(uint16_t *k, uint16_t *v, int NL, int B, int Hkv, int64_t cap, int D,
                            int ring, const uint16_t *kn, const uint16_t *vn, int64_t ld_new,
                            int M, const int64_t *base, uint16_t *sk, uint16_t *sv, int32_t *err,
                            hipStream_t stream) {
  KvArgs a{k, v, kn, vn, sk, sv, base, nullptr, err, cap, ld_new, B, Hkv, D, M, ring};
  hipLaunchKernelGGL(kv_append_kernel, dim3(NL * B * Hkv), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_restore(uint16_t *k, uint16_t *v, int NL, int B, int Hkv, int64_t cap, int D,
                             int ring, int M, const int64_t *base, const int64_t *roll,
                             const uint16_t *sk, const uint16_t *sv, int32_t *err,
                             hipStream_t stream) {
  if (!ring) return hipSuccess;             // a linear cache's length is the rollback index itself
  KvArgs a{k, v, nullptr, nullptr, const_cast<uint16_t *>(sk), const_cast<uint16_t *>(sv),
           base, roll, err, cap, 0, B, Hkv, D, M, ring};
  hipLaunchKernelGGL(kv_restore_kernel, dim3(NL * B * Hkv), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mtp
