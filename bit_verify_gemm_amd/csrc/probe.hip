// Read-bandwidth probe: a measurement aid beside the verify kernels, not a
// step of the verify pass.  It reads every 16-byte piece of a buffer once
// (non-temporal vector loads, grid-stride, in one of a few launch shapes)
// and folds them with XOR so that the loads cannot be dropped; a thread writes only if its fold hits one fixed
// value, so the probe moves next to no bytes besides the reads.  Timed over
// the same sizes and rotating copies as a verify GEMM, the best of its
// shapes gives the read rate one launch of that size can reach.
#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace mtp {
namespace {

constexpr int kProbeThreads = 256;

// launch shapes: loads in flight per thread and the largest grid
struct ProbeShape { int unroll, max_groups; };
constexpr ProbeShape kShapes[] = {{1, 2048}, {2, 2048}, {4, 2048}, {8, 2048}, {4, 8192}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

template <int U>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *src, size_t n,
                                                                   uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

int read_probe_shapes() { return kNumShapes; }

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int shape,
                             hipStream_t stream) {
  const size_t n = bytes / 16;
  const ProbeShape s = kShapes[shape];
  const size_t per_group = (size_t)kProbeThreads * s.unroll;
  const int groups = (int)std::min<size_t>((n + per_group - 1) / per_group, s.max_groups);
  if (groups == 0) return hipSuccess;
  const u32x4 *p = static_cast<const u32x4 *>(src);
  switch (s.unroll) {
    case 1: hipLaunchKernelGGL(read_probe_kernel<1>, dim3(groups), dim3(kProbeThreads), 0, stream, p, n, sink); break;
    case 2: hipLaunchKernelGGL(read_probe_kernel<2>, dim3(groups), dim3(kProbeThreads), 0, stream, p, n, sink); break;
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, dim3(groups), dim3(kProbeThreads), 0, stream, p, n, sink); break;
    default: hipLaunchKernelGGL(read_probe_kernel<8>, dim3(groups), dim3(kProbeThreads), 0, stream, p, n, sink); break;
  }
  return hipGetLastError();
}

}  // namespace mtp
