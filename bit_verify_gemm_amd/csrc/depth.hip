// Draft-depth controller on the device: the live per-position acceptance
// statistics are updated from the accept call's counts on the stream, and
// the next depth is chosen there too, so that the host needs no read-back
// per step.
//
// Ollama mtp.go commit log, the controller message: the engine drafts the
// depth that maximises committed tokens per wall-clock from live
// per-position acceptance and the measured cost per width.  "Faster Gemma 4
// on MLX with multi-token prediction", fourth and fifth paragraphs: the
// runtime tunes itself from acceptance and verify timings, and the pass runs
// on the GPU with no return to the CPU.  The arithmetic is that of the host
// functions in controller.cpp (the same fp64 operations in the same order,
// no contraction), so the two agree bit for bit.
#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace mtp {
namespace {

constexpr int kLanes = 64;   // dmax <= 63: one lane per position

// One wave.  Lane i (< dmax) holds position i + 1.
__global__ __launch_bounds__(kLanes) void depth_observe_kernel(double *reached, double *accepted,
                                                               int dmax, int depth,
                                                               const int32_t *counts, double keep,
                                                               const double *cost, int32_t *choice,
                                                               double *prob, int32_t *err) {
  const int lane = threadIdx.x;
  const int n = counts[0];   // drafts accepted by the step
  const bool ok = n >= 0 && n <= depth;
  double r = 0.0, a = 0.0;
  if (lane < dmax) {
    r = reached[lane];
    a = accepted[lane];
    if (ok) {
      const int i = lane + 1;
      r *= keep;
      a *= keep;
      if (i <= depth && i <= n + 1) r += 1.0;
      if (i <= depth && i <= n) a += 1.0;
      reached[lane] = r;
      accepted[lane] = a;
    }
  }
  const double pr = (a + 1.0) / (r + 2.0);   // Laplace's rule
  if (prob && lane < dmax) prob[lane] = pr;
  if (err && lane == 0) *err = ok ? 0 : 1;
  if (!choice) return;
  // E(d) / cost[d] over d = 0..dmax, in order, on lane 0 (the probabilities
  // gathered from the other lanes); the smallest depth wins a tie
  int best = 0;
  bool bad = false;
  double best_rate = 0.0, e = 1.0, prod = 1.0;
  for (int d = 0; d <= dmax; ++d) {
    if (d > 0) {
      prod *= __shfl(pr, d - 1);
      e += prod;
    }
    const double c = cost[d];
    bad |= !(c > 0.0);
    const double rate = e / c;
    if (d == 0 || rate > best_rate) {
      best = d;
      best_rate = rate;
    }
  }
  if (lane == 0) {
    *choice = bad ? 0 : best;
    if (err && bad) *err = 2;
  }
}

}  // namespace

hipError_t launch_depth_observe(double *reached, double *accepted, int dmax, int depth,
                                const int32_t *counts, double keep, const double *cost,
                                int32_t *choice, double *prob, int32_t *err, hipStream_t stream) {
  hipLaunchKernelGGL(depth_observe_kernel, dim3(1), dim3(kLanes), 0, stream, reached, accepted,
                     dmax, depth, counts, keep, cost, choice, prob, err);
  return hipGetLastError();
}

}  // namespace mtp
