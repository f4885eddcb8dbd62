// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtp {

// ---- verify GEMM -----------------------------------------------------------

struct GemmPlan {
  int splits;      // K-ranges processed by separate workgroups
  int split_k;     // length of each K-range (multiple of 128, last one ragged)
  size_t ws_bytes; // fp32 partials [splits][M][N] when splits > 1
};

GemmPlan gemm_plan(int M, int N, int K);

hipError_t launch_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                       const uint8_t *codes, const void *scales, float gscale, float *y,
                       int64_t ldy, uint16_t *yb, int64_t ldyb, void *ws, const GemmPlan &plan,
                       hipStream_t stream);

// ---- acceptance ------------------------------------------------------------

size_t accept_ws_bytes(int M, int V);

hipError_t launch_accept_greedy(const float *logits, int M, int V, int64_t ldl,
                                const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                int32_t *counts, int64_t *rollback, void *ws, hipStream_t stream);

hipError_t launch_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                                   const float *q, int64_t ldq, const int32_t *drafts,
                                   const float *u, float temperature, float top_p,
                                   int64_t base_len, int32_t *tokens, int32_t *counts,
                                   int64_t *rollback, void *ws, hipStream_t stream);

// ---- MoE -------------------------------------------------------------------

size_t moe_ws_bytes(int T, int H, int F, int E, int topk);

hipError_t launch_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                      const int32_t *ids, const float *gw, const uint8_t *gu_codes,
                      const void *gu_scales, const float *gu_global, const uint8_t *dn_codes,
                      const void *dn_scales, const float *dn_global, float *out,
                      uint16_t *h_out, void *ws, hipStream_t stream);

}  // namespace mtp
