// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtp {

// ---- packing and the verify GEMM -------------------------------------------

size_t packed_weight_bytes(int N, int K);

hipError_t launch_pack(int format, int count, int N, int K, const uint8_t *codes,
                       const void *scales, uint8_t *packed, hipStream_t stream);

// Launch shape of the dense GEMM (see engine.h for the terms).
struct GemmPlan {
  int T, P;          // tiles of 16 rows, pairs of 256 K
  int S, ppj;        // K slices and pairs per slice (shape only)
  int J, KG, TW;     // slices per workgroup, workgroups per tile group, tiles per workgroup
  int TG, G, grid;   // tile groups, workgroups per K group, total workgroups
  int threads;
  size_t lds;
  size_t ws_bytes;   // arrival counters + slice partials when KG > 1
  int PP;            // weight blocks each wave keeps in flight
};

GemmPlan gemm_plan(int format, int M, int N, int K);
GemmPlan finish_plan(GemmPlan pl);   // fills G, grid, PP and ws_bytes from the rest

// Workspace that covers every M for this shape (0 when K has one slice).
size_t gemm_ws_bytes(int N, int K);

hipError_t launch_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                       const uint8_t *packed, float gscale, float *y, int64_t ldy, uint16_t *yb,
                       int64_t ldyb, void *ws, const GemmPlan &plan, hipStream_t stream);

// ---- acceptance ------------------------------------------------------------

size_t accept_ws_bytes(int M, int V);

// Sampled acceptance of B sequences (mtp_accept_sampled), arguments checked.
struct SampledCall {
  const float *logits;
  int B, M, V;
  int64_t ldl;
  const int32_t *history, *history_len;
  int64_t ldh;
  const int32_t *drafts;
  const float *q;
  int64_t ldq;
  const int32_t *q_ids;
  const float *q_probs;
  int Kq;
  const float *uniforms;
  float temperature, top_p, min_p;
  int top_k;
  float repeat_penalty, presence_penalty, frequency_penalty;
  int penalty_last_n;
  const int64_t *base_len;
  int32_t *tokens, *counts;
  int64_t *rollback;
  int32_t *out_ids;
  float *out_probs;
};

size_t sampled_ws_bytes(int B, int M, int V, int top_k, bool penalties);

// ---- multi-row verify attention ---------------------------------------------

size_t attention_ws_bytes(int M, int Hq, int Hkv, int D, int L);
hipError_t launch_verify_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   int64_t ldk, int M, int Hq, int Hkv, int D, int L, float scale,
                                   float *out, void *ws, hipStream_t stream);
hipError_t launch_accept_sampled(const SampledCall &c, void *ws, hipStream_t stream);

hipError_t launch_accept_greedy(const float *logits, int M, int V, int64_t ldl,
                                const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                int32_t *counts, int64_t *rollback, void *ws, hipStream_t stream);

// Greedy acceptance on the library's own static device scratch (no workspace).
size_t greedy_static_bytes(int M, int V);
size_t greedy_static_max_bytes();
hipError_t launch_accept_greedy_static(const float *logits, int M, int V, int64_t ldl,
                                       const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                       int32_t *counts, int64_t *rollback, hipStream_t stream);

hipError_t launch_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                                   const float *q, int64_t ldq, const int32_t *drafts,
                                   const float *u, float temperature, float top_p,
                                   int64_t base_len, int32_t *tokens, int32_t *counts,
                                   int64_t *rollback, void *ws, hipStream_t stream);

// ---- read-bandwidth probe (measurement aid) -------------------------------

int read_probe_shapes();
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int shape,
                             hipStream_t stream);

// ---- KV-cache rollback ------------------------------------------------------

hipError_t launch_kv_append(uint16_t *k, uint16_t *v, int NL, int B, int Hkv, int64_t cap, int D,
                            int ring, const uint16_t *kn, const uint16_t *vn, int64_t ld_new,
                            int M, const int64_t *base, uint16_t *sk, uint16_t *sv, int32_t *err,
                            hipStream_t stream);
hipError_t launch_kv_restore(uint16_t *k, uint16_t *v, int NL, int B, int Hkv, int64_t cap, int D,
                             int ring, int M, const int64_t *base, const int64_t *roll,
                             const uint16_t *sk, const uint16_t *sv, int32_t *err,
                             hipStream_t stream);

// ---- MoE -------------------------------------------------------------------

size_t moe_ws_bytes(int T, int H, int F, int E, int topk);

// Whether the staged rows of one expert pass fit a workgroup's LDS.
bool moe_fits(int format, int T, int H, int F);

hipError_t launch_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                      const int32_t *ids, const float *gw, const uint8_t *gu_packed,
                      const float *gu_global, const uint8_t *dn_packed, const float *dn_global,
                      float *out, uint16_t *h_out, void *ws, hipStream_t stream);

// depth.hip
hipError_t launch_depth_observe(double *reached, double *accepted, int dmax, int depth,
                                const int32_t *counts, double keep, const double *cost,
                                int32_t *choice, double *prob, int32_t *err, hipStream_t stream);

}  // namespace mtp
