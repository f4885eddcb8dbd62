// C ABI of the verify-pass library: argument checks on the host, workspace
// sizing, and dispatch to the HIP launchers.  Every check runs before any HIP
// call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mtp_verify.h"
#include "internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) {
    g_error.clear();
    return MTP_OK;
  }
  return fail(MTP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_format(int f) { return f == MTP_FMT_NVFP4 || f == MTP_FMT_Q4_0; }

// Checks shared by the dense GEMM and the MoE weight sets.
int check_packed(const char *who, int format, int K, const void *packed) {
  if (!valid_format(format)) return fail(MTP_ERR_FORMAT, "%s: unknown weight format %d", who, format);
  if (K < 32 || K % 32) return fail(MTP_ERR_SHAPE, "%s: K=%d must be a positive multiple of 32", who, K);
  if (!packed) return fail(MTP_ERR_NULL, "%s: packed weights are required", who);
  if (!aligned(packed, 16)) return fail(MTP_ERR_ALIGN, "%s: packed weights must be 16-byte aligned", who);
  return MTP_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr int kMaxAcceptRows = 64;
constexpr int kMaxVocab = 1 << 26;
constexpr int kMaxSampledSeqs = 1024;
constexpr int kMaxPenaltyWindow = 4096;

int check_accept_common(const char *who, const float *logits, int M, int V, int64_t ldl,
                        const int32_t *drafts, int32_t *tokens, int32_t *counts,
                        int64_t *rollback, void *ws, size_t ws_bytes) {
  if (M < 1 || M > kMaxAcceptRows) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, %d]", who, M, kMaxAcceptRows);
  if (V < 1 || V > kMaxVocab) return fail(MTP_ERR_SHAPE, "%s: V=%d out of [1, %d]", who, V, kMaxVocab);
  if (ldl < V) return fail(MTP_ERR_SHAPE, "%s: ldl=%lld < V=%d", who, (long long)ldl, V);
  if (!logits || !tokens || !counts || !rollback)
    return fail(MTP_ERR_NULL, "%s: logits and outputs are required", who);
  if (M > 1 && !drafts) return fail(MTP_ERR_NULL, "%s: draft_ids required for M > 1", who);
  if (!aligned(logits, 4)) return fail(MTP_ERR_ALIGN, "%s: logits must be 4-byte aligned", who);
  const size_t need = mtp::accept_ws_bytes(M, V);
  if (!ws || ws_bytes < need)
    return fail(MTP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(MTP_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  return MTP_OK;
}

}  // namespace

extern "C" {

int mtp_abi_version(void) { return MTP_ABI_VERSION; }

const char *mtp_last_error(void) { return g_error.c_str(); }

size_t mtp_packed_weight_bytes(int N, int K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return mtp::packed_weight_bytes(N, K);
}

int mtp_pack_weights(int format, int count, int N, int K, const uint8_t *codes,
                     const void *scales, uint8_t *packed, void *stream) {
  const char *who = "mtp_pack_weights";
  if (!valid_format(format)) return fail(MTP_ERR_FORMAT, "%s: unknown weight format %d", who, format);
  if (K < 32 || K % 32) return fail(MTP_ERR_SHAPE, "%s: K=%d must be a positive multiple of 32", who, K);
  if (N < 1 || count < 1) return fail(MTP_ERR_SHAPE, "%s: N=%d and count=%d must be positive", who, N, count);
  const int64_t blocks = (int64_t)count * ((N + 15) / 16) * ((K + 255) / 256);
  if (blocks > INT32_MAX) return fail(MTP_ERR_SHAPE, "%s: %lld blocks exceed one launch", who, (long long)blocks);
  if (!codes || !scales || !packed) return fail(MTP_ERR_NULL, "%s: codes, scales and packed are required", who);
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(packed, 16))
    return fail(MTP_ERR_ALIGN, "%s: codes, scales and packed must be 16-byte aligned", who);
  const size_t cb = (size_t)count * N * (K / 2);
  const size_t sb = (size_t)count * N * (format == MTP_FMT_NVFP4 ? K / 16 : (K / 32) * 2);
  const size_t pb = (size_t)count * mtp::packed_weight_bytes(N, K);
  if (overlaps(packed, pb, codes, cb) || overlaps(packed, pb, scales, sb))
    return fail(MTP_ERR_SHAPE, "%s: packed output overlaps the source", who);
  return hip_status(mtp::launch_pack(format, count, N, K, codes, scales, packed,
                                     static_cast<hipStream_t>(stream)),
                    who);
}

size_t mtp_gemm_workspace_bytes(int N, int K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return mtp::gemm_ws_bytes(N, K);
}

int mtp_verify_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                    const uint8_t *packed, float global_scale, float *y, int64_t ldy,
                    uint16_t *y_bf16, int64_t ldyb, void *ws, size_t ws_bytes, void *stream) {
  const char *who = "mtp_verify_gemm";
  if (int rc = check_packed(who, format, K, packed)) return rc;
  if (M < 1 || M > MTP_MAX_M) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, %d]", who, M, MTP_MAX_M);
  if (N < 1) return fail(MTP_ERR_SHAPE, "%s: N=%d must be positive", who, N);
  if (!x) return fail(MTP_ERR_NULL, "%s: x is required", who);
  if (!y && !y_bf16) return fail(MTP_ERR_NULL, "%s: y or y_bf16 is required", who);
  if (ldx < K) return fail(MTP_ERR_SHAPE, "%s: ldx=%lld < K=%d", who, (long long)ldx, K);
  if (ldx % 8 || !aligned(x, 16)) return fail(MTP_ERR_ALIGN, "%s: x must be 16-byte aligned with ldx %% 8 == 0", who);
  if (((int64_t)(M - 1) * ldx + K) * 2 >= ((int64_t)1 << 31))
    return fail(MTP_ERR_SHAPE, "%s: the %d activation rows span 2 GiB or more", who, M);
  if (y && ldy < N) return fail(MTP_ERR_SHAPE, "%s: ldy=%lld < N=%d", who, (long long)ldy, N);
  if (y_bf16 && ldyb < N) return fail(MTP_ERR_SHAPE, "%s: ldyb=%lld < N=%d", who, (long long)ldyb, N);
  if (y && !aligned(y, 4)) return fail(MTP_ERR_ALIGN, "%s: y must be 4-byte aligned", who);
  if (y_bf16 && !aligned(y_bf16, 2)) return fail(MTP_ERR_ALIGN, "%s: y_bf16 must be 2-byte aligned", who);
  const mtp::GemmPlan plan = mtp::gemm_plan(format, M, N, K);
  if (plan.ws_bytes && (!ws || ws_bytes < plan.ws_bytes))
    return fail(MTP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who,
                plan.ws_bytes, ws ? ws_bytes : (size_t)0);
  if (plan.ws_bytes && !aligned(ws, 256)) return fail(MTP_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  return hip_status(mtp::launch_gemm(format, M, N, K, x, ldx, packed, global_scale, y, ldy,
                                     y_bf16, ldyb, plan.ws_bytes ? ws : nullptr, plan,
                                     static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_gemm_plan_info(int format, int M, int N, int K, int32_t *info, int n) {
  const char *who = "mtp_gemm_plan_info";
  if (!valid_format(format)) return fail(MTP_ERR_FORMAT, "%s: unknown weight format %d", who, format);
  if (M < 1 || M > MTP_MAX_M || N < 1 || K < 32 || K % 32)
    return fail(MTP_ERR_SHAPE, "%s: bad shape M=%d N=%d K=%d", who, M, N, K);
  if (!info || n < 1) return fail(MTP_ERR_NULL, "%s: info is required", who);
  const mtp::GemmPlan p = mtp::gemm_plan(format, M, N, K);
  const int32_t v[14] = {p.T,       p.P,       p.S,    p.ppj,         p.J,
                         p.KG,      p.TW,      p.TG,   p.G,           p.grid,
                         p.threads, (int32_t)p.lds,    (int32_t)p.ws_bytes, p.PP};
  for (int i = 0; i < n && i < 14; ++i) info[i] = v[i];
  g_error.clear();
  return MTP_OK;
}

size_t mtp_moe_workspace_bytes(int T, int H, int F, int E, int topk) {
  if (T < 1 || topk < 1 || (int64_t)T * topk > 1024 || E < 1 || H < 32 || H % 32 || F < 32 || F % 32)
    return 0;
  return mtp::moe_ws_bytes(T, H, F, E, topk);
}

int mtp_verify_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                   const int32_t *topk_ids, const float *topk_w, const uint8_t *gu_packed,
                   const float *gu_global, const uint8_t *dn_packed, const float *dn_global,
                   float *out, uint16_t *h_out, void *ws, size_t ws_bytes, void *stream) {
  const char *who = "mtp_verify_moe";
  if (!valid_format(format)) return fail(MTP_ERR_FORMAT, "%s: unknown weight format %d", who, format);
  if (T < 1 || topk < 1 || (int64_t)T * topk > 1024)
    return fail(MTP_ERR_SHAPE, "%s: need T >= 1, topk >= 1, T*topk <= 1024 (T=%d, topk=%d)", who, T, topk);
  if (E < 1 || E > (1 << 20)) return fail(MTP_ERR_SHAPE, "%s: E=%d out of [1, 2^20]", who, E);
  if (int rc = check_packed(who, format, H, gu_packed)) return rc;
  if (int rc = check_packed(who, format, F, dn_packed)) return rc;
  if (!x || !topk_ids || !topk_w || !out) return fail(MTP_ERR_NULL, "%s: x, ids, weights and out are required", who);
  if (!aligned(x, 16)) return fail(MTP_ERR_ALIGN, "%s: x must be 16-byte aligned", who);
  if (!mtp::moe_fits(format, T, H, F))
    return fail(MTP_ERR_SHAPE, "%s: H=%d, F=%d too large for one expert pass", who, H, F);
  const size_t need = mtp::moe_ws_bytes(T, H, F, E, topk);
  if (!ws || ws_bytes < need)
    return fail(MTP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(MTP_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  return hip_status(mtp::launch_moe(format, T, H, F, E, topk, x, topk_ids, topk_w, gu_packed,
                                    gu_global, dn_packed, dn_global, out, h_out, ws,
                                    static_cast<hipStream_t>(stream)),
                    who);
}

size_t mtp_accept_workspace_bytes(int M, int V) {
  if (M < 1 || M > kMaxAcceptRows || V < 1 || V > kMaxVocab) return 0;
  return mtp::accept_ws_bytes(M, V);
}

int mtp_accept_greedy(const float *logits, int M, int V, int64_t ldl, const int32_t *draft_ids,
                      int64_t base_len, int32_t *out_tokens, int32_t *out_counts,
                      int64_t *out_rollback, void *ws, size_t ws_bytes, void *stream) {
  const char *who = "mtp_accept_greedy";
  if (int rc = check_accept_common(who, logits, M, V, ldl, draft_ids, out_tokens, out_counts,
                                   out_rollback, ws, ws_bytes))
    return rc;
  return hip_status(mtp::launch_accept_greedy(logits, M, V, ldl, draft_ids, base_len, out_tokens,
                                              out_counts, out_rollback, ws,
                                              static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_accept_greedy_static(const float *logits, int M, int V, int64_t ldl,
                             const int32_t *draft_ids, int64_t base_len, int32_t *out_tokens,
                             int32_t *out_counts, int64_t *out_rollback, void *stream) {
  const char *who = "mtp_accept_greedy_static";
  if (M < 1 || M > kMaxAcceptRows) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, %d]", who, M, kMaxAcceptRows);
  if (V < 1 || V > kMaxVocab) return fail(MTP_ERR_SHAPE, "%s: V=%d out of [1, %d]", who, V, kMaxVocab);
  if (ldl < V) return fail(MTP_ERR_SHAPE, "%s: ldl=%lld < V=%d", who, (long long)ldl, V);
  if (!logits || !out_tokens || !out_counts || !out_rollback)
    return fail(MTP_ERR_NULL, "%s: logits and outputs are required", who);
  if (M > 1 && !draft_ids) return fail(MTP_ERR_NULL, "%s: draft_ids required for M > 1", who);
  if (!aligned(logits, 4)) return fail(MTP_ERR_ALIGN, "%s: logits must be 4-byte aligned", who);
  const size_t need = mtp::greedy_static_bytes(M, V), have = mtp::greedy_static_max_bytes();
  if (need > have)
    return fail(MTP_ERR_SHAPE, "%s: M=%d, V=%d needs %zu bytes of scratch, the library holds %zu",
                who, M, V, need, have);
  return hip_status(mtp::launch_accept_greedy_static(logits, M, V, ldl, draft_ids, base_len,
                                                     out_tokens, out_counts, out_rollback,
                                                     static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_depth_observe_device(double *reached, double *accepted, int dmax, int depth,
                             const int32_t *counts, double keep, const double *cost,
                             int32_t *choice, double *prob, int32_t *err, void *stream) {
  const char *who = "mtp_depth_observe_device";
  if (!reached || !accepted || !counts)
    return fail(MTP_ERR_NULL, "%s: reached, accepted and counts are required", who);
  if (choice && !cost) return fail(MTP_ERR_NULL, "%s: cost is required with choice", who);
  if (dmax < 1 || dmax > 63) return fail(MTP_ERR_SHAPE, "%s: dmax=%d out of [1, 63]", who, dmax);
  if (depth < 0) return fail(MTP_ERR_SHAPE, "%s: depth=%d < 0", who, depth);
  if (!(keep >= 0.0 && keep <= 1.0))
    return fail(MTP_ERR_VALUE, "%s: keep=%g out of [0, 1]", who, keep);
  return hip_status(mtp::launch_depth_observe(reached, accepted, dmax, depth, counts, keep, cost,
                                              choice, prob, err,
                                              static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                         const float *draft_probs, int64_t ldq, const int32_t *draft_ids,
                         const float *uniforms, float temperature, float top_p, int64_t base_len,
                         int32_t *out_tokens, int32_t *out_counts, int64_t *out_rollback,
                         void *ws, size_t ws_bytes, void *stream) {
  const char *who = "mtp_accept_rejection";
  if (int rc = check_accept_common(who, logits, M, V, ldl, draft_ids, out_tokens, out_counts,
                                   out_rollback, ws, ws_bytes))
    return rc;
  if (!(temperature >= 0.0f) || temperature != temperature)
    return fail(MTP_ERR_VALUE, "%s: temperature must be >= 0 (got %g)", who, (double)temperature);
  if (top_p != top_p) return fail(MTP_ERR_VALUE, "%s: top_p is NaN", who);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (temperature == 0.0f)
    return hip_status(mtp::launch_accept_greedy(logits, M, V, ldl, draft_ids, base_len,
                                                out_tokens, out_counts, out_rollback, ws, s),
                      who);
  if (!uniforms) return fail(MTP_ERR_NULL, "%s: uniforms are required", who);
  if (M > 1 && !draft_probs) return fail(MTP_ERR_NULL, "%s: draft_probs required for M > 1", who);
  if (M > 1 && ldq < V) return fail(MTP_ERR_SHAPE, "%s: ldq=%lld < V=%d", who, (long long)ldq, V);
  return hip_status(mtp::launch_accept_rejection(logits, M, V, ldl, draft_probs, ldq, draft_ids,
                                                 uniforms, temperature, top_p, base_len,
                                                 out_tokens, out_counts, out_rollback, ws, s),
                    who);
}

static int check_attention(const char *who, int M, int Hq, int Hkv, int D, int L) {
  if (M < 1 || M > 16) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, 16]", who, M);
  if (D != 64 && D != 128 && D != 256)
    return fail(MTP_ERR_SHAPE, "%s: head dim %d is not 64, 128 or 256", who, D);
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv)
    return fail(MTP_ERR_SHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", who, Hq, Hkv);
  if ((int64_t)M * (Hq / Hkv) > 128)
    return fail(MTP_ERR_SHAPE, "%s: M * Hq / Hkv = %lld query rows per KV head above 128", who,
                (long long)M * (Hq / Hkv));
  if (L < 0 || (int64_t)(L + M) * D * 2 >= ((int64_t)1 << 31))
    return fail(MTP_ERR_SHAPE, "%s: L=%d out of range", who, L);
  if (Hkv > 65535) return fail(MTP_ERR_SHAPE, "%s: Hkv=%d above 65535", who, Hkv);
  return MTP_OK;
}

size_t mtp_verify_attention_workspace_bytes(int M, int Hq, int Hkv, int D, int L) {
  if (check_attention("mtp_verify_attention_workspace_bytes", M, Hq, Hkv, D, L)) return 0;
  return mtp::attention_ws_bytes(M, Hq, Hkv, D, L);
}

int mtp_verify_attention(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         int64_t ldk, int M, int Hq, int Hkv, int D, int L, float scale,
                         float *out, void *ws, size_t ws_bytes, void *stream) {
  const char *who = "mtp_verify_attention";
  if (int rc = check_attention(who, M, Hq, Hkv, D, L)) return rc;
  if (!q || !k_cache || !v_cache || !out)
    return fail(MTP_ERR_NULL, "%s: q, caches and out are required", who);
  if (ldk < (int64_t)L + M)
    return fail(MTP_ERR_SHAPE, "%s: ldk=%lld < L + M=%d", who, (long long)ldk, L + M);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(MTP_ERR_ALIGN, "%s: q, caches and out must be 16-byte aligned", who);
  if (!(scale == scale)) return fail(MTP_ERR_VALUE, "%s: scale is NaN", who);
  const size_t need = mtp::attention_ws_bytes(M, Hq, Hkv, D, L);
  if (!ws || ws_bytes < need)
    return fail(MTP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(MTP_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  return hip_status(mtp::launch_verify_attention(q, k_cache, v_cache, ldk, M, Hq, Hkv, D, L, scale,
                                                 out, ws, static_cast<hipStream_t>(stream)),
                    who);
}

static int check_kv(const char *who, const void *k, const void *v, int NL, int B, int Hkv,
                    int64_t cap, int D, int ring, int M, const int64_t *base, const void *sk,
                    const void *sv) {
  if (NL < 1 || B < 1 || Hkv < 1 || (int64_t)NL * B * Hkv > ((int64_t)1 << 24))
    return fail(MTP_ERR_SHAPE, "%s: NL=%d, B=%d, Hkv=%d (each >= 1, product <= 2^24)", who, NL, B,
                Hkv);
  if (D < 8 || D > 512 || D % 8) return fail(MTP_ERR_SHAPE, "%s: D=%d (8..512, a multiple of 8)", who, D);
  if (M < 1 || M > kMaxAcceptRows) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, %d]", who, M, kMaxAcceptRows);
  if (cap < M) return fail(MTP_ERR_SHAPE, "%s: cap=%lld below M=%d", who, (long long)cap, M);
  if (ring != 0 && ring != 1) return fail(MTP_ERR_VALUE, "%s: ring=%d is not 0 or 1", who, ring);
  if (!k || !v || !base) return fail(MTP_ERR_NULL, "%s: caches and base_len are required", who);
  if (ring && (!sk || !sv)) return fail(MTP_ERR_NULL, "%s: a rotating cache needs snapshots", who);
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(sk, 16) || !aligned(sv, 16) ||
      !aligned(base, 8))
    return fail(MTP_ERR_ALIGN, "%s: caches and snapshots must be 16-byte aligned", who);
  return MTP_OK;
}

int mtp_kv_append(uint16_t *k_cache, uint16_t *v_cache, int NL, int B, int Hkv, int64_t cap,
                  int D, int ring, const uint16_t *k_new, const uint16_t *v_new, int64_t ld_new,
                  int M, const int64_t *base_len, uint16_t *snap_k, uint16_t *snap_v,
                  int32_t *err, void *stream) {
  const char *who = "mtp_kv_append";
  if (int rc = check_kv(who, k_cache, v_cache, NL, B, Hkv, cap, D, ring, M, base_len, snap_k, snap_v))
    return rc;
  if (!k_new || !v_new) return fail(MTP_ERR_NULL, "%s: k_new and v_new are required", who);
  if (ld_new < (int64_t)Hkv * D || ld_new % 8)
    return fail(MTP_ERR_SHAPE, "%s: ld_new=%lld (>= Hkv * D = %d, a multiple of 8)", who,
                (long long)ld_new, Hkv * D);
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(MTP_ERR_ALIGN, "%s: k_new and v_new must be 16-byte aligned", who);
  return hip_status(mtp::launch_kv_append(k_cache, v_cache, NL, B, Hkv, cap, D, ring, k_new, v_new,
                                          ld_new, M, base_len, snap_k, snap_v, err,
                                          static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_kv_restore(uint16_t *k_cache, uint16_t *v_cache, int NL, int B, int Hkv, int64_t cap,
                   int D, int ring, int M, const int64_t *base_len, const int64_t *rollback,
                   const uint16_t *snap_k, const uint16_t *snap_v, int32_t *err, void *stream) {
  const char *who = "mtp_kv_restore";
  if (int rc = check_kv(who, k_cache, v_cache, NL, B, Hkv, cap, D, ring, M, base_len, snap_k, snap_v))
    return rc;
  if (!rollback) return fail(MTP_ERR_NULL, "%s: rollback is required", who);
  if (!aligned(rollback, 8)) return fail(MTP_ERR_ALIGN, "%s: rollback must be 8-byte aligned", who);
  if (rollback < base_len + B && base_len < rollback + B)
    return fail(MTP_ERR_VALUE, "%s: rollback overlaps base_len", who);
  return hip_status(mtp::launch_kv_restore(k_cache, v_cache, NL, B, Hkv, cap, D, ring, M, base_len,
                                           rollback, snap_k, snap_v, err,
                                           static_cast<hipStream_t>(stream)),
                    who);
}

int mtp_read_probe(const void *src, size_t bytes, uint32_t *sink, int shape, void *stream) {
  const char *who = "mtp_read_probe";
  if (shape < 0) return mtp::read_probe_shapes();
  if (shape >= mtp::read_probe_shapes())
    return fail(MTP_ERR_VALUE, "%s: shape %d out of [0, %d)", who, shape, mtp::read_probe_shapes());
  if (!src || !sink) return fail(MTP_ERR_NULL, "%s: src and sink are required", who);
  if (!aligned(src, 16) || bytes % 16 || !aligned(sink, 4))
    return fail(MTP_ERR_ALIGN, "%s: src and bytes must be multiples of 16", who);
  return hip_status(
      mtp::launch_read_probe(src, bytes, sink, shape, static_cast<hipStream_t>(stream)), who);
}

size_t mtp_accept_sampled_workspace_bytes(int B, int M, int V, int top_k, int penalties) {
  if (B < 1 || B > kMaxSampledSeqs || M < 1 || M > kMaxAcceptRows || V < 1 || V > kMaxVocab ||
      top_k < 1 || top_k > MTP_MAX_TOP_K)
    return 0;
  return mtp::sampled_ws_bytes(B, M, V, top_k, penalties != 0);
}

int mtp_accept_sampled(const float *logits, int B, int M, int V, int64_t ldl,
                       const int32_t *history, const int32_t *history_len, int64_t ldh,
                       const int32_t *draft_ids, const float *draft_probs, int64_t ldq,
                       const int32_t *draft_topk_ids, const float *draft_topk_probs, int Kq,
                       const float *uniforms, const mtp_sampler *params, const int64_t *base_len,
                       int32_t *out_tokens, int32_t *out_counts, int64_t *out_rollback,
                       int32_t *out_target_ids, float *out_target_probs, void *ws,
                       size_t ws_bytes, void *stream) {
  const char *who = "mtp_accept_sampled";
  if (!params) return fail(MTP_ERR_NULL, "%s: params are required", who);
  const mtp_sampler s = *params;
  if (B < 1 || B > kMaxSampledSeqs)
    return fail(MTP_ERR_SHAPE, "%s: B=%d out of [1, %d]", who, B, kMaxSampledSeqs);
  if (M < 1 || M > kMaxAcceptRows) return fail(MTP_ERR_SHAPE, "%s: M=%d out of [1, %d]", who, M, kMaxAcceptRows);
  if (V < 1 || V > kMaxVocab) return fail(MTP_ERR_SHAPE, "%s: V=%d out of [1, %d]", who, V, kMaxVocab);
  if (ldl < V) return fail(MTP_ERR_SHAPE, "%s: ldl=%lld < V=%d", who, (long long)ldl, V);
  if (!logits || !uniforms || !out_tokens || !out_counts || !out_rollback)
    return fail(MTP_ERR_NULL, "%s: logits, uniforms and outputs are required", who);
  if (!aligned(logits, 4)) return fail(MTP_ERR_ALIGN, "%s: logits must be 4-byte aligned", who);
  if (!(s.temperature >= 0.0f))
    return fail(MTP_ERR_VALUE, "%s: temperature must be >= 0 (got %g)", who, (double)s.temperature);
  if (s.top_p != s.top_p || s.min_p != s.min_p || s.repeat_penalty != s.repeat_penalty ||
      s.presence_penalty != s.presence_penalty || s.frequency_penalty != s.frequency_penalty)
    return fail(MTP_ERR_VALUE, "%s: NaN sampler parameter", who);
  if (s.top_k < 1 || s.top_k > MTP_MAX_TOP_K)
    return fail(MTP_ERR_VALUE, "%s: top_k=%d out of [1, %d] (this path keeps the top-k entries)",
                who, s.top_k, MTP_MAX_TOP_K);
  if (!(s.repeat_penalty > 0.0f))
    return fail(MTP_ERR_VALUE, "%s: repeat_penalty must be > 0", who);
  if (s.penalty_last_n > kMaxPenaltyWindow)
    return fail(MTP_ERR_VALUE, "%s: penalty_last_n=%d above %d", who, s.penalty_last_n,
                kMaxPenaltyWindow);
  if (history && !history_len) return fail(MTP_ERR_NULL, "%s: history needs history_len", who);
  if (history && ldh < 1) return fail(MTP_ERR_SHAPE, "%s: ldh=%lld < 1", who, (long long)ldh);
  if (M > 1) {
    if (!draft_ids) return fail(MTP_ERR_NULL, "%s: draft_ids required for M > 1", who);
    if (draft_probs) {
      if (ldq < V) return fail(MTP_ERR_SHAPE, "%s: ldq=%lld < V=%d", who, (long long)ldq, V);
    } else {
      if (!draft_topk_ids || !draft_topk_probs)
        return fail(MTP_ERR_NULL, "%s: dense or sparse draft distributions required for M > 1",
                    who);
      if (Kq < 1 || Kq > MTP_MAX_TOP_K)
        return fail(MTP_ERR_SHAPE, "%s: Kq=%d out of [1, %d]", who, Kq, MTP_MAX_TOP_K);
    }
  }
  if ((out_target_ids == nullptr) != (out_target_probs == nullptr))
    return fail(MTP_ERR_NULL, "%s: target ids and probs are written together", who);
  const bool pen = s.penalty_last_n > 0 &&
                   (s.repeat_penalty != 1.0f || s.presence_penalty != 0.0f ||
                    s.frequency_penalty != 0.0f);
  const size_t need = mtp::sampled_ws_bytes(B, M, V, s.top_k, pen);
  if (!ws || ws_bytes < need)
    return fail(MTP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(MTP_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  mtp::SampledCall c;
  c.logits = logits; c.B = B; c.M = M; c.V = V; c.ldl = ldl;
  c.history = history; c.history_len = history_len; c.ldh = ldh;
  c.drafts = draft_ids; c.q = draft_probs; c.ldq = ldq;
  c.q_ids = draft_probs ? nullptr : draft_topk_ids;
  c.q_probs = draft_probs ? nullptr : draft_topk_probs;
  c.Kq = draft_probs ? 0 : Kq;
  c.uniforms = uniforms;
  c.temperature = s.temperature; c.top_p = s.top_p; c.min_p = s.min_p; c.top_k = s.top_k;
  c.repeat_penalty = s.repeat_penalty; c.presence_penalty = s.presence_penalty;
  c.frequency_penalty = s.frequency_penalty; c.penalty_last_n = s.penalty_last_n;
  c.base_len = base_len;
  c.tokens = out_tokens; c.counts = out_counts; c.rollback = out_rollback;
  c.out_ids = out_target_ids; c.out_probs = out_target_probs;
  return hip_status(mtp::launch_accept_sampled(c, ws, static_cast<hipStream_t>(stream)), who);
}

}  // extern "C\"
