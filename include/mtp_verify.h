/*
 * mtp_verify.h -- the verification pass of multi-token-prediction (MTP)
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages' own sections):
 *
 *  - The verify GEMM.  "Faster Gemma 4 on MLX with multi-token prediction"
 *    (Ollama news item), sixth paragraph: verification costs most of an MTP
 *    step; its batch of 2-8 tokens sits between matrix-vector and large
 *    matrix-matrix shapes; the kernel reads and unpacks every block of nvfp4
 *    weights once and reuses it for the whole batch, with computation
 *    identical to the per-token product.  The Qiita roofline article (§2-3)
 *    adds that the weight bytes stay the same while only the arithmetic
 *    grows with the batch, and ("前提") fixes Q4-class weights at about half
 *    a byte per parameter.
 *  - The MoE variant.  Same article, §3-2: a verify mini-batch routes its
 *    tokens to more distinct experts ("expert scattering"), so the unique
 *    expert bytes grow with the batch; each unique expert is read once here.
 *  - Acceptance.  Gemini Nano summary, analysis §3, and the Qiita article,
 *    §2-4: greedy verification keeps the longest prefix agreeing with the
 *    target and always commits one more token.  MTPLX blog post, "Why it is
 *    interesting on a Mac specifically": Leviathan/Chen rejection sampling
 *    with residual correction at temperature 0.6, top_p 0.95.  Ollama mtp.go
 *    commit log, sampler rework and "greedy is a special case": temperature,
 *    softmax, top-p, normalise, categorical; at temperature 0 acceptance is
 *    argmax matching.  Ollama news item, fifth paragraph: a rollback point is
 *    recorded so that a rejection rewinds to the last accepted token.
 *  - Around the pass: the full sampler (penalties, top-k, top-p, min-p) in
 *    the acceptance of B sequences (Ollama mtp.go commit log, MLX sampler
 *    rework); the draft-depth controller (same log, controller message);
 *    multi-row verify attention over a shared KV prefix (Qiita roofline
 *    article, §2-3); cache rollback with lazy snapshots (same log, snapshot
 *    rework).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory, including the workspace; the library never allocates, frees or
 *    keeps device memory, and keeps no pointer after it returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) of the calling thread's current
 *    device.  The library never synchronises.  Buffers must stay alive
 *    until the stream passes the work.
 *  - Return value: MTP_OK (0) or a negative MTP_ERR_* code.  Arguments are
 *    checked on the host before anything is enqueued; on error nothing is
 *    enqueued and mtp_last_error() describes the problem.  Launch failures
 *    return MTP_ERR_HIP.  Device faults surface at the caller's next
 *    synchronisation.  Device-resident data (ids, uniforms) is never read on
 *    the host; out-of-range ids are handled as documented per call.
 *  - Calls are reentrant; the only global state is the thread-local error
 *    string.  Calls that share a workspace must be ordered on one stream.
 *
 * Weight formats (the pages name "nvfp4" and "Q4"; the layouts are this
 * library's).  A K x N matrix used as y = x . W is given per output row n in
 * the row-major SOURCE layout:
 *   codes : uint8 [N][K/2]; weight (n, k) is the low nibble of byte
 *           n*K/2 + k/2 for even k and the high nibble for odd k.
 *   MTP_FMT_NVFP4: nibble = E2M1 (bit3 sign, bits2..1 exponent bias 1, bit0
 *           mantissa); scales = uint8 E4M3 "FN" [N][K/16] (bias 7, 0x7F/0xFF
 *           NaN); w = global_scale * e4m3(scale[n][k/16]) * e2m1(nibble).
 *   MTP_FMT_Q4_0: nibble u = offset-binary int4; scales = IEEE fp16
 *           [N][K/32]; w = global_scale * f16(scale[n][k/32]) * (u - 8).
 *   K must be a positive multiple of 32.
 * The GEMM reads weights in a PACKED layout made once (at load time) by
 * mtp_pack_weights: for tile t (rows 16t .. 16t+15) and pair p (k = 256p ..
 * 256p+255) a 2304-byte block at byte (t * ceil(K/256) + p) * 2304.  With
 * lane l = 16g + r (row 16t + r), k0 = 256p + 32g and k1 = k0 + 128:
 *   nvfp4: bytes [16l, 16l+16)       source code bytes of k0 .. k0+31
 *          bytes [1024+16l, +16)     source code bytes of k1 .. k1+31
 *          bytes [2048+4l, +4)       scales of k0, k0+16, k1, k1+16
 *   Q4_0:  bytes [16l + 4q, +4)      source code bytes of k = 256p + 32q + 8g
 *                                    .. +7 (q = 0..3), bytes [1024 + 16l + 4q,
 *                                    +4) the same with k + 128
 *          bytes [2048+16r, +16)     the 8 fp16 scales of row 16t+r, blocks
 *                                    8p .. 8p+7
 * Rows past N and k past K are zero codes with zero scales.  This is the
 * order in which the matrix cores consume operands, so each wave streams
 * 1 KiB-contiguous loads and decodes every weight once.  Matrices stacked
 * along N (fused Q/K/V, gate||up) are just more rows.
 * Activations: bf16 bit patterns (uint16), row-major with a row stride in
 * elements; accumulation is fp32.
 */
#ifndef MTP_VERIFY_H
#define MTP_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_ABI_VERSION 8

enum {
  MTP_OK = 0,
  MTP_ERR_NULL = -1,      /* a required pointer is NULL                       */
  MTP_ERR_SHAPE = -2,     /* a size, count or stride is out of range          */
  MTP_ERR_ALIGN = -3,     /* a pointer or stride breaks an alignment rule     */
  MTP_ERR_FORMAT = -4,    /* unknown weight format                            */
  MTP_ERR_WORKSPACE = -5, /* workspace missing or smaller than required       */
  MTP_ERR_HIP = -6,       /* a HIP launch failed                              */
  MTP_ERR_VALUE = -7      /* a scalar argument is out of range (temperature)  */
};

enum { MTP_FMT_NVFP4 = 1, MTP_FMT_Q4_0 = 2 };

/* Largest row count of one verify pass (drafts + 1). */
#define MTP_MAX_M 16

/*
 * Bytes of one packed K x N matrix: ceil(N/16) * ceil(K/256) * 2304.
 * Returns 0 for N < 1 or K not a positive multiple of 32.
 */
size_t mtp_packed_weight_bytes(int N, int K);

/*
 * Repack `count` stacked source matrices (codes [count][N][K/2], scales
 * [count][N][K/16] bytes for nvfp4 or [count][N][K/32] fp16 for Q4_0) into
 * the packed layout, matrix i at packed + i * mtp_packed_weight_bytes(N, K).
 * A pure data movement (no arithmetic on weights); run once at load time.
 *   codes, scales  device, 16-byte aligned; packed  device, 16-byte aligned,
 *   not overlapping the sources.  count >= 1, N >= 1, K as above.
 */
int mtp_pack_weights(int format, int count, int N, int K, const uint8_t *codes,
                     const void *scales, uint8_t *packed, void *stream);

/*
 * Verify GEMM: y[m][n] = global_scale * sum_k x[m][k] * w(n, k) for
 * m < M, n < N, with every weight byte read once for all M rows.
 *   format       MTP_FMT_NVFP4 or MTP_FMT_Q4_0
 *   M            1..MTP_MAX_M rows (the committed token plus the drafts)
 *   N, K         output columns (>= 1) and reduction length (multiple of 32)
 *   x, ldx       bf16 [M][ldx], ldx >= K, ldx % 8 == 0, x 16-byte aligned;
 *                the M rows span less than 2 GiB ((M - 1) * ldx + K < 2^30)
 *   packed       the weight matrix in the packed layout (mtp_pack_weights),
 *                16-byte aligned
 *   global_scale (host) fp32 multiplier applied to every weight
 *   y, ldy       fp32 output [M][ldy], ldy >= N; may be NULL if y_bf16 is set
 *   y_bf16,ldyb  optional bf16 copy of y (round to nearest even) [M][ldyb];
 *                may be NULL.  At least one of y and y_bf16 must be non-NULL.
 *   ws, ws_bytes workspace of at least mtp_gemm_workspace_bytes(N, K) bytes
 *                (NULL allowed when that is 0), 256-byte aligned.  Its first
 *                max(256 KiB, 4 * ceil(N/16)) bytes hold arrival counters
 *                that must be ZERO before its first use (fill it with zeros
 *                once); every call leaves them zero again, and the partial
 *                sums follow them.  One workspace (of the largest size
 *                needed) may serve any sequence of matrices with N <=
 *                1048576; a matrix with more rows needs one of its own (or
 *                a refill with zeros before and after it).  Between GEMM
 *                calls nothing else may write it, and calls sharing it must
 *                be ordered on one stream.
 * Accuracy: |y - exact| <= 1e-3 * sum_k |x * w| + 1e-5 (fp32 accumulation).
 * An infinity or NaN in x[m] makes every output of row m non-finite: nvfp4
 * follows IEEE products and sums (+-inf, NaN where an infinity meets a zero
 * weight); Q4_0 gives NaN (its per-block offset correction subtracts the
 * infinite block sum).
 * Results are deterministic, and row m's result depends only on x[m] and W
 * (not on M or the other rows): the K split is a function of (N, K) alone.
 */
int mtp_verify_gemm(int format, int M, int N, int K, const uint16_t *x, int64_t ldx,
                    const uint8_t *packed, float global_scale, float *y, int64_t ldy,
                    uint16_t *y_bf16, int64_t ldyb, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for mtp_verify_gemm on an N x K matrix, any M (may be 0). */
size_t mtp_gemm_workspace_bytes(int N, int K);

/*
 * Diagnostic: the launch shape mtp_verify_gemm uses for (format, M, N, K).
 * Writes min(n, 14) int32 values to host array `info`: tiles T (16 rows),
 * pairs P (256 K), K slices S, pairs per slice, slices per workgroup J,
 * workgroups per tile group KG, tiles per workgroup TW, tile groups, resident
 * workgroups per K group, grid size, threads per workgroup, dynamic LDS bytes,
 * workspace bytes this M needs, weight blocks each wave keeps in flight.
 * Enqueues nothing.
 */
int mtp_gemm_plan_info(int format, int M, int N, int K, int32_t *info, int n);

/*
 * Routed MoE verify pass for T token rows, each routed to `topk` of E
 * experts.  Expert e is a gated FFN H -> F -> H:
 *   a = W_gu[e] . x_t   (2F outputs: rows [0, F) gate, rows [F, 2F) up)
 *   h = bf16_rne( silu(a_gate) * a_up ),  silu(v) = v / (1 + exp(-v))
 *   y = W_d[e] . h      (H outputs)
 *   out[t] = sum over slots s = 0..topk-1, in slot order, of topk_w[t][s] * y
 * Each expert that at least one token selects is read once for all of its
 * tokens (the grouping and deduplication run on the device).
 *   format          both weight sets use it
 *   T, H, F, E, topk  1 <= T, 1 <= topk, T*topk <= 1024, 1 <= E,
 *                   H and F multiples of 32
 *   x               bf16 [T][H] (row stride H), 16-byte aligned
 *   topk_ids        int32 [T][topk]; an id outside [0, E) contributes nothing
 *   topk_w          fp32 [T][topk]
 *   gu_packed       the E gate||up matrices (N = 2F rows, K = H), packed
 *                   and stacked: expert e at e * mtp_packed_weight_bytes(2F, H)
 *   gu_global       device fp32 [E] per-expert global scales, or NULL (1.0)
 *   dn_packed/dn_global  the same for the down projections (N = H, K = F),
 *                   expert e at e * mtp_packed_weight_bytes(H, F)
 *   out             fp32 [T][H] (must not overlap the inputs)
 *   h_out           optional bf16 [T*topk][F] copy of h (pair p = t*topk+s;
 *                   rows of out-of-range ids are zero); may be NULL
 *   ws, ws_bytes    at least mtp_moe_workspace_bytes(T, H, F, E, topk)
 */
int mtp_verify_moe(int format, int T, int H, int F, int E, int topk, const uint16_t *x,
                   const int32_t *topk_ids, const float *topk_w, const uint8_t *gu_packed,
                   const float *gu_global, const uint8_t *dn_packed, const float *dn_global,
                   float *out, uint16_t *h_out, void *ws, size_t ws_bytes, void *stream);

size_t mtp_moe_workspace_bytes(int T, int H, int F, int E, int topk);

/*
 * Greedy acceptance over M verified rows.  Row i of `logits` is the target's
 * next-token scores after row i's input (row 0: the last committed token,
 * row i+1: draft i).  g_i = argmax of row i (NaN ranks below every number,
 * the lowest index wins ties, an all-NaN row gives 0).  a = number of leading
 * drafts with draft_ids[i] == g_i.  Outputs, written together:
 *   out_tokens[0..a] = g_0..g_a (a accepted drafts, then the correction or
 *                      bonus token), out_tokens[a+1..M-1] = -1
 *   out_counts       = {a, a + 1}   (accepted, committed)
 *   out_rollback     = base_len + a + 1 (cache length to restore to)
 *   logits, ldl      fp32 [M][ldl], 1 <= M <= 64, 1 <= V <= ldl
 *   draft_ids        int32 [M-1] (may be NULL when M == 1)
 *   ws, ws_bytes     at least mtp_accept_workspace_bytes(M, V), zero-filled
 *                    before its first use.  Its first 282 KiB hold counters
 *                    and tags that mtp_accept_rejection leaves ready for the
 *                    next call (of either kind and any shape that fits);
 *                    nothing else is kept between calls.  Calls that share
 *                    one workspace must not overlap in time.
 */
int mtp_accept_greedy(const float *logits, int M, int V, int64_t ldl, const int32_t *draft_ids,
                      int64_t base_len, int32_t *out_tokens, int32_t *out_counts,
                      int64_t *out_rollback, void *ws, size_t ws_bytes, void *stream);

/*
 * Rejection-sampling acceptance (Leviathan/Chen) with residual correction.
 * Target of row i, in fp64: e_j = exp((z_j - max z) / temperature); order j
 * by (z descending, j ascending); the nucleus is the shortest prefix whose
 * mass reaches top_p * sum(e) (top_p >= 1 keeps all, top_p <= 0 keeps one);
 * p'_j = e_j / (nucleus mass) inside the nucleus, 0 outside.
 * For i = 0..M-2: accept draft x_i iff u_i * q_i(x_i) < p'_i(x_i) (an id
 * outside [0, V) is rejected); stop at the first rejection a.  Then draw the
 * last committed token with u_{M-1}: from max(0, p'_a - q_a) if a < M-1
 * (from p'_a if that is all zero), else from p'_{M-1} (bonus).  A draw from
 * weights w picks the smallest j with w_0 + .. + w_j > u * sum(w).
 * temperature == 0 gives exactly mtp_accept_greedy; temperature < 0 or NaN
 * is MTP_ERR_VALUE.  Logits must be finite.
 *   draft_probs, ldq fp32 [M-1][ldq] (the draft's final distributions)
 *   uniforms         fp32 [M] in [0, 1), supplied by the caller (reproducible)
 *   other arguments and outputs as for mtp_accept_greedy
 */
int mtp_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                         const float *draft_probs, int64_t ldq, const int32_t *draft_ids,
                         const float *uniforms, float temperature, float top_p, int64_t base_len,
                         int32_t *out_tokens, int32_t *out_counts, int64_t *out_rollback,
                         void *ws, size_t ws_bytes, void *stream);

size_t mtp_accept_workspace_bytes(int M, int V);

/*
 * mtp_accept_greedy without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, fixed serving loops, harnesses
 * that forbid allocation).  Same computation, outputs and argument rules as
 * mtp_accept_greedy (1 <= M <= 64, 1 <= V <= 2^26, ldl >= V); its scratch
 * (the per-block partial maxima, at most 64 KiB: 8 bytes per row per block
 * of the row, 128 blocks per row at most) is a static device array inside
 * the library, one per GPU, held until the process ends.  The call
 * allocates nothing (no hipMalloc, no library allocator); a shape whose
 * scratch would exceed the array is MTP_ERR_SHAPE.  Every call on a GPU
 * writes that GPU's array before reading it, so nothing needs clearing, but
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must be ordered by the caller.
 */
int mtp_accept_greedy_static(const float *logits, int M, int V, int64_t ldl,
                             const int32_t *draft_ids, int64_t base_len, int32_t *out_tokens,
                             int32_t *out_counts, int64_t *out_rollback, void *stream);

/*
 * Sampler parameters of mtp_accept_sampled, applied in the order of the
 * Ollama mtp.go commit log's MLX sampler rework: (1) penalties, (2) top-k,
 * (3) temperature/softmax, (4) top-p, (5) min-p, (6) normalize,
 * (7) categorical.  The pages name the steps only; the formulas are the
 * usual ones:
 *   (1) for a token seen c > 0 times in the row's penalty window (the last
 *       penalty_last_n tokens of history ++ the drafts before the row; none
 *       if penalty_last_n <= 0), in fp32, each operation rounded on its own:
 *       z = z > 0 ? z / repeat_penalty : z * repeat_penalty (skipped when it
 *       is 1), then z = (z - c * frequency_penalty) - presence_penalty.
 *   (2) keep the top_k entries first in the order (z desc, index asc).
 *   (3) e = exp((z - z_max) / temperature) in fp64 (temperature 0: a point
 *       mass at the first entry of the order).
 *   (4) keep the shortest prefix of that order whose e-mass reaches top_p
 *       times the kept mass (top_p >= 1 keeps all, top_p <= 0 the first).
 *   (5) drop entries with e < min_p, i.e. p < min_p * max p (min_p <= 0:
 *       off); the first entry always stays.
 *   (6) p' = e / (mass of what is left).
 *   (7) a draw picks the smallest id with cumulative weight > u * total.
 */
typedef struct {
  float temperature;        /* >= 0 */
  float top_p;
  float min_p;
  int32_t top_k;            /* 1 .. MTP_MAX_TOP_K */
  float repeat_penalty;     /* > 0; 1 = none */
  float presence_penalty;
  float frequency_penalty;
  int32_t penalty_last_n;   /* <= MTP_MAX_PENALTY_WINDOW; <= 0: no penalties */
} mtp_sampler;

#define MTP_MAX_TOP_K 1024
#define MTP_MAX_PENALTY_WINDOW 4096

/*
 * Sampled acceptance (Leviathan/Chen rejection sampling with residual
 * correction) of B sequences of M verified rows each, on the sparse top-k
 * path: each row's target p' is built by the sampler pipeline above and kept
 * as at most top_k (id, probability) pairs on the GPU; acceptance, the
 * residual draw max(0, p'_a - q_a) (from p'_a if it is all zero) and the
 * bonus draw from p'_{M-1} reuse them (same article).  Per sequence b, with
 * u = uniforms[b]: accept draft x_i iff u_i * q_i(x_i) < p'_i(x_i), stop at
 * the first rejection a; the draws use u_{M-1}.  Outputs per sequence as
 * for mtp_accept_greedy; rollback[b] = base_len[b] + a + 1.
 *   logits, ldl      fp32 [B*M][ldl], row b*M + i (finite values)
 *   history, ldh     int32 [B][ldh] committed tokens, oldest first, or NULL;
 *   history_len      int32 [B] (device), clamped to [0, ldh]
 *   draft_ids        int32 [B][M-1]
 *   draft_probs, ldq dense fp32 [B*(M-1)][ldq], or NULL and then
 *   draft_topk_ids / draft_topk_probs: sparse [B*(M-1)][Kq] (an id not listed
 *                    has probability 0; the first listing of an id counts)
 *   uniforms         fp32 [B][M] in [0, 1)
 *   params           (host) the sampler
 *   base_len         int64 [B] (device), or NULL (0)
 *   out_tokens [B][M], out_counts [B][2], out_rollback [B]
 *   out_target_ids / out_target_probs  optional int32 / fp32 [B*M][K],
 *                    K = min(top_k, V): each row's p' in order of
 *                    probability, -1 / 0 past its support
 *   ws, ws_bytes     at least mtp_accept_sampled_workspace_bytes(B, M, V,
 *                    top_k, penalties on), zero-filled before its first use.
 *                    Its first 20 KiB hold row and sequence counters that
 *                    every call leaves zero for the next (of any shape);
 *                    nothing else is kept between calls.  Calls sharing it
 *                    must not overlap in time.
 * Errors: MTP_ERR_VALUE for temperature < 0 or NaN, a NaN parameter, top_k
 * outside [1, MTP_MAX_TOP_K], repeat_penalty <= 0 or a window above
 * MTP_MAX_PENALTY_WINDOW; 1 <= B <= 1024, 1 <= M <= 64.
 */
int mtp_accept_sampled(const float *logits, int B, int M, int V, int64_t ldl,
                       const int32_t *history, const int32_t *history_len, int64_t ldh,
                       const int32_t *draft_ids, const float *draft_probs, int64_t ldq,
                       const int32_t *draft_topk_ids, const float *draft_topk_probs, int Kq,
                       const float *uniforms, const mtp_sampler *params, const int64_t *base_len,
                       int32_t *out_tokens, int32_t *out_counts, int64_t *out_rollback,
                       int32_t *out_target_ids, float *out_target_probs, void *ws,
                       size_t ws_bytes, void *stream);

/* penalties: nonzero when penalty_last_n > 0 and a penalty differs from its
 * neutral value (the penalised rows then take a workspace copy). */
size_t mtp_accept_sampled_workspace_bytes(int B, int M, int V, int top_k, int penalties);

/*
 * Multi-row verify attention over a shared KV prefix.  Qiita roofline
 * article, §2-3: at long context the KV reads also take bandwidth, but the
 * candidates of one verify pass look at the same prefix, so one KV read
 * serves all of them (as with the weights).  For the M verify rows of one
 * sequence, row i (absolute position L + i) of query head h attends
 * causally to keys 0 .. L + i of KV head h / (Hq / Hkv):
 *   out[i][h] = softmax_j(scale * q[i][h] . k[h/G][j]) . v[h/G][j]
 * Each KV head's keys are read once for all M * Hq/Hkv query rows.  The M
 * verify tokens' own K and V must already be in the cache at positions
 * L .. L + M - 1.  Arithmetic: bf16 products with fp32 accumulation on the
 * matrix cores, fp32 online softmax, the probabilities rounded to bf16 for
 * the product with V (|error| <= 2^-8 * sum_j p_j |v_j| from that rounding).
 *   q            bf16 [M][Hq][D], 16-byte aligned
 *   k_cache,
 *   v_cache, ldk bf16 [Hkv][ldk][D] (ldk >= L + M), 16-byte aligned
 *   M            1..16; D 64, 128 or 256; Hq a multiple of Hkv with
 *                M * Hq / Hkv <= 128
 *   scale        the score scale (e.g. 1 / sqrt(D))
 *   out          fp32 [M][Hq][D]
 *   ws, ws_bytes at least mtp_verify_attention_workspace_bytes(...)
 */
int mtp_verify_attention(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         int64_t ldk, int M, int Hq, int Hkv, int D, int L, float scale,
                         float *out, void *ws, size_t ws_bytes, void *stream);
size_t mtp_verify_attention_workspace_bytes(int M, int Hq, int Hkv, int D, int L);

/*
 * KV-cache rollback with lazy snapshots.  Ollama mtp.go commit log, the
 * snapshot rework: a cache snapshots itself as a verify write crosses each
 * offset and the runner commits a batch by restoring to the accepted count;
 * a KV or rotating capture points into the live buffer and holds no copy of
 * its own until a destructive write forces one, so rejecting costs nothing.
 * Ollama news item, fifth paragraph: the restore point is the rollback index
 * that the accept calls emit (out_rollback = base_len + a + 1).
 *
 * Layout.  One call covers NL layers of the same shape: a cache is
 *   k_cache, v_cache  bf16 [NL][B][Hkv][cap][D] (contiguous, 16-byte aligned)
 * for B sequences.  A LINEAR cache (ring = 0) keeps position p in row p and
 * must have room for it (p < cap).  A ROTATING cache (ring = 1) keeps
 * position p in row p mod cap; writing p >= cap destroys position p - cap,
 * which is the one write that takes a copy.  (A rotating cache that serves a
 * sliding window of W keys to M verify rows at once needs cap >= W + M - 1.)
 *
 * mtp_kv_append: writes the M verify rows of every sequence b at positions
 *   base_len[b] .. base_len[b] + M - 1.  Before a rotating-cache row that
 *   holds a live position is overwritten, its old contents are copied to
 *   snap_k/snap_v [NL][B][Hkv][M][D] at index m = p - base_len[b]; no other
 *   snapshot row is touched, and a linear cache copies nothing (its snapshot
 *   is base_len itself; snap_k and snap_v may be NULL).
 *     k_new, v_new  bf16; row m of sequence b of layer l starts at element
 *                   ((l * B + b) * M + m) * ld_new, and holds head h at
 *                   h * D .. h * D + D - 1 (ld_new >= Hkv * D, a multiple
 *                   of 8), so a fused projection's K or V columns can be
 *                   passed in place
 *     base_len      int64 [B] (device): the cache length before the write
 *                   (e.g. the previous step's out_rollback)
 * mtp_kv_restore: commits to rollback[b] (device int64 [B], clamped into
 *   [base_len[b], base_len[b] + M]): the positions rollback[b] .. base_len[b]
 *   + M - 1 are dropped, and every rotating-cache row they overwrote gets its
 *   snapshot back, so the cache equals one that only ever received the first
 *   rollback[b] - base_len[b] rows.  For a linear cache nothing is launched
 *   and nothing is read: the new length is rollback[b] itself.  base_len, M and the snapshot must
 *   be those of the append being undone; base_len must not overlap rollback.
 *   Run it after the append and before the next write to the same cache.
 * err (device int32, may be NULL): set to a nonzero value (never cleared) if
 *   a position was negative, did not fit a linear cache (that row is not
 *   written), or a rollback lay outside its range (it is clamped).
 * Limits: 1 <= M <= 64, M <= cap, 1 <= D <= 512 a multiple of 8,
 *   NL * B * Hkv <= 2^24.
 */
int mtp_kv_append(uint16_t *k_cache, uint16_t *v_cache, int NL, int B, int Hkv, int64_t cap,
                  int D, int ring, const uint16_t *k_new, const uint16_t *v_new, int64_t ld_new,
                  int M, const int64_t *base_len, uint16_t *snap_k, uint16_t *snap_v,
                  int32_t *err, void *stream);
int mtp_kv_restore(uint16_t *k_cache, uint16_t *v_cache, int NL, int B, int Hkv, int64_t cap,
                   int D, int ring, int M, const int64_t *base_len, const int64_t *rollback,
                   const uint16_t *snap_k, const uint16_t *snap_v, int32_t *err, void *stream);

/*
 * Draft-depth controller (host functions; no GPU work).  Ollama mtp.go
 * commit log: the depth drafted is the one that maximises committed tokens
 * per wall-clock, from live per-position acceptance and the measured forward
 * cost per width, with no depth cap; MTPLX blog post: plain decoding stays
 * the baseline.  A step of depth d verifies M = d + 1 rows and commits
 * E(d) = 1 + sum_{i=1..d} prod_{j<=i} accept_prob[j-1] tokens in
 * expectation.
 *
 * mtp_choose_draft_depth: returns the d in [0, dmax] with the largest
 *   E(d) / cost[d] (the smallest d on a tie; d = 0 is plain decoding) and
 *   writes E(d) / cost[d] to rate[0..dmax] if rate is not NULL.
 *   accept_prob [dmax] in [0, 1]; cost [dmax + 1] > 0 (e.g. microseconds of
 *   the verify pass at M = d + 1 plus drafting d tokens); dmax in [0, 63].
 *   Errors: MTP_ERR_NULL, MTP_ERR_SHAPE (dmax), MTP_ERR_VALUE (a cost <= 0
 *   or NaN, a probability outside [0, 1]).
 * mtp_depth_observe: after a step of depth `depth` that accepted n_accepted
 *   drafts, positions 1..min(n_accepted + 1, depth) were reached and
 *   1..n_accepted accepted; reached[] and accepted[] (length dmax, caller
 *   owned, start at 0) are multiplied by keep in [0, 1] (1: plain counts),
 *   then counted.
 * mtp_depth_estimate: prob[i] = (accepted[i] + 1) / (reached[i] + 2)
 *   (Laplace's rule: 1/2 before any evidence).
 */
int mtp_choose_draft_depth(const double *accept_prob, const double *cost, int dmax, double *rate);
int mtp_depth_observe(double *reached, double *accepted, int dmax, int depth, int n_accepted,
                      double keep);
int mtp_depth_estimate(const double *reached, const double *accepted, int dmax, double *prob);

/*
 * The same controller on the device, enqueued on `stream` after the accept
 * call of a step of depth `depth`, so that the host reads nothing per step
 * ("Faster Gemma 4 on MLX with multi-token prediction", fourth and fifth
 * paragraphs: the runtime tunes the depth from acceptance and verify
 * timings, with no return to the CPU).  With n = counts[0] (the accepted
 * count the accept call wrote, device int32):
 *   reached, accepted   device fp64 [dmax], updated as mtp_depth_observe
 *                       updates them (the same fp64 operations, so the two
 *                       agree bit for bit);
 *   prob (optional)     device fp64 [dmax]: mtp_depth_estimate of the update;
 *   choice (optional)   device int32 [1]: mtp_choose_draft_depth of prob and
 *                       cost (device fp64 [dmax + 1], required with choice).
 * The host may read choice whenever it likes (for instance with an
 * asynchronous copy behind an event), or a drafting kernel may read it on
 * the device.  Device-side errors go to err (optional, device int32 [1]):
 * 0 ok; 1 counts[0] outside [0, depth] (the statistics are left as they
 * were); 2 a cost <= 0 or NaN (choice 0).  Host errors, returned before
 * anything is enqueued: MTP_ERR_NULL (reached, accepted or counts; cost with
 * choice), MTP_ERR_SHAPE (dmax outside [1, 63], depth < 0), MTP_ERR_VALUE
 * (keep outside [0, 1]).
 */
int mtp_depth_observe_device(double *reached, double *accepted, int dmax, int depth,
                             const int32_t *counts, double keep, const double *cost,
                             int32_t *choice, double *prob, int32_t *err, void *stream);

/*
 * Read-bandwidth probe (a measurement aid, not a step of the verify pass):
 * reads every 16-byte piece of src[0 .. bytes) once with non-temporal vector
 * loads in launch shape `shape` (0 .. n-1: loads in flight per thread and
 * grid size) and folds them so that no load can be dropped; *sink (device,
 * 4-byte aligned) is written only when the fold equals one fixed value.
 * Timed on buffers of a verify matrix's size, the best shape gives the read
 * rate a launch of that size reaches: the ceiling the verify GEMM is
 * compared with.  shape < 0 returns n (the number of shapes).
 * Errors: MTP_ERR_VALUE (shape >= n), MTP_ERR_NULL, MTP_ERR_ALIGN (src not
 * 16-byte aligned, bytes not a multiple of 16).
 */
int mtp_read_probe(const void *src, size_t bytes, uint32_t *sink, int shape, void *stream);

/* Thread-local message for the last non-zero status of this thread. */
const char *mtp_last_error(void);

int mtp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTP_VERIFY_H */
