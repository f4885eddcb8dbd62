/*
 * CPU oracle for the multi-token-prediction verification pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Everything here is the plain definition, written for a reader to check by
 * eye, evaluated serially in fp64:
 *
 *   - "Faster Gemma 4 on MLX with multi-token prediction" (Ollama news item),
 *     sixth paragraph: the verify pass multiplies a batch of 2-8 token rows by
 *     nvfp4 block-quantised weights, reading and unpacking every weight block
 *     once for the whole batch, with computation identical to the per-token
 *     product.  The oracle is that product: y[m][n] = sum_k x[m][k] * w[k][n].
 *   - Qiita roofline article, "前提" and §2-3: Q4-class weights (about half a
 *     byte per parameter); verification turns a matrix-vector product into a
 *     skinny matrix-matrix product over the same weights.
 *   - Same article, §2-4, and the Gemini Nano summary, analysis §3: greedy
 *     verification keeps the longest prefix matching the target's own choice
 *     and always commits one more token (the correction).
 *   - MTPLX blog post, "Why it is interesting on a Mac specifically":
 *     Leviathan/Chen rejection sampling with residual correction at
 *     temperature 0.6, top_p 0.95.
 *   - Ollama mtp.go commit log, the sampler rework (pipeline order
 *     temperature/softmax -> top-p -> normalize -> categorical) and the
 *     "greedy is a special case of sampled decoding" message (temperature 0
 *     gives a point mass, so rejection acceptance reduces to argmax match).
 *   - Ollama news item, fifth paragraph: a rollback point before each
 *     proposal; a rejection rewinds to the last accepted token.
 *   - Ollama mtp.go commit log, the snapshot rework: the runner commits a
 *     verify batch by restoring the caches to the accepted count.  The
 *     oracle is what that restore must produce: the cache as if only the
 *     accepted rows had ever been written (orc_kv_write of those rows).
 *
 * Element formats (the pages only name "nvfp4" and "Q4"; the readings used):
 *   E2M1 nibble: bit3 sign, bits2..1 exponent (bias 1), bit0 mantissa.
 *   E4M3 byte ("FN"): bit7 sign, bits6..3 exponent (bias 7), bits2..0
 *     mantissa, exponent 0 subnormal, 0x7F/0xFF NaN, no infinities.
 *   fp16: IEEE binary16.  bf16: upper half of an IEEE binary32.
 *   Weight (n,k) of a K x N matrix stored per output row n: code nibble in
 *     byte n*K/2 + k/2 (low nibble for even k).  nvfp4: one E4M3 scale per 16
 *     weights, w = g * e4m3(s[n][k/16]) * e2m1(c).  Q4_0-style: one fp16 scale
 *     per 32 weights, w = g * f16(d[n][k/32]) * (u - 8).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_NVFP4 1
#define ORC_Q4_0 2

/* ------------------------------------------------------------------------ */
/* element decoders                                                          */
/* ------------------------------------------------------------------------ */

double orc_e2m1(uint32_t code) {
    uint32_t s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

double orc_e4m3(uint32_t b) {
    uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

double orc_f16(uint32_t h) {
    uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    double mag;
    if (e == 0) mag = ldexp((double)m, -24);
    else if (e == 31) mag = m ? NAN : INFINITY;
    else mag = ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
    return s ? -mag : mag;
}

double orc_bf16(uint32_t b) {
    uint32_t u = (b & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), in one step. */
uint16_t orc_bf16_rne(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r;
    int e;
    (void)frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    if (e - 1 >= -126) {
        /* normal range: 8 significant bits */
        r = ldexp(rint(ldexp(a, 8 - e)), e - 8);
    } else {
        /* subnormal range: quantum 2^-133 */
        r = ldexp(rint(ldexp(a, 133)), -133);
    }
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)r;                  /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

static double g_e2m1[16];
static double g_e4m3[256];
static double g_f16[65536];
static pthread_once_t g_once = PTHREAD_ONCE_INIT;

static void tables_init(void) {
    for (uint32_t i = 0; i < 16; ++i) g_e2m1[i] = orc_e2m1(i);
    for (uint32_t i = 0; i < 256; ++i) g_e4m3[i] = orc_e4m3(i);
    for (uint32_t i = 0; i < 65536; ++i) g_f16[i] = orc_f16(i);
}

/* Weight (n, k) of one matrix, exactly, in fp64. */
static double weight_nk(int fmt, int K, const uint8_t *codes, const void *scales, double g,
                        int64_t n, int64_t k) {
    uint8_t byte = codes[n * (K / 2) + k / 2];
    uint32_t nib = (k & 1) ? (byte >> 4) : (byte & 15u);
    if (fmt == ORC_NVFP4) {
        uint8_t s = ((const uint8_t *)scales)[n * (K / 16) + k / 16];
        return g * g_e4m3[s] * g_e2m1[nib];
    }
    uint16_t d = ((const uint16_t *)scales)[n * (K / 32) + k / 32];
    return g * g_f16[d] * (double)((int)nib - 8);
}

double orc_weight(int fmt, int K, const uint8_t *codes, const void *scales, float g, int64_t n,
                  int64_t k) {
    pthread_once(&g_once, tables_init);
    return weight_nk(fmt, K, codes, scales, (double)g, n, k);
}

/* ------------------------------------------------------------------------ */
/* verify GEMM: y[m][n] = sum_k x[m][k] * w(n, k), serial fp64 sum over k    */
/* b[m][n] = sum_k |x[m][k] * w(n, k)|  (the error scale of the product)     */
/* ------------------------------------------------------------------------ */

typedef struct {
    int fmt, M, K;
    const double *xd;            /* [M][K] widened activations */
    const uint8_t *codes;
    const void *scales;
    double g;
    const int64_t *cols;         /* output columns to compute */
    int64_t ncols;
    double *y, *b;               /* [M][ncols] */
    int64_t begin, end;
} gemm_job;

static void *gemm_worker(void *arg) {
    gemm_job *j = (gemm_job *)arg;
    double acc[16], mag[16];
    for (int64_t c = j->begin; c < j->end; ++c) {
        int64_t n = j->cols[c];
        for (int m = 0; m < j->M; ++m) acc[m] = 0.0, mag[m] = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            double w = weight_nk(j->fmt, j->K, j->codes, j->scales, j->g, n, k);
            for (int m = 0; m < j->M; ++m) {
                double p = j->xd[(int64_t)m * j->K + k] * w;
                acc[m] += p;
                mag[m] += fabs(p);
            }
        }
        for (int m = 0; m < j->M; ++m) {
            j->y[(int64_t)m * j->ncols + c] = acc[m];
            if (j->b) j->b[(int64_t)m * j->ncols + c] = mag[m];
        }
    }
    return NULL;
}

/*
 * fmt: 1 nvfp4, 2 Q4_0-style.  x: bf16 bits [M][ldx].  cols: the output
 * columns wanted (ncols of them; NULL = all N in order).  y, b: [M][ncols]
 * (b may be NULL).  Returns 0, or -1 on bad arguments.
 */
int orc_gemm(int fmt, int M, int N, int K, const uint16_t *x, int64_t ldx, const uint8_t *codes,
             const void *scales, float g, const int64_t *cols, int64_t ncols, double *y,
             double *b, int nthreads) {
    if (M < 1 || M > 16 || K < 32 || K % 32 || N < 1 || (fmt != ORC_NVFP4 && fmt != ORC_Q4_0))
        return -1;
    pthread_once(&g_once, tables_init);
    int64_t *all = NULL;
    if (!cols) {
        all = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
        if (!all) return -1;
        for (int64_t n = 0; n < N; ++n) all[n] = n;
        cols = all;
        ncols = N;
    }
    double *xd = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!xd) { free(all); return -1; }
    for (int m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) xd[(int64_t)m * K + k] = orc_bf16(x[m * ldx + k]);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > ncols) nthreads = (int)(ncols > 0 ? ncols : 1);
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        gemm_job *j = &jobs[t];
        j->fmt = fmt; j->M = M; j->K = K; j->xd = xd; j->codes = codes; j->scales = scales;
        j->g = (double)g; j->cols = cols; j->ncols = ncols; j->y = y; j->b = b;
        j->begin = ncols * t / nthreads;
        j->end = ncols * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    gemm_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(xd);
    free(all);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* routed MoE: for each token t and slot s with expert e = ids[t][s]:        */
/*   a = W_gu[e] x_t  (rows [0,F) gate, [F,2F) up)                           */
/*   h = bf16_rne( silu(a_gate) * a_up ),  silu(v) = v / (1 + exp(-v))       */
/*   y = W_d[e] h                                                            */
/*   out[t] = sum over slots s, in slot order, of w[t][s] * y                */
/* An id outside [0, E) contributes nothing and leaves its h row at zero.    */
/* ------------------------------------------------------------------------ */

typedef struct {
    int fmt, T, H, F, E, topk;
    const double *xd;            /* [T][H] */
    const int32_t *ids;
    const float *gw;
    const uint8_t *gu_codes, *dn_codes;
    const void *gu_scales, *dn_scales;
    const float *gu_g, *dn_g;
    double *y, *yb;              /* [T*topk][H] */
    uint16_t *h;                 /* [T*topk][F] */
    double *a_out, *ab_out;      /* [T*topk][2F] pre-activations and their error scale, or NULL */
    int64_t begin, end;
} moe_job;

static void *moe_worker(void *arg) {
    moe_job *j = (moe_job *)arg;
    const int H = j->H, F = j->F;
    double *a = (double *)malloc(sizeof(double) * 2 * (size_t)F);
    double *hd = (double *)malloc(sizeof(double) * (size_t)F);
    for (int64_t p = j->begin; p < j->end; ++p) {
        int64_t t = p / j->topk;
        int32_t e = j->ids[p];
        uint16_t *hrow = j->h + p * F;
        double *yrow = j->y + p * H, *ybrow = j->yb + p * H;
        if (e < 0 || e >= j->E) {
            for (int f = 0; f < F; ++f) hrow[f] = 0;
            for (int n = 0; n < 2 * F; ++n) {
                if (j->a_out) j->a_out[p * 2 * F + n] = 0.0;
                if (j->ab_out) j->ab_out[p * 2 * F + n] = 0.0;
            }
            for (int n = 0; n < H; ++n) yrow[n] = 0.0, ybrow[n] = 0.0;
            continue;
        }
        const uint8_t *gc = j->gu_codes + (int64_t)e * (2 * F) * (H / 2);
        const uint8_t *dc = j->dn_codes + (int64_t)e * H * (F / 2);
        const void *gs, *ds;
        if (j->fmt == ORC_NVFP4) {
            gs = (const uint8_t *)j->gu_scales + (int64_t)e * (2 * F) * (H / 16);
            ds = (const uint8_t *)j->dn_scales + (int64_t)e * H * (F / 16);
        } else {
            gs = (const uint16_t *)j->gu_scales + (int64_t)e * (2 * F) * (H / 32);
            ds = (const uint16_t *)j->dn_scales + (int64_t)e * H * (F / 32);
        }
        double ggu = j->gu_g ? (double)j->gu_g[e] : 1.0;
        double gdn = j->dn_g ? (double)j->dn_g[e] : 1.0;
        for (int n = 0; n < 2 * F; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < H; ++k) {
                double pr = j->xd[t * H + k] * weight_nk(j->fmt, H, gc, gs, ggu, n, k);
                acc += pr;
                mag += fabs(pr);
            }
            a[n] = acc;
            if (j->a_out) j->a_out[p * 2 * F + n] = acc;
            if (j->ab_out) j->ab_out[p * 2 * F + n] = mag;
        }
        for (int f = 0; f < F; ++f) {
            double gate = a[f], up = a[F + f];
            double silu = gate / (1.0 + exp(-gate));
            hrow[f] = orc_bf16_rne(silu * up);
            hd[f] = orc_bf16(hrow[f]);
        }
        for (int n = 0; n < H; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int f = 0; f < F; ++f) {
                double pr = hd[f] * weight_nk(j->fmt, F, dc, ds, gdn, n, f);
                acc += pr;
                mag += fabs(pr);
            }
            yrow[n] = acc;
            ybrow[n] = mag;
        }
    }
    free(a);
    free(hd);
    return NULL;
}

/*
 * x: bf16 bits [T][H].  ids, gw: [T][topk].  Experts e are stored back to back:
 * gate/up codes [E][2F][H/2], scales [E][2F][H/bs]; down codes [E][H][F/2],
 * scales [E][H][F/bs].  gu_g, dn_g: per-expert global scales or NULL (1.0).
 * Outputs: out [T][H] and outb [T][H] = sum_s |w| * sum_f |h * w_d| (error
 * scale), h [T*topk][F] bf16 bits, and optionally the gate/up
 * pre-activations a_out [T*topk][2F] with their error scale ab_out
 * (sum_k |x * w|).  Returns 0 or -1.
 */
int orc_moe(int fmt, int T, int H, int F, int E, int topk, const uint16_t *x, const int32_t *ids,
            const float *gw, const uint8_t *gu_codes, const void *gu_scales, const float *gu_g,
            const uint8_t *dn_codes, const void *dn_scales, const float *dn_g, double *out,
            double *outb, uint16_t *h, double *a_out, double *ab_out, int nthreads) {
    if (T < 1 || topk < 1 || E < 1 || H < 32 || H % 32 || F < 32 || F % 32 ||
        (fmt != ORC_NVFP4 && fmt != ORC_Q4_0))
        return -1;
    pthread_once(&g_once, tables_init);
    int64_t P = (int64_t)T * topk;
    double *xd = (double *)malloc(sizeof(double) * (size_t)T * (size_t)H);
    double *y = (double *)malloc(sizeof(double) * (size_t)P * (size_t)H);
    double *yb = (double *)malloc(sizeof(double) * (size_t)P * (size_t)H);
    if (!xd || !y || !yb) { free(xd); free(y); free(yb); return -1; }
    for (int64_t i = 0; i < (int64_t)T * H; ++i) xd[i] = orc_bf16(x[i]);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > P) nthreads = (int)P;
    pthread_t th[256];
    moe_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        moe_job *j = &jobs[t];
        j->fmt = fmt; j->T = T; j->H = H; j->F = F; j->E = E; j->topk = topk; j->xd = xd;
        j->ids = ids; j->gw = gw; j->gu_codes = gu_codes; j->dn_codes = dn_codes;
        j->gu_scales = gu_scales; j->dn_scales = dn_scales; j->gu_g = gu_g; j->dn_g = dn_g;
        j->y = y; j->yb = yb; j->h = h; j->a_out = a_out; j->ab_out = ab_out;
        j->begin = P * t / nthreads;
        j->end = P * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, moe_worker, &jobs[t]);
    moe_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < T; ++t) {
        for (int n = 0; n < H; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int s = 0; s < topk; ++s) {
                int64_t p = (int64_t)t * topk + s;
                double w = (double)gw[p];
                acc += w * y[p * H + n];
                mag += fabs(w) * yb[p * H + n];
            }
            out[(int64_t)t * H + n] = acc;
            if (outb) outb[(int64_t)t * H + n] = mag;
        }
    }
    free(xd);
    free(y);
    free(yb);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* acceptance                                                                */
/* ------------------------------------------------------------------------ */

/* Row argmax: NaN ranks below every number, the lowest index wins ties, a
 * row of NaN gives 0. */
int32_t orc_argmax(const float *z, int V) {
    int32_t best = 0;
    float bv = z[0];
    for (int j = 1; j < V; ++j) {
        float v = z[j];
        if (isnan(v)) continue;
        if (isnan(bv) || v > bv) { best = j; bv = v; }
    }
    return best;
}

static void write_run(int M, const int32_t *run, int a, int64_t base_len, int32_t *tokens,
                      int32_t *counts, int64_t *rollback) {
    for (int i = 0; i < M; ++i) tokens[i] = (i <= a) ? run[i] : -1;
    counts[0] = a;
    counts[1] = a + 1;
    *rollback = base_len + a + 1;
}

/*
 * Greedy verification.  Row i of logits is the target's distribution after
 * row i's token; draft i is checked against row i's argmax g_i.  a = number
 * of leading drafts equal to g_0, g_1, ...; the committed run is g_0..g_a
 * (a accepted drafts plus the correction or bonus token).  Rollback index =
 * base_len + a + 1.
 */
int orc_accept_greedy(const float *logits, int M, int V, int64_t ldl, const int32_t *drafts,
                      int64_t base_len, int32_t *tokens, int32_t *counts, int64_t *rollback) {
    if (M < 1 || V < 1 || ldl < V) return -1;
    int32_t run[64];
    if (M > 64) return -1;
    int a = 0;
    run[0] = orc_argmax(logits, V);
    while (a < M - 1 && drafts[a] == run[a]) {
        ++a;
        run[a] = orc_argmax(logits + (int64_t)a * ldl, V);
    }
    write_run(M, run, a, base_len, tokens, counts, rollback);
    return 0;
}

typedef struct { float z; int32_t j; } zkey;

static int zkey_cmp(const void *pa, const void *pb) {
    const zkey *a = (const zkey *)pa, *b = (const zkey *)pb;
    if (a->z > b->z) return -1;
    if (a->z < b->z) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

/*
 * Target distribution of one row after temperature and top-p:
 *   e_j = exp((z_j - max z) / T) in fp64, S = sum_j e_j;
 *   order j by (z descending, j ascending) -- the order of probability with
 *   ties broken by index; the nucleus is the shortest prefix whose e-mass
 *   reaches top_p * S (top_p >= 1 keeps all, top_p <= 0 keeps the first);
 *   S' = e-mass of the nucleus; p'_j = e_j / S' inside, 0 outside.
 * Writes e (masked to the nucleus) and returns S'.  *margin receives the
 * relative distance of the nucleus cut from its threshold.
 */
static double target_row(const float *z, int V, double T, double top_p, double *e,
                         zkey *keys, double *margin) {
    float zm = z[0];
    for (int j = 1; j < V; ++j) zm = (z[j] > zm) ? z[j] : zm;
    double S = 0.0;
    for (int j = 0; j < V; ++j) {
        e[j] = exp(((double)z[j] - (double)zm) / T);
        S += e[j];
    }
    *margin = INFINITY;
    if (top_p >= 1.0) return S;
    for (int j = 0; j < V; ++j) keys[j].z = z[j], keys[j].j = j;
    qsort(keys, (size_t)V, sizeof(zkey), zkey_cmp);
    double thr = top_p * S;
    double cum = 0.0;
    int c = 0;
    if (top_p <= 0.0) {
        cum = e[keys[0].j];
        c = 1;
    } else {
        while (c < V) {
            double prev = cum;
            cum += e[keys[c].j];
            ++c;
            if (cum >= thr) {
                double m1 = fabs(cum - thr) / S, m0 = fabs(prev - thr) / S;
                *margin = m1 < m0 ? m1 : m0;
                break;
            }
        }
    }
    for (int i = c; i < V; ++i) e[keys[i].j] = 0.0;
    return cum;
}

/* Categorical draw from unnormalised weights w (index order): the smallest j
 * with w_0 + ... + w_j > u * (w_0 + ... + w_{V-1}); if rounding passes the end,
 * the last j with w_j > 0.  *margin = distance of u*W from the nearest
 * cumulative boundary, relative to W. */
static int32_t draw(const double *w, int V, double u, double *margin) {
    double W = 0.0;
    for (int j = 0; j < V; ++j) W += w[j];
    double t = u * W, cum = 0.0;
    *margin = INFINITY;
    for (int j = 0; j < V; ++j) {
        double prev = cum;
        cum += w[j];
        if (cum > t) {
            double m1 = fabs(cum - t), m0 = fabs(t - prev);
            *margin = (m1 < m0 ? m1 : m0) / W;
            return j;
        }
    }
    for (int j = V - 1; j >= 0; --j)
        if (w[j] > 0.0) { *margin = 0.0; return j; }
    *margin = 0.0;
    return V - 1;
}

/*
 * Rejection-sampling verification (Leviathan/Chen).  Row i (i < M-1) tests
 * draft x_i ~ q_i against the target p'_i: accept iff u_i * q_i(x_i) < p'_i(x_i)
 * (u, q widened to fp64, product exact).  At the first rejection i = a, draw
 * the correction from r = max(0, p'_a - q_a) (from p'_a if r sums to zero);
 * if every draft is accepted, draw a bonus token from p'_{M-1}.  Both draws use
 * u_{M-1}.  A draft id outside [0, V) is rejected.  temperature == 0 gives the
 * greedy result; temperature < 0 is an error.
 * margins (optional, [M+1]): per-row acceptance margins |u*q - p'| / p',
 * then the draw margin, then the smallest nucleus margin seen.
 */
int orc_accept_rejection(const float *logits, int M, int V, int64_t ldl, const float *q,
                         int64_t ldq, const int32_t *drafts, const float *u, float temperature,
                         float top_p, int64_t base_len, int32_t *tokens, int32_t *counts,
                         int64_t *rollback, double *margins) {
    if (M < 1 || M > 64 || V < 1 || ldl < V || (M > 1 && ldq < V) || !(temperature >= 0.0f))
        return -1;
    if (temperature == 0.0f)
        return orc_accept_greedy(logits, M, V, ldl, drafts, base_len, tokens, counts, rollback);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    zkey *keys = (zkey *)malloc(sizeof(zkey) * (size_t)V);
    if (!e || !r || !keys) { free(e); free(r); free(keys); return -1; }
    int32_t run[64];
    double nuc_margin = INFINITY, m_nuc, m_draw = INFINITY;
    const double T = (double)temperature, P = (double)top_p;
    if (margins)
        for (int i = 0; i <= M; ++i) margins[i] = INFINITY;
    int a = 0;
    int32_t last = -1;
    for (;;) {
        double Sp = target_row(logits + (int64_t)a * ldl, V, T, P, e, keys, &m_nuc);
        if (m_nuc < nuc_margin) nuc_margin = m_nuc;
        if (a == M - 1) {                       /* every draft accepted: bonus */
            last = draw(e, V, (double)u[M - 1], &m_draw);
            break;
        }
        int32_t x = drafts[a];
        const float *qa = q + (int64_t)a * ldq;
        double px = (x >= 0 && x < V) ? e[x] / Sp : 0.0;
        double qx = (x >= 0 && x < V) ? (double)qa[x] : 0.0;
        double lhs = (double)u[a] * qx;
        if (margins) margins[a] = (px > 0.0) ? fabs(lhs - px) / px : INFINITY;
        if (lhs < px) {
            run[a] = x;
            ++a;
            continue;
        }
        double W = 0.0;
        for (int j = 0; j < V; ++j) {
            double pj = e[j] / Sp, d = pj - (double)qa[j];
            r[j] = d > 0.0 ? d : 0.0;
            W += r[j];
        }
        last = (W > 0.0) ? draw(r, V, (double)u[M - 1], &m_draw)
                         : draw(e, V, (double)u[M - 1], &m_draw);
        break;
    }
    run[a] = last;
    write_run(M, run, a, base_len, tokens, counts, rollback);
    if (margins) {
        margins[M - 1] = m_draw;
        margins[M] = nuc_margin;
    }
    free(e);
    free(r);
    free(keys);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* sampled acceptance with the full sampler pipeline                         */
/* ------------------------------------------------------------------------ */

/*
 * Ollama mtp.go commit log, the MLX sampler rework: the target distribution
 * of a row is built by an explicit pipeline -- (1) penalties, (2) top-k,
 * (3) temperature/softmax, (4) top-p, (5) min-p, (6) normalize,
 * (7) categorical -- and the common top-k path keeps sparse per-row token
 * ids and probabilities, which sampled MTP reuses for acceptance, the bonus
 * draw and the residual draw.  The pages name the steps but not their
 * formulas; the readings taken here (the usual ones):
 *
 *   (1) the penalty window of row i of a sequence is the last penalty_last_n
 *       tokens of (history ++ drafts[0..i-1]) (none if penalty_last_n <= 0);
 *       for a token t seen c_t > 0 times in it, in fp32 with every operation
 *       rounded on its own:
 *         z = (z > 0) ? z / repeat_penalty : z * repeat_penalty
 *         z = (z - c_t * frequency_penalty) - presence_penalty
 *       (the repeat step is skipped when repeat_penalty == 1); ids outside
 *       [0, V) in the window are ignored.
 *   (2) top-k keeps the top_k entries first in the order (z desc, index asc)
 *       (top_k <= 0 or >= V keeps all).
 *   (3) e_j = exp((z_j - z_max) / T) in fp64 over the kept entries;
 *       T == 0 makes the target a point mass at the first entry of the order.
 *   (4) top-p keeps the shortest prefix of the order whose e-mass reaches
 *       top_p * (sum of e) (top_p >= 1 keeps all, top_p <= 0 the first).
 *   (5) min-p then drops entries with e_j < min_p (that is, p_j below min_p
 *       times the largest p); the first entry always stays.
 *   (6) p'_j = e_j / (e-mass of what is left), 0 elsewhere.
 *   (7) a draw picks, in index order, the smallest j with
 *       w_0 + .. + w_j > u * sum(w) (the last j with w_j > 0 if rounding
 *       passes the end).
 * Acceptance of draft x_i ~ q_i: accept iff u_i * q_i(x_i) < p'_i(x_i); the
 * first rejection a draws from max(0, p'_a - q_a) (from p'_a if that is all
 * zero); if every draft is accepted, a bonus is drawn from p'_{M-1}; both
 * draws use u_{M-1}.  q_i is dense [V] or sparse (ids, probs; an id not listed
 * has probability 0, the first listing of an id counts).
 */
typedef struct {
    float temperature, top_p, min_p;
    int32_t top_k;
    float repeat_penalty, presence_penalty, frequency_penalty;
    int32_t penalty_last_n;
} orc_sampler;

/* Penalised copy of one row (step 1). */
static void penalise_row(const float *z, int V, const int32_t *window, int W,
                         const orc_sampler *s, float *zp) {
    for (int j = 0; j < V; ++j) zp[j] = z[j];
    for (int w = 0; w < W; ++w) {
        int32_t t = window[w];
        if (t < 0 || t >= V) continue;
        int first = 1;
        for (int v = 0; v < w; ++v)
            if (window[v] == t) { first = 0; break; }
        if (!first) continue;
        int c = 0;
        for (int v = 0; v < W; ++v) c += (window[v] == t);
        volatile float x = z[t];
        if (s->repeat_penalty != 1.0f) x = (x > 0.0f) ? x / s->repeat_penalty : x * s->repeat_penalty;
        volatile float cf = (float)c * s->frequency_penalty;
        x = x - cf;
        x = x - s->presence_penalty;
        zp[t] = x;
    }
}

/*
 * Target distribution of one row (steps 2-6) from its penalised logits:
 * writes p'[V] (0 outside the kept entries) and returns the number kept.
 * margin: relative distance of the top-p and min-p cuts from their
 * thresholds.
 */
static int sampled_row(const float *zp, int V, const orc_sampler *s, double *p, zkey *keys,
                       double *margin) {
    for (int j = 0; j < V; ++j) keys[j].z = zp[j], keys[j].j = j;
    qsort(keys, (size_t)V, sizeof(zkey), zkey_cmp);
    int n = (s->top_k > 0 && s->top_k < V) ? s->top_k : V;
    for (int j = 0; j < V; ++j) p[j] = 0.0;
    *margin = INFINITY;
    if (s->temperature == 0.0f) {
        p[keys[0].j] = 1.0;
        return 1;
    }
    const double T = (double)s->temperature, zm = (double)keys[0].z;
    double S = 0.0;
    for (int c = 0; c < n; ++c) {
        p[keys[c].j] = exp(((double)keys[c].z - zm) / T);
        S += p[keys[c].j];
    }
    int c_p = n;
    if (s->top_p < 1.0f) {
        double thr = (double)s->top_p * S, cum = 0.0;
        c_p = 1;
        if (s->top_p > 0.0f) {
            for (c_p = 0; c_p < n;) {
                double prev = cum;
                cum += p[keys[c_p].j];
                ++c_p;
                if (cum >= thr) {
                    double m1 = fabs(cum - thr) / S, m0 = fabs(prev - thr) / S;
                    *margin = m1 < m0 ? m1 : m0;
                    break;
                }
            }
        }
    }
    int c_m = n;
    if (s->min_p > 0.0f) {
        for (c_m = 1; c_m < n; ++c_m) {
            double e = p[keys[c_m].j];
            double m = fabs(e - (double)s->min_p) / (double)s->min_p;
            if (m < *margin) *margin = m;
            if (e < (double)s->min_p) break;
        }
    }
    int kept = c_p < c_m ? c_p : c_m;
    double Sp = 0.0;
    for (int c = 0; c < kept; ++c) Sp += p[keys[c].j];
    for (int c = 0; c < kept; ++c) p[keys[c].j] /= Sp;
    for (int c = kept; c < n; ++c) p[keys[c].j] = 0.0;
    return kept;
}

static double q_of(const float *q, const int32_t *q_ids, const float *q_probs, int Kq, int32_t x) {
    if (q) return (double)q[x];
    for (int k = 0; k < Kq; ++k)
        if (q_ids[k] == x) return (double)q_probs[k];
    return 0.0;
}

/*
 * B sequences of M rows each; row i of sequence b is logits row b*M + i.
 * history[b][0..history_len[b]-1] (row stride ldh), drafts [B][M-1],
 * uniforms [B][M], base_len [B]; q dense [B][M-1][ldq] or, if q is NULL,
 * sparse q_ids / q_probs [B][M-1][Kq].  Outputs tokens [B][M], counts [B][2],
 * rollback [B].  Optional: target_p [B*M][V] receives every row's p';
 * margins [B][M+1] as in orc_accept_rejection (acceptance margins per row,
 * the draw margin, then the smallest cut margin).
 */
int orc_accept_sampled(int B, int M, int V, const float *logits, int64_t ldl,
                       const int32_t *history, const int32_t *history_len, int64_t ldh,
                       const int32_t *drafts, const float *q, int64_t ldq, const int32_t *q_ids,
                       const float *q_probs, int Kq, const float *u, const orc_sampler *s,
                       const int64_t *base_len, int32_t *tokens, int32_t *counts,
                       int64_t *rollback, double *target_p, double *margins) {
    if (B < 1 || M < 1 || M > 64 || V < 1 || ldl < V || !(s->temperature >= 0.0f)) return -1;
    if (M > 1 && !q && (!q_ids || !q_probs || Kq < 1)) return -1;
    float *zp = (float *)malloc(sizeof(float) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V * (size_t)M);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    zkey *keys = (zkey *)malloc(sizeof(zkey) * (size_t)V);
    int32_t *window = NULL;
    int maxw = 0;
    for (int b = 0; b < B; ++b) {
        int w = (history ? history_len[b] : 0) + M;
        if (w > maxw) maxw = w;
    }
    window = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxw + 1));
    if (!zp || !p || !r || !keys || !window) {
        free(zp); free(p); free(r); free(keys); free(window);
        return -1;
    }
    for (int b = 0; b < B; ++b) {
        const int Lh = history ? history_len[b] : 0;
        const int32_t *d = drafts ? drafts + (int64_t)b * (M - 1) : NULL;
        double *mg = margins ? margins + (int64_t)b * (M + 1) : NULL;
        double cut_margin = INFINITY, m_cut, m_draw = INFINITY;
        if (mg)
            for (int i = 0; i <= M; ++i) mg[i] = INFINITY;
        for (int i = 0; i < M; ++i) {
            /* the penalty window: last penalty_last_n of history ++ drafts[0..i-1] */
            int W = 0;
            if (s->penalty_last_n > 0) {
                int total = Lh + i, w0 = total - s->penalty_last_n;
                if (w0 < 0) w0 = 0;
                for (int c = w0; c < total; ++c)
                    window[W++] = (c < Lh) ? history[(int64_t)b * ldh + c] : d[c - Lh];
            }
            penalise_row(logits + ((int64_t)b * M + i) * ldl, V, window, W, s, zp);
            sampled_row(zp, V, s, p + (int64_t)i * V, keys, &m_cut);
            if (m_cut < cut_margin) cut_margin = m_cut;
            if (target_p)
                memcpy(target_p + ((int64_t)b * M + i) * V, p + (int64_t)i * V,
                       sizeof(double) * (size_t)V);
        }
        int32_t run[64];
        int a = 0;
        int32_t last = -1;
        const float *ub = u + (int64_t)b * M;
        for (;;) {
            const double *pa = p + (int64_t)a * V;
            if (a == M - 1) {
                last = draw(pa, V, (double)ub[M - 1], &m_draw);
                break;
            }
            const int32_t x = d[a];
            const float *qa = q ? q + ((int64_t)b * (M - 1) + a) * ldq : NULL;
            const int32_t *qia = q ? NULL : q_ids + ((int64_t)b * (M - 1) + a) * Kq;
            const float *qpa = q ? NULL : q_probs + ((int64_t)b * (M - 1) + a) * Kq;
            const double px = (x >= 0 && x < V) ? pa[x] : 0.0;
            const double qx = (x >= 0 && x < V) ? q_of(qa, qia, qpa, Kq, x) : 0.0;
            const double lhs = (double)ub[a] * qx;
            if (mg) mg[a] = (px > 0.0) ? fabs(lhs - px) / px : INFINITY;
            if (lhs < px) {
                run[a] = x;
                ++a;
                continue;
            }
            double Wr = 0.0;
            for (int j = 0; j < V; ++j) {
                double dj = pa[j] - (pa[j] > 0.0 ? q_of(qa, qia, qpa, Kq, j) : 0.0);
                r[j] = dj > 0.0 ? dj : 0.0;
                Wr += r[j];
            }
            last = (Wr > 0.0) ? draw(r, V, (double)ub[M - 1], &m_draw)
                              : draw(pa, V, (double)ub[M - 1], &m_draw);
            break;
        }
        run[a] = last;
        write_run(M, run, a, base_len ? base_len[b] : 0, tokens + (int64_t)b * M, counts + 2 * b,
                  rollback + b);
        if (mg) {
            mg[M - 1] = m_draw;
            mg[M] = cut_margin;
        }
    }
    free(zp); free(p); free(r); free(keys); free(window);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* draft-depth controller                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Ollama mtp.go commit log (the controller that replaced the heuristic
 * schedule): draft the depth that maximises committed tokens per unit of
 * wall-clock, from live per-position acceptance and the measured forward
 * cost per width, with no cap on the depth; MTPLX blog post, "Why it is
 * interesting on a Mac specifically": plain decoding stays the baseline.
 *
 * With a_i the probability that draft i (1-based) is accepted given drafts
 * 1..i-1 were, a step of depth d commits E(d) = 1 + sum_{i=1..d} prod_{j<=i}
 * a_j tokens in expectation (the accepted run plus the correction or bonus
 * token) and costs cost[d] (the verify pass at M = d + 1 rows, plus drafting
 * d tokens); the chosen depth maximises E(d) / cost[d], the smallest d on a
 * tie, d = 0 (plain decoding, one token per step) included.
 */
int orc_choose_draft_depth(const double *accept_prob, const double *cost, int dmax,
                           double *rate) {
    if (dmax < 0 || dmax > 63) return -1;
    for (int d = 0; d <= dmax; ++d)
        if (!(cost[d] > 0.0)) return -1;
    for (int i = 0; i < dmax; ++i)
        if (!(accept_prob[i] >= 0.0 && accept_prob[i] <= 1.0)) return -1;
    int best = 0;
    double best_rate = 0.0;
    for (int d = 0; d <= dmax; ++d) {
        double e = 1.0;
        for (int i = 1; i <= d; ++i) {
            double prod = 1.0;
            for (int j = 1; j <= i; ++j) prod *= accept_prob[j - 1];
            e += prod;
        }
        double r = e / cost[d];
        if (rate) rate[d] = r;
        if (d == 0 || r > best_rate) {
            best = d;
            best_rate = r;
        }
    }
    return best;
}

/*
 * Live per-position acceptance: after a step of depth d that accepted a
 * drafts, positions i = 1..min(a + 1, d) were reached and positions 1..a
 * accepted; counts decay by `keep` per step (1 = plain counts).  The estimate
 * a_i = (accepted_i + 1) / (reached_i + 2) (Laplace's rule, 1/2 before any
 * evidence).
 */
void orc_depth_observe(double *reached, double *accepted, int dmax, int d, int a, double keep) {
    for (int i = 1; i <= dmax; ++i) {
        reached[i - 1] *= keep;
        accepted[i - 1] *= keep;
        if (i <= d && i <= a + 1) reached[i - 1] += 1.0;
        if (i <= d && i <= a) accepted[i - 1] += 1.0;
    }
}

void orc_depth_estimate(const double *reached, const double *accepted, int dmax, double *prob) {
    for (int i = 0; i < dmax; ++i) prob[i] = (accepted[i] + 1.0) / (reached[i] + 2.0);
}

/* ------------------------------------------------------------------------ */
/* multi-row verify attention over a shared KV prefix                        */
/* ------------------------------------------------------------------------ */

/*
 * Qiita roofline article, §2-3: at long context the KV reads also take
 * bandwidth, but the K candidates of a verify pass look at the same prefix,
 * so one KV read serves all of them, as with the weights.  The oracle is the
 * plain definition of causal attention for the M verify rows of one
 * sequence (grouped heads: query head h reads KV head h / G):
 *   row i sits at position L + i and sees keys 0 .. L + i (the prefix and
 *   the verify tokens up to itself, whose K and V are already in the cache);
 *   s_j = scale * sum_d q[i][h][d] * k[h/G][j][d]; p = softmax(s);
 *   o[i][h][d] = sum_j p_j * v[h/G][j][d];
 * in fp64 from the bf16 inputs.  ob[i][h][d] = sum_j p_j |v[h/G][j][d]| is
 * the error scale of the result.
 */
static void *attn_worker(void *arg);
typedef struct {
    int M, Hq, Hkv, D, L;
    int64_t ldk;
    const uint16_t *q, *k, *v;
    double scale;
    double *o, *ob;
    int h0, h1;
} attn_job;

static void *attn_worker(void *arg) {
    attn_job *J = (attn_job *)arg;
    const int G = J->Hq / J->Hkv, D = J->D;
    double *s = (double *)malloc(sizeof(double) * (size_t)(J->L + J->M));
    if (!s) return NULL;
    for (int h = J->h0; h < J->h1; ++h) {
        const int kh = h / G;
        const uint16_t *K = J->k + (int64_t)kh * J->ldk * D;
        const uint16_t *V = J->v + (int64_t)kh * J->ldk * D;
        for (int i = 0; i < J->M; ++i) {
            const uint16_t *q = J->q + ((int64_t)i * J->Hq + h) * D;
            const int n = J->L + i + 1;
            double mx = -INFINITY;
            for (int j = 0; j < n; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += orc_bf16(q[d]) * orc_bf16(K[(int64_t)j * D + d]);
                s[j] = J->scale * acc;
                if (s[j] > mx) mx = s[j];
            }
            double l = 0.0;
            for (int j = 0; j < n; ++j) {
                s[j] = exp(s[j] - mx);
                l += s[j];
            }
            double *o = J->o + ((int64_t)i * J->Hq + h) * D;
            double *ob = J->ob + ((int64_t)i * J->Hq + h) * D;
            for (int d = 0; d < D; ++d) o[d] = ob[d] = 0.0;
            for (int j = 0; j < n; ++j) {
                const double p = s[j] / l;
                for (int d = 0; d < D; ++d) {
                    const double vv = orc_bf16(V[(int64_t)j * D + d]);
                    o[d] += p * vv;
                    ob[d] += p * fabs(vv);
                }
            }
        }
    }
    free(s);
    return NULL;
}

/* q [M][Hq][D], k and v [Hkv][ldk][D] (positions 0 .. L+M-1 hold keys),
 * o and ob [M][Hq][D]. */
int orc_verify_attention(int M, int Hq, int Hkv, int D, int L, int64_t ldk, const uint16_t *q,
                         const uint16_t *k, const uint16_t *v, double scale, double *o,
                         double *ob, int nthreads) {
    if (M < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || D < 1 || L < 0 || ldk < (int64_t)L + M)
        return -1;
    tables_init();
    if (nthreads < 1) nthreads = 1;
    if (nthreads > Hq) nthreads = Hq;
    pthread_t th[64];
    attn_job jobs[64];
    if (nthreads > 64) nthreads = 64;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (attn_job){M, Hq, Hkv, D, L, ldk, q, k, v, scale, o, ob,
                             (int)((int64_t)Hq * t / nthreads), (int)((int64_t)Hq * (t + 1) / nthreads)};
        pthread_create(&th[t], NULL, attn_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* KV-cache commit                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Ollama mtp.go commit log, the snapshot rework: restoring a cache to the
 * accepted count must leave it as if the rejected rows had never been
 * written.  The plain definition of a write: position p of one head goes to
 * row p of a linear cache (ring = 0; positions at or past cap are not
 * stored) or row p mod cap of a rotating one (ring = 1), replacing what was
 * there.  Writing n rows of D elements, rows[m * ld + d], one position at a
 * time from base upwards.  Called with n = accepted count on a copy of the
 * cache taken before the verify write, it gives the committed cache.
 */
void orc_kv_write(uint16_t *cache, int64_t cap, int D, int ring, int64_t base,
                  const uint16_t *rows, int64_t ld, int n) {
  for (int m = 0; m < n; m++) {
    int64_t p = base + m;
    if (p < 0) continue;
    int64_t row;
    if (ring) {
      row = p % cap;
    } else {
      if (p >= cap) continue;
      row = p;
    }
    for (int d = 0; d < D; d++) cache[row * D + d] = rows[(int64_t)m * ld + d];
  }
}
