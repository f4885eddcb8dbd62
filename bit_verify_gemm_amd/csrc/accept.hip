// Acceptance step of the verify pass: greedy prefix match and Leviathan/Chen
// rejection sampling with residual correction, plus the rollback index.
//
// Gemini Nano summary, analysis §3, and Qiita roofline article, §2-4: greedy
// verification keeps the longest prefix that agrees with the target and
// always commits one more (correction) token.  MTPLX blog post, "Why it is
// interesting on a Mac specifically": rejection sampling with residual
// correction preserves the target's output at temperature 0.6, top_p 0.95.
// Ollama mtp.go commit log: the sampler pipeline is temperature/softmax ->
// top-p -> normalise -> categorical, target distributions are reused for
// acceptance, bonus and residual draws, and at temperature 0 acceptance is
// argmax matching.  Ollama news item, fifth paragraph: a rollback point lets
// a rejection rewind to the last accepted token without a return to the CPU.
//
// Everything runs on the device.  Probability mass is computed in fp64 and
// summed as exact 128-bit fixed-point integers (resolution 2^-100), so sums
// are independent of thread order and the outputs are a deterministic
// function of the inputs.  The top-p nucleus is found by a 4-pass radix
// select over the order-preserving 32-bit key of each logit, with per-digit
// mass histograms; ties at the cut are broken by index.
#include "../../include/mtp_verify.h"
#include "device.h"
#include "internal.h"

namespace mtp {
namespace {

typedef unsigned long long u64;

constexpr int kBlock = 256;
constexpr int kMaxBlocksPerRow = 128;
constexpr int kBins = 256;

int blocks_per_row(int V) {
  int nb = (V + 2047) / 2048;
  return nb < 1 ? 1 : (nb > kMaxBlocksPerRow ? kMaxBlocksPerRow : nb);
}

// ---- 128-bit fixed point (value * 2^100) -----------------------------------

struct Fx {
  u64 lo, hi;
};

__device__ __forceinline__ Fx fx_zero() { return Fx{0ull, 0ull}; }

// floor(v * 2^100) for 0 <= v < 2^27 (values below 2^-100 become 0).
__device__ __forceinline__ Fx to_fx(double v) {
  Fx r = fx_zero();
  if (!(v > 0.0)) return r;
  const u64 bits = (u64)__double_as_longlong(v);
  const int ex = (int)((bits >> 52) & 0x7FF);
  if (ex == 0) return r;
  const u64 mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int sh = ex - 975;  // v * 2^100 = mant * 2^(ex - 1075 + 100)
  if (sh >= 64) {
    r.hi = mant << (sh - 64);
  } else if (sh > 0) {
    r.lo = mant << sh;
    r.hi = mant >> (64 - sh);
  } else if (sh == 0) {
    r.lo = mant;
  } else if (sh > -64) {
    r.lo = mant >> (-sh);
  }
  return r;
}

__device__ __forceinline__ void fx_add(Fx &a, const Fx &b) {
  const u64 lo = a.lo + b.lo;
  a.hi += b.hi + (lo < a.lo ? 1ull : 0ull);
  a.lo = lo;
}

__device__ __forceinline__ Fx fx_sum(Fx a, const Fx &b) {
  fx_add(a, b);
  return a;
}

__device__ __forceinline__ bool fx_ge(const Fx &a, const Fx &b) {
  return a.hi > b.hi || (a.hi == b.hi && a.lo >= b.lo);
}

__device__ __forceinline__ bool fx_gt(const Fx &a, const Fx &b) {
  return a.hi > b.hi || (a.hi == b.hi && a.lo > b.lo);
}

__device__ __forceinline__ bool fx_nonzero(const Fx &a) { return (a.lo | a.hi) != 0ull; }

__device__ __forceinline__ double fx_to_double(const Fx &a) {
  return ldexp((double)a.hi, -36) + ldexp((double)a.lo, -100);
}

__device__ __forceinline__ void fx_atomic_add(u64 *p, Fx v) {
  if (v.lo) {
    const u64 old = atomicAdd(p, v.lo);
    if (old + v.lo < old) v.hi += 1ull;
  }
  if (v.hi) atomicAdd(p + 1, v.hi);
}

__device__ __forceinline__ Fx fx_load(const u64 *p) { return Fx{p[0], p[1]}; }

__device__ __forceinline__ Fx fx_shfl_xor(const Fx &a, int m) {
  return Fx{(u64)__shfl_xor((long long)a.lo, m), (u64)__shfl_xor((long long)a.hi, m)};
}

// Exact wave-wide sum (integer adds commute).
__device__ __forceinline__ Fx fx_wave_sum(Fx a) {
  for (int m = kWave / 2; m > 0; m >>= 1) fx_add(a, fx_shfl_xor(a, m));
  return a;
}

// Block-wide sum; result valid in every thread.  `red` holds kBlock/kWave Fx.
__device__ Fx fx_block_sum(Fx a, Fx *red) {
  a = fx_wave_sum(a);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = a;
  __syncthreads();
  Fx s = fx_zero();
  for (int i = 0; i < kBlock / kWave; ++i) fx_add(s, red[i]);
  return s;
}

// Order-preserving key: a < b as floats  <=>  key(a) < key(b).
__device__ __forceinline__ uint32_t fkey(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- workspace layout -------------------------------------------------------

struct RowState {
  float zmax;
  uint32_t kappa;   // key of the last nucleus value (all keys >= kappa)
  int32_t cutoff;   // entries with key == kappa and index <= cutoff are inside
  int32_t all;      // 1: the nucleus is the whole row
  double mass;      // nucleus mass S' (sum of e over the nucleus)
};

struct Global {
  int32_t a;        // accepted drafts
  int32_t row;      // row of the final draw
  int32_t residual; // 1: draw from max(0, p' - q), else from p'
  int32_t pad;
};

struct Layout {
  size_t maxp, hist, total, rows, glob, blk, gpart, bytes;
};

Layout layout(int M, int V) {
  const size_t nb = (size_t)blocks_per_row(V);
  Layout L;
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  L.maxp = take(sizeof(float) * M * nb);
  L.hist = take(sizeof(u64) * 3 * kBins * 4 * M);
  L.total = take(sizeof(u64) * 2 * M);
  L.rows = take(sizeof(RowState) * M);
  L.glob = take(sizeof(Global));
  L.blk = take(sizeof(u64) * 4 * nb);
  L.gpart = take(sizeof(float) * 2 * M * nb);
  L.bytes = o;
  return L;
}

struct RejArgs {
  const float *z;
  int64_t ldl;
  const float *q;
  int64_t ldq;
  const int32_t *drafts;
  const float *u;
  double T;
  double top_p;
  int M, V, nb, chunk;
  int64_t base_len;
  int32_t *tokens;
  int32_t *counts;
  int64_t *rollback;
  float *maxp;
  u64 *hist;     // [pass][row][bin][lo, hi, count]
  u64 *total;    // [row][lo, hi]
  RowState *rows;
  Global *glob;
  u64 *blk;      // [block][res lo, res hi, e lo, e hi]
};

__device__ __forceinline__ u64 *hist_at(const RejArgs &p, int pass, int row) {
  return p.hist + ((size_t)(pass * p.M + row) * kBins) * 3;
}

// ---- greedy -------------------------------------------------------------------

// Better candidate: a number beats NaN, larger beats smaller, lower index
// breaks ties.
__device__ __forceinline__ bool better(float v, int j, float bv, int bj) {
  if (isnan(v)) return false;
  if (isnan(bv)) return true;
  return v > bv || (v == bv && j < bj);
}

__global__ __launch_bounds__(kBlock) void greedy_partial(const float *z, int64_t ldl, int V,
                                                         int nb, int chunk, float *pv, int *pj) {
  const int b = blockIdx.x, row = blockIdx.y;
  const float *zr = z + (int64_t)row * ldl;
  const int j0 = b * chunk, j1 = min(V, j0 + chunk);
  float bv = __int_as_float(0x7FC00000);
  int bj = 0x7FFFFFFF;
  for (int j = j0 + threadIdx.x; j < j1; j += kBlock) {
    const float v = zr[j];
    if (better(v, j, bv, bj)) { bv = v; bj = j; }
  }
  for (int m = kWave / 2; m > 0; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oj = __shfl_xor(bj, m);
    if (better(ov, oj, bv, bj)) { bv = ov; bj = oj; }
  }
  __shared__ float sv[kBlock / kWave];
  __shared__ int sj[kBlock / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) { sv[threadIdx.x / kWave] = bv; sj[threadIdx.x / kWave] = bj; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBlock / kWave; ++w)
      if (better(sv[w], sj[w], bv, bj)) { bv = sv[w]; bj = sj[w]; }
    pv[row * nb + b] = bv;
    pj[row * nb + b] = bj;
  }
}

__global__ __launch_bounds__(64) void greedy_final(const float *pv, const int *pj, int M, int nb,
                                                   const int32_t *drafts, int64_t base_len,
                                                   int32_t *tokens, int32_t *counts,
                                                   int64_t *rollback) {
  __shared__ int g[64];
  const int row = threadIdx.x;
  if (row < M) {
    float bv = __int_as_float(0x7FC00000);
    int bj = 0x7FFFFFFF;
    for (int b = 0; b < nb; ++b)
      if (better(pv[row * nb + b], pj[row * nb + b], bv, bj)) { bv = pv[row * nb + b]; bj = pj[row * nb + b]; }
    g[row] = (bj == 0x7FFFFFFF) ? 0 : bj;  // all-NaN row: index 0
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < M - 1 && drafts[a] == g[a]) ++a;
    for (int i = 0; i < M; ++i) tokens[i] = (i <= a) ? g[i] : -1;
    counts[0] = a;
    counts[1] = a + 1;
    *rollback = base_len + a + 1;
  }
}

// ---- rejection sampling ----------------------------------------------------

__device__ __forceinline__ double e_of(float z, float zmax, double T) {
  return exp(((double)z - (double)zmax) / T);
}

__device__ __forceinline__ float row_max_from_partials(const RejArgs &p, int row) {
  float m = -__builtin_inff();
  for (int b = 0; b < p.nb; ++b) m = fmaxf(m, p.maxp[row * p.nb + b]);
  return m;
}

// Nucleus threshold in fixed point: top_p * S (at least one unit, so that
// top_p <= 0 keeps exactly the first entry).
__device__ __forceinline__ Fx threshold(const RejArgs &p, int row) {
  const double S = fx_to_double(fx_load(p.total + 2 * row));
  Fx t = to_fx(p.top_p > 0.0 ? p.top_p * S : 0.0);
  if (!fx_nonzero(t)) t.lo = 1ull;
  return t;
}

// Walk the bins of one pass from the top: the chosen bin is the first whose
// inclusion brings the mass to the threshold (or the lowest occupied bin if
// rounding never gets there).  `above` is updated to the mass strictly above.
__device__ int select_bin(const u64 *h, const Fx &thr, Fx &above) {
  Fx cum = above;
  int last = -1;
  Fx last_above = cum;
  for (int b = kBins - 1; b >= 0; --b) {
    const u64 cnt = h[3 * b + 2];
    if (!cnt) continue;
    const Fx mass = Fx{h[3 * b], h[3 * b + 1]};
    const Fx next = fx_sum(cum, mass);
    if (fx_ge(next, thr)) {
      above = cum;
      return b;
    }
    last = b;
    last_above = cum;
    cum = next;
  }
  above = last_above;
  return last;
}

// Selected key prefix after `passes` passes (8 bits per pass, from the top).
__device__ uint32_t prefix_after(const RejArgs &p, int row, int passes, Fx &above) {
  const Fx thr = threshold(p, row);
  above = fx_zero();
  uint32_t prefix = 0;
  for (int s = 0; s < passes; ++s) {
    const int b = select_bin(hist_at(p, s, row), thr, above);
    prefix = (prefix << 8) | (uint32_t)(b < 0 ? 0 : b);
  }
  return prefix;
}

// Row maxima (partial) and zeroing of this call's accumulators.
__global__ __launch_bounds__(kBlock) void rej_rowmax(RejArgs p) {
  const int b = blockIdx.x, row = blockIdx.y;
  const float *zr = p.z + (int64_t)row * p.ldl;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  float m = -__builtin_inff();
  for (int j = j0 + threadIdx.x; j < j1; j += kBlock) m = fmaxf(m, zr[j]);
  for (int s = kWave / 2; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  __shared__ float sm[kBlock / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) sm[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBlock / kWave; ++w) m = fmaxf(m, sm[w]);
    p.maxp[row * p.nb + b] = m;
  }
  // zero this row's histograms (4 passes) and total, spread over the row's blocks
  const int words = 4 * kBins * 3;
  for (int i = b * kBlock + threadIdx.x; i < words; i += p.nb * kBlock) {
    const int pass = i / (kBins * 3), w = i - pass * kBins * 3;
    hist_at(p, pass, row)[w] = 0ull;
  }
  if (b == 0 && threadIdx.x < 2) p.total[2 * row + threadIdx.x] = 0ull;
}

// Radix pass `pass` (0..3): histogram of e-mass by key digit for the entries
// matching the prefix selected so far; pass 0 also sums the row's total mass.
__global__ __launch_bounds__(kBlock) void rej_pass(RejArgs p, int pass, int with_hist) {
  __shared__ u64 sh[kBins * 3];
  __shared__ Fx red[kBlock / kWave];
  const int b = blockIdx.x, row = blockIdx.y;
  const float zmax = row_max_from_partials(p, row);
  uint32_t prefix = 0;
  if (pass > 0) {
    Fx above;
    prefix = prefix_after(p, row, pass, above);
  }
  for (int i = threadIdx.x; i < kBins * 3; i += kBlock) sh[i] = 0ull;
  __syncthreads();
  const float *zr = p.z + (int64_t)row * p.ldl;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  const int shift = 24 - 8 * pass;
  Fx tot = fx_zero();
  for (int j = j0 + threadIdx.x; j < j1; j += kBlock) {
    const float zj = zr[j];
    const uint32_t key = fkey(zj);
    if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
    const Fx e = to_fx(e_of(zj, zmax, p.T));
    if (pass == 0) fx_add(tot, e);
    if (with_hist) {
      const int d = (key >> shift) & 0xFF;
      u64 *bin = sh + 3 * d;
      if (e.lo) {
        const u64 old = atomicAdd(bin, e.lo);
        atomicAdd(bin + 1, e.hi + ((old + e.lo < old) ? 1ull : 0ull));
      } else if (e.hi) {
        atomicAdd(bin + 1, e.hi);
      }
      atomicAdd(bin + 2, 1ull);
    }
  }
  if (pass == 0) {
    tot = fx_block_sum(tot, red);
    if (threadIdx.x == 0) fx_atomic_add(p.total + 2 * row, tot);
  }
  if (with_hist) {
    __syncthreads();
    u64 *gh = hist_at(p, pass, row);
    for (int d = threadIdx.x; d < kBins; d += kBlock) {
      if (sh[3 * d + 2]) {
        fx_atomic_add(gh + 3 * d, Fx{sh[3 * d], sh[3 * d + 1]});
        atomicAdd(gh + 3 * d + 2, sh[3 * d + 2]);
      }
    }
  }
}

// Index of the t-th (1-based) entry of row `zr` with key == kappa, scanning in
// index order with the whole block.  Returns V-1 if there are fewer.
__device__ int find_tth_tie(const float *zr, int V, uint32_t kappa, int t) {
  __shared__ int cnt[kBlock];
  const int per = (V + kBlock - 1) / kBlock;
  const int j0 = threadIdx.x * per, j1 = min(V, j0 + per);
  int c = 0;
  for (int j = j0; j < j1; ++j) c += (fkey(zr[j]) == kappa);
  cnt[threadIdx.x] = c;
  __syncthreads();
  __shared__ int found;
  if (threadIdx.x == 0) {
    found = V - 1;
    int acc = 0;
    for (int i = 0; i < kBlock; ++i) {
      if (acc + cnt[i] >= t) {
        int need = t - acc;
        const int a0 = i * per, a1 = min(V, a0 + per);
        for (int j = a0; j < a1; ++j)
          if (fkey(zr[j]) == kappa && --need == 0) { found = j; break; }
        break;
      }
      acc += cnt[i];
    }
  }
  __syncthreads();
  const int r = found;
  __syncthreads();
  return r;
}

__device__ __forceinline__ bool in_nucleus(const RowState &rs, float z, int j) {
  if (rs.all) return true;
  const uint32_t k = fkey(z);
  return k > rs.kappa || (k == rs.kappa && j <= rs.cutoff);
}

// Per-row nucleus description, then the sequential acceptance tests.
__global__ __launch_bounds__(kBlock) void rej_decide(RejArgs p) {
  for (int row = 0; row < p.M; ++row) {
    RowState rs;
    rs.zmax = row_max_from_partials(p, row);
    const double S = fx_to_double(fx_load(p.total + 2 * row));
    if (p.top_p >= 1.0) {
      rs.all = 1; rs.kappa = 0; rs.cutoff = p.V; rs.mass = S;
    } else {
      Fx above;
      const uint32_t kappa = prefix_after(p, row, 4, above);
      const u64 *h3 = hist_at(p, 3, row) + 3 * (kappa & 0xFF);
      const u64 n = h3[2];
      const double ek = e_of(key_to_float(kappa), rs.zmax, p.T);
      const double above_d = fx_to_double(above);
      const Fx thr = threshold(p, row);
      const double thr_d = fx_to_double(thr);
      double tt = ceil((thr_d - above_d) / ek);
      u64 t = (tt < 1.0) ? 1ull : (tt >= (double)n ? n : (u64)tt);
      rs.all = 0;
      rs.kappa = kappa;
      if (t >= n) {
        rs.cutoff = p.V;
      } else {
        rs.cutoff = find_tth_tie(p.z + (int64_t)row * p.ldl, p.V, kappa, (int)t);
      }
      rs.mass = above_d + (double)t * ek;
    }
    if (threadIdx.x == 0) p.rows[row] = rs;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int a = 0;
    int residual = 0;
    while (a < p.M - 1) {
      const int x = p.drafts[a];
      const RowState rs = p.rows[a];
      double px = 0.0, qx = 0.0;
      if (x >= 0 && x < p.V) {
        const float zx = p.z[(int64_t)a * p.ldl + x];
        if (in_nucleus(rs, zx, x)) px = e_of(zx, rs.zmax, p.T) / rs.mass;
        qx = (double)p.q[(int64_t)a * p.ldq + x];
      }
      if ((double)p.u[a] * qx < px) {
        ++a;
      } else {
        residual = 1;
        break;
      }
    }
    p.glob->a = a;
    p.glob->row = a;
    p.glob->residual = residual;
  }
}

// Weights of the final draw for entry j of row `row`.
__device__ __forceinline__ void draw_weights(const RejArgs &p, const RowState &rs, int row,
                                             bool residual, int j, Fx &wres, Fx &we) {
  const float zj = p.z[(int64_t)row * p.ldl + j];
  double e = 0.0;
  if (in_nucleus(rs, zj, j)) e = e_of(zj, rs.zmax, p.T);
  we = to_fx(e);
  if (residual) {
    const double d = e / rs.mass - (double)p.q[(int64_t)row * p.ldq + j];
    wres = to_fx(d > 0.0 ? d : 0.0);
  } else {
    wres = fx_zero();
  }
}

__global__ __launch_bounds__(kBlock) void rej_draw_sums(RejArgs p) {
  __shared__ Fx red[kBlock / kWave];
  const Global gl = *p.glob;
  const RowState rs = p.rows[gl.row];
  const int b = blockIdx.x;
  const int j0 = b * p.chunk, j1 = min(p.V, j0 + p.chunk);
  Fx sr = fx_zero(), se = fx_zero();
  for (int j = j0 + threadIdx.x; j < j1; j += kBlock) {
    Fx wr, we;
    draw_weights(p, rs, gl.row, gl.residual != 0, j, wr, we);
    fx_add(sr, wr);
    fx_add(se, we);
  }
  sr = fx_block_sum(sr, red);
  se = fx_block_sum(se, red);
  if (threadIdx.x == 0) {
    u64 *o = p.blk + 4 * b;
    o[0] = sr.lo; o[1] = sr.hi; o[2] = se.lo; o[3] = se.hi;
  }
}

// Smallest j with prefix weight > u * total (index order); the last j with a
// positive weight if rounding passes the end.  Writes the committed run.
__global__ __launch_bounds__(kBlock) void rej_draw_final(RejArgs p) {
  __shared__ Fx part[kBlock];
  __shared__ int s_blk, s_use_res, s_pick;
  __shared__ Fx s_before, s_target;
  const Global gl = *p.glob;
  const RowState rs = p.rows[gl.row];
  if (threadIdx.x == 0) {
    Fx wres = fx_zero(), we = fx_zero();
    for (int b = 0; b < p.nb; ++b) {
      fx_add(wres, fx_load(p.blk + 4 * b));
      fx_add(we, fx_load(p.blk + 4 * b + 2));
    }
    const int use_res = gl.residual && fx_nonzero(wres);
    const Fx W = use_res ? wres : we;
    const Fx target = to_fx((double)p.u[p.M - 1] * fx_to_double(W));
    Fx cum = fx_zero();
    int blk = -1, last_nz = -1;
    Fx last_before = fx_zero();
    for (int b = 0; b < p.nb; ++b) {
      const Fx s = fx_load(p.blk + 4 * b + (use_res ? 0 : 2));
      const Fx next = fx_sum(cum, s);
      if (fx_gt(next, target)) { blk = b; break; }
      if (fx_nonzero(s)) { last_nz = b; last_before = cum; }
      cum = next;
    }
    s_use_res = use_res;
    s_target = target;
    if (blk >= 0) {
      s_blk = blk;
      s_before = cum;
      s_pick = -1;
    } else {
      s_blk = last_nz;       // rounding passed the end
      s_before = last_before;
      s_pick = -2;
    }
  }
  __syncthreads();
  const int blk = s_blk;
  int pick = p.V - 1;
  if (blk >= 0) {
    const int j0 = blk * p.chunk, j1 = min(p.V, j0 + p.chunk);
    const int per = (j1 - j0 + kBlock - 1) / kBlock;
    const int a0 = j0 + threadIdx.x * per, a1 = min(j1, a0 + per);
    Fx mine = fx_zero();
    for (int j = a0; j < a1; ++j) {
      Fx wr, we;
      draw_weights(p, rs, gl.row, gl.residual != 0, j, wr, we);
      fx_add(mine, s_use_res ? wr : we);
    }
    part[threadIdx.x] = mine;
    __syncthreads();
    if (threadIdx.x == 0) {
      if (s_pick == -1) {
        Fx cum = s_before;
        for (int i = 0; i < kBlock && s_pick == -1; ++i) {
          const Fx next = fx_sum(cum, part[i]);
          if (fx_gt(next, s_target)) {
            const int b0 = j0 + i * per, b1 = min(j1, b0 + per);
            for (int j = b0; j < b1; ++j) {
              Fx wr, we;
              draw_weights(p, rs, gl.row, gl.residual != 0, j, wr, we);
              fx_add(cum, s_use_res ? wr : we);
              if (fx_gt(cum, s_target)) { s_pick = j; break; }
            }
            if (s_pick == -1) s_pick = b1 - 1;
          } else {
            cum = next;
          }
        }
        if (s_pick == -1) s_pick = j1 - 1;
      } else {
        // last entry with a positive weight in the last occupied block
        s_pick = j1 - 1;
        for (int j = j1 - 1; j >= j0; --j) {
          Fx wr, we;
          draw_weights(p, rs, gl.row, gl.residual != 0, j, wr, we);
          if (fx_nonzero(s_use_res ? wr : we)) { s_pick = j; break; }
        }
      }
    }
    __syncthreads();
    pick = s_pick;
  }
  if (threadIdx.x == 0) {
    const int a = gl.a;
    for (int i = 0; i < p.M; ++i) p.tokens[i] = (i < a) ? p.drafts[i] : (i == a ? pick : -1);
    p.counts[0] = a;
    p.counts[1] = a + 1;
    *p.rollback = p.base_len + a + 1;
  }
}

}  // namespace

size_t accept_ws_bytes(int M, int V) { return layout(M, V).bytes; }

hipError_t launch_accept_greedy(const float *logits, int M, int V, int64_t ldl,
                                const int32_t *drafts, int64_t base_len, int32_t *tokens,
                                int32_t *counts, int64_t *rollback, void *ws, hipStream_t stream) {
  const Layout L = layout(M, V);
  const int nb = blocks_per_row(V);
  const int chunk = (V + nb - 1) / nb;
  uint8_t *w = static_cast<uint8_t *>(ws);
  float *pv = reinterpret_cast<float *>(w + L.gpart);
  int *pj = reinterpret_cast<int *>(pv + (size_t)M * nb);
  hipLaunchKernelGGL(greedy_partial, dim3(nb, M), dim3(kBlock), 0, stream, logits, ldl, V, nb,
                     chunk, pv, pj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_final, dim3(1), dim3(64), 0, stream, pv, pj, M, nb, drafts, base_len,
                     tokens, counts, rollback);
  return hipGetLastError();
}

hipError_t launch_accept_rejection(const float *logits, int M, int V, int64_t ldl,
                                   const float *q, int64_t ldq, const int32_t *drafts,
                                   const float *u, float temperature, float top_p,
                                   int64_t base_len, int32_t *tokens, int32_t *counts,
                                   int64_t *rollback, void *ws, hipStream_t stream) {
  const Layout L = layout(M, V);
  uint8_t *w = static_cast<uint8_t *>(ws);
  RejArgs p;
  p.z = logits; p.ldl = ldl; p.q = q; p.ldq = ldq; p.drafts = drafts; p.u = u;
  p.T = (double)temperature; p.top_p = (double)top_p;
  p.M = M; p.V = V; p.nb = blocks_per_row(V); p.chunk = (V + p.nb - 1) / p.nb;
  p.base_len = base_len; p.tokens = tokens; p.counts = counts; p.rollback = rollback;
  p.maxp = reinterpret_cast<float *>(w + L.maxp);
  p.hist = reinterpret_cast<u64 *>(w + L.hist);
  p.total = reinterpret_cast<u64 *>(w + L.total);
  p.rows = reinterpret_cast<RowState *>(w + L.rows);
  p.glob = reinterpret_cast<Global *>(w + L.glob);
  p.blk = reinterpret_cast<u64 *>(w + L.blk);
  const dim3 rows_grid(p.nb, M);
  hipLaunchKernelGGL(rej_rowmax, rows_grid, dim3(kBlock), 0, stream, p);
  const int with_hist = (p.top_p < 1.0) ? 1 : 0;
  const int passes = with_hist ? 4 : 1;
  for (int pass = 0; pass < passes; ++pass)
    hipLaunchKernelGGL(rej_pass, rows_grid, dim3(kBlock), 0, stream, p, pass, with_hist);
  hipLaunchKernelGGL(rej_decide, dim3(1), dim3(kBlock), 0, stream, p);
  hipLaunchKernelGGL(rej_draw_sums, dim3(p.nb), dim3(kBlock), 0, stream, p);
  hipLaunchKernelGGL(rej_draw_final, dim3(1), dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mtp
