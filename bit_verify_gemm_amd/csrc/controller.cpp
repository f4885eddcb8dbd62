// Draft-depth controller (host code).
//
// Ollama mtp.go commit log: an engine-level controller replaced the
// heuristic draft schedule; it drafts the depth that maximises committed
// tokens per wall-clock from live per-position acceptance and the measured
// forward cost per width, with no cap on the depth.  MTPLX blog post, "Why
// it is interesting on a Mac specifically": plain decoding stays the
// baseline a depth has to beat.
//
// A step of depth d verifies M = d + 1 rows.  With a_i the probability that
// draft i (1-based) is accepted given drafts 1..i-1 were, it commits
// E(d) = 1 + sum_{i=1..d} prod_{j<=i} a_j tokens in expectation (the
// accepted run plus the correction or bonus token); its cost is the caller's
// measured cost[d] (the verify pass at M = d + 1, plus drafting d tokens).
#include "../../include/mtp_verify.h"

#pragma clang fp contract(off)

extern "C" {

int mtp_choose_draft_depth(const double *accept_prob, const double *cost, int dmax, double *rate) {
  if (!cost || (dmax > 0 && !accept_prob)) return MTP_ERR_NULL;
  if (dmax < 0 || dmax > 63) return MTP_ERR_SHAPE;
  for (int d = 0; d <= dmax; ++d)
    if (!(cost[d] > 0.0)) return MTP_ERR_VALUE;
  for (int i = 0; i < dmax; ++i)
    if (!(accept_prob[i] >= 0.0 && accept_prob[i] <= 1.0)) return MTP_ERR_VALUE;
  int best = 0;
  double best_rate = 0.0, e = 1.0, prod = 1.0;
  for (int d = 0; d <= dmax; ++d) {
    if (d > 0) {
      prod *= accept_prob[d - 1];   // P(drafts 1..d all accepted)
      e += prod;
    }
    const double r = e / cost[d];
    if (rate) rate[d] = r;
    if (d == 0 || r > best_rate) {   // the smallest depth wins a tie
      best = d;
      best_rate = r;
    }
  }
  return best;
}

int mtp_depth_observe(double *reached, double *accepted, int dmax, int depth, int n_accepted,
                      double keep) {
  if (!reached || !accepted) return MTP_ERR_NULL;
  if (dmax < 1 || dmax > 63 || depth < 0 || n_accepted < 0 || n_accepted > depth)
    return MTP_ERR_SHAPE;
  if (!(keep >= 0.0 && keep <= 1.0)) return MTP_ERR_VALUE;
  for (int i = 1; i <= dmax; ++i) {
    reached[i - 1] *= keep;
    accepted[i - 1] *= keep;
    if (i <= depth && i <= n_accepted + 1) reached[i - 1] += 1.0;
    if (i <= depth && i <= n_accepted) accepted[i - 1] += 1.0;
  }
  return MTP_OK;
}

int mtp_depth_estimate(const double *reached, const double *accepted, int dmax, double *prob) {
  if (!reached || !accepted || !prob) return MTP_ERR_NULL;
  if (dmax < 1 || dmax > 63) return MTP_ERR_SHAPE;
  for (int i = 0; i < dmax; ++i) prob[i] = (accepted[i] + 1.0) / (reached[i] + 2.0);
  return MTP_OK;
}

}  // extern "C"
