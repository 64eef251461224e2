// Verify-budget scheduling (host code).
//
// What is computed (DSpark, "Hardware-aware prefix scheduler" and the method
// section on confidence-scheduled verification): every draft position k of
// request i carries a conditional survival probability c[i][k] (the chance
// that draft k is accepted once drafts 1..k-1 were); its cumulative survival
// S[i][k] = c[i][1] * ... * c[i][k] is the chance that the prefix up to k is
// accepted.  The scheduler sorts all (request, position) candidates by S,
// admits them one at a time on top of the requests' root rows, and after
// each admission evaluates Theta = tau * SPS(B): B = verify rows in the batch,
// tau = expected tokens the step emits (one bonus token per request plus the
// admitted S values), SPS = the engine's measured verify steps per second at
// B rows.  It keeps the batch with the largest Theta.
//
// Because S does not grow along a request's positions, every prefix of the
// sorted order admits whole prefixes of each request's drafts (equal values
// are ordered by position), and it is the largest tau for its B: the greedy
// batch is the best prefix-closed batch for every B.
#include <math.h>

#include <algorithm>
#include <vector>

#include "sv_internal.h"

namespace {

struct Cand {
  double s;  // cumulative survival
  int i, k;  // request, draft position (1-based)
};

// SPS at b rows: linear interpolation in the table, clamped at its ends
double sps_at(const float *rows, const float *value, int n, double b) {
  if (b <= rows[0]) return value[0];
  if (b >= rows[n - 1]) return value[n - 1];
  int j = 1;
  while (rows[j] < b) ++j;
  const double t = (b - rows[j - 1]) / ((double)rows[j] - rows[j - 1]);
  return value[j - 1] + t * ((double)value[j] - value[j - 1]);
}

}  // namespace

extern "C" int spec_verify_budget(const float *cond_survival, const int32_t *cu_draft, int batch,
                                  const float *sps_rows, const float *sps_value, int n_sps,
                                  int32_t *verify_len, int32_t *batch_rows, double *theta) {
  if (batch < 0 || n_sps < 1) return SV_ERR_SHAPE;
  if (!cu_draft || !sps_rows || !sps_value || !verify_len || !batch_rows || !theta) return SV_ERR_NULL;
  if (cu_draft[0] != 0) return SV_ERR_SHAPE;
  for (int i = 0; i < batch; ++i) {
    const int g = cu_draft[i + 1] - cu_draft[i];
    if (g < 0 || g > sv::kMaxTokens - 1) return SV_ERR_SHAPE;
  }
  const int n_cand = batch > 0 ? cu_draft[batch] : 0;
  if (n_cand > 0 && !cond_survival) return SV_ERR_NULL;
  for (int j = 0; j < n_sps; ++j) {
    if (!(sps_rows[j] > 0.f) || !isfinite(sps_rows[j]) || !(sps_value[j] >= 0.f) || !isfinite(sps_value[j]))
      return SV_ERR_SHAPE;
    if (j > 0 && !(sps_rows[j] > sps_rows[j - 1])) return SV_ERR_SHAPE;
  }
  std::vector<Cand> cand;
  cand.reserve(n_cand);
  for (int i = 0; i < batch; ++i) {
    double s = 1.0;
    for (int k = 1; k <= cu_draft[i + 1] - cu_draft[i]; ++k) {
      const float c = cond_survival[cu_draft[i] + k - 1];
      if (!(c >= 0.f && c <= 1.f)) return SV_ERR_SHAPE;  // also rejects NaN
      s *= c;
      cand.push_back(Cand{s, i, k});
    }
  }
  // S descending; equal S: earlier position, then lower request
  std::stable_sort(cand.begin(), cand.end(), [](const Cand &a, const Cand &b) {
    if (a.s != b.s) return a.s > b.s;
    if (a.k != b.k) return a.k < b.k;
    return a.i < b.i;
  });
  // admit one candidate at a time; keep the first batch with the largest Theta
  double tau = batch;
  double best = batch > 0 ? tau * sps_at(sps_rows, sps_value, n_sps, batch) : 0.0;
  size_t best_m = 0;
  for (size_t m = 1; m <= cand.size(); ++m) {
    tau += cand[m - 1].s;
    const double th = tau * sps_at(sps_rows, sps_value, n_sps, (double)batch + m);
    if (th > best) {
      best = th;
      best_m = m;
    }
  }
  for (int i = 0; i < batch; ++i) verify_len[i] = 0;
  for (size_t m = 0; m < best_m; ++m) verify_len[cand[m].i] = std::max(verify_len[cand[m].i], cand[m].k);
  *batch_rows = batch + (int)best_m;
  *theta = best;
  return SV_OK;
}
