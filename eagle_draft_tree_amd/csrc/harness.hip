// EAGLE-4 Harness: cost-aware control of the draft tree (EAGLE-4 blog, the
// EAGLE-Harness paragraph; the section on converging trends for the
// confidence and the threshold that rises with depth).
//
// A warm-up measures the time of one drafter round and of one
// verification step over batch sizes, context lengths and tokens per
// request; each round then compares the expected extra accepted tokens per
// extra millisecond with a threshold, in three places: one more draft
// layer, the number of drafted tokens sent to verification, and the branch
// cap (8 or 4 children per node).  The confidence of a node is the product
// of its path's draft probabilities, exp of the tree's float32 score.
//
// Host code: the rules read a few scores per request that
// eagle3_tree_confidence copies out of the tree state, and a table of a few
// dozen measured times.  Arithmetic in double, sums in index order.
#include <math.h>

#include "eagle3.h"
#include "harness.hpp"

namespace e3 {

namespace {
// the smallest measured value >= x, or the largest
int snap_up(const int32_t* vals, int n, int x) {
  for (int i = 0; i < n; ++i)
    if (vals[i] >= x) return i;
  return n - 1;
}
}  // namespace

double harness_cost(const eagle3_cost_table& t, int kind, int B, int ctx, double n) {
  const int ib = snap_up(t.batch, t.n_batch, B), ic = snap_up(t.ctx, t.n_ctx, ctx);
  const float* row = (kind == EAGLE3_COST_DRAFT ? t.draft_ms : t.verify_ms) + ((size_t)ib * t.n_ctx + ic) * t.n_tok;
  const int nt = t.n_tok;
  // linear interpolation over the measured token counts, clamped at the ends
  if (n <= (double)t.tok[0]) return (double)row[0];
  if (n >= (double)t.tok[nt - 1]) return (double)row[nt - 1];
  int j = 0;
  while (j + 1 < nt && (double)t.tok[j + 1] <= n) ++j;
  if (n == (double)t.tok[j]) return (double)row[j];
  const double slope = ((double)row[j + 1] - (double)row[j]) / ((double)t.tok[j + 1] - (double)t.tok[j]);
  return slope * (n - (double)t.tok[j]) + (double)row[j];
}

int harness_continue(const eagle3_cost_table& t, int B, int ctx, int k, int depth, const float* logconf,
                     double tau0, double alpha, double* total_gain) {
  double gain = 0.0;
  for (int b = 0; b < B; ++b) {
    double gb = 0.0;
    for (int j = 0; j < k; ++j) gb += exp((double)logconf[(size_t)b * k + j]);
    gain += gb;
  }
  if (total_gain) *total_gain = gain;
  const double ms = harness_cost(t, EAGLE3_COST_DRAFT, B, ctx, (double)k);
  if (!(ms > 0.0)) return 1;
  return gain / ms > tau0 * (1.0 + alpha * depth) ? 1 : 0;
}

int harness_verify_count(const eagle3_cost_table& t, int B, int ctx, int m_max, const float* logconf, double tau) {
  int n = 0;
  while (n < m_max) {
    double gain = 0.0;
    for (int b = 0; b < B; ++b) gain += exp((double)logconf[(size_t)b * m_max + n]);
    const double dt = harness_cost(t, EAGLE3_COST_VERIFY, B, ctx, (double)(n + 2)) -
                      harness_cost(t, EAGLE3_COST_VERIFY, B, ctx, (double)(n + 1));
    if (dt > 0.0 && !(gain / dt > tau)) break;
    ++n;
  }
  return n;
}

int harness_branch_cap(const eagle3_cost_table& t, int B, int ctx, const float* root_lp, double tau) {
  double gain = 0.0;
  for (int b = 0; b < B; ++b)
    for (int i = 4; i < 8; ++i) gain += exp((double)root_lp[(size_t)b * 8 + i]);
  const double dt = harness_cost(t, EAGLE3_COST_DRAFT, B, ctx, 8.0) - harness_cost(t, EAGLE3_COST_DRAFT, B, ctx, 4.0);
  return (dt <= 0.0 || gain / dt > tau) ? 8 : 4;
}

}  // namespace e3
