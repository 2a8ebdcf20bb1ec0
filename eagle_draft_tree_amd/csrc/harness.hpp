// Internal interface of the EAGLE-4 Harness rules (host code) and of the
// kernel that reads the confidences they need out of the tree state.
#pragma once
#include <hip/hip_runtime.h>

#include "eagle3.h"

namespace e3 {
double harness_cost(const eagle3_cost_table& t, int kind, int B, int ctx, double n);
int harness_continue(const eagle3_cost_table& t, int B, int ctx, int k, int depth, const float* logconf,
                     double tau0, double alpha, double* total_gain);
int harness_verify_count(const eagle3_cost_table& t, int B, int ctx, int m_max, const float* logconf, double tau);
int harness_branch_cap(const eagle3_cost_table& t, int B, int ctx, const float* root_lp, double tau);
hipError_t launch_tree_confidence(int B, int k, int D, int m_max, const void* state, float* frontier,
                                  float* pool_sorted, hipStream_t st);
}  // namespace e3
