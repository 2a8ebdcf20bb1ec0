// Strict target verification of the draft tree ("EAGLE-3 精读" §5: with the
// drafter treated as a proposal, the standard verifier keeps the greedy
// sequence, or -- with the residual correction -- the sampling distribution).
//
// One workgroup per request walks the tree from the root: at every visited
// node it reduces that node's target-logit row (argmax, or fp64 weights and
// their total), tries the node's children in sibling order and either moves
// on or emits the bonus token.  Tree children are deterministic top-k picks,
// so each candidate's proposal is a point mass: candidate x is accepted with
// probability p(x) of the remaining support, and a rejected token leaves the
// support -- the residual max(p - q, 0) renormalised.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int VF_THREADS = 1024;
constexpr int VF_WAVES = VF_THREADS / 64;

struct ArgRed {
  float v;
  int id;
};

__device__ __forceinline__ ArgRed arg_better(ArgRed a, ArgRed b) {
  return better(b.v, b.id, a.v, a.id) ? b : a;
}

__global__ __launch_bounds__(VF_THREADS) void verify_kernel(int m, int V, int Dmax,
                                                            const int32_t* v_tok,
                                                            const int32_t* v_parent,
                                                            const float* logits, int mode,
                                                            float temperature, const double* u_try,
                                                            const double* u_res,
                                                            int32_t* accept_len, int32_t* accepted,
                                                            int32_t* bonus, int32_t* status) {
  const int b = blockIdx.x;
  const int M1 = m + 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ ArgRed ared[VF_WAVES];
  __shared__ double dred[VF_WAVES];
  __shared__ int nan_s;
  __shared__ int kids[EAGLE3_MAX_TREE_SLOTS];
  __shared__ int nkids_s;
  __shared__ int rejected[EAGLE3_MAX_TREE_SLOTS];
  __shared__ int nrej_s;
  __shared__ double seg_s[VF_THREADS];
  __shared__ int bonus_s;

  const int32_t* tok = v_tok + (size_t)b * M1;
  const int32_t* par = v_parent + (size_t)b * M1;
  int node = 0, nacc = 0, out_bonus = -1, st = 0;
  const double invT = 1.0 / (double)temperature;
  for (int iter = 0; iter <= M1; ++iter) {
    const float* row = logits + ((size_t)b * M1 + node) * V;
    if (threadIdx.x == 0) nan_s = 0;
    // children of `node` in sibling (= verify index) order
    if (threadIdx.x == 0) {
      int c = 0;
      for (int i = 1; i < M1; ++i)
        if (par[i] == node) kids[c++] = i;
      nkids_s = c;
    }
    __syncthreads();
    // argmax / max of the row (NaN flagged)
    ArgRed best{-INFINITY, INT_MAX};
    int hasnan = 0;
    for (int y = threadIdx.x; y < V; y += VF_THREADS) {
      const float v = row[y];
      if (v != v) hasnan = 1;
      else if (better(v, y, best.v, best.id)) best = ArgRed{v, y};
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ArgRed d{__shfl_xor(best.v, o, 64), __shfl_xor(best.id, o, 64)};
      best = arg_better(best, d);
    }
    if (hasnan) nan_s = 1;
    if (lane == 0) ared[w] = best;
    __syncthreads();
    best = ared[0];
    for (int i = 1; i < VF_WAVES; ++i) best = arg_better(best, ared[i]);
    if (nan_s) {
      st = EAGLE3_ENUMERIC;
      nacc = 0;
      out_bonus = -1;
      break;
    }
    const int nk = nacc < Dmax ? nkids_s : 0;  // a walk cut at Dmax ends as at a leaf
    if (mode == EAGLE3_GREEDY) {
      int next = -1;
      for (int c = 0; c < nk; ++c)
        if (tok[kids[c]] == best.id) next = kids[c];
      __syncthreads();
      if (next >= 0) {
        if (threadIdx.x == 0) accepted[(size_t)b * Dmax + nacc] = next;
        ++nacc;
        node = next;
        continue;
      }
      out_bonus = best.id;
      break;
    }
    // ---- sampling: w(y) = exp((L[y] - max) / T) in fp64
    const double mx = (double)best.v;
    double part = 0.0;
    for (int y = threadIdx.x; y < V; y += VF_THREADS) part += exp(((double)row[y] - mx) * invT);
    part = wave_sum_d(part);
    if (lane == 0) dred[w] = part;
    __syncthreads();
    double Rm = 0.0;
    for (int i = 0; i < VF_WAVES; ++i) Rm += dred[i];
    int next = -1, nrej = 0;
    for (int c = 0; c < nk; ++c) {
      const int ci = kids[c];
      const int t = tok[ci];
      const double wt = exp(((double)row[t] - mx) * invT);
      if (u_try[(size_t)b * M1 + ci] * Rm < wt) {
        next = ci;
        break;
      }
      if (threadIdx.x == 0) rejected[nrej] = t;
      ++nrej;
      Rm = Rm - wt;
    }
    if (next >= 0) {
      __syncthreads();
      if (threadIdx.x == 0) accepted[(size_t)b * Dmax + nacc] = next;
      ++nacc;
      node = next;
      continue;
    }
    if (threadIdx.x == 0) nrej_s = nrej;
    __syncthreads();
    // bonus: inverse CDF over the remaining support in token-id order.
    // Thread t owns the contiguous id segment [t*seg, (t+1)*seg); the
    // cumulative weight of y is (sum of the earlier segments, in order) +
    // (running sum inside y's segment).  The bonus is the smallest y whose
    // cumulative weight exceeds u_res * Rm.
    const double thr = u_res[(size_t)b * M1 + node] * Rm;
    const int seg = (V + VF_THREADS - 1) / VF_THREADS;
    const int lo = min(V, threadIdx.x * seg), hi = min(V, lo + seg);
    const int nrj = nrej_s;
    auto weight = [&](int y) -> double {
      for (int r = 0; r < nrj; ++r)
        if (rejected[r] == y) return 0.0;
      return exp(((double)row[y] - mx) * invT);
    };
    double s = 0.0;
    for (int y = lo; y < hi; ++y) s += weight(y);
    seg_s[threadIdx.x] = s;
    if (threadIdx.x == 0) bonus_s = INT_MAX;
    __syncthreads();
    if (threadIdx.x == 0) {  // exclusive prefix over segments, in order
      double acc = 0.0;
      for (int t = 0; t < VF_THREADS; ++t) {
        const double v = seg_s[t];
        seg_s[t] = acc;
        acc += v;
      }
    }
    __syncthreads();
    {
      double acc = seg_s[threadIdx.x];
      int first = INT_MAX;
      for (int y = lo; y < hi; ++y) {
        acc += weight(y);
        if (acc > thr) {
          first = y;
          break;
        }
      }
      if (first != INT_MAX) atomicMin(&bonus_s, first);
    }
    __syncthreads();
    if (bonus_s == INT_MAX && threadIdx.x == 0) {  // no crossing: last y with w > 0
      for (int y = V - 1; y >= 0; --y)
        if (weight(y) > 0.0) {
          bonus_s = y;
          break;
        }
    }
    __syncthreads();
    out_bonus = bonus_s;
    break;
  }
  if (threadIdx.x == 0) {
    accept_len[b] = nacc;
    for (int i = nacc; i < Dmax; ++i) accepted[(size_t)b * Dmax + i] = -1;
    if (st != 0)
      for (int i = 0; i < Dmax; ++i) accepted[(size_t)b * Dmax + i] = -1;
    bonus[b] = out_bonus;
    status[b] = st;
  }
}

hipError_t launch_verify(int B, int m, int V, int Dmax, const int32_t* v_tok,
                         const int32_t* v_parent, const float* logits, int mode, float temperature,
                         const double* u_try, const double* u_res, int32_t* accept_len,
                         int32_t* accepted, int32_t* bonus, int32_t* status, hipStream_t st) {
  verify_kernel<<<B, VF_THREADS, 0, st>>>(m, V, Dmax, v_tok, v_parent, logits, mode, temperature,
                                          u_try, u_res, accept_len, accepted, bonus, status);
  return hipGetLastError();
}

}  // namespace e3
