// Per-row top-k and log-probabilities over the vocabulary (the LM head's
// per-node top-k that drives the dynamic tree: "EAGLE-3 精读" §2; EAGLE-4
// blog, 关于 Efficient LM Head: the draft LM head is a large share of the
// draft forward).
//
// Phase 1: the row is cut into PS-wide partitions; every thread keeps a
// sorted top-KMAX list of its strided elements in registers plus an online
// (max, sum exp) pair; the block then pops the k best heads by wavefront
// shuffles.  Phase 2 merges the partitions of a row (rank selection, fixed
// order LSE).  Order everywhere: value desc, id asc.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int TK_THREADS = 256;
constexpr int TK_PS = 4096;  // elements per partition

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Cand d{__shfl_xor(c.v, o, 64), __shfl_xor(c.id, o, 64)};
    if (better(d.v, d.id, c.v, c.id)) c = d;
  }
  return c;
}

template <int KMAX>
__global__ __launch_bounds__(TK_THREADS) void topk_partial_kernel(const float* __restrict__ logits,
                                                                  int V, int k, int nparts,
                                                                  float* pv, int* pid, float* pm,
                                                                  float* ps) {
  const int part = blockIdx.x, row = blockIdx.y;
  const float* x = logits + (size_t)row * V;
  const int lo = part * TK_PS, hi = min(V, lo + TK_PS);
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lv[j] = -INFINITY;
    li[j] = INT_MAX;
  }
  float m = -INFINITY, s = 0.f;
  for (int y = lo + threadIdx.x; y < hi; y += TK_THREADS) {
    const float v = x[y];
    if (v > m) {
      s = s * expf(m - v) + 1.f;
      m = v;
    } else if (v > -INFINITY) {
      s += expf(v - m);
    }
    if (better(v, y, lv[KMAX - 1], li[KMAX - 1])) {
      lv[KMAX - 1] = v;
      li[KMAX - 1] = y;
#pragma unroll
      for (int j = KMAX - 1; j > 0; --j) {
        if (better(lv[j], li[j], lv[j - 1], li[j - 1])) {
          const float tv = lv[j];
          lv[j] = lv[j - 1];
          lv[j - 1] = tv;
          const int ti = li[j];
          li[j] = li[j - 1];
          li[j - 1] = ti;
        }
      }
    }
  }
  __shared__ Cand wbest[TK_THREADS / 64];
  __shared__ float red[TK_THREADS / 64];
  __shared__ float mred[TK_THREADS / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t o = (size_t)row * nparts + part;
  // block (max, sum): max first, then rescaled sums in a fixed order
  float wm = wave_max(m);
  if (lane == 0) mred[w] = wm;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < TK_THREADS / 64; ++i) M = fmaxf(M, mred[i]);
  const float mine = (m == -INFINITY) ? 0.f : s * expf(m - M);
  const float S = block_sum(mine, red);
  if (threadIdx.x == 0) {
    pm[o] = M;
    ps[o] = S;
  }
  // k rounds of block argmax over the list heads
  for (int r = 0; r < k; ++r) {
    Cand c = wave_best(Cand{lv[0], li[0]});
    __syncthreads();
    if (lane == 0) wbest[w] = c;
    __syncthreads();
    Cand best = wbest[0];
    for (int i = 1; i < TK_THREADS / 64; ++i)
      if (better(wbest[i].v, wbest[i].id, best.v, best.id)) best = wbest[i];
    if (threadIdx.x == 0) {
      pv[o * k + r] = best.v;
      pid[o * k + r] = best.id;
    }
    if (li[0] == best.id) {  // the owner pops its head
#pragma unroll
      for (int j = 0; j < KMAX - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = INT_MAX;
    }
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(int k, int nparts, const float* pv,
                                                                const int* pid, const float* pm,
                                                                const float* ps, int32_t* ids,
                                                                float* lp, float* lse_out) {
  const int row = blockIdx.x;
  extern __shared__ unsigned char smem[];
  const int n = nparts * k;
  float* cv = (float*)smem;
  int* ci = (int*)(cv + n);
  __shared__ float lse_s;
  for (int i = threadIdx.x; i < n; i += TK_THREADS) {
    cv[i] = pv[(size_t)row * n + i];
    ci[i] = pid[(size_t)row * n + i];
  }
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, pm[(size_t)row * nparts + p]);
    float S = 0.f;
    for (int p = 0; p < nparts; ++p) {
      const float mp = pm[(size_t)row * nparts + p];
      if (mp != -INFINITY) S += ps[(size_t)row * nparts + p] * expf(mp - M);
    }
    lse_s = M + logf(S);
  }
  __syncthreads();
  const float L = lse_s;
  for (int i = threadIdx.x; i < n; i += TK_THREADS) {
    if (ci[i] == INT_MAX) continue;  // padding of a short partition
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (ci[j] != INT_MAX) && better(cv[j], ci[j], cv[i], ci[i]);
    if (rank < k) {
      ids[(size_t)row * k + rank] = ci[i];
      lp[(size_t)row * k + rank] = cv[i] - L;
    }
  }
  if (lse_out && threadIdx.x == 0) lse_out[row] = L;
}

size_t topk_ws_bytes(int rows, int V) {
  const size_t nparts = (V + TK_PS - 1) / TK_PS;
  return (size_t)rows * nparts * (EAGLE3_MAX_TOPK * 8 + 8) + 256;
}

hipError_t launch_topk(const float* logits, int rows, int V, int k, int32_t* ids, float* lp,
                       float* lse, void* ws, hipStream_t st) {
  const int nparts = (V + TK_PS - 1) / TK_PS;
  float* pv = (float*)ws;
  int* pid = (int*)(pv + (size_t)rows * nparts * k);
  float* pm = (float*)(pid + (size_t)rows * nparts * k);
  float* ps = pm + (size_t)rows * nparts;
  dim3 g1(nparts, rows);
  if (k <= 1) topk_partial_kernel<1><<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  else if (k <= 2) topk_partial_kernel<2><<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  else if (k <= 4) topk_partial_kernel<4><<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  else if (k <= 8) topk_partial_kernel<8><<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  else topk_partial_kernel<16><<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  const size_t sm = (size_t)nparts * k * 8;
  topk_merge_kernel<<<rows, TK_THREADS, sm, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  return hipGetLastError();
}

}  // namespace e3
