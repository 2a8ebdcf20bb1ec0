// Per-row top-k and log-probabilities over the vocabulary (the LM head's
// per-node top-k that drives the dynamic tree: "EAGLE-3 精读" §2; EAGLE-4
// blog, 关于 Efficient LM Head: the draft LM head is a large share of the
// draft forward).
//
// Phase 1 (grid: partitions x rows): a workgroup loads its TK_PS logits with
// 16-byte loads into registers (all loads in flight at once), keeps a sorted
// top-KMAX list per thread, then each wave pops its k best heads with
// wavefront shuffles and wave 0 pops the k best of the 4 wave lists.
// It also writes the partition's (max, sum exp(x - max)).
// Phase 2 (grid: rows, one wave each): the partitions' candidates sit in
// registers and k rounds of wave argmax select the top-k; the LSE merges the
// partition pairs with shuffle reductions.  Order everywhere: value desc, id
// asc.  Every selection is a register/shuffle computation, so no step waits
// on a chain of dependent memory accesses.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int TK_THREADS = 256;
constexpr int TK_PER_THREAD = 16;
constexpr int TK_PS = TK_THREADS * TK_PER_THREAD;  // 4096 elements per partition

struct Cand {
  float v;
  int id;
};

template <int KMAX>
__device__ __forceinline__ void list_insert(float (&lv)[KMAX], int (&li)[KMAX], float v, int y) {
  if (!better(v, y, lv[KMAX - 1], li[KMAX - 1])) return;
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

template <int KMAX>
__global__ __launch_bounds__(TK_THREADS) void topk_partial_kernel(const float* __restrict__ logits,
                                                                  int V, int k, int nparts,
                                                                  float* __restrict__ pv,
                                                                  int* __restrict__ pid,
                                                                  float* __restrict__ pm,
                                                                  float* __restrict__ ps) {
  const int part = blockIdx.x, row = blockIdx.y;
  const float* x = logits + (size_t)row * V;
  const int lo = part * TK_PS;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // element e of this thread: lo + 4*(threadIdx.x + 256*j) + c, j < 4, c < 4
  float v[TK_PER_THREAD];
  const bool vec_ok = (V & 3) == 0;
#pragma unroll
  for (int j = 0; j < TK_PER_THREAD / 4; ++j) {
    const int y0 = lo + 4 * (threadIdx.x + TK_THREADS * j);
    if (vec_ok && y0 + 3 < V) {
      const float4 f = *(const float4*)(x + y0);
      v[4 * j] = f.x;
      v[4 * j + 1] = f.y;
      v[4 * j + 2] = f.z;
      v[4 * j + 3] = f.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * j + c] = y0 + c < V ? x[y0 + c] : -INFINITY;
    }
  }
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lv[j] = -INFINITY;
    li[j] = INT_MAX;
  }
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e) m = fmaxf(m, v[e]);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e) {
    const int y = lo + 4 * (threadIdx.x + TK_THREADS * (e >> 2)) + (e & 3);
    if (y < V) {
      if (v[e] > -INFINITY) s += expf(v[e] - m);
      list_insert<KMAX>(lv, li, v[e], y);
    }
  }
  __shared__ float mred[TK_THREADS / 64];
  __shared__ float sred[TK_THREADS / 64];
  __shared__ Cand wl[TK_THREADS / 64][KMAX];
  // (max, sum): max first, then sums rescaled to it, added in a fixed order
  const float wm = wave_max(m);
  if (lane == 0) mred[w] = wm;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < TK_THREADS / 64; ++i) M = fmaxf(M, mred[i]);
  const float mine = (m == -INFINITY) ? 0.f : s * expf(m - M);
  const float ws = wave_sum(mine);
  if (lane == 0) sred[w] = ws;
  // per-wave top-k: k rounds of wavefront argmax over the list heads
  for (int r = 0; r < k; ++r) {
    Cand c{lv[0], li[0]};
    wave_argmax(c.v, c.id);
    if (lane == 0) wl[w][r] = c;
    if (li[0] == c.id && c.id != INT_MAX) {  // the owner pops its head
#pragma unroll
      for (int j = 0; j < KMAX - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = INT_MAX;
    }
  }
  __syncthreads();
  const size_t o = (size_t)row * nparts + part;
  if (w == 0) {
    if (lane == 0) {
      float S = 0.f;
#pragma unroll
      for (int i = 0; i < TK_THREADS / 64; ++i) S += sred[i];
      pm[o] = M;
      ps[o] = S;
    }
    // lane i holds candidate i of the 4 wave lists; k rounds of wave argmax
    const int nc = (TK_THREADS / 64) * k;  // <= 64
    Cand mine{-INFINITY, INT_MAX};
    if (lane < nc) {
      const int ww = lane / k;
      mine = wl[ww][lane - ww * k];
    }
    for (int r = 0; r < k; ++r) {
      Cand c = mine;
      wave_argmax(c.v, c.id);
      if (lane == 0) {
        pv[o * k + r] = c.v;
        pid[o * k + r] = c.id;
      }
      if (mine.id == c.id) mine = Cand{-INFINITY, INT_MAX};
    }
  }
}

// Phase 2: one wave per row.  Lane l holds candidates l, l+64, ... (<= 16
// per lane), then k rounds of wave argmax pop the best; the LSE merges the
// partition (max, sum) pairs with shuffle reductions (fixed order).
constexpr int TK_MERGE_PER_LANE = 16;

__global__ __launch_bounds__(64) void topk_merge_kernel(int k, int nparts, const float* __restrict__ pv,
                                                        const int* __restrict__ pid, const float* __restrict__ pm,
                                                        const float* __restrict__ ps, int32_t* __restrict__ ids,
                                                        float* __restrict__ lp, float* __restrict__ lse_out) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = nparts * k;
  float cv[TK_MERGE_PER_LANE];
  int ci[TK_MERGE_PER_LANE];
#pragma unroll
  for (int j = 0; j < TK_MERGE_PER_LANE; ++j) {
    const int i = lane + 64 * j;
    cv[j] = i < n ? pv[(size_t)row * n + i] : -INFINITY;
    ci[j] = i < n ? pid[(size_t)row * n + i] : INT_MAX;
  }
  float pmv[2], psv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = lane + 64 * j;
    pmv[j] = p < nparts ? pm[(size_t)row * nparts + p] : -INFINITY;
    psv[j] = p < nparts ? ps[(size_t)row * nparts + p] : 0.f;
  }
  const float M = wave_max(fmaxf(pmv[0], pmv[1]));
  float sl = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) sl += pmv[j] == -INFINITY ? 0.f : psv[j] * expf(pmv[j] - M);
  const float L = M + logf(wave_sum(sl));
  for (int r = 0; r < k; ++r) {
    // this lane's best remaining candidate
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < TK_MERGE_PER_LANE; ++j)
      if (better(cv[j], ci[j], bv, bi)) {
        bv = cv[j];
        bi = ci[j];
      }
    float wv = bv;
    int wi = bi;
    wave_argmax(wv, wi);
    if (lane == 0) {
      ids[(size_t)row * k + r] = wi;
      lp[(size_t)row * k + r] = wv - L;
    }
#pragma unroll
    for (int j = 0; j < TK_MERGE_PER_LANE; ++j)
      if (ci[j] == wi) {
        cv[j] = -INFINITY;
        ci[j] = INT_MAX;
      }
  }
  if (lse_out && lane == 0) lse_out[row] = L;
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
  topk_merge_kernel<<<rows, 64, 0, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  return hipGetLastError();
}

}  // namespace e3
