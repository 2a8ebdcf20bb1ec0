// Per-row top-k and log-probabilities over the vocabulary (the LM head's
// per-node top-k that drives the dynamic tree: "EAGLE-3 精读" §2; EAGLE-4
// blog, 关于 Efficient LM Head: the draft LM head is a large share of the
// draft forward).
//
// Phase 1 (grid: partitions x rows): a workgroup loads its TK_PS logits with
// 16-byte loads into registers (all loads in flight at once); each wave
// selects its k best in k rounds of wavefront argmax over the lanes' bests,
// and wave 0 pops the k best of the 4 wave lists.
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

// Phase 1.  Lane-level selection keeps no sorted lists: each lane tracks the
// best of its 16 values not yet taken (a removal bit mask, so every register
// index is static), each of the k rounds is one wavefront argmax, and only
// the lane that owned the winner rescans its 16 values.
__global__ __launch_bounds__(TK_THREADS) void topk_partial_kernel(const float* __restrict__ logits, int V, int k,
                                                                  int nparts, float* __restrict__ pv,
                                                                  int* __restrict__ pid, float* __restrict__ pm,
                                                                  float* __restrict__ ps) {
  const int part = blockIdx.x, row = blockIdx.y;
  const float* x = logits + (size_t)row * V;
  const int lo = part * TK_PS;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // element e of this thread: id lo + 4*(threadIdx.x + 256*(e/4)) + e%4 (ids rise with e)
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
  auto id_of = [&](int e) { return lo + 4 * (threadIdx.x + TK_THREADS * (e >> 2)) + (e & 3); };
  uint32_t taken = 0;  // removed or past V
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e)
    if (id_of(e) >= V) taken |= 1u << e;
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e) m = fmaxf(m, v[e]);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e)
    if (!((taken >> e) & 1u) && v[e] > -INFINITY) s += expf(v[e] - m);
  float bv;
  int bi, be;
  auto rescan = [&]() {
    bv = -INFINITY;
    bi = INT_MAX;
    be = 0;
#pragma unroll
    for (int e = 0; e < TK_PER_THREAD; ++e) {
      const int y = id_of(e);
      if (!((taken >> e) & 1u) && better(v[e], y, bv, bi)) {
        bv = v[e];
        bi = y;
        be = e;
      }
    }
  };
  rescan();
  __shared__ float mred[TK_THREADS / 64];
  __shared__ float sred[TK_THREADS / 64];
  __shared__ Cand wl[TK_THREADS / 64][EAGLE3_MAX_TOPK];
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
  // per-wave top-k: k rounds of wavefront argmax over the lanes' bests
  for (int r = 0; r < k; ++r) {
    Cand c{bv, bi};
    wave_argmax(c.v, c.id);
    if (lane == 0) wl[w][r] = c;
    if (bi == c.id && c.id != INT_MAX) {  // the owner takes it and rescans
      taken |= 1u << be;
      rescan();
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
    Cand mc{-INFINITY, INT_MAX};
    if (lane < nc) {
      const int ww = lane / k;
      mc = wl[ww][lane - ww * k];
    }
    for (int r = 0; r < k; ++r) {
      Cand c = mc;
      wave_argmax(c.v, c.id);
      if (lane == 0) {
        pv[o * k + r] = c.v;
        pid[o * k + r] = c.id;
      }
      if (mc.id == c.id) mc = Cand{-INFINITY, INT_MAX};
    }
  }
}

// Phase 2: one wave per row.  Lane l holds candidates l, l+64, ... (SLOTS
// per lane), then k rounds of wave argmax pop the best; the LSE merges the
// partition (max, sum) pairs with shuffle reductions (fixed order).
template <int SLOTS>
__global__ __launch_bounds__(64) void topk_merge_kernel(int k, int nparts, const float* __restrict__ pv,
                                                        const int* __restrict__ pid, const float* __restrict__ pm,
                                                        const float* __restrict__ ps, int32_t* __restrict__ ids,
                                                        float* __restrict__ lp, float* __restrict__ lse_out) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = nparts * k;
  float cv[SLOTS];
  int ci[SLOTS];
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int i = lane + 64 * j;
    cv[j] = i < n ? pv[(size_t)row * n + i] : -INFINITY;
    ci[j] = i < n ? pid[(size_t)row * n + i] : INT_MAX;
  }
  float pmv = lane < nparts ? pm[(size_t)row * nparts + lane] : -INFINITY;
  float psv = lane < nparts ? ps[(size_t)row * nparts + lane] : 0.f;
  const float M = wave_max(pmv);
  const float L = M + logf(wave_sum(pmv == -INFINITY ? 0.f : psv * expf(pmv - M)));
  float bv = -INFINITY;
  int bi = INT_MAX;
  auto rescan = [&]() {
    bv = -INFINITY;
    bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j)
      if (better(cv[j], ci[j], bv, bi)) {
        bv = cv[j];
        bi = ci[j];
      }
  };
  rescan();
  for (int r = 0; r < k; ++r) {
    float wv = bv;
    int wi = bi;
    wave_argmax(wv, wi);
    if (lane == 0) {
      ids[(size_t)row * k + r] = wi;
      lp[(size_t)row * k + r] = wv - L;
    }
    if (bi == wi) {
#pragma unroll
      for (int j = 0; j < SLOTS; ++j)
        if (ci[j] == wi) {
          cv[j] = -INFINITY;
          ci[j] = INT_MAX;
        }
      rescan();
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
  topk_partial_kernel<<<g1, TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps);
  const int n = nparts * k;  // nparts <= 64 (V <= 262144), k <= 16
  if (n <= 128) topk_merge_kernel<2><<<rows, 64, 0, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  else if (n <= 256) topk_merge_kernel<4><<<rows, 64, 0, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  else if (n <= 512) topk_merge_kernel<8><<<rows, 64, 0, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  else topk_merge_kernel<16><<<rows, 64, 0, st>>>(k, nparts, pv, pid, pm, ps, ids, lp, lse);
  return hipGetLastError();
}

}  // namespace e3
