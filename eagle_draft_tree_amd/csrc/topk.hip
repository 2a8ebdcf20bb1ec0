// Per-row top-k and log-probabilities over the vocabulary (the LM head's
// per-node top-k that drives the dynamic tree: "EAGLE-3 精读" §2; EAGLE-4
// blog, 关于 Efficient LM Head: the draft LM head is a large share of the
// draft forward).
//
// One kernel, grid (partitions of 4096 logits) x rows.  A workgroup loads
// its logits with 16-byte loads (all in flight at once) and writes the
// partition's (max, sum exp(x - max)) and its k best (value desc, id asc).
// Selection by threshold and rank: each wave finds the k-th largest of its
// 64 lanes' maxima, so at least k of the partition's logits reach the
// largest of the four wave thresholds and the partition's k best are all
// among the logits at or above it (about 3k of 4096 for Gaussian logits);
// those candidates go to LDS and each one's rank is counted against the
// others.  The last workgroup of a row to finish (a per-row arrival
// counter, zeroed by a small kernel before the launch) merges the
// partitions the same way: the threshold is the larger of the k-th largest
// partition maximum and the largest partition k-th value.  A candidate set larger than the LDS list
// (many equal logits) falls back to k rounds of wavefront argmax, which
// gives the same result.  Ties: value desc, then id asc, everywhere.
//
// Cross-workgroup hand-off without an L2 write-back: the partials are
// written with agent-scope atomic stores (write-through to the device's
// coherence point), each wave waits for its stores to complete before the
// barrier that precedes the counter increment, and the merging workgroup
// reads them with agent-scope atomic loads.
#include <limits.h>

#include "common.hpp"
#include "gemm_rows.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int TK_THREADS = 256;
constexpr int TK_PER_THREAD = 16;
constexpr int TK_PS = TK_THREADS * TK_PER_THREAD;  // 4096 elements per partition
constexpr int TK_CMAX = 256;                       // candidates ranked in LDS

struct Cand {
  float v;
  int id;
};

template <typename X>
__device__ __forceinline__ void st_dev(X* p, X v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename X>
__device__ __forceinline__ X ld_dev(const X* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// k-th largest of the wave's values counted with multiplicity (at least k
// lanes hold a value >= the result), or -inf when fewer than k lanes hold a
// finite value.  Uniform result.
__device__ __forceinline__ float wave_kth_largest(float x, int k) {
  int got = 0;
  float t = -INFINITY;
  while (got < k) {
    const float mx = wave_max(x);
    if (mx == -INFINITY) return -INFINITY;
    got += __popcll(__ballot(x == mx));
    if (x == mx) x = -INFINITY;
    t = mx;
  }
  return t;
}

// Rank each of the C <= TK_CMAX candidates (value, id bits) among the others
// and write the k best in order; slots past C get (-inf, INT_MAX).  The list
// is padded with (-inf, INT_MAX) entries to a multiple of 8, which are never
// better than a candidate.
template <bool DEV>
__device__ __forceinline__ void rank_and_write(const float2* cand, int C, int k, float* ov, int32_t* oi, float sub) {
  auto put = [&](int r, float v, int id) {
    if (DEV) {
      st_dev(ov + r, v);
      st_dev(oi + r, id);
    } else {
      ov[r] = v;
      oi[r] = id;
    }
  };
  const int t = threadIdx.x;
  if (t < C) {
    const float2 me = cand[t];
    const int id = __float_as_int(me.y);
    int r = 0;
    for (int j0 = 0; j0 < C; j0 += 8) {
      float2 c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = cand[j0 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += better(c[u].x, __float_as_int(c[u].y), me.x, id) ? 1 : 0;
    }
    if (r < k) put(r, me.x - sub, id);
  } else if (t < k) {
    put(t, -INFINITY - sub, INT_MAX);
  }
}

// Append (v, id) to the LDS candidate list (dropped past TK_CMAX; the
// caller then takes the fallback).
__device__ __forceinline__ void push_cand(float2* cand, int* ncand, float v, int id) {
  const int pos = atomicAdd(ncand, 1);
  if (pos < TK_CMAX) cand[pos] = make_float2(v, __int_as_float(id));
}

// Pad the list read back as C entries to a multiple of 8 (call between two
// barriers).
__device__ __forceinline__ void pad_cand(float2* cand, int C) {
  const int t = threadIdx.x;
  if (C <= TK_CMAX && t >= C && t < ((C + 7) & ~7)) cand[t] = make_float2(-INFINITY, __int_as_float(INT_MAX));
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* __restrict__ logits, int V, int k, int nparts,
                                                          float* pv, int* pid, float* pm, float* ps,
                                                          unsigned* done, int32_t* __restrict__ ids,
                                                          float* __restrict__ lp, float* __restrict__ lse_out) {
  const int part = blockIdx.x, row = blockIdx.y;
  const float* x = logits + (size_t)row * V;
  const int lo = part * TK_PS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float2 cand[TK_CMAX + 8];
  __shared__ float mred[TK_THREADS / 64], sred[TK_THREADS / 64], tred[TK_THREADS / 64];
  __shared__ Cand wl[TK_THREADS / 64][EAGLE3_MAX_TOPK];
  __shared__ int ncand, last;
  __shared__ float rowL, rowT;
  if (tid == 0) ncand = 0;

  // element e of this thread: id lo + 4*(tid + 256*(e/4)) + e%4 (ids rise with e)
  float v[TK_PER_THREAD];
  const bool vec_ok = (V & 3) == 0;
#pragma unroll
  for (int j = 0; j < TK_PER_THREAD / 4; ++j) {
    const int y0 = lo + 4 * (tid + TK_THREADS * j);
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
  auto id_of = [&](int e) { return lo + 4 * (tid + TK_THREADS * (e >> 2)) + (e & 3); };
  uint32_t taken = 0;  // past V (and, in the fallback, removed)
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
  // (max, sum): max first, then sums rescaled to it, added in a fixed order
  const float wm = wave_max(m);
  const float tw = wave_kth_largest(m, k);
  if (lane == 0) {
    mred[w] = wm;
    tred[w] = tw;
  }
  __syncthreads();
  float M = -INFINITY, T = -INFINITY;
#pragma unroll
  for (int i = 0; i < TK_THREADS / 64; ++i) {
    M = fmaxf(M, mred[i]);
    T = fmaxf(T, tred[i]);
  }
  const float mine = (m == -INFINITY) ? 0.f : s * expf(m - M);
  const float ws = wave_sum(mine);
  if (lane == 0) sred[w] = ws;
  // candidates: every logit at or above the threshold
#pragma unroll
  for (int e = 0; e < TK_PER_THREAD; ++e)
    if (!((taken >> e) & 1u) && v[e] >= T) push_cand(cand, &ncand, v[e], id_of(e));
  __syncthreads();
  const int C = ncand;
  pad_cand(cand, C);
  __syncthreads();
  const size_t o = (size_t)row * nparts + part;
  if (tid == 0) {
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < TK_THREADS / 64; ++i) S += sred[i];
    st_dev(pm + o, M);
    st_dev(ps + o, S);
  }
  if (C <= TK_CMAX) {
    rank_and_write<true>(cand, C, k, pv + o * k, pid + o * k, 0.f);
  } else {
    // fallback: per-wave k best by k rounds of wavefront argmax over the
    // lanes' bests, then wave 0 pops the k best of the four wave lists
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
    for (int r = 0; r < k; ++r) {
      Cand c{bv, bi};
      wave_argmax(c.v, c.id);
      if (lane == 0) wl[w][r] = c;
      if (bi == c.id && c.id != INT_MAX) {
        taken |= 1u << be;
        rescan();
      }
    }
    __syncthreads();
    if (w == 0) {
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
          st_dev(pv + o * k + r, c.v);
          st_dev(pid + o * k + r, c.id);
        }
        if (mc.id == c.id) mc = Cand{-INFINITY, INT_MAX};
      }
    }
  }

  // ---- the row's last workgroup merges the partitions
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
  __syncthreads();
  if (tid == 0) last = atomicAdd(&done[row], 1u) == (unsigned)(nparts - 1);
  __syncthreads();
  if (!last) return;
  const int n = nparts * k;  // <= 64 * 16
  const float* rv = pv + (size_t)row * n;
  const int* ri = pid + (size_t)row * n;
  // every list entry of the row, loaded at once (4 per thread)
  float lv[4];
  int li[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + TK_THREADS * j;
    lv[j] = i < n ? ld_dev(rv + i) : -INFINITY;
    li[j] = i < n ? ld_dev(ri + i) : INT_MAX;
  }
  if (w == 0) {
    // LSE over the partitions' (max, sum) pairs (nparts <= 64), fixed order
    const float pmv = lane < nparts ? ld_dev(pm + (size_t)row * nparts + lane) : -INFINITY;
    const float psv = lane < nparts ? ld_dev(ps + (size_t)row * nparts + lane) : 0.f;
    const float head = lane < nparts ? ld_dev(rv + lane * k) : -INFINITY;
    const float kth = lane < nparts ? ld_dev(rv + lane * k + k - 1) : -INFINITY;
    const float M2 = wave_max(pmv);
    const float L = M2 + logf(wave_sum(pmv == -INFINITY ? 0.f : psv * expf(pmv - M2)));
    // threshold: at least k list entries reach it
    const float T2 = fmaxf(wave_kth_largest(head, k), wave_max(kth));
    if (lane == 0) {
      rowL = L;
      rowT = T2;
      ncand = 0;
      if (lse_out) lse_out[row] = L;
    }
  }
  __syncthreads();
  const float L = rowL, T2 = rowT;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (li[j] != INT_MAX && lv[j] >= T2) push_cand(cand, &ncand, lv[j], li[j]);
  __syncthreads();
  const int C2 = ncand;
  pad_cand(cand, C2);
  __syncthreads();
  if (C2 <= TK_CMAX) {
    rank_and_write<false>(cand, C2, k, lp + (size_t)row * k, ids + (size_t)row * k, L);
  } else if (w == 0) {
    // fallback: lane l holds list entries l, l+64, ...; k rounds of argmax
    constexpr int SLOTS = 16;
    float cv[SLOTS];
    int ci[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int i = lane + 64 * j;
      cv[j] = i < n ? ld_dev(rv + i) : -INFINITY;
      ci[j] = i < n ? ld_dev(ri + i) : INT_MAX;
    }
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
  }
}

// Top-1 from (max, sum exp(x - max), argmax) partials: one workgroup per
// row; the maximum and its lowest id by (value desc, id asc), then the LSE
// with each thread's partials added in index order and the threads' sums in
// a fixed order.
__global__ __launch_bounds__(256) void top1_merge_kernel(const float4* __restrict__ part, int nparts,
                                                         int32_t* __restrict__ ids, float* __restrict__ lp) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float4* p = part + (size_t)row * nparts;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int i = tid; i < nparts; i += 256) {
    const float4 c = p[i];
    if (better(c.x, __float_as_int(c.z), bv, bi)) {
      bv = c.x;
      bi = __float_as_int(c.z);
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    wv[w] = bv;
    wi[w] = bi;
  }
  __syncthreads();
  float M = wv[0];
  int id = wi[0];
  for (int u = 1; u < 4; ++u)
    if (better(wv[u], wi[u], M, id)) {
      M = wv[u];
      id = wi[u];
    }
  float s = 0.f;
  for (int i = tid; i < nparts; i += 256) {
    const float4 c = p[i];
    if (c.x > -INFINITY) s += c.y * expf(c.x - M);
  }
  s = wave_sum(s);
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) {
    const float L = M + logf((red[0] + red[1]) + (red[2] + red[3]));
    ids[row] = id;
    lp[row] = M - L;
  }
}

hipError_t launch_top1_merge(const float4* part, int rows, int nparts, int32_t* ids, float* lp, hipStream_t st) {
  top1_merge_kernel<<<rows, 256, 0, st>>>(part, nparts, ids, lp);
  return hipGetLastError();
}

// Top-k from the LM head's per-tile statistics (EpiLogitsTiles, one launch
// of at most 64 rows): one workgroup per row.  Thread t holds the
// {max, sum exp} pairs of slots t, t + 512, ... (padding slots hold
// {-inf, 0}).  Each 16-lane row of threads takes its maximum: 32 group
// maxima, each a logit of a different group.  The threshold T is the largest
// group maximum that at least k group maxima reach (every wave counts this
// itself from LDS, no serial k rounds): k distinct logits are >= T, so the k
// best logits are all >= T and lie in the tiles whose maximum reaches T.
// Only those tiles' logits are read back (16 bytes per thread, all loads in
// flight together); the ones >= T are ranked in LDS.  The LSE adds each
// thread's pairs in slot order and the wave sums in a fixed order.  Too many
// candidate tiles or logits (many equal values) take k rounds of block
// argmax over the whole row, each restricted to what ranks after the
// previous pick: the same result.
constexpr int TT_THREADS = 512;
constexpr int TT_TPT = 33;      // slots per thread: vocab <= 262144 plus slot padding
constexpr int TT_TILES = 1024;  // candidate tiles
constexpr int TT_CMAX = 1024;   // candidate logits

__global__ __launch_bounds__(TT_THREADS) void topk_tiles_kernel(const float* __restrict__ logits,
                                                                const float2* __restrict__ part, TileSlots sl,
                                                                int V, int k, int32_t* __restrict__ ids,
                                                                float* __restrict__ lp) {
  constexpr int NW = TT_THREADS / 64;
  constexpr int NG = TT_THREADS / 16;  // 16-lane groups
  static_assert(NG == 32 && NG >= EAGLE3_MAX_TOPK, "one wave counts the group maxima; k <= groups");
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* x = logits + (size_t)row * V;
  const int ns = sl.count();
  const float2* p = part + (size_t)row * ns;
  __shared__ float2 cand[TT_CMAX + 8];
  __shared__ int tlist[TT_TILES];
  __shared__ __attribute__((aligned(16))) float gmax[NG];
  __shared__ float sred[NW];
  __shared__ float bval[NW];
  __shared__ int bidx[NW];
  __shared__ int ncand, ntile;
  if (tid == 0) {
    ncand = 0;
    ntile = 0;
  }
  float mx[TT_TPT], sx[TT_TPT];
#pragma unroll
  for (int j = 0; j < TT_TPT; ++j) {
    const int s = tid + TT_THREADS * j;
    const float2 pr = s < ns ? p[s] : make_float2(-INFINITY, 0.f);
    mx[j] = pr.x;
    sx[j] = pr.y;
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < TT_TPT; ++j) m = fmaxf(m, mx[j]);
  const float gm = row16_max(m);
  if ((lane & 15) == 0) gmax[tid >> 4] = gm;
  __syncthreads();
  // every wave: lane l < 32 counts the group maxima >= group maximum l
  float T, M;
  {
    const float mine = gmax[lane & (NG - 1)];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < NG; q += 4) {
      const float4 o = *(const float4*)(gmax + q);
      cnt += (o.x >= mine) + (o.y >= mine) + (o.z >= mine) + (o.w >= mine);
    }
    T = wave_max(cnt >= k ? mine : -INFINITY);
    M = wave_max(mine);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < TT_TPT; ++j)
    if (mx[j] > -INFINITY) s += sx[j] * expf(mx[j] - M);
  s = wave_sum(s);
  if (lane == 0) sred[w] = s;
  // the unrolled loop only compares and appends slot indices; the tile of a
  // slot (two integer divisions) is taken in a rolled pass over the listed
  // slots, which keeps the kernel's code (fetched cold by each of its few
  // workgroups) small
#pragma unroll
  for (int j = 0; j < TT_TPT; ++j) {
    const int sj = tid + TT_THREADS * j;
    if (sj < ns && mx[j] >= T) {
      const int pos = atomicAdd(&ntile, 1);
      if (pos < TT_TILES) tlist[pos] = sj;
    }
  }
  __syncthreads();
  // a padding slot (no tile) becomes -1, skipped below: it holds -inf, so it
  // reaches T only when T is -inf
  for (int i = tid; i < min(ntile, TT_TILES); i += TT_THREADS) tlist[i] = sl.tile(tlist[i]);
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < NW; i += 2) S += sred[i] + sred[i + 1];
  const float L = M + logf(S);
  const int NT = ntile;
  if (NT <= TT_TILES) {
    // quarter q of candidate tile i: 4 logits from one 16-byte load, two
    // loads per thread in flight per pass
    for (int e0 = 0; e0 < 4 * NT; e0 += 2 * TT_THREADS) {
      float4 f[2];
      int id0[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = e0 + tid + u * TT_THREADS;
        const int tt = e < 4 * NT ? tlist[e >> 2] : -1;  // -1: past the list, or a padding slot
        id0[u] = tt >= 0 ? tt * 16 + (e & 3) * 4 : -1;
        f[u] = id0[u] >= 0 ? *(const float4*)(x + id0[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (id0[u] < 0) continue;
        const float v4[4] = {f[u].x, f[u].y, f[u].z, f[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (v4[c] >= T) {
            const int pos = atomicAdd(&ncand, 1);
            if (pos < TT_CMAX) cand[pos] = make_float2(v4[c], __int_as_float(id0[u] + c));
          }
      }
    }
  }
  __syncthreads();
  const int C = ncand;
  int32_t* oi = ids + (size_t)row * k;
  float* ov = lp + (size_t)row * k;
  if (NT <= TT_TILES && C <= TT_CMAX) {
    const int C8 = (C + 7) & ~7;
    for (int i = C + tid; i < C8; i += TT_THREADS) cand[i] = make_float2(-INFINITY, __int_as_float(INT_MAX));
    __syncthreads();
    for (int c = tid; c < C; c += TT_THREADS) {
      const float2 me = cand[c];
      const int id = __float_as_int(me.y);
      int r = 0;
      for (int j0 = 0; j0 < C8; j0 += 8) {
        float2 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = cand[j0 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) r += better(o[u].x, __float_as_int(o[u].y), me.x, id) ? 1 : 0;
      }
      if (r < k) {
        oi[r] = id;
        ov[r] = me.x - L;
      }
    }
    for (int r = C + tid; r < k; r += TT_THREADS) {
      oi[r] = INT_MAX;
      ov[r] = -INFINITY;
    }
    return;
  }
  // fallback: k rounds of block argmax; round r takes the best (value desc,
  // id asc) among the logits that rank after round r-1's pick
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int id = tid; id < V; id += TT_THREADS) {
      const float v = x[id];
      if (better(pv, pi, v, id) && better(v, id, bv, bi)) {
        bv = v;
        bi = id;
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
      bval[w] = bv;
      bidx[w] = bi;
    }
    __syncthreads();
    bv = bval[0];
    bi = bidx[0];
#pragma unroll
    for (int i = 1; i < NW; ++i)
      if (better(bval[i], bidx[i], bv, bi)) {
        bv = bval[i];
        bi = bidx[i];
      }
    __syncthreads();
    if (tid == 0) {
      oi[r] = bi;
      ov[r] = bv - L;
    }
    pv = bv;
    pi = bi;
  }
}

hipError_t launch_topk_tiles(const float* logits, const float2* part, int tiles_per_wg, int rows, int V, int k,
                             int32_t* ids, float* lp, hipStream_t st) {
  const TileSlots sl = tile_slots(V / 16, tiles_per_wg);
  if (rows > 64 || sl.count() > TT_THREADS * TT_TPT) return hipErrorInvalidValue;
  topk_tiles_kernel<<<rows, TT_THREADS, 0, st>>>(logits, part, sl, V, k, ids, lp);
  return hipGetLastError();
}

__global__ void topk_zero_kernel(unsigned* done, int rows) {
  for (int i = threadIdx.x; i < rows; i += blockDim.x) done[i] = 0u;
}

static size_t topk_parts(int V) { return (V + TK_PS - 1) / TK_PS; }

size_t topk_ws_bytes(int rows, int V) {
  return (size_t)rows * topk_parts(V) * (EAGLE3_MAX_TOPK * 8 + 8) + (size_t)rows * 4 + 256;
}

static unsigned* topk_counters(void* ws, int rows, int V) {
  return (unsigned*)((unsigned char*)ws + (size_t)rows * topk_parts(V) * (EAGLE3_MAX_TOPK * 8 + 8));
}

hipError_t launch_topk(const float* logits, int rows, int V, int k, int32_t* ids, float* lp, float* lse, void* ws,
                       hipStream_t st) {
  const int nparts = (int)topk_parts(V);  // <= 64 (V <= 262144)
  float* pv = (float*)ws;
  int* pid = (int*)(pv + (size_t)rows * nparts * k);
  float* pm = (float*)(pid + (size_t)rows * nparts * k);
  float* ps = pm + (size_t)rows * nparts;
  unsigned* done = topk_counters(ws, rows, V);
  topk_zero_kernel<<<1, 256, 0, st>>>(done, rows);
  topk_kernel<<<dim3(nparts, rows), TK_THREADS, 0, st>>>(logits, V, k, nparts, pv, pid, pm, ps, done, ids, lp, lse);
  return hipGetLastError();
}

}  // namespace e3
