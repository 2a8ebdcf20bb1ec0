// Strict target verification of the draft tree ("EAGLE-3 精读" §5: with the
// drafter treated as a proposal, the standard verifier keeps the greedy
// sequence, or -- with the residual correction -- the sampling distribution).
//
// Tree children are deterministic top-k picks, so each candidate's proposal
// is a point mass: candidate x is accepted with probability p(x) of the
// remaining support, and a rejected token leaves the support -- the
// residual max(p - q, 0) renormalised.
//
// One kernel, grid (partition groups x requests * rows).  Every workgroup
// reduces two 4096-token partitions of one verify row: argmax (value
// desc, id asc), NaN flag and, for sampling, the partition max and sum of
// exp((L - max)/T) in fp64.  The last workgroup of a request to finish
// (arrival counters, each reset by its last arrival) walks the request's
// tree on those partials; at the last node of a sampling walk it locates the
// partition where the residual CDF crosses u_res * Rm and scans only that
// partition.  Arrival is counted in two levels, each counter on a 64-byte
// line of its own: a row's workgroups count on the row's counter, and the
// last of them on the request's counter (same-line atomics from hundreds
// of workgroups serialise).  The partials cross workgroups (and XCDs) through agent-scope
// stores and loads, each wave waiting for its stores before the barrier that
// precedes the counter increment: no L2 write-back.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int VR_THREADS = 256;  // threads per partition
constexpr int VR_EPT = 16;                   // tokens per thread (four 16-byte loads)
constexpr int VR_PS = VR_THREADS * VR_EPT;  // tokens per partition
constexpr int VR_PARTS = 2;      // partitions per workgroup
constexpr int VW_THREADS = VR_THREADS * VR_PARTS;
constexpr int VW_WAVES = VW_THREADS / 64;
constexpr int VCNT_STRIDE = 16;  // uints between arrival counters (one 64-byte line each)

template <typename X>
__device__ __forceinline__ void st_dev(X* p, X v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename X>
__device__ __forceinline__ X ld_dev(const X* p) {
  return __hip_atomic_load((X*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ArgRed {
  float v;
  int id;
};

__device__ __forceinline__ ArgRed arg_better(ArgRed a, ArgRed b) {
  return better(b.v, b.id, a.v, a.id) ? b : a;
}

__device__ __forceinline__ ArgRed wave_arg(ArgRed a) {
  wave_argmax(a.v, a.id);
  return a;
}

// ---------------------------------------------------------------- the rows
// A workgroup of VW_THREADS reduces VR_PARTS partitions of one row: part
// sg (VR_THREADS threads, VR_EPT tokens each) takes partition blockIdx.x *
// VR_PARTS + sg.  Every barrier is reached by all parts (a part past the
// last partition reduces nothing).
__device__ __forceinline__ void verify_rows(
    int V, int nparts, const float* __restrict__ logits, int sample, double invT,
    float* __restrict__ pa_v, int* __restrict__ pa_id, float* __restrict__ pmax,
    double* __restrict__ psum, int* __restrict__ pnan) {
  constexpr int QW = VR_THREADS / 64;  // waves per quarter
  const int sg = threadIdx.x / VR_THREADS, lt = threadIdx.x - sg * VR_THREADS;
  const int part = blockIdx.x * VR_PARTS + sg;
  const bool valid = part < nparts;
  const size_t row = blockIdx.y;  // request * (m+1) + node
  const float* x = logits + row * V;
  const int lo = part * VR_PS;
  const int lane = lt & 63, w = lt >> 6;
  float v[VR_EPT];
  const bool vec_ok = (V & 3) == 0;
#pragma unroll
  for (int j = 0; j < VR_EPT / 4; ++j) {
    const int y0 = lo + 4 * (lt + VR_THREADS * j);
    if (valid && vec_ok && y0 + 3 < V) {
      const float4 f = *(const float4*)(x + y0);
      v[4 * j] = f.x;
      v[4 * j + 1] = f.y;
      v[4 * j + 2] = f.z;
      v[4 * j + 3] = f.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * j + c] = valid && y0 + c < V ? x[y0 + c] : -INFINITY;
    }
  }
  ArgRed best{-INFINITY, INT_MAX};
  int nan = 0;
#pragma unroll
  for (int e = 0; e < VR_EPT; ++e) {
    const int y = lo + 4 * (lt + VR_THREADS * (e >> 2)) + (e & 3);
    if (v[e] != v[e]) nan = 1;
    else if (y < V && better(v[e], y, best.v, best.id)) best = ArgRed{v[e], y};
  }
  __shared__ ArgRed ared[VR_PARTS * QW];
  __shared__ double dred[VR_PARTS * QW];
  __shared__ int nred[VR_PARTS * QW];
  best = wave_arg(best);
  const int wn = __any(nan) ? 1 : 0;
  if (lane == 0) {
    ared[sg * QW + w] = best;
    nred[sg * QW + w] = wn;
  }
  __syncthreads();
  ArgRed b = ared[sg * QW];
  int anynan = nred[sg * QW];
#pragma unroll
  for (int i = 1; i < QW; ++i) {
    b = arg_better(b, ared[sg * QW + i]);
    anynan |= nred[sg * QW + i];
  }
  const size_t o = row * nparts + part;
  if (sample) {  // uniform over the workgroup: the barrier below is too
    const double mx = (double)b.v;
    double s = 0.0;
    if (!anynan) {
#pragma unroll
      for (int e = 0; e < VR_EPT; ++e) {
        const int y = lo + 4 * (lt + VR_THREADS * (e >> 2)) + (e & 3);
        if (y < V && v[e] > -INFINITY) s += exp(((double)v[e] - mx) * invT);
      }
    }
    s = wave_sum_d(s);
    if (lane == 0) dred[sg * QW + w] = s;
    __syncthreads();
    if (lt == 0 && valid && !anynan) {
      double t = 0.0;
#pragma unroll
      for (int i = 0; i < QW; ++i) t += dred[sg * QW + i];
      st_dev(psum + o, t);
    }
  }
  if (lt == 0 && valid) {
    st_dev(pa_v + o, b.v);
    st_dev(pa_id + o, b.id);
    st_dev(pmax + o, b.v);
    st_dev(pnan + o, anynan);
  }
}

// ---------------------------------------------------------------- the walk
__device__ void verify_walk(
    int b, int m, int V, int Dmax, int nparts, const int32_t* __restrict__ v_tok,
    const int32_t* __restrict__ v_parent, const float* __restrict__ logits, int mode, double invT,
    const double* __restrict__ u_try, const double* __restrict__ u_res, const float* __restrict__ pa_v,
    const int* __restrict__ pa_id, const float* __restrict__ pmax, const double* __restrict__ psum,
    const int* __restrict__ pnan, int32_t* accept_len, int32_t* accepted, int32_t* bonus,
    int32_t* status) {
  const int M1 = m + 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ int kids[EAGLE3_MAX_TREE_SLOTS];
  __shared__ int nkids_s;
  __shared__ int rejected[EAGLE3_MAX_TREE_SLOTS];
  __shared__ double wpart[64];  // remaining weight of each partition (<= 64 partitions handled per pass)
  __shared__ double wsum[VW_WAVES];
  __shared__ int bonus_s;
  __shared__ ArgRed rowbest_s;
  __shared__ double rm_s, mx_s;
  __shared__ int nan_s;

  const int32_t* tok = v_tok + (size_t)b * M1;
  const int32_t* par = v_parent + (size_t)b * M1;
  int node = 0, nacc = 0, out_bonus = -1, st = 0;
  for (int iter = 0; iter <= M1; ++iter) {
    const size_t row = (size_t)b * M1 + node;
    const float* L = logits + row * V;
    if (w == 0) {
      // children of `node` in verify-index order: ballot over the parent array
      const int pi = (lane >= 1 && lane < M1) ? par[lane] : -2;
      const unsigned long long km = __ballot(pi == node);
      if (pi == node) kids[__popcll(km & ((1ull << lane) - 1ull))] = lane;
      // the row's partitions: lanes own p = lane, lane + 64, ...
      ArgRed bb{-INFINITY, INT_MAX};
      int nn = 0;
      for (int p = lane; p < nparts; p += 64) {
        bb = arg_better(bb, ArgRed{ld_dev(pa_v + row * nparts + p), ld_dev(pa_id + row * nparts + p)});
        nn |= ld_dev(pnan + row * nparts + p);
      }
      bb = wave_arg(bb);
      const int anynan = __any(nn) ? 1 : 0;
      double R = 0.0;
      if (mode == EAGLE3_SAMPLE && !anynan) {
        const double M = (double)bb.v;
        for (int p = lane; p < nparts; p += 64) {
          const float mp = ld_dev(pmax + row * nparts + p);
          if (mp > -INFINITY) R += ld_dev(psum + row * nparts + p) * exp(((double)mp - M) * invT);
        }
        R = wave_sum_d(R);
      }
      if (lane == 0) {
        nkids_s = __popcll(km);
        rowbest_s = bb;
        nan_s = anynan;
        rm_s = R;
        mx_s = (double)bb.v;
      }
    }
    __syncthreads();
    const ArgRed best = rowbest_s;
    if (nan_s) {
      st = EAGLE3_ENUMERIC;
      nacc = 0;
      out_bonus = -1;
      break;
    }
    const int nk = nacc < Dmax ? nkids_s : 0;  // a walk cut at Dmax ends as at a leaf
    if (mode == EAGLE3_GREEDY) {
      int next = -1;
      for (int c = 0; c < nk && next < 0; ++c)  // the first matching child in sibling order
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
    // ---- sampling: w(y) = exp((L[y] - max) / T) in fp64; Rm = remaining mass
    const double mx = mx_s;
    double Rm = rm_s;
    int next = -1, nrej = 0;
    for (int c = 0; c < nk; ++c) {
      const int ci = kids[c];
      const int t = tok[ci];
      const double wt = exp(((double)L[t] - mx) * invT);
      if (u_try[(size_t)b * M1 + ci] * Rm < wt) {
        next = ci;
        break;
      }
      if (threadIdx.x == 0) rejected[nrej] = t;
      ++nrej;
      Rm = Rm - wt;
    }
    __syncthreads();
    if (next >= 0) {
      if (threadIdx.x == 0) accepted[(size_t)b * Dmax + nacc] = next;
      ++nacc;
      node = next;
      continue;
    }
    // bonus: the smallest y outside the rejected set whose cumulative weight
    // (partitions in order; inside a partition, per-thread 8-token segments
    // in order) exceeds u_res[node] * Rm.
    const double thr = u_res[(size_t)b * M1 + node] * Rm;
    auto weight = [&](int y) -> double {
      for (int r = 0; r < nrej; ++r)
        if (rejected[r] == y) return 0.0;
      return exp(((double)L[y] - mx) * invT);
    };
    if (threadIdx.x == 0) bonus_s = INT_MAX;
    double before = 0.0;  // cumulative weight of the partitions already passed
    for (int p0 = 0; p0 < nparts; p0 += 64) {
      const int np = min(64, nparts - p0);
      // remaining weight of each partition: its sum rescaled, minus rejected tokens in it
      if (threadIdx.x < np) {
        const int p = p0 + threadIdx.x;
        const float mp = ld_dev(pmax + row * nparts + p);
        double s = mp > -INFINITY ? ld_dev(psum + row * nparts + p) * exp(((double)mp - mx) * invT) : 0.0;
        for (int r = 0; r < nrej; ++r)
          if (rejected[r] / VR_PS == p) s -= exp(((double)L[rejected[r]] - mx) * invT);
        wpart[threadIdx.x] = s > 0.0 ? s : 0.0;
      }
      __syncthreads();
      bool done = false;
      for (int q = 0; q < np && !done; ++q) {
        const double s = wpart[q];
        if (before + s <= thr) {
          before += s;
          continue;
        }
        // the crossing lies in partition p0 + q (or just after, by rounding): scan it
        const int lo = (p0 + q) * VR_PS;
        constexpr int SEG = VR_PS / VW_THREADS;  // tokens per thread
        const int y0 = lo + SEG * threadIdx.x;
        double seg = 0.0;
        double wy[SEG];
#pragma unroll
        for (int c = 0; c < SEG; ++c) {
          wy[c] = y0 + c < V ? weight(y0 + c) : 0.0;
          seg += wy[c];
        }
        // exclusive scan of the segment sums (waves, then wave totals)
        double incl = seg;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        double wbase = 0.0;
        for (int i = 0; i < w; ++i) wbase += wsum[i];
        double acc = before + wbase + (incl - seg);
#pragma unroll
        for (int c = 0; c < SEG; ++c) {
          acc += wy[c];
          if (wy[c] > 0.0 && acc > thr) {
            atomicMin(&bonus_s, y0 + c);
            break;
          }
        }
        __syncthreads();
        if (bonus_s != INT_MAX) {
          done = true;
        } else {
          // no crossing after all: continue from the total just scanned, the
          // same sum the scan compared against, not the partition's estimate
          double tot = 0.0;
          for (int i = 0; i < VW_WAVES; ++i) tot += wsum[i];
          before += tot;
        }
        __syncthreads();
      }
      if (done) break;
      __syncthreads();
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

__global__ __launch_bounds__(VW_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void verify_kernel(
    int m, int V, int Dmax, int nparts, const int32_t* __restrict__ v_tok, const int32_t* __restrict__ v_parent,
    const float* __restrict__ logits, int mode, double invT, const double* __restrict__ u_try,
    const double* __restrict__ u_res, float* pa_v, int* pa_id, float* pmax, double* psum, int* pnan,
    unsigned* arrive, int32_t* accept_len, int32_t* accepted, int32_t* bonus, int32_t* status) {
  verify_rows(V, nparts, logits, mode == EAGLE3_SAMPLE, invT, pa_v, pa_id, pmax, psum, pnan);
  __shared__ int last;
  const int row = blockIdx.y, b = row / (m + 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    // counters: row r at arrive[16 r], request b at arrive[16 (rows + b)]
    unsigned* rc = arrive + (size_t)row * VCNT_STRIDE;
    unsigned* qc = arrive + ((size_t)gridDim.y + b) * VCNT_STRIDE;
    int l = 0;
    if (atomicAdd(rc, 1u) == gridDim.x - 1) {
      *rc = 0u;  // every arrival of the row has been counted: ready for the next call
      if (atomicAdd(qc, 1u) == (unsigned)m) {
        *qc = 0u;
        l = 1;
      }
    }
    last = l;
  }
  __syncthreads();
  if (!last) return;
  verify_walk(b, m, V, Dmax, nparts, v_tok, v_parent, logits, mode, invT, u_try, u_res, pa_v, pa_id, pmax, psum,
              pnan, accept_len, accepted, bonus, status);
}

// Partials [B*(m+1)][nparts] (psum fp64, argmax value and id, max, NaN flag)
// from the start of the buffer; arrival counters (one per row, then one per
// request, 64 bytes apart) in its last sixth, from byte
// verify_cnt_off(ws_bytes).  The counter region depends on
// the buffer size alone, never on (B, m, V): calls of any shape that fit the
// buffer keep their partials below it, and every call leaves the counters it
// used at zero, so one zero fill serves every later call.
static size_t verify_cnt_off(size_t ws_bytes) { return (ws_bytes / 6 * 5) & ~(size_t)255; }

size_t verify_ws_bytes(int B, int m, int V) {
  const size_t nparts = (V + VR_PS - 1) / VR_PS;
  const size_t n = (size_t)B * (m + 1) * nparts;
  // S >= 1.2 (24 n + 1024) gives verify_cnt_off(S) >= 24 n; S >= 6 C + 1024
  // leaves the counters' C bytes in the last sixth.
  const size_t cnt = ((size_t)B * (m + 1) + B) * VCNT_STRIDE * 4;
  const size_t s1 = (n * (4 + 4 + 4 + 8 + 4) + 1024) * 6 / 5 + 1024, s2 = 6 * cnt + 1024;
  return s1 > s2 ? s1 : s2;
}

hipError_t launch_verify(int B, int m, int V, int Dmax, const int32_t* v_tok,
                         const int32_t* v_parent, const float* logits, int mode, float temperature,
                         const double* u_try, const double* u_res, int32_t* accept_len,
                         int32_t* accepted, int32_t* bonus, int32_t* status, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  const int nparts = (V + VR_PS - 1) / VR_PS;
  const size_t n = (size_t)B * (m + 1) * nparts;
  double* psum = (double*)ws;
  float* pa_v = (float*)(psum + n);
  int* pa_id = (int*)(pa_v + n);
  float* pmax = (float*)(pa_id + n);
  int* pnan = (int*)(pmax + n);
  unsigned* arrive = (unsigned*)((unsigned char*)ws + verify_cnt_off(ws_bytes));
  const double invT = mode == EAGLE3_SAMPLE ? 1.0 / (double)temperature : 1.0;
  dim3 ga((nparts + VR_PARTS - 1) / VR_PARTS, B * (m + 1));
  verify_kernel<<<ga, VW_THREADS, 0, st>>>(m, V, Dmax, nparts, v_tok, v_parent, logits, mode, invT, u_try, u_res,
                                           pa_v, pa_id, pmax, psum, pnan, arrive, accept_len, accepted, bonus,
                                           status);
  return hipGetLastError();
}

}  // namespace e3
