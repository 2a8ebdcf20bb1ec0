// EAGLE-2 confidence-value dynamic tree ("EAGLE-3 精读" §2: inference keeps
// EAGLE-2's dynamic tree; EAGLE-4 blog, 几条技术路线正在收敛: confidence is
// the product of draft probabilities -- kept here as a float32 sum of
// log-probs) and the top-m rerank that chooses what is sent to verification.
//
// One workgroup per request.  The candidate pool lives in the caller's tree
// state buffer; selections are computed by parallel rank counting, so every
// decision is deterministic and independent of thread timing.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int TREE_THREADS = 256;
constexpr int HDR_INTS = 64;  // round, root_tok, root_pos, npool, frontier[16], ...

struct Pool {
  int* hdr;
  int *tok, *parent, *depth, *flat, *rank, *slot;
  float* score;
  uint64_t* anc;
};

static __host__ __device__ inline int pool_max(int k, int D) { return k + (D - 1) * k * k; }

static __host__ __device__ inline size_t state_bytes(int k, int D) {
  const size_t P = pool_max(k, D);
  size_t b = HDR_INTS * 4 + P * (6 * 4 + 4) ;
  b = (b + 7) & ~(size_t)7;
  b += P * 8;
  return (b + 255) & ~(size_t)255;
}

size_t tree_state_bytes_per_req(int k, int D) { return state_bytes(k, D); }

__device__ inline Pool pool_of(void* state, int b, int k, int D) {
  unsigned char* base = (unsigned char*)state + (size_t)b * state_bytes(k, D);
  const int P = pool_max(k, D);
  Pool p;
  p.hdr = (int*)base;
  p.tok = p.hdr + HDR_INTS;
  p.parent = p.tok + P;
  p.depth = p.parent + P;
  p.flat = p.depth + P;
  p.rank = p.flat + P;
  p.slot = p.rank + P;
  p.score = (float*)(p.slot + P);
  size_t off = HDR_INTS * 4 + (size_t)P * 28;
  off = (off + 7) & ~(size_t)7;
  p.anc = (uint64_t*)(base + off);
  return p;
}

// (score desc, flat asc) -- frontier order inside one depth
__device__ __forceinline__ bool front_better(float sa, int fa, float sb, int fb) {
  return sa > sb || (sa == sb && fa < fb);
}
// (score desc, depth asc, flat asc) -- rerank order over the pool
__device__ __forceinline__ bool pool_better(float sa, int da, int fa, float sb, int db, int fb) {
  return sa > sb || (sa == sb && (da < db || (da == db && fa < fb)));
}

// Give the frontier nodes of depth j their tree slots (j-1)k + rank and emit
// the rows of the next draft step.
__device__ void emit_frontier(Pool& P, const int* front, int b, int k, int j, int root_pos,
                              int32_t* next_tok, int32_t* next_parent_slot, int32_t* next_pos,
                              uint64_t* next_anc) {
  for (int rho = threadIdx.x; rho < k; rho += blockDim.x) {
    const int n = front[rho];
    const int s = (j - 1) * k + rho;
    const int par = P.parent[n];
    const uint64_t pa = par >= 0 ? P.anc[par] : 0ull;
    P.slot[n] = s;
    P.anc[n] = pa | (1ull << s);
    next_tok[b * k + rho] = P.tok[n];
    next_parent_slot[b * k + rho] = par >= 0 ? 1 + P.slot[par] : 0;
    next_pos[b * k + rho] = root_pos + j;
    next_anc[b * k + rho] = pa | (1ull << s);
  }
}

__global__ __launch_bounds__(TREE_THREADS) void tree_init_kernel(
    int k, int D, const int32_t* root_tok, const int32_t* root_pos, void* state,
    const int32_t* ids, const float* lp, int32_t* next_tok, int32_t* next_parent_slot,
    int32_t* next_pos, uint64_t* next_anc) {
  const int b = blockIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ int front[EAGLE3_MAX_TOPK];
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    front[i] = i;
    P.tok[i] = ids[b * k + i];
    P.parent[i] = -1;
    P.depth[i] = 1;
    P.flat[i] = i;
    P.rank[i] = i;
    P.slot[i] = -1;
    P.score[i] = lp[b * k + i];
    P.anc[i] = 0ull;
    P.hdr[4 + i] = i;
  }
  if (threadIdx.x == 0) {
    P.hdr[0] = 1;
    P.hdr[1] = root_tok[b];
    P.hdr[2] = root_pos[b];
    P.hdr[3] = k;
  }
  __syncthreads();
  if (D > 1) emit_frontier(P, front, b, k, 1, root_pos[b], next_tok, next_parent_slot, next_pos, next_anc);
}

__global__ __launch_bounds__(TREE_THREADS) void tree_step_kernel(
    int k, int D, void* state, const int32_t* ids, const float* lp, int32_t* next_tok,
    int32_t* next_parent_slot, int32_t* next_pos, uint64_t* next_anc) {
  const int b = blockIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ int front[EAGLE3_MAX_TOPK];
  __shared__ int newfront[EAGLE3_MAX_TOPK];
  __shared__ float csc[EAGLE3_MAX_TOPK * EAGLE3_MAX_TOPK];
  const int j = P.hdr[0] + 1;
  if (j > D) return;  // the tree already has depth D
  const int base = P.hdr[3];
  const int root_pos = P.hdr[2];
  for (int i = threadIdx.x; i < k; i += blockDim.x) front[i] = P.hdr[4 + i];
  __syncthreads();
  const int kk = k * k;
  for (int c = threadIdx.x; c < kk; c += blockDim.x) {
    const int rho = c / k, i = c - rho * k;
    const int par = front[rho];
    const float sc = P.score[par] + lp[(size_t)(b * k + rho) * k + i];  // one fp32 add
    const int n = base + c;
    P.tok[n] = ids[(size_t)(b * k + rho) * k + i];
    P.parent[n] = par;
    P.depth[n] = j;
    P.flat[n] = c;
    P.rank[n] = i;
    P.slot[n] = -1;
    P.score[n] = sc;
    P.anc[n] = 0ull;
    csc[c] = sc;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < kk; c += blockDim.x) {
    int r = 0;
    for (int o = 0; o < kk; ++o) r += front_better(csc[o], o, csc[c], c);
    if (r < k) newfront[r] = base + c;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += blockDim.x) P.hdr[4 + i] = newfront[i];
  if (threadIdx.x == 0) {
    P.hdr[0] = j;
    P.hdr[3] = base + kk;
  }
  __syncthreads();
  if (j < D) emit_frontier(P, newfront, b, k, j, root_pos, next_tok, next_parent_slot, next_pos, next_anc);
}

constexpr int MAX_POOL = EAGLE3_MAX_TOPK + (EAGLE3_MAX_TREE_SLOTS)*EAGLE3_MAX_TOPK;

__global__ __launch_bounds__(TREE_THREADS) void tree_final_kernel(
    int k, int D, int m, void* state, int32_t* v_tok, int32_t* v_parent, int32_t* v_depth,
    int32_t* v_pos, uint64_t* v_anc) {
  const int b = blockIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ float sc[MAX_POOL];
  __shared__ short dp[MAX_POOL];
  __shared__ short fl[MAX_POOL];
  __shared__ short rk[MAX_POOL];
  __shared__ short par[MAX_POOL];
  __shared__ short vidx[MAX_POOL];  // -1 dropped, -2 kept (index pending), else verify index
  __shared__ short vnew[MAX_POOL];
  __shared__ uint64_t anc_s[EAGLE3_MAX_TREE_SLOTS];
  __shared__ int cnt_s[EAGLE3_MAX_TREE_SLOTS + 2];
  const int n = P.hdr[3];
  const int root_pos = P.hdr[2];
  const int M1 = m + 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    sc[i] = P.score[i];
    dp[i] = (short)P.depth[i];
    fl[i] = (short)P.flat[i];
    rk[i] = (short)P.rank[i];
    par[i] = (short)P.parent[i];
  }
  __syncthreads();
  // keep the first m by (score desc, depth asc, flat asc)
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int r = 0;
    const float s = sc[i];
    const int d = dp[i], f = fl[i];
    for (int o = 0; o < n; ++o) r += pool_better(sc[o], dp[o], fl[o], s, d, f);
    vidx[i] = r < m ? -2 : -1;
  }
  __syncthreads();
  // kept nodes per depth -> first verify index of each depth
  if (threadIdx.x == 0) {
    for (int d = 0; d <= D; ++d) cnt_s[d] = 0;
    for (int i = 0; i < n; ++i)
      if (vidx[i] == -2) cnt_s[dp[i]]++;
    int acc = 1;
    for (int d = 1; d <= D; ++d) {
      const int c = cnt_s[d];
      cnt_s[d] = acc;
      acc += c;
    }
  }
  __syncthreads();
  // canonical order, one depth at a time: (parent's verify index, child rank)
  for (int dep = 1; dep <= D; ++dep) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      if (vidx[i] != -2 || dp[i] != dep) continue;
      const int pv = par[i] < 0 ? 0 : vidx[par[i]];
      int pos = 0;
      for (int o = 0; o < n; ++o) {
        if (vidx[o] != -2 || dp[o] != dep) continue;
        const int pvo = par[o] < 0 ? 0 : vidx[par[o]];
        pos += (pvo < pv) || (pvo == pv && rk[o] < rk[i]);
      }
      vnew[i] = (short)(cnt_s[dep] + pos);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      if (vidx[i] == -2 && dp[i] == dep) vidx[i] = vnew[i];
    __syncthreads();
  }
  // bitsets: parents first (their indices are smaller), one depth at a time
  if (threadIdx.x == 0) anc_s[0] = 1ull;
  __syncthreads();
  for (int dep = 1; dep <= D; ++dep) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      if (vidx[i] < 0 || dp[i] != dep) continue;
      const int vi = vidx[i];
      const int pv = par[i] < 0 ? 0 : vidx[par[i]];
      anc_s[vi] = anc_s[pv] | (1ull << vi);
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    if (vidx[i] < 0) continue;
    const int vi = vidx[i];
    v_tok[b * M1 + vi] = P.tok[i];
    v_parent[b * M1 + vi] = par[i] < 0 ? 0 : vidx[par[i]];
    v_depth[b * M1 + vi] = dp[i];
    v_pos[b * M1 + vi] = root_pos + dp[i];
    v_anc[b * M1 + vi] = anc_s[vi];
  }
  if (threadIdx.x == 0) {
    v_tok[b * M1] = P.hdr[1];
    v_parent[b * M1] = -1;
    v_depth[b * M1] = 0;
    v_pos[b * M1] = root_pos;
    v_anc[b * M1] = 1ull;
  }
}

hipError_t launch_tree_expand(int phase, int B, int k, int D, int m, const int32_t* root_tok,
                              const int32_t* root_pos, void* state, const int32_t* topk_id,
                              const float* topk_lp, int32_t* next_tok, int32_t* next_parent_slot,
                              int32_t* next_pos, uint64_t* next_anc, int32_t* v_tok,
                              int32_t* v_parent, int32_t* v_depth, int32_t* v_pos, uint64_t* v_anc,
                              hipStream_t st) {
  if (phase == EAGLE3_INIT)
    tree_init_kernel<<<B, TREE_THREADS, 0, st>>>(k, D, root_tok, root_pos, state, topk_id, topk_lp,
                                                 next_tok, next_parent_slot, next_pos, next_anc);
  else if (phase == EAGLE3_STEP)
    tree_step_kernel<<<B, TREE_THREADS, 0, st>>>(k, D, state, topk_id, topk_lp, next_tok,
                                                 next_parent_slot, next_pos, next_anc);
  else
    tree_final_kernel<<<B, TREE_THREADS, 0, st>>>(k, D, m, state, v_tok, v_parent, v_depth, v_pos,
                                                  v_anc);
  return hipGetLastError();
}

}  // namespace e3
