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
#include "harness.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int TREE_THREADS = 256;

// Per-request header: the round, the root, the pool size and the current
// frontier with everything the next step needs from it (its nodes' scores,
// tree slots, ancestor bits and path keys), so a step reads one header
// instead of chasing pool entries.
struct Hdr {
  int round, root_tok, root_pos, npool;
  int front[EAGLE3_MAX_TOPK];
  float fscore[EAGLE3_MAX_TOPK];
  int fslot[EAGLE3_MAX_TOPK];
  int pad[EAGLE3_MAX_TOPK % 2 + 2];
  uint64_t fanc[EAGLE3_MAX_TOPK];
  uint64_t fpath[EAGLE3_MAX_TOPK];
};
constexpr int HDR_BYTES = ((int)sizeof(Hdr) + 255) & ~255;

struct Pool {
  Hdr* hdr;
  int *tok, *parent, *depth, *flat, *rank, *slot;
  float* score;
  uint64_t* anc;
  uint64_t* path;  // child ranks along the root path, base k, the depth-1 ancestor's rank first
};

static __host__ __device__ inline int pool_max(int k, int D) { return k + (D - 1) * k * k; }

static __host__ __device__ inline size_t state_bytes(int k, int D) {
  const size_t P = pool_max(k, D);
  size_t b = HDR_BYTES + P * (6 * 4 + 4);
  b = (b + 7) & ~(size_t)7;
  b += P * 16;  // anc, path
  return (b + 255) & ~(size_t)255;
}

size_t tree_state_bytes_per_req(int k, int D) { return state_bytes(k, D); }

__device__ inline Pool pool_of(void* state, int b, int k, int D) {
  unsigned char* base = (unsigned char*)state + (size_t)b * state_bytes(k, D);
  const int P = pool_max(k, D);
  Pool p;
  p.hdr = (Hdr*)base;
  p.tok = (int*)(base + HDR_BYTES);
  p.parent = p.tok + P;
  p.depth = p.parent + P;
  p.flat = p.depth + P;
  p.rank = p.flat + P;
  p.slot = p.rank + P;
  p.score = (float*)(p.slot + P);
  size_t off = HDR_BYTES + (size_t)P * 28;
  off = (off + 7) & ~(size_t)7;
  p.anc = (uint64_t*)(base + off);
  p.path = p.anc + P;
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

// Give the frontier nodes of depth j their tree slots (j-1)k + rank, emit
// the rows of the next draft step and record the frontier in the header.
// front[rho] = pool node with token ftok[rho], fpar[rho] = its parent's
// frontier index in the previous header (-1 for depth 1), with that header's
// slot/anc (pslot, panc).
__device__ void emit_frontier(Pool& P, const int* front, const int* ftok, const int* fpar, const float* fsc,
                              const uint64_t* fpath, const int* pslot, const uint64_t* panc, int b, int k, int j,
                              int root_pos, int32_t* next_tok, int32_t* next_parent_slot, int32_t* next_pos,
                              uint64_t* next_anc) {
  for (int rho = threadIdx.x; rho < k; rho += blockDim.x) {
    const int n = front[rho];
    const int s = (j - 1) * k + rho;
    const int pr = fpar[rho];
    const uint64_t pa = pr >= 0 ? panc[pr] : 0ull;
    const uint64_t a = pa | (1ull << s);
    P.hdr->front[rho] = n;
    P.hdr->fscore[rho] = fsc[rho];
    P.hdr->fslot[rho] = s;
    P.hdr->fanc[rho] = a;
    P.hdr->fpath[rho] = fpath[rho];
    next_tok[b * k + rho] = ftok[rho];
    next_parent_slot[b * k + rho] = pr >= 0 ? 1 + pslot[pr] : 0;
    next_pos[b * k + rho] = root_pos + j;
    next_anc[b * k + rho] = a;
  }
}

__global__ __launch_bounds__(TREE_THREADS) void tree_init_kernel(
    int k, int D, const int32_t* root_tok, const int32_t* root_pos, void* state,
    const int32_t* ids, const float* lp, int32_t* next_tok, int32_t* next_parent_slot,
    int32_t* next_pos, uint64_t* next_anc) {
  const int b = blockIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ int front[EAGLE3_MAX_TOPK], ftok[EAGLE3_MAX_TOPK], fpar[EAGLE3_MAX_TOPK];
  __shared__ float fsc[EAGLE3_MAX_TOPK];
  __shared__ uint64_t fpath[EAGLE3_MAX_TOPK];
  const int rp = root_pos[b];
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    const int t = ids[b * k + i];
    const float sc = lp[b * k + i];
    front[i] = i;
    ftok[i] = t;
    fpar[i] = -1;
    fsc[i] = sc;
    fpath[i] = (uint64_t)i;
    P.tok[i] = t;
    P.parent[i] = -1;
    P.depth[i] = 1;
    P.flat[i] = i;
    P.rank[i] = i;
    P.score[i] = sc;
    P.path[i] = (uint64_t)i;
  }
  if (threadIdx.x == 0) {
    P.hdr->round = 1;
    P.hdr->root_tok = root_tok[b];
    P.hdr->root_pos = rp;
    P.hdr->npool = k;
  }
  __syncthreads();
  if (D > 1) emit_frontier(P, front, ftok, fpar, fsc, fpath, nullptr, nullptr, b, k, 1, rp, next_tok,
                           next_parent_slot, next_pos, next_anc);
  else
    for (int rho = threadIdx.x; rho < k; rho += blockDim.x) {  // depth-1 tree: the header still lists the frontier
      P.hdr->front[rho] = rho;
      P.hdr->fscore[rho] = fsc[rho];
      P.hdr->fslot[rho] = -1;
      P.hdr->fanc[rho] = 0ull;
      P.hdr->fpath[rho] = fpath[rho];
    }
}

// One depth step: the k*k candidates (frontier row rho, its i-th best token)
// get score = frontier score + lp, in one fp32 add; the k best by (score
// desc, flat index asc) become the next frontier.  Thread c owns candidate
// c (kk <= 256 = TREE_THREADS) and loads its id and log-prob before the
// header arrives; the selection counts each candidate's rank in LDS.
__global__ __launch_bounds__(TREE_THREADS) void tree_step_kernel(
    int k, int D, void* state, const int32_t* ids, const float* lp, int32_t* next_tok,
    int32_t* next_parent_slot, int32_t* next_pos, uint64_t* next_anc) {
  static_assert(TREE_THREADS >= EAGLE3_MAX_TOPK * EAGLE3_MAX_TOPK, "one thread per candidate");
  const int b = blockIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ int front[EAGLE3_MAX_TOPK], pslot[EAGLE3_MAX_TOPK];
  __shared__ float pscore[EAGLE3_MAX_TOPK];
  __shared__ uint64_t panc[EAGLE3_MAX_TOPK], ppath[EAGLE3_MAX_TOPK];
  __shared__ int newfront[EAGLE3_MAX_TOPK], newtok[EAGLE3_MAX_TOPK], newpar[EAGLE3_MAX_TOPK];
  __shared__ float newsc[EAGLE3_MAX_TOPK];
  __shared__ uint64_t newpath[EAGLE3_MAX_TOPK];
  __shared__ __attribute__((aligned(16))) float csc[EAGLE3_MAX_TOPK * EAGLE3_MAX_TOPK];
  const int kk = k * k;
  const int c = threadIdx.x;
  int ctok = 0;
  float clp = 0.f;
  if (c < kk) {  // ids/lp rows b*k + rho, column i: element b*kk + c
    ctok = ids[(size_t)b * kk + c];
    clp = lp[(size_t)b * kk + c];
  }
  const int j = P.hdr->round + 1;
  if (j > D) return;  // the tree already has depth D (same value in every thread)
  const int base = P.hdr->npool;
  const int root_pos = P.hdr->root_pos;
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    front[i] = P.hdr->front[i];
    pscore[i] = P.hdr->fscore[i];
    pslot[i] = P.hdr->fslot[i];
    panc[i] = P.hdr->fanc[i];
    ppath[i] = P.hdr->fpath[i];
  }
  __syncthreads();
  float sc = -INFINITY;
  uint64_t path = 0ull;
  if (c < kk) {
    const int rho = c / k, i = c - rho * k;
    sc = pscore[rho] + clp;  // one fp32 add
    path = ppath[rho] * (uint64_t)k + (uint64_t)i;
    const int n = base + c;
    P.tok[n] = ctok;
    P.parent[n] = front[rho];
    P.depth[n] = j;
    P.flat[n] = c;
    P.rank[n] = i;
    P.score[n] = sc;
    P.path[n] = path;
    csc[c] = sc;
  }
  for (int e = kk + c; e < ((kk + 3) & ~3); e += TREE_THREADS) csc[e] = -INFINITY;  // pad to a multiple of 4
  __syncthreads();
  if (c < kk) {
    // rank: candidates better by (score desc, flat asc); pads (-inf, flat >= kk) never are
    int r = 0;
    for (int q = 0; q < kk; q += 4) {
      const float4 o = *(const float4*)(csc + q);
      r += front_better(o.x, q, sc, c) + front_better(o.y, q + 1, sc, c) + front_better(o.z, q + 2, sc, c) +
           front_better(o.w, q + 3, sc, c);
    }
    if (r < k) {
      newfront[r] = base + c;
      newtok[r] = ctok;
      newpar[r] = c / k;
      newsc[r] = sc;
      newpath[r] = path;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    P.hdr->round = j;
    P.hdr->npool = base + kk;
  }
  if (j < D) {
    emit_frontier(P, newfront, newtok, newpar, newsc, newpath, pslot, panc, b, k, j, root_pos, next_tok,
                  next_parent_slot, next_pos, next_anc);
  } else {
    for (int rho = threadIdx.x; rho < k; rho += blockDim.x) {  // last depth: no more rows to draft
      P.hdr->front[rho] = newfront[rho];
      P.hdr->fscore[rho] = newsc[rho];
      P.hdr->fslot[rho] = -1;
      P.hdr->fanc[rho] = 0ull;
      P.hdr->fpath[rho] = newpath[rho];
    }
  }
}

constexpr int MAX_POOL = EAGLE3_MAX_TOPK + (EAGLE3_MAX_TREE_SLOTS)*EAGLE3_MAX_TOPK;

// Rerank key: smaller = better.  (score desc, depth asc, flat asc) packed
// into one 64-bit integer (the float's order-preserving bit image, negated).
__device__ __forceinline__ unsigned long long rerank_key(float score, int depth, int flat) {
  if (score == 0.f) score = 0.f;  // -0 and +0 compare equal
  uint32_t u = __float_as_uint(score);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in score
  return ((unsigned long long)(~u) << 32) | ((unsigned long long)depth << 16) | (unsigned)flat;
}

constexpr int FIN_THREADS = 256;
constexpr int FIN_SORT_MAX = 2048;  // power of two >= MAX_POOL

// Rerank and layout.  The whole pool's rerank keys (unique: (depth, flat)
// names a node) are sorted ascending with a bitonic network in LDS and the
// first m are kept.  The kept set holds every kept node's parent (a child's
// score is its parent's plus a log-probability <= 0, and ties prefer the
// shallower node), so the canonical verify order -- depth by depth, by
// (parent's verify index, child rank) -- is the order of (depth, path key):
// a node's path key lists the child ranks along its root path, most
// significant first, and the parents' verify order is their own path order.
// Wave 0 ranks the kept nodes by that key, then builds the ancestor bitsets
// depth by depth.
__global__ __launch_bounds__(FIN_THREADS) void tree_final_kernel(int k, int D, int m, void* state, int32_t* v_tok,
                                                                 int32_t* v_parent, int32_t* v_depth, int32_t* v_pos,
                                                                 uint64_t* v_anc) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  Pool P = pool_of(state, b, k, D);
  __shared__ unsigned long long sk[FIN_SORT_MAX];
  __shared__ unsigned long long ck[EAGLE3_MAX_TREE_SLOTS];
  __shared__ short vidx_of[MAX_POOL];  // verify index of each kept pool node
  __shared__ uint64_t anc_s[EAGLE3_MAX_TREE_SLOTS];
  const int n = P.hdr->npool;
  const int root_pos = P.hdr->root_pos;
  const int M1 = m + 1;
  const int mk = min(m, n);  // nodes kept
  int N = 64;
  while (N < n) N <<= 1;
  // 1. sort the pool's rerank keys (padding ~0 sorts last)
  for (int i = tid; i < N; i += FIN_THREADS) sk[i] = i < n ? rerank_key(P.score[i], P.depth[i], P.flat[i]) : ~0ull;
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (N >> 1); t += FIN_THREADS) {
        const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1)), j = i | stride;
        const unsigned long long x = sk[i], y = sk[j];
        if ((x > y) == ((i & size) == 0)) {
          sk[i] = y;
          sk[j] = x;
        }
      }
      __syncthreads();
    }
  }
  // 2. lane e < mk of wave 0: the e-th kept node and its canonical key
  int my_node = -1, my_dep = 0, my_par = -1;
  unsigned long long my_ck = ~0ull;
  if (tid < 64 && lane < mk) {
    const unsigned long long key = sk[lane];
    my_dep = (int)((key >> 16) & 0xffff);
    const int flat = (int)(key & 0xffff);
    my_node = my_dep == 1 ? flat : k + (my_dep - 2) * k * k + flat;
    my_par = P.parent[my_node];
    my_ck = ((unsigned long long)my_dep << 58) | P.path[my_node];
    ck[lane] = my_ck;
  }
  __syncthreads();
  int my_vidx = -1;
  if (my_node >= 0) {
    int r = 0;
    for (int e = 0; e < mk; ++e) r += ck[e] < my_ck ? 1 : 0;
    my_vidx = 1 + r;
    vidx_of[my_node] = (short)my_vidx;
  }
  if (tid == 0) anc_s[0] = 1ull;
  __syncthreads();
  const int my_pv = my_node >= 0 ? (my_par < 0 ? 0 : vidx_of[my_par]) : 0;
  // 3. ancestor bitsets, parents first
  for (int dep = 1; dep <= D; ++dep) {
    if (my_node >= 0 && my_dep == dep) anc_s[my_vidx] = anc_s[my_pv] | (1ull << my_vidx);
    __syncthreads();
  }
  if (my_node >= 0) {
    v_tok[b * M1 + my_vidx] = P.tok[my_node];
    v_parent[b * M1 + my_vidx] = my_pv;
    v_depth[b * M1 + my_vidx] = my_dep;
    v_pos[b * M1 + my_vidx] = root_pos + my_dep;
    v_anc[b * M1 + my_vidx] = anc_s[my_vidx];
  }
  if (tid == 0) {
    v_tok[b * M1] = P.hdr->root_tok;
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
    tree_final_kernel<<<B, FIN_THREADS, 0, st>>>(k, D, m, state, v_tok, v_parent, v_depth, v_pos, v_anc);
  return hipGetLastError();
}

// Confidences the harness rules read (EAGLE-4 blog, EAGLE-Harness): the
// frontier's log-confidences in frontier-rank order, and the pool's in
// rerank order -- descending; equal scores are equal values, so their order
// does not matter -- with -inf past the pool.  One workgroup per request;
// a bitonic sort of order-preserving keys in LDS.
__device__ __forceinline__ uint32_t desc_key(float s) {
  if (s == 0.f) s = 0.f;  // -0 and +0 compare equal
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in s
  return ~u;                                        // ascending in -s
}
__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t u = ~key;
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__global__ __launch_bounds__(FIN_THREADS) void tree_confidence_kernel(int k, int D, int m_max, void* state,
                                                                      float* __restrict__ frontier,
                                                                      float* __restrict__ pool_sorted) {
  const int b = blockIdx.x, tid = threadIdx.x;
  Pool P = pool_of(state, b, k, D);
  __shared__ uint32_t sk[FIN_SORT_MAX];
  const int n = P.hdr->npool;
  if (frontier && tid < k) frontier[(size_t)b * k + tid] = P.hdr->fscore[tid];
  int N = 64;
  while (N < n) N <<= 1;
  for (int i = tid; i < N; i += FIN_THREADS) sk[i] = i < n ? desc_key(P.score[i]) : 0xffffffffu;
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (N >> 1); t += FIN_THREADS) {
        const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1)), j = i | stride;
        const uint32_t x = sk[i], y = sk[j];
        if ((x > y) == ((i & size) == 0)) {
          sk[i] = y;
          sk[j] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < m_max; i += FIN_THREADS) pool_sorted[(size_t)b * m_max + i] = i < n ? key_score(sk[i]) : -INFINITY;
}

hipError_t launch_tree_confidence(int B, int k, int D, int m_max, const void* state, float* frontier,
                                  float* pool_sorted, hipStream_t st) {
  tree_confidence_kernel<<<B, FIN_THREADS, 0, st>>>(k, D, m_max, (void*)state, frontier, pool_sorted);
  return hipGetLastError();
}

}  // namespace e3
