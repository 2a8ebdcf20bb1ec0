// Tree-masked decode attention for the drafter ("EAGLE-3 精读" §1-§2: the
// draft decoder attends over the committed prefix plus the growing draft
// tree; the tree mask is an ancestor bitset per row).
//
// Split-K over the keys: workgroup (split s, kv head g / query group,
// request b) walks `cpw` consecutive 64-key chunks of the committed rows
// (or, for the last split index, the 64 tree slots) for every query vector
// (row, q head) of that KV head's GQA group, with an online softmax across
// its chunks.  K/V of a chunk are staged once in LDS and shared by all the
// group's query heads; the next chunk's K/V loads are in flight while the
// current chunk is computed.  Each workgroup writes a partial (max, sum,
// o[hd]); a merge kernel combines the splits in index order (deterministic).
//
// bf16 caches use attn_mfma_kernel (below): matrix-core scores and P.V with
// each wave streaming its own 32-key sub-chunks; fp32 caches use the
// vector-ALU attn_partial_kernel.

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int CH = 64;  // keys per chunk
constexpr int ATT_THREADS = 256;

struct AttnArgs {
  const void* q;   // [Rtot][Hq][hd]
  const void* kc;  // committed cache (contiguous or paged)
  const void* vc;
  const void* tk;  // tree slots [B][64][Hkv][hd]
  const void* tv;
  const int32_t* ctx_len;
  const int32_t* block_table;
  const uint64_t* anc;  // [Rtot] (TREE) or NULL
  int cap, max_blocks, block_size;
  int bs_log2;     // log2(block_size) when it is a power of two, else -1
  int B, rows, hq, hkv, mode, n_commit_splits, cpw, n_qgroups;
  int n_cache_sub, spw, nsplits;  // attn_mfma_kernel: cache sub-chunks, sub-chunks per wave, wave splits
  float scale;
  float* part_o;   // [Rtot*Hq][partials][hd]: partials = nsplits, or ceil(nsplits/4) merged
  float* part_ml;  // [Rtot*Hq][partials][2]
};

// 16-byte vector of T elements, unpacked to float.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};

// QG: query vectors per workgroup (8 or 32).  In the P.V phase thread t owns
// the (query, 16-byte vector) pair t % PAIRS over key range t / PAIRS of
// KSPL equal ranges: with few query vectors (QG = 8) the four waves split
// each chunk's keys, and the ranges are summed once per split.
constexpr int MAX_SPLIT_BLOCKS = 64;  // paged-table entries staged per split

template <typename T, int HD, int QG>
__global__ __launch_bounds__(ATT_THREADS) void attn_partial_kernel(AttnArgs a) {
  constexpr int EPV = Vec16<T>::N;             // elements per 16-byte vector
  constexpr int VPR = HD / EPV;                // vectors per key row
  constexpr int KPV = VPR + 1;                 // padded LDS row (vectors): spreads banks
  constexpr int LPT = CH * VPR / ATT_THREADS;  // staged vectors per thread (K and V each)
  constexpr int QPW = QG / 4;                  // query vectors per wave (score / softmax phase)
  constexpr int PAIRS = QG * VPR;              // (query, vector) pairs
  constexpr int KSPL = PAIRS >= ATT_THREADS ? 1 : ATT_THREADS / PAIRS;  // key ranges in P.V
  constexpr int PVJ = (PAIRS + ATT_THREADS - 1) / ATT_THREADS;           // pairs per thread
  constexpr int KPR = CH / KSPL;               // keys per range
  __shared__ uint4 ks[CH * KPV];
  __shared__ uint4 vs[CH * VPR];
  __shared__ float4 qs[QG * HD / 4];  // query vectors as float
  __shared__ float sc[QG * CH];
  __shared__ float alpha_s[QG];
  __shared__ int blk_s[MAX_SPLIT_BLOCKS];

  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_qgroups, qgrp = blockIdx.y - g * a.n_qgroups;
  const int b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int nq_total = a.rows * G;
  const int q0 = qgrp * QG;
  const int nq = min(QG, nq_total - q0);
  const int nsplits = a.n_commit_splits + 1;
  const bool tree_split = split == a.n_commit_splits;
  const int ctx = a.ctx_len[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (nq <= 0) return;
  const int nchunk = tree_split ? 1 : a.cpw;
  const int maxvis = a.mode == EAGLE3_TREE ? ctx : ctx + a.rows;  // rows visible to the last query
  auto chunk_keys = [&](int cc) {
    if (tree_split) return a.mode == EAGLE3_TREE ? (int)EAGLE3_MAX_TREE_SLOTS : 0;
    return min(CH, maxvis - (split * a.cpw + cc) * CH);
  };
  auto out_index = [&](int qi) {
    const int rr = (q0 + qi) / G, gi = (q0 + qi) - rr * G;
    const int row = b * a.rows + rr, h = g * G + gi;
    return (size_t)(row * a.hq + h) * nsplits + split;
  };
  // Tree slots no row of this request can see may hold stale data: they
  // are staged as zeros so that masked keys never feed NaN into P.V.
  // (anc exists only in TREE mode; in COMMIT mode the tree split has no keys.)
  uint64_t any_vis = ~0ull;
  if (tree_split && a.mode == EAGLE3_TREE) {
    any_vis = 0ull;
    for (int rr = 0; rr < a.rows; ++rr) any_vis |= a.anc[b * a.rows + rr];
  }
  // paged cache: the split's block-table entries, staged once when they fit
  const bool paged = a.block_table != nullptr && !tree_split;
  const int key0 = split * a.cpw * CH;
  const int nb = paged ? (a.cpw * CH + a.block_size - 1) / a.block_size + 1 : 0;
  const bool staged_table = paged && nb <= MAX_SPLIT_BLOCKS;
  if (staged_table) {
    for (int i = threadIdx.x; i < nb; i += ATT_THREADS) {
      const int lb = key0 / a.block_size + i;
      blk_s[i] = lb < a.max_blocks ? a.block_table[(size_t)b * a.max_blocks + lb] : 0;
    }
    __syncthreads();
  }
  uint4 kreg[LPT], vreg[LPT];
  auto load_chunk = [&](int cc) {
    const int nk = chunk_keys(cc);
    const int p0 = (split * a.cpw + cc) * CH;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int e = threadIdx.x + ATT_THREADS * j;
      const int p = e / VPR, c = e - p * VPR;
      kreg[j] = vreg[j] = make_uint4(0, 0, 0, 0);
      if (p < nk && ((any_vis >> p) & 1ull)) {
        size_t off;
        const T *kb, *vb;
        if (tree_split) {
          off = ((size_t)(b * EAGLE3_MAX_TREE_SLOTS + p) * a.hkv + g) * HD;
          kb = (const T*)a.tk;
          vb = (const T*)a.tv;
        } else {
          const int pos = p0 + p;
          if (paged) {
            const int blk = staged_table ? blk_s[pos / a.block_size - key0 / a.block_size]
                                         : a.block_table[(size_t)b * a.max_blocks + pos / a.block_size];
            off = (((size_t)blk * a.block_size + pos % a.block_size) * a.hkv + g) * HD;
          } else {
            off = (((size_t)b * a.cap + pos) * a.hkv + g) * HD;
          }
          kb = (const T*)a.kc;
          vb = (const T*)a.vc;
        }
        kreg[j] = *((const uint4*)(kb + off) + c);
        vreg[j] = *((const uint4*)(vb + off) + c);
      }
    }
  };
  // query vectors (q head h = g*G + gi of row rr), unpacked to float
  {
    const T* Q = (const T*)a.q;
    for (int e = threadIdx.x; e < nq * VPR; e += ATT_THREADS) {
      const int qi = e / VPR, c = e - qi * VPR;
      const int rr = (q0 + qi) / G, gi = (q0 + qi) - rr * G;
      const size_t row = (size_t)b * a.rows + rr;
      float f[EPV];
      Vec16<T>::unpack(*((const uint4*)(Q + (row * a.hq + g * G + gi) * HD) + c), f);
#pragma unroll
      for (int i = 0; i < EPV; i += 4) qs[(qi * HD + c * EPV + i) / 4] = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
    }
  }
  float m_run[QPW], l_run[QPW];
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }
  float acc[PVJ][EPV];
#pragma unroll
  for (int j = 0; j < PVJ; ++j)
#pragma unroll
    for (int i = 0; i < EPV; ++i) acc[j][i] = 0.f;

  if (chunk_keys(0) > 0) load_chunk(0);
  for (int cc = 0; cc < nchunk; ++cc) {
    const int nkeys = chunk_keys(cc);
    if (nkeys <= 0) break;
    const int p0 = (split * a.cpw + cc) * CH;
    __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int e = threadIdx.x + ATT_THREADS * j;
      const int p = e / VPR, c = e - p * VPR;
      ks[p * KPV + c] = kreg[j];
      vs[p * VPR + c] = vreg[j];
    }
    __syncthreads();
    if (cc + 1 < nchunk && chunk_keys(cc + 1) > 0) load_chunk(cc + 1);  // in flight during this chunk
    // scores: lane = key, wave w takes query vectors w, w+4, ...
    float s[QPW];
#pragma unroll
    for (int t = 0; t < QPW; ++t) s[t] = 0.f;
#pragma unroll 4
    for (int c = 0; c < VPR; ++c) {
      float kf[EPV];
      Vec16<T>::unpack(ks[lane * KPV + c], kf);
#pragma unroll
      for (int t = 0; t < QPW; ++t) {
        const int qi = wave + 4 * t;
        if (qi < nq) {
#pragma unroll
          for (int i = 0; i < EPV; i += 4) {
            const float4 q4v = qs[(qi * HD + c * EPV + i) / 4];
            s[t] = fmaf(q4v.x, kf[i], s[t]);
            s[t] = fmaf(q4v.y, kf[i + 1], s[t]);
            s[t] = fmaf(q4v.z, kf[i + 2], s[t]);
            s[t] = fmaf(q4v.w, kf[i + 3], s[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < QPW; ++t) {
      const int qi = wave + 4 * t;
      if (qi >= nq) continue;  // uniform per wave
      const int rr = (q0 + qi) / G;
      bool vis = lane < nkeys;
      if (tree_split) {
        vis = vis && ((a.anc[b * a.rows + rr] >> lane) & 1ull);
      } else {
        const int lim = a.mode == EAGLE3_TREE ? ctx : ctx + rr + 1;
        vis = vis && p0 + lane < lim;
      }
      const float sv = vis ? s[t] * a.scale : -INFINITY;
      const float m_new = fmaxf(m_run[t], wave_max(sv));
      const float al = m_new == -INFINITY ? 1.f : expf(m_run[t] - m_new);
      const float p = m_new == -INFINITY ? 0.f : expf(sv - m_new);
      l_run[t] = l_run[t] * al + wave_sum(p);
      m_run[t] = m_new;
      sc[qi * CH + lane] = p;
      if (lane == 0) alpha_s[qi] = al;
    }
    __syncthreads();
    // o[qi][c-th vector] = alpha * o + sum_p P[qi][p] V[p][c-th vector] over this
    // thread's key range (masked keys carry P = 0)
#pragma unroll
    for (int j = 0; j < PVJ; ++j) {
      const int e = threadIdx.x + ATT_THREADS * j;
      const int pr = KSPL > 1 ? e % PAIRS : e, kr = KSPL > 1 ? e / PAIRS : 0;
      if (pr < nq * VPR) {
        const int qi = pr / VPR, c = pr - qi * VPR;
        const float al = alpha_s[qi];
#pragma unroll
        for (int i = 0; i < EPV; ++i) acc[j][i] *= al;
        const int pend = min(nkeys, (kr + 1) * KPR);
#pragma unroll 8
        for (int p = kr * KPR; p < pend; ++p) {
          const float w = sc[qi * CH + p];
          float f[EPV];
          Vec16<T>::unpack(vs[p * VPR + c], f);
#pragma unroll
          for (int i = 0; i < EPV; ++i) acc[j][i] = fmaf(w, f[i], acc[j][i]);
        }
      }
    }
  }
  if (KSPL > 1) {  // combine the key ranges in a fixed order (range 0 keeps the sum)
    float* red = (float*)ks;  // free after the last chunk: PAIRS * KSPL * EPV floats
    __syncthreads();
    const int e = threadIdx.x;
    const int pr = e % PAIRS, kr = e / PAIRS;
    if (kr > 0) {
#pragma unroll
      for (int i = 0; i < EPV; ++i) red[((kr - 1) * PAIRS + pr) * EPV + i] = acc[0][i];
    }
    __syncthreads();
    if (kr == 0) {
      for (int r = 1; r < KSPL; ++r)
#pragma unroll
        for (int i = 0; i < EPV; ++i) acc[0][i] += red[((r - 1) * PAIRS + pr) * EPV + i];
    }
  }
  // partials (unnormalised, relative to m_run)
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    const int qi = wave + 4 * t;
    if (qi < nq && lane == 0) {
      const size_t o = out_index(qi);
      a.part_ml[2 * o] = m_run[t];
      a.part_ml[2 * o + 1] = l_run[t];
    }
  }
#pragma unroll
  for (int j = 0; j < PVJ; ++j) {
    const int e = threadIdx.x + ATT_THREADS * j;
    if (e < nq * VPR && (KSPL == 1 || e < PAIRS)) {
      const int qi = e / VPR, c = e - qi * VPR;
      float* dst = a.part_o + out_index(qi) * HD + c * EPV;
#pragma unroll
      for (int i = 0; i < EPV; ++i) dst[i] = acc[j][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode attention for bf16 caches.
//
// Work unit: one wave = (request b, KV head g, group of 16 query vectors,
// wave split w < nsplits).  A request's key space is its committed cache
// rows in 32-key sub-chunks followed, in TREE mode, by the 64 tree slots as
// two more sub-chunks; the sub-chunks holding visible keys are dealt out in
// equal contiguous runs over the nsplits waves of (b, g, group), so short
// prefixes do not leave a few waves with all of the work.  Each wave keeps an
// online softmax over its run.  A workgroup's four waves are four
// consecutive splits of one (b, g, group), and consecutive workgroups are
// the KV heads of one split group; after the key loop the four waves'
// (m, l, o) are merged in LDS in wave order and the workgroup writes one
// partial per query vector (an empty run counts as m = -inf); the
// attn_merge_kernel combines the split groups' partials.
//
// Per sub-chunk, with the 16x16x32 bf16 MFMA:
//   S^T[key][query] = K Q^T: the K fragment (16 keys x 32 head dims) is read
//     straight from the cache (16 contiguous bytes per lane), Q^T is loaded
//     once per wave;
//   online softmax on S^T: lane l holds query l%16 and keys 4(l/16)+i of
//     each 16-key tile, so a query's maximum needs two cross-row shuffles;
//   O^T[dim][query] += V^T P^T: P^T is already in B-operand layout if the
//     k-slots of lane group j are taken as keys {4j..4j+3, 16+4j..16+4j+3};
//     V^T takes the same key order with the LDS transpose read
//     (ds_read_b64_tr_b16) from the wave's V tile, two reads per 16 dims.
//   P is split into bf16 hi + lo halves (two MFMAs), so the probabilities
//     keep about 16 significant bits; K, Q and V are bf16 already, products
//     are exact and accumulate in fp32.
// Keys that are out of range or never visible read the cache's first row
// (always mapped) and are zeroed in registers, so stale rows never feed NaN
// into P.V; their scores are set to -inf.  The registers fit two waves per
// SIMD: latency is hidden by the other waves rather than by a deeper
// per-wave pipeline.
constexpr int SUB = 32;  // keys per sub-chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

__device__ __forceinline__ float xor_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum16_32(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 cat_bf16x8(s16x4 a, s16x4 b) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// 8 floats -> bf16 hi (round to nearest even) and lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 uh, ul;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t h2 = f2bf2(x[2 * t], x[2 * t + 1]);
    uh[t] = h2;
    ul[t] = f2bf2(x[2 * t] - __uint_as_float(h2 << 16), x[2 * t + 1] - __uint_as_float(h2 & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, uh);
  lo = __builtin_bit_cast(bf16x8, ul);
}

// KVM: cache addressing, 0 = contiguous, 1 = paged with the wave's block
// entries staged in lanes (at most 64), 2 = paged with a table load per key.
// MERGE: a workgroup's four waves are four splits merged before the store.
// QG: 16-query groups per wave (1 or 2).  Every K/V sub-chunk a wave loads
// serves all of its QG groups, so many query rows (a verification forward's
// m+1 rows times the GQA group) load each key QG times fewer.
template <int HD, int KVM, bool MERGE, int QG>
__global__ __launch_bounds__(ATT_THREADS)
__attribute__((amdgpu_waves_per_eu(QG == 1 ? 3 : 2))) void attn_mfma_kernel(AttnArgs a) {
  constexpr int KS = HD / 32;             // k-steps of S
  constexpr int HT = HD / 16;             // head-dim tiles of O^T
  constexpr int VROW = HD + 16;           // padded V tile row (elements)
  constexpr int VLD = SUB * HD / 8 / 64;  // 16-byte V loads per lane per sub-chunk
  __shared__ __attribute__((aligned(16))) bf16 vtile[4][SUB * VROW];
  __shared__ float mred[4][16], lred[4][16];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar control flow
  const int c16 = lane & 15, g16 = lane >> 4;
  // MERGE: workgroup -> (split group, KV head) with the head fastest (the
  // workgroups reading the same cache rows run side by side); its four waves
  // take the group's four consecutive splits and merge them before the
  // store.  Otherwise wave -> (split, KV head) with the head fastest, and
  // every wave stores its own partial.
  constexpr bool merge4 = MERGE;
  const int nsg = (a.nsplits + 3) >> 2;
  int wsplit, g;
  if constexpr (merge4) {
    const int sgi = blockIdx.x / a.hkv;
    g = blockIdx.x - sgi * a.hkv;
    wsplit = sgi * 4 + w;  // past the last split: an empty key range
  } else {
    const int wid = blockIdx.x * 4 + w;
    wsplit = wid / a.hkv;
    g = wid - wsplit * a.hkv;
  }
  const int b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int nq_total = a.rows * G;
  const int q0 = blockIdx.y * QG * 16;          // the wave's first query vector
  if (q0 >= nq_total) return;                   // uniform over the workgroup
  if (!merge4 && wsplit >= a.nsplits) return;  // no workgroup barrier without MERGE
  const int ctx = a.ctx_len[b];
  const bool tree = a.mode == EAGLE3_TREE;
  const int maxvis = tree ? ctx : ctx + a.rows;  // cache rows visible to some query
  // active sub-chunks: cache 0..ncs-1, then (TREE) tree slots 0-31, 32-63
  const int ncs = min((maxvis + SUB - 1) / SUB, a.n_cache_sub);
  const int n_act = ncs + (tree ? 2 : 0);
  const int per = (n_act + a.nsplits - 1) / a.nsplits;
  const int i0 = min(wsplit * per, n_act), i1 = min(i0 + per, n_act);
  bf16* vt = vtile[w];

  // the lane's query vector of group u: qi = q0 + 16u + c16, row qi / G,
  // head g*G + qi % G (none past nq_total: qrow = -1, zero q)
  int qrow[QG];
  bf16x8 qf[QG][KS];
  uint64_t vis_tree[QG];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const int qi = q0 + 16 * u + c16;
    qrow[u] = qi < nq_total ? qi / G : -1;
    const int h = g * G + (qi - (qi / G) * G);
    const bf16* qp = (const bf16*)a.q + ((size_t)(b * a.rows + max(qrow[u], 0)) * a.hq + h) * HD + 8 * g16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = *(const u32x4*)(qp + ks * 32);
      qf[u][ks] = as_bf16x8(qrow[u] >= 0 ? v : u32x4{0u, 0u, 0u, 0u});
    }
    vis_tree[u] = (tree && qrow[u] >= 0) ? a.anc[b * a.rows + qrow[u]] : 0ull;
  }
  // tree slots some row can see (others are never loaded): the rows' masks
  // are loaded across the lanes and OR-reduced
  uint64_t any_vis = ~0ull;
  if (tree && i1 > ncs) {
    uint64_t v = 0ull;
    for (int rr = lane; rr < a.rows; rr += 64) v |= a.anc[b * a.rows + rr];
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      lo |= (uint32_t)__shfl_xor((int)lo, sh);
      hi |= (uint32_t)__shfl_xor((int)hi, sh);
    }
    any_vis = ((uint64_t)hi << 32) | lo;
  }
  // paged cache (KVM 1): the run's block-table entries, one per lane, read
  // with a lane shuffle (no dependent global load before a sub-chunk's copies)
  int blk0 = 0, blk_reg = 0;
  if (KVM == 1 && i0 < ncs) {
    blk0 = (i0 * SUB) / a.block_size;
    const int blk_end = min((min(i1, ncs) * SUB + a.block_size - 1) / a.block_size, a.max_blocks);
    if (blk0 + lane < blk_end) blk_reg = a.block_table[(size_t)b * a.max_blocks + blk0 + lane];
    // an identity DPP move: the wait for the table load happens once, here,
    // instead of before every shuffle of it
    blk_reg = __builtin_amdgcn_update_dpp(0, blk_reg, 0xE4, 0xF, 0xF, false);
  }

  float m_run[QG], l_run[QG];
  f32x4 o[QG][HT];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) o[u][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Source row of key p (0..31) of active sub-chunk i, and whether it is a
  // real, possibly visible key.  Every lane calls it (the block shuffle
  // reads other lanes' registers).
  auto key_row = [&](int i, int p, const void* cache, const void* tslots, bool& ok)
                     __attribute__((always_inline)) -> const bf16* {
    if (i < ncs) {
      const int pos = i * SUB + p;
      ok = pos < maxvis;
      size_t off;
      if (KVM == 0) {
        off = (((size_t)b * a.cap + pos) * a.hkv + g) * HD;
      } else {
        // power-of-two blocks (the usual 16): a shift and a mask instead of
        // an integer division per key row
        const int bi = a.bs_log2 >= 0 ? pos >> a.bs_log2 : pos / a.block_size;
        const int po = pos - bi * a.block_size;
        int blk;
        if (KVM == 1) blk = __shfl(blk_reg, min(max(bi - blk0, 0), 63));
        else blk = ok ? a.block_table[(size_t)b * a.max_blocks + bi] : 0;
        off = (((size_t)blk * a.block_size + po) * a.hkv + g) * HD;
      }
      return ok ? (const bf16*)cache + off : (const bf16*)cache;
    }
    const int slot = (i - ncs) * SUB + p;
    ok = ((any_vis >> slot) & 1ull) != 0;
    return ok ? (const bf16*)tslots + ((size_t)(b * EAGLE3_MAX_TREE_SLOTS + slot) * a.hkv + g) * HD
              : (const bf16*)tslots;
  };

  for (int i = i0; i < i1; ++i) {
    // copies: K fragments (keys kt*16 + c16) and V rows, all issued at once
    const bf16* kr[2];
    const bf16* vr[VLD];
    uint32_t okm = 0;  // bit kt: K row real; bit 2 + v: V row real
    bool ok;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      kr[kt] = key_row(i, kt * 16 + c16, a.kc, a.tk, ok);
      okm |= (uint32_t)ok << kt;
    }
#pragma unroll
    for (int v = 0; v < VLD; ++v) {
      const int e = v * 64 + lane, pk = e / (HD / 8), c = e - pk * (HD / 8);
      vr[v] = key_row(i, pk, a.vc, a.tv, ok) + 8 * c;
      okm |= (uint32_t)ok << (2 + v);
    }
    u32x4 kf[2][KS], vf[VLD];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kt][ks] = *(const u32x4*)(kr[kt] + ks * 32 + 8 * g16);
#pragma unroll
    for (int v = 0; v < VLD; ++v) vf[v] = *(const u32x4*)vr[v];
    // V into the wave's tile (rows in key order), masked rows as zeros
#pragma unroll
    for (int v = 0; v < VLD; ++v) {
      const int e = v * 64 + lane, pk = e / (HD / 8), c = e - pk * (HD / 8);
      const uint32_t keep = 0u - ((okm >> (2 + v)) & 1u);
      *(u32x4*)(vt + pk * VROW + 8 * c) = vf[v] & keep;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint32_t keep = 0u - ((okm >> kt) & 1u);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kt][ks] &= keep;
    }
    const bool is_tree = i >= ncs;
    const int p0 = is_tree ? (i - ncs) * SUB : i * SUB;
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      // S^T = K Q^T for the two 16-key tiles
      f32x4 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kt][ks]), qf[u][ks], sc[kt], 0, 0, 0);
      }
      // mask and scale: key p0 + kt*16 + 4*g16 + t for the lane's query row
      const int lim = tree ? ctx : ctx + qrow[u] + 1;
      float x[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int pk = p0 + kt * 16 + 4 * g16 + t;
          const bool vis = qrow[u] >= 0 && (is_tree ? ((vis_tree[u] >> pk) & 1ull) != 0 : pk < lim);
          x[kt * 4 + t] = vis ? sc[kt][t] * a.scale : -INFINITY;
          mloc = fmaxf(mloc, x[kt * 4 + t]);
        }
      const float m_new = fmaxf(m_run[u], xor_max16_32(mloc));
      const float al = m_new == -INFINITY ? 1.f : expf(m_run[u] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = m_new == -INFINITY ? 0.f : expf(x[t] - m_new);
        psum += x[t];
      }
      l_run[u] = l_run[u] * al + psum;
      m_run[u] = m_new;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) o[u][ht] *= al;
      bf16x8 phi, plo;
      split_bf16x8(x, phi, plo);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        // V^T fragment: dims ht*16 + c16, keys {4*g16 + t} and {16 + 4*g16 + t}, t < 4
        const bf16* src = vt + (4 * g16 + (c16 >> 2)) * VROW + ht * 16 + 4 * (c16 & 3);
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)src);
        const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(src + 16 * VROW));
        const bf16x8 vfr = cat_bf16x8(va, vb);
        o[u][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, phi, o[u][ht], 0, 0, 0);
        o[u][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, plo, o[u][ht], 0, 0, 0);
      }
    }
  }
  // the wave's split: (m, l) per query and o (unnormalised, relative to m)
  if constexpr (!merge4) {
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const float l = xor_sum16_32(l_run[u]);
      if (qrow[u] < 0) continue;
      const int qi = q0 + 16 * u + c16;
      const int h = g * G + (qi - qrow[u] * G);
      const size_t oi = ((size_t)(b * a.rows + qrow[u]) * a.hq + h) * a.nsplits + wsplit;
      if (g16 == 0) {
        a.part_ml[2 * oi] = m_run[u];
        a.part_ml[2 * oi + 1] = l;
      }
      float* dst = a.part_o + oi * HD + 4 * g16;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        *(float4*)(dst + ht * 16) = make_float4(o[u][ht][0], o[u][ht][1], o[u][ht][2], o[u][ht][3]);
    }
    return;
  }
  // MERGE, one query group at a time: into the wave's own V-tile space as
  // [query][HD + 4] floats, then the four splits in wave order
  constexpr int OROW = HD + 4;  // padded: the 16 queries' float4 stores hit distinct banks
  static_assert(16 * OROW * 4 <= SUB * VROW * 2, "merge rows fit the V tile");
  const int sgi = wsplit >> 2;
  constexpr int DPT = HD / 16;
  const int qc = threadIdx.x >> 4, j = threadIdx.x & 15;
  float* ow = (float*)vt;
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const float l = xor_sum16_32(l_run[u]);
    __syncthreads();  // the V tiles (and the previous group's merge rows) are no longer read
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
      *(float4*)(ow + c16 * OROW + ht * 16 + 4 * g16) = make_float4(o[u][ht][0], o[u][ht][1], o[u][ht][2],
                                                                    o[u][ht][3]);
    if (g16 == 0) {
      mred[w][c16] = m_run[u];
      lred[w][c16] = l;
    }
    __syncthreads();
    // thread t takes query t/16 and dims DPT*(t%16) ..; the merged partial is the split group's
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      mw[s4] = mred[s4][qc];
      M = fmaxf(M, mw[s4]);
    }
    float wt[4], L = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      wt[s4] = mw[s4] == -INFINITY ? 0.f : expf(mw[s4] - M);
      L += lred[s4][qc] * wt[s4];
    }
    float acc[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) acc[d] = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float* src = (const float*)vtile[s4] + qc * OROW + DPT * j;
#pragma unroll
      for (int d = 0; d < DPT; d += 4) {
        const float4 v = *(const float4*)(src + d);
        acc[d] = fmaf(v.x, wt[s4], acc[d]);
        acc[d + 1] = fmaf(v.y, wt[s4], acc[d + 1]);
        acc[d + 2] = fmaf(v.z, wt[s4], acc[d + 2]);
        acc[d + 3] = fmaf(v.w, wt[s4], acc[d + 3]);
      }
    }
    const int qim = q0 + 16 * u + qc;
    if (qim < nq_total) {
      const int qrm = qim / G;
      const int h = g * G + (qim - qrm * G);
      const size_t oi = ((size_t)(b * a.rows + qrm) * a.hq + h) * nsg + sgi;
      if (j == 0) {
        a.part_ml[2 * oi] = M;
        a.part_ml[2 * oi + 1] = L;
      }
      float* dst = a.part_o + oi * HD + DPT * j;
#pragma unroll
      for (int d = 0; d < DPT; d += 4) *(float4*)(dst + d) = make_float4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
    }
  }
}

// out[row][h*hd + i] = merged attention output, rounded to T.  One
// workgroup per (row, head): wave 0 computes the partials' weights
// exp(m_c - M) (lanes over partials) and L; wave w then sums the weighted
// partial vectors c = w, w+4, ... and the four sums are added in wave order.
// Each wave's first partial vectors are loaded before the weights, so the
// two loads share one round trip.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int nchunks, int hq,
                                                         T* __restrict__ out) {
  constexpr int MAXC = 512;
  constexpr int EPL = HD / 64;  // elements per lane
  __shared__ float wc[MAXC];
  __shared__ float red[4][HD];
  __shared__ float sL;
  const size_t rh = blockIdx.x;  // row*hq + h
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // every wave's first PRE partial vectors (c = w, w+4, ...) are loaded
  // before the weights are known, so their round trip overlaps wave 0's
  const float* po = part_o + rh * nchunks * HD;
  constexpr int PRE = 5;
  float pv[PRE][EPL];
#pragma unroll
  for (int u = 0; u < PRE; ++u)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int c = w + 4 * u;
      pv[u][j] = c < nchunks ? po[(size_t)c * HD + lane + 64 * j] : 0.f;
    }
  if (w == 0) {
    const float* ml = part_ml + 2 * rh * nchunks;
    float mloc = -INFINITY;
    for (int c = lane; c < nchunks; c += 64) mloc = fmaxf(mloc, ml[2 * c]);
    const float M = wave_max(mloc);
    float lloc = 0.f;
    for (int c = lane; c < nchunks; c += 64) {
      const float m = ml[2 * c];
      const float wgt = m == -INFINITY ? 0.f : expf(m - M);
      wc[c] = wgt;
      lloc += ml[2 * c + 1] * wgt;
    }
    const float L = wave_sum(lloc);
    if (lane == 0) sL = L;
  }
  __syncthreads();
  // partials in the order c = w, w+4, w+8, ...
  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int u = 0; u < PRE; ++u) {
    const int c = w + 4 * u;
    if (c < nchunks)
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] = fmaf(pv[u][j], wc[c], acc[j]);
  }
  int c = w + 4 * PRE;
  for (; c + 12 < nchunks; c += 16) {
    float v[4][EPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[u][j] = po[(size_t)(c + 4 * u) * HD + lane + 64 * j];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] = fmaf(v[u][j], wc[c + 4 * u], acc[j]);
  }
  for (; c < nchunks; c += 4)
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = fmaf(po[(size_t)c * HD + lane + 64 * j], wc[c], acc[j]);
#pragma unroll
  for (int j = 0; j < EPL; ++j) red[w][lane + 64 * j] = acc[j];
  __syncthreads();
  if (w == 0) {
    const float L = sL;
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int i = lane + 64 * j;
      Elem<T>::st(out, rh * HD + i, ((red[0][i] + red[1][i]) + red[2][i] + red[3][i]) * inv);
    }
  }
}

// partial slots per (row, head): the 32-key sub-chunks plus the two tree
// sub-chunks, at most 512 (the merge kernel's limit); covers the fp32 kernel's
// 64-key chunks too
int attn_num_chunks(int cap_rows) {
  const int n = (cap_rows + SUB - 1) / SUB + 2;
  return n < 512 ? n : 512;
}

hipError_t launch_attention(const AttnLaunch& L, hipStream_t st) {
  AttnArgs a;
  a.q = L.q;
  a.kc = L.kc;
  a.vc = L.vc;
  a.tk = L.tk;
  a.tv = L.tv;
  a.ctx_len = L.ctx_len;
  a.block_table = L.block_table;
  a.anc = L.anc;
  a.cap = L.cap;
  a.max_blocks = L.max_blocks;
  a.block_size = L.block_size;
  a.bs_log2 = -1;
  if (L.block_size > 0 && (L.block_size & (L.block_size - 1)) == 0)
    for (a.bs_log2 = 0; (1 << a.bs_log2) < L.block_size; ++a.bs_log2) {
    }
  a.B = L.B;
  a.rows = L.rows;
  a.hq = L.hq;
  a.hkv = L.hkv;
  a.mode = L.mode;
  const int G = L.hq / L.hkv;
  const int nq = L.rows * G;
  const int rtot = L.B * L.rows;
  a.scale = 1.0f / sqrtf((float)L.hd);
  a.part_o = L.part_o;
  a.part_ml = L.part_ml;
  if (L.bf16) {
    // workgroups: (split group of 4 waves, KV head, 16-query group, request).
    // A request's visible sub-chunks are dealt out over its nsplits waves;
    // nsplits is sized so that the launch holds about 8192 waves of
    // capacity-sized work.
    a.n_qgroups = (nq + 15) / 16;
    // query groups per wave: two when many rows share the keys (the 70B
    // verification forward's 61 rows x 8 GQA heads, about 9 % faster), one
    // otherwise (measured: the 8B forward's 16 groups run faster with one,
    // and four per wave, at one wave per SIMD, is slower everywhere)
    const int QG = a.n_qgroups > 16 ? 2 : 1;
    const int nwq = (a.n_qgroups + QG - 1) / QG;
    a.n_cache_sub = (L.cap_rows + SUB - 1) / SUB;
    const int n_sub = a.n_cache_sub + (L.mode == EAGLE3_TREE ? 2 : 0);
    const long units = (long)n_sub * L.hkv * nwq * L.B;
    int spw = (int)((units + 8191) / 8192);
    // at most 96 splits: the 70B tree's 130 sub-chunks (4096 keys) run two
    // per wave (70B cycle +0.6 %), the 8B tree's 66 one per wave (two: -0.3 %)
    const int spw_min = (n_sub + 95) / 96;
    spw = spw < spw_min ? spw_min : spw;
    a.spw = spw;
    a.nsplits = (n_sub + spw - 1) / spw;  // <= attn_num_chunks(cap_rows)
    a.cpw = 0;
    a.n_commit_splits = 0;
    // paged: a wave's run spans at most 32*ceil(n_sub/nsplits)/block_size + 1 blocks
    const int run = (n_sub + a.nsplits - 1) / a.nsplits;
    const int kvm = !L.block_table ? 0 : ((SUB * run + L.block_size - 1) / L.block_size + 1 <= 64 ? 1 : 2);
    // many splits (short runs, batch-1 shapes), or at least 8 splits whose
    // waves each hold a full group of 16 query vectors (the target's batch
    // of 4-row chains: a partial is 8 KB per wave, 57 MB per call at 64 x 4
    // rows): a workgroup merges its four waves' splits, so four times fewer
    // partials are written and merged (8B target over 64 x 4 rows 12.25 ->
    // 11.91 ms per step; the batch-64 drafter's 4 query vectors per wave
    // write little and lost 0.6 % merging)
    const bool merge4 = a.nsplits >= 32 || (a.nsplits >= 8 && nq >= 16);
    const int nsg = (a.nsplits + 3) / 4;
    const int nparts = merge4 ? nsg : a.nsplits;
    dim3 grid(merge4 ? nsg * L.hkv : (a.nsplits * L.hkv + 3) / 4, nwq, L.B);
#define E3_MFMA_Q(HD, KV, M)                                                      \
  do {                                                                            \
    if (QG == 1) attn_mfma_kernel<HD, KV, M, 1><<<grid, ATT_THREADS, 0, st>>>(a); \
    else attn_mfma_kernel<HD, KV, M, 2><<<grid, ATT_THREADS, 0, st>>>(a);         \
  } while (0)
#define E3_MFMA_K(HD, M)                   \
  do {                                     \
    if (kvm == 0) E3_MFMA_Q(HD, 0, M);     \
    else if (kvm == 1) E3_MFMA_Q(HD, 1, M); \
    else E3_MFMA_Q(HD, 2, M);              \
  } while (0)
#define E3_MFMA(HD)              \
  do {                           \
    if (merge4) E3_MFMA_K(HD, true); \
    else E3_MFMA_K(HD, false);   \
  } while (0)
    if (L.hd == 128) {
      E3_MFMA(128);
      attn_merge_kernel<bf16, 128><<<rtot * L.hq, 256, 0, st>>>(L.part_o, L.part_ml, nparts, L.hq, (bf16*)L.out);
    } else {
      E3_MFMA(64);
      attn_merge_kernel<bf16, 64><<<rtot * L.hq, 256, 0, st>>>(L.part_o, L.part_ml, nparts, L.hq, (bf16*)L.out);
    }
#undef E3_MFMA
#undef E3_MFMA_K
#undef E3_MFMA_Q
    return hipGetLastError();
  }
  // fp32 caches (head_dim 64, validated by the caller): vector-ALU kernel
  const int qg = nq <= 8 ? 8 : 32;
  a.n_qgroups = (nq + qg - 1) / qg;
  // chunks per workgroup: one while the (chunk, head group, request) tasks
  // alone fill the chip a few times over, more for large batches
  const int nchunks = (L.cap_rows + CH - 1) / CH;
  const long tasks = (long)nchunks * L.hkv * a.n_qgroups * L.B;
  int cpw = (int)((tasks + 2047) / 2048);
  cpw = cpw < 1 ? 1 : (cpw > 8 ? 8 : cpw);
  a.cpw = cpw;
  a.n_commit_splits = (nchunks + cpw - 1) / cpw;
  a.n_cache_sub = 0;
  a.spw = 0;
  const int nsplits = a.n_commit_splits + 1;  // <= attn_num_chunks(cap_rows): the workspace bound
  a.nsplits = nsplits;
  dim3 grid(nsplits, L.hkv * a.n_qgroups, L.B);
#define E3_ATTN(T, HD, QGV) attn_partial_kernel<T, HD, QGV><<<grid, ATT_THREADS, 0, st>>>(a)
  if (qg == 8) E3_ATTN(float, 64, 8); else E3_ATTN(float, 64, 32);
  attn_merge_kernel<float, 64><<<rtot * L.hq, 256, 0, st>>>(L.part_o, L.part_ml, nsplits, L.hq, (float*)L.out);
#undef E3_ATTN
  return hipGetLastError();
}

}  // namespace e3
