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
  int B, rows, hq, hkv, mode, n_commit_splits, cpw, n_qgroups;
  float scale;
  float* part_o;   // [Rtot*Hq][nsplits][hd]
  float* part_ml;  // [Rtot*Hq][nsplits][2]
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

// out[row][h*hd + i] = merged attention output, rounded to T.  One wave per
// (row, head): chunk maxima and weights first (lanes over chunks), then the
// weighted sum of the chunk partials in chunk order.
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml, int nchunks, int hq,
                                                        T* __restrict__ out) {
  constexpr int MAXC = 512;
  __shared__ float wc[MAXC];
  const size_t rh = blockIdx.x;  // row*hq + h
  const int lane = threadIdx.x;
  const float* ml = part_ml + 2 * rh * nchunks;
  float mloc = -INFINITY;
  for (int c = lane; c < nchunks; c += 64) mloc = fmaxf(mloc, ml[2 * c]);
  const float M = wave_max(mloc);
  float lloc = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
    const float m = ml[2 * c];
    const float w = m == -INFINITY ? 0.f : expf(m - M);
    wc[c] = w;
    lloc += ml[2 * c + 1] * w;
  }
  const float L = wave_sum(lloc);
  __syncthreads();
  float acc[HD / 64];
#pragma unroll
  for (int j = 0; j < HD / 64; ++j) acc[j] = 0.f;
  const float* po = part_o + rh * nchunks * HD;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    float v[8][HD / 64];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < HD / 64; ++j) v[u][j] = po[(size_t)(c + u) * HD + lane + 64 * j];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < HD / 64; ++j) acc[j] = fmaf(v[u][j], wc[c + u], acc[j]);
  }
  for (; c < nchunks; ++c)
#pragma unroll
    for (int j = 0; j < HD / 64; ++j) acc[j] = fmaf(po[(size_t)c * HD + lane + 64 * j], wc[c], acc[j]);
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int j = 0; j < HD / 64; ++j) Elem<T>::st(out, rh * HD + lane + 64 * j, acc[j] * inv);
}

int attn_num_chunks(int cap_rows) { return (cap_rows + CH - 1) / CH + 1; }

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
  a.B = L.B;
  a.rows = L.rows;
  a.hq = L.hq;
  a.hkv = L.hkv;
  a.mode = L.mode;
  const int G = L.hq / L.hkv;
  const int nq = L.rows * G;
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
  a.scale = 1.0f / sqrtf((float)L.hd);
  a.part_o = L.part_o;
  a.part_ml = L.part_ml;
  const int nsplits = a.n_commit_splits + 1;  // <= attn_num_chunks(cap_rows): the workspace bound
  dim3 grid(nsplits, L.hkv * a.n_qgroups, L.B);
  const int rtot = L.B * L.rows;
#define E3_ATTN(T, HD, QGV) attn_partial_kernel<T, HD, QGV><<<grid, ATT_THREADS, 0, st>>>(a)
  if (L.bf16) {
    if (L.hd == 128) {
      if (qg == 8) E3_ATTN(bf16, 128, 8); else E3_ATTN(bf16, 128, 32);
      attn_merge_kernel<bf16, 128><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nsplits, L.hq, (bf16*)L.out);
    } else {
      if (qg == 8) E3_ATTN(bf16, 64, 8); else E3_ATTN(bf16, 64, 32);
      attn_merge_kernel<bf16, 64><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nsplits, L.hq, (bf16*)L.out);
    }
  } else {  // fp32 drafters: head_dim 64 (validated by the caller)
    if (qg == 8) E3_ATTN(float, 64, 8); else E3_ATTN(float, 64, 32);
    attn_merge_kernel<float, 64><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nsplits, L.hq, (float*)L.out);
  }
#undef E3_ATTN
  return hipGetLastError();
}

}  // namespace e3
