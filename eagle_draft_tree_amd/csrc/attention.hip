// Tree-masked decode attention for the drafter ("EAGLE-3 精读" §1-§2: the
// draft decoder attends over the committed prefix plus the growing draft
// tree; the tree mask is an ancestor bitset per row).
//
// Split-K over the keys: workgroup (chunk c, kv head g / query group, request
// b) handles CH consecutive committed rows, or -- for the last chunk index --
// the 64 tree slots, for every query vector (row, q head) of that KV head's
// GQA group.  K/V of the chunk are staged once in LDS and shared by all the
// group's query heads.  Each workgroup writes a partial (max, sum, o[hd]);
// a merge kernel combines the chunks in index order (deterministic).
#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int CH = 64;       // keys per chunk
constexpr int QG = 32;       // query vectors per workgroup
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
  int B, rows, hq, hkv, mode, n_commit_chunks, n_qgroups;
  float scale;
  float* part_o;   // [Rtot*Hq][nchunks][hd]
  float* part_ml;  // [Rtot*Hq][nchunks][2]
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

template <typename T, int HD>
__global__ __launch_bounds__(ATT_THREADS) void attn_partial_kernel(AttnArgs a) {
  constexpr int EPV = Vec16<T>::N;         // elements per 16-byte vector
  constexpr int VPR = HD / EPV;            // vectors per key row
  constexpr int KPV = VPR + 1;             // padded LDS row (vectors): spreads banks
  __shared__ uint4 ks[CH * KPV];
  __shared__ uint4 vs[CH * VPR];
  __shared__ float qs[QG * HD];
  __shared__ float sc[QG * CH];

  const int chunk = blockIdx.x;
  const int g = blockIdx.y / a.n_qgroups, qgrp = blockIdx.y - g * a.n_qgroups;
  const int b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int nq_total = a.rows * G;
  const int q0 = qgrp * QG;
  const int nq = min(QG, nq_total - q0);
  const int nchunks = a.n_commit_chunks + 1;
  const bool tree_chunk = chunk == a.n_commit_chunks;
  const int ctx = a.ctx_len[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (nq <= 0) return;

  // Keys of this chunk and how many exist.
  const int p0 = chunk * CH;
  int nkeys;
  if (tree_chunk) {
    nkeys = a.mode == EAGLE3_TREE ? EAGLE3_MAX_TREE_SLOTS : 0;
  } else {
    const int maxvis = a.mode == EAGLE3_TREE ? ctx : ctx + a.rows;  // rows visible to the last query
    nkeys = min(CH, maxvis - p0);
  }
  auto out_index = [&](int qi) {
    const int rr = (q0 + qi) / G, gi = (q0 + qi) - rr * G;
    const int row = b * a.rows + rr, h = g * G + gi;
    return (size_t)(row * a.hq + h) * nchunks + chunk;
  };
  if (nkeys <= 0) {
    for (int qi = threadIdx.x; qi < nq; qi += ATT_THREADS) {
      const size_t o = out_index(qi);
      a.part_ml[2 * o] = -INFINITY;
      a.part_ml[2 * o + 1] = 0.f;
    }
    for (int e = threadIdx.x; e < nq * HD; e += ATT_THREADS) {
      const int qi = e / HD, i = e - qi * HD;
      a.part_o[out_index(qi) * HD + i] = 0.f;
    }
    return;
  }
  // Tree slots no row of this request can see may hold stale data: they
  // are staged as zeros so that masked keys never feed NaN into P.V.
  uint64_t any_vis = ~0ull;
  if (tree_chunk) {
    any_vis = 0ull;
    for (int rr = 0; rr < a.rows; ++rr) any_vis |= a.anc[b * a.rows + rr];
  }
  // Stage K/V rows of the chunk with 16-byte loads.
  for (int e = threadIdx.x; e < nkeys * VPR; e += ATT_THREADS) {
    const int p = e / VPR, c = e - p * VPR;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if ((any_vis >> p) & 1ull) {
      size_t off;
      const T *kb, *vb;
      if (tree_chunk) {
        off = ((size_t)(b * EAGLE3_MAX_TREE_SLOTS + p) * a.hkv + g) * HD;
        kb = (const T*)a.tk;
        vb = (const T*)a.tv;
      } else {
        const int pos = p0 + p;
        if (a.block_table) {
          const int blk = a.block_table[(size_t)b * a.max_blocks + pos / a.block_size];
          off = (((size_t)blk * a.block_size + pos % a.block_size) * a.hkv + g) * HD;
        } else {
          off = (((size_t)b * a.cap + pos) * a.hkv + g) * HD;
        }
        kb = (const T*)a.kc;
        vb = (const T*)a.vc;
      }
      kv = *((const uint4*)(kb + off) + c);
      vv = *((const uint4*)(vb + off) + c);
    }
    ks[p * KPV + c] = kv;
    vs[p * VPR + c] = vv;
  }
  // Stage the query vectors (q head h = g*G + gi of row rr) as float.
  const T* Q = (const T*)a.q;
  for (int e = threadIdx.x; e < nq * VPR; e += ATT_THREADS) {
    const int qi = e / VPR, c = e - qi * VPR;
    const int rr = (q0 + qi) / G, gi = (q0 + qi) - rr * G;
    const size_t row = (size_t)b * a.rows + rr;
    const uint4 u = *((const uint4*)(Q + (row * a.hq + g * G + gi) * HD) + c);
    float f[EPV];
    Vec16<T>::unpack(u, f);
#pragma unroll
    for (int j = 0; j < EPV; ++j) qs[qi * HD + c * EPV + j] = f[j];
  }
  __syncthreads();
  // Scores: lane = key, waves split the query vectors.
  if (lane < nkeys) {
    float kf[HD];
#pragma unroll
    for (int c = 0; c < VPR; ++c) Vec16<T>::unpack(ks[lane * KPV + c], kf + c * EPV);
    for (int qi = wave; qi < nq; qi += ATT_THREADS / 64) {
      const int rr = (q0 + qi) / G;
      bool vis;
      if (tree_chunk) {
        vis = (a.anc[b * a.rows + rr] >> lane) & 1ull;
      } else {
        const int lim = a.mode == EAGLE3_TREE ? ctx : ctx + rr + 1;
        vis = p0 + lane < lim;
      }
      const float4* q4 = (const float4*)(qs + qi * HD);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < HD / 4; i += 2) {
        const float4 x = q4[i], y = q4[i + 1];
        s0 = fmaf(x.x, kf[4 * i], s0);
        s0 = fmaf(x.y, kf[4 * i + 1], s0);
        s0 = fmaf(x.z, kf[4 * i + 2], s0);
        s0 = fmaf(x.w, kf[4 * i + 3], s0);
        s1 = fmaf(y.x, kf[4 * i + 4], s1);
        s1 = fmaf(y.y, kf[4 * i + 5], s1);
        s1 = fmaf(y.z, kf[4 * i + 6], s1);
        s1 = fmaf(y.w, kf[4 * i + 7], s1);
      }
      sc[qi * CH + lane] = vis ? (s0 + s1) * a.scale : -INFINITY;
    }
  } else {
    for (int qi = wave; qi < nq; qi += ATT_THREADS / 64) sc[qi * CH + lane] = -INFINITY;
  }
  __syncthreads();
  // Partial softmax per query vector (one wave per vector).
  for (int qi = wave; qi < nq; qi += ATT_THREADS / 64) {
    const float s = sc[qi * CH + lane];
    const float mx = wave_max(s);
    const float p = (mx == -INFINITY) ? 0.f : expf(s - mx);
    const float l = wave_sum(p);
    sc[qi * CH + lane] = p;
    if (lane == 0) {
      const size_t o = out_index(qi);
      a.part_ml[2 * o] = mx;
      a.part_ml[2 * o + 1] = l;
    }
  }
  __syncthreads();
  // o[qi][i..i+EPV) = sum_p P[qi][p] V[p][i..i+EPV): VPR threads per query.
  for (int e = threadIdx.x; e < nq * VPR; e += ATT_THREADS) {
    const int qi = e / VPR, c = e - qi * VPR;
    float acc[EPV];
#pragma unroll
    for (int j = 0; j < EPV; ++j) acc[j] = 0.f;
    for (int p = 0; p < nkeys; ++p) {
      const float w = sc[qi * CH + p];
      float f[EPV];
      Vec16<T>::unpack(vs[p * VPR + c], f);
#pragma unroll
      for (int j = 0; j < EPV; ++j) acc[j] = fmaf(w, f[j], acc[j]);
    }
    float* dst = a.part_o + out_index(qi) * HD + c * EPV;
#pragma unroll
    for (int j = 0; j < EPV; ++j) dst[j] = acc[j];
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
  a.n_commit_chunks = attn_num_chunks(L.cap_rows) - 1;
  const int G = L.hq / L.hkv;
  a.n_qgroups = (L.rows * G + QG - 1) / QG;
  a.scale = 1.0f / sqrtf((float)L.hd);
  a.part_o = L.part_o;
  a.part_ml = L.part_ml;
  const int nchunks = a.n_commit_chunks + 1;
  dim3 grid(nchunks, L.hkv * a.n_qgroups, L.B);
  const int rtot = L.B * L.rows;
  if (L.bf16) {
    if (L.hd == 128) {
      attn_partial_kernel<bf16, 128><<<grid, ATT_THREADS, 0, st>>>(a);
      attn_merge_kernel<bf16, 128><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nchunks, L.hq, (bf16*)L.out);
    } else {
      attn_partial_kernel<bf16, 64><<<grid, ATT_THREADS, 0, st>>>(a);
      attn_merge_kernel<bf16, 64><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nchunks, L.hq, (bf16*)L.out);
    }
  } else {  // fp32 drafters: head_dim 64 (validated by the caller)
    attn_partial_kernel<float, 64><<<grid, ATT_THREADS, 0, st>>>(a);
    attn_merge_kernel<float, 64><<<rtot * L.hq, 64, 0, st>>>(L.part_o, L.part_ml, nchunks, L.hq, (float*)L.out);
  }
  return hipGetLastError();
}

}  // namespace e3
