// Pieces of one decoder layer shared by the drafter step and the target's
// verification forward: the row kernels' thread layout, split-K partial
// sums, the FFN RMSNorm, the split-K QKV finish (RoPE + KV scatter) and the
// rows-GEMM dispatch (skinny / register-weight / LDS-tiled kernels by row
// count and layout).  Split-K partials are added in split order by the
// consumer, so every result is deterministic.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "gemm_rows.hpp"
#include "rows_dma.hpp"
#include "rows_rx.hpp"
#include "timing.hpp"

namespace e3 {

constexpr int RT = 1024;      // threads of the row kernels
constexpr int EPT_MAX = 8;    // elements per thread: d <= 8192

// ---------------------------------------------------------------------------
// row kernels: every thread owns elements i = threadIdx.x + RT*j, j < EPT_MAX,
// and issues all of its loads before using any of them.

// v[j] += sum over splits of part[s][row][i] (fixed split order).  Four
// splits' loads are issued before any of them is added, so a row's 8 or 16
// splits take two to four memory round trips instead of one each.
__device__ __forceinline__ void add_partials(float (&v)[EPT_MAX], const float* __restrict__ part, int splits,
                                             size_t split_stride, size_t row_off, int d) {
  constexpr int SG = 4;
  for (int s0 = 0; s0 < splits; s0 += SG) {
    float p[SG][EPT_MAX];
#pragma unroll
    for (int u = 0; u < SG; ++u)
#pragma unroll
      for (int j = 0; j < EPT_MAX; ++j) {
        const int i = threadIdx.x + RT * j;
        p[u][j] = (s0 + u < splits && i < d) ? part[(size_t)(s0 + u) * split_stride + row_off + i] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < SG; ++u)
      if (s0 + u < splits)
#pragma unroll
        for (int j = 0; j < EPT_MAX; ++j) v[j] += p[u][j];
  }
}

// h1 = res + sum of o partials (splits > 0), or h1 already complete;
// pre-norm (post == 0): u = rms(h1) * gain (dtype); post-norm (post != 0):
// h1 = rms(h1) * gain is stored and u = h1 (dtype), the FFN's input.
template <typename T>
__global__ __launch_bounds__(RT) void ffn_norm_kernel(const float* __restrict__ res, const float* __restrict__ part,
                                                      int splits, int R, int d, const float* __restrict__ gain,
                                                      float eps, float* __restrict__ h1, T* __restrict__ u,
                                                      int post = 0) {
  __shared__ float red[RT / 64];
  const int r = blockIdx.x;
  float v[EPT_MAX];
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    v[j] = i < d ? (splits > 0 ? res[(size_t)r * d + i] : h1[(size_t)r * d + i]) : 0.f;
  }
  if (splits > 0) add_partials(v, part, splits, (size_t)R * d, (size_t)r * d, d);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) ss = fmaf(v[j], v[j], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    if (i < d) {
      const float nv = v[j] * inv * gain[i];
      if (post) {
        h1[(size_t)r * d + i] = nv;
      } else if (splits > 0) {
        h1[(size_t)r * d + i] = v[j];
      }
      Elem<T>::st(u, (size_t)r * d + i, nv);
    }
  }
}

// QKV after split-K: one workgroup per (row, head); thread i < hd/2 owns the
// RoPE pair (i, i + hd/2).  Sum partials in split order, rotate q and k at
// the row's position, round, write q to ws and k/v to the KV destination.
template <typename T>
__global__ __launch_bounds__(64) void qkv_finish_kernel(const float* __restrict__ part, int splits, int R,
                                                        int N, const int32_t* __restrict__ pos,
                                                        KVDest dst, T* __restrict__ q_out, int hq,
                                                        float theta) {
  const int r = blockIdx.x, head = blockIdx.y;
  const int hd = dst.hd, half = hd >> 1;
  for (int i = threadIdx.x; i < half; i += 64) {
    const size_t n0 = (size_t)head * hd + i;
    // the rotation first: its fp64 angle and cos/sin need no partial sum,
    // so their latency overlaps the partials' loads
    float c = 1.f, sn = 0.f;
    if (head < hq + dst.hkv) {
      const double inv = pow((double)theta, -(2.0 * i) / (double)hd);
      const double ang = (double)pos[r] * inv;
      c = (float)cos(ang);
      sn = (float)sin(ang);
    }
    float p0[16], p1[16];
    float a = 0.f, b = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 16) {
      const int ns = min(16, splits - s0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < ns) {
          p0[s] = part[(size_t)(s0 + s) * R * N + (size_t)r * N + n0];
          p1[s] = part[(size_t)(s0 + s) * R * N + (size_t)r * N + n0 + half];
        }
      }
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < ns) {
          a += p0[s];
          b += p1[s];
        }
    }
    if (head < hq + dst.hkv) {  // q or k: rotate
      const float a2 = a * c - b * sn, b2 = b * c + a * sn;
      a = a2;
      b = b2;
    }
    if (head < hq) {
      const size_t o = (size_t)r * hq * hd + (size_t)head * hd;
      Elem<T>::st(q_out, o + i, a);
      Elem<T>::st(q_out, o + i + half, b);
    } else {
      const bool isk = head < hq + dst.hkv;
      const int g = isk ? head - hq : head - hq - dst.hkv;
      bool tree;
      const size_t o = dst.off(r, g, tree);
      T* base = (T*)(isk ? (tree ? dst.tk : dst.k) : (tree ? dst.tv : dst.v));
      Elem<T>::st(base, o + i, a);
      Elem<T>::st(base, o + i + half, b);
    }
  }
}

// LM head for 17..64 rows: weights straight into registers (rx_gemm_kernel),
// eight waves of four 16-row weight tiles, so 32 tiles (512 vocabulary
// columns) per workgroup and one workgroup per CU.  The 8B batch-64 LM head
// streams about 20 % faster this way than through the LDS-copy skinny kernel
// (measured, 172 vs 215 us with partial stores); the smaller layer GEMMs
// keep the skinny kernel, which is faster on their few workgroups.
constexpr int LM_RX_WT = 4, LM_RX_KU = 2, LM_RX_WAVES = 8;
constexpr int LM_RX_TPW = LM_RX_WT * LM_RX_WAVES;  // tiles per workgroup
static inline bool lm_rx_ok(int R, int K, bool packed) { return sk_ok(R, K, packed) && K % (32 * LM_RX_KU) == 0; }

// ---------------------------------------------------------------------------
// rows-GEMM dispatch.  The epilogue sees rows 0..R-1 of one launch; row
// chunks beyond 64 are launched separately with shifted pointers (no split).
template <typename TW, int T, int NT, int U, int WAVES, class Epi>
static hipError_t rows_gemm_launch(const TW* X, int ldx, int R, const TW* W, int K, int N, RowMap map,
                                   const Epi& epi, const RowsPlan& p, bool packed, hipStream_t st, int kc = -1) {
  const int nt16 = N / 16;
  const int grid = p.tiles * p.splits;
  const size_t lds = sizeof(TW) == 2 ? (size_t)WAVES * T * NT * 256 * sizeof(float) : 0;
  if (packed)
    launch_timed(kc, rows_gemm_kernel<TW, T, NT, U, WAVES, true, Epi>, dim3(grid), dim3(WAVES * 64), lds, st, X, ldx,
                 R, W, K, nt16, p.splits, map, epi);
  else
    launch_timed(kc, rows_gemm_kernel<TW, T, NT, U, WAVES, false, Epi>, dim3(grid), dim3(WAVES * 64), lds, st, X, ldx,
                 R, W, K, nt16, p.splits, map, epi);
  return hipGetLastError();
}

// The template arguments below must match plan_rows (T, U, waves per NT).
// kc >= 0: the launch is the principal kernel of timing class kc (kernel mode)
template <typename TW, class Epi>
static hipError_t rows_gemm(const TW* X, int ldx, int R, const TW* W, int K, int N, RowMap map,
                            const Epi& epi, const RowsPlan& p, bool packed, hipStream_t st, int kc = -1) {
  if constexpr (std::is_same<Epi, EpiPartial>::value) {
    // split-K layer GEMMs of 17..64 rows: weights streamed into registers
    if (sizeof(TW) == 2 && sk_ok(R, K, packed) && p.splits > 1 && p.splits == rx_splits(K)) {
      constexpr int WT = 2, WAVES = 4, NB = WT * WAVES;
      const int nt16 = N / 16;
      const int grid = (nt16 + NB - 1) / NB * p.splits;
      rx_gemm_kernel<WT, RX_SPLIT_KU, Epi, WAVES><<<grid, WAVES * 64, 0, st>>>(
          (const bf16*)X, ldx, R, (const bf16*)W, K, nt16, p.splits, epi, 1);
      return hipGetLastError();
    }
  }
  if (sizeof(TW) == 2 && sk_ok(R, K, packed)) {
    const int nt16 = N / 16;
    const int bn = sk_bn(nt16, p.splits);
    const int grid = (nt16 + bn / 16 - 1) / (bn / 16) * p.splits;
    const bf16* Xb = (const bf16*)X;
    const bf16* Wb = (const bf16*)W;
    if (bn == 128)
      launch_timed(kc, skinny_gemm_kernel<128, Epi>, dim3(grid), dim3(256), 0, st, Xb, ldx, R, Wb, K, nt16, p.splits, epi);
    else
      launch_timed(kc, skinny_gemm_kernel<64, Epi>, dim3(grid), dim3(256), 0, st, Xb, ldx, R, Wb, K, nt16, p.splits, epi);
    return hipGetLastError();
  }
  if (sizeof(TW) == 2) {
    switch (p.nt) {
      case 1:
        if (p.t == 1) return rows_gemm_launch<TW, 1, 1, 4, 8>(X, ldx, R, W, K, N, map, epi, p, packed, st, kc);
        return rows_gemm_launch<TW, 2, 1, 4, 8>(X, ldx, R, W, K, N, map, epi, p, packed, st, kc);
      case 2: return rows_gemm_launch<TW, 4, 2, 2, 4>(X, ldx, R, W, K, N, map, epi, p, packed, st, kc);
      case 3: return rows_gemm_launch<TW, 4, 3, 2, 4>(X, ldx, R, W, K, N, map, epi, p, packed, st, kc);
      default: return rows_gemm_launch<TW, 4, 4, 2, 4>(X, ldx, R, W, K, N, map, epi, p, packed, st, kc);
    }
  }
  if (p.nt == 1) return rows_gemm_launch<TW, 1, 1, 1, 4>(X, ldx, R, W, K, N, map, epi, p, false, st, kc);
  return rows_gemm_launch<TW, 1, 4, 1, 4>(X, ldx, R, W, K, N, map, epi, p, false, st, kc);
}

// The drafter's gate/up GEMM (unsplit, SwiGLU epilogue): at 17..64 rows with
// packed weights on the register-weight kernel, measured 1.4 % faster per
// 8B batch-64 chain cycle than the skinny kernel (the target's 61-row
// forward keeps the skinny kernel through rows_gemm: 2 % faster there).
template <typename TW>
static hipError_t rows_gemm_gate_up(const TW* X, int ldx, int R, const TW* W, int K, int N, RowMap map,
                                    const EpiSwiGLU<TW>& epi, const RowsPlan& p, bool packed, hipStream_t st) {
  if constexpr (sizeof(TW) == 2) {
    if (sk_ok(R, K, packed) && p.splits == 1 && (K / 32) % RX_SPLIT_KU == 0) {
      constexpr int WT = 2, WAVES = 4, NB = WT * WAVES;
      const int nt16 = N / 16;
      rx_gemm_kernel<WT, RX_SPLIT_KU, EpiSwiGLU<TW>, WAVES><<<(nt16 + NB - 1) / NB, WAVES * 64, 0, st>>>(
          (const bf16*)X, ldx, R, (const bf16*)W, K, nt16, 1, epi, 1);
      return hipGetLastError();
    }
  }
  return rows_gemm<TW>(X, ldx, R, W, K, N, map, epi, p, packed, st);
}

// ---------------------------------------------------------------------------
// More than 64 rows (a verification forward over a batch of chains): the row
// chunks of 64 in one launch on the register-weight kernel (chunk_of_block),
// so that the chunks of a weight tile read it together: split-K GEMMs
// (EpiPartial with split stride R * N, splits = rx_splits_chunked(K)), the
// unsplit gate/up GEMM (EpiSwiGLU) and, with the LM-head kernel's tiling,
// the LM head (EpiStore).  Every chunk holds 17..64 rows.
//
// k-steps per chunk in the chunked launches: four, so that the activation
// stages and the epilogue tile fit four workgroups per CU in LDS (37 KB
// each, against 64 KB at eight steps): 12.3 against 12.7 ms per 8B
// verification step over 4 x 64 rows (two steps: 12.5)
constexpr int RX_CHUNK_KU = 4;

static inline bool rows_chunked_ok(int R, int K, bool packed) {
  const int last = R % 64 == 0 ? 64 : R % 64;
  return packed && R > 64 && last > 16 && K % (32 * RX_CHUNK_KU) == 0;
}

// Splits of a chunked split-K launch: the chunks already multiply the grid,
// and at rx_splits(K) splits the partials of all R rows are as large as the
// weights, so half as many (8B target at 4 x 64 rows: 13.5 against 13.9 ms
// per verification step, a quarter 13.6); every split still holds whole KU
// chunks.
static inline int rx_splits_chunked(int K) {
  const int s0 = rx_splits(K);
  if (s0 <= 0) return 0;
  const int ns = K / 32;
  int s = s0 / 2;
  while (s > 1 && (ns % s || (ns / s) % RX_CHUNK_KU)) s >>= 1;
  return s;
}

template <class Epi>
static hipError_t rows_gemm_chunked(const bf16* X, int ldx, int R, const bf16* W, int K, int N, const Epi& epi,
                                    int splits, hipStream_t st, int kc = -1) {
  static_assert(EpiRebase<Epi>::value, "a chunked launch needs an epilogue that can be rebased to its chunk");
  const int nt16 = N / 16, nchunk = (R + 63) / 64;
  if constexpr (std::is_same<Epi, EpiPartial>::value) {
    if (splits < 1 || splits != rx_splits_chunked(K)) return hipErrorInvalidValue;
    constexpr int WT = 2, WAVES = 4, NB = WT * WAVES;
    const int grid = chunked_grid((nt16 + NB - 1) / NB * splits, nchunk);
    // weights through the cache (not nontemporal as in the one-chunk
    // launches), so that a unit's chunks share them in L2: 13.0 against
    // 13.5 ms per verification step
    launch_timed(kc, rx_gemm_kernel<WT, RX_CHUNK_KU, Epi, WAVES, false>, dim3(grid), dim3(WAVES * 64), 0, st, X, ldx,
                 R, W, K, nt16, splits, epi, nchunk);
  } else if constexpr (std::is_same<Epi, EpiStore<float>>::value) {
    // cached weight loads as above: 457 against 496 us per 256-row LM head
    const int grid = chunked_grid((nt16 + LM_RX_TPW - 1) / LM_RX_TPW, nchunk);
    launch_timed(kc, rx_gemm_kernel<LM_RX_WT, LM_RX_KU, Epi, LM_RX_WAVES, false>, dim3(grid), dim3(LM_RX_WAVES * 64), 0,
                 st, X, ldx, R, W, K, nt16, 1, epi, nchunk);
  } else {
    // unsplit (gate/up): the register-weight kernel with cached weights,
    // 12.8 against 13.0 ms per verification step on the skinny kernel
    constexpr int WT = 2, WAVES = 4, NB = WT * WAVES;
    if ((K / 32) % RX_CHUNK_KU) return hipErrorInvalidValue;
    const int grid = chunked_grid((nt16 + NB - 1) / NB, nchunk);
    launch_timed(kc, rx_gemm_kernel<WT, RX_CHUNK_KU, Epi, WAVES, false>, dim3(grid), dim3(WAVES * 64), 0, st, X, ldx,
                 R, W, K, nt16, 1, epi, nchunk);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Workspace layout (shared by the size query and the calls).
struct Bump {
  size_t off = 0;
  unsigned char* base = nullptr;
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

}  // namespace e3
