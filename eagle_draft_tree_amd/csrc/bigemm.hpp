// Tiled MFMA GEMM for many rows (the training-time-test forward):
//   C[r, n] = sum_k A[r, k] * W[n, k]
// A: activations [M][K] bf16 row-major; W: weights in packed fragment order
// (eagle3_pack_weights) or row-major read through a row map.  fp32
// accumulation on v_mfma_f32_16x16x32_bf16.
//
// Workgroup tile 256 x 256, four waves in a 2 x 2 grid (wave tile 128 x 128
// = 8 x 8 MFMA tiles, 256 accumulator registers), K step 64.  Both operands
// are staged in LDS in MFMA fragment order (a 16 x 32 fragment is 64 lanes x
// 16 bytes; lane l holds row l%16, k-slice 8(l/16)), so an MFMA operand is
// one 16-byte LDS read per lane.  A-tile fragments are stored with an XOR
// swizzle on the lane slot that keeps both the row-wise stores and the
// fragment reads free of bank conflicts.  LDS is double-buffered: the
// global loads of step s+1 are in flight during the MFMAs of step s.
//
// Block order: 8 row tiles share a column tile (grouped order), and block
// ids are remapped so that consecutive logical tiles run on the same XCD
// (hardware dispatch places block b on XCD b % 8) and share its L2.
#pragma once
#include "common.hpp"
#include "gemm_rows.hpp"

namespace e3 {

constexpr int BG_BM = 256, BG_BN = 256, BG_BK = 64;
constexpr int BG_THREADS = 256;
constexpr int BG_FRAGS = (BG_BM / 16) * (BG_BK / 32);  // 32 fragments per operand per stage
constexpr int BG_STAGE_U4 = 2 * BG_FRAGS * 64;           // A + B of one stage, in uint4

static inline int bg_grid(int M, int N) { return ((M + BG_BM - 1) / BG_BM) * ((N / 16 + 15) / 16); }

// Lane slot of fragment lane `pos` (row pos%16, k-slice pos/16) of k-chunk
// `cc` in the swizzled A layout.
__device__ __forceinline__ int bg_swz(int pos, int cc) { return pos ^ ((pos >> 4) | (cc << 2) | ((pos & 1) << 3)); }

template <bool PACKED, class Epi>
__global__ __launch_bounds__(BG_THREADS) void big_gemm_kernel(const bf16* __restrict__ A, int lda, int M,
                                                              const bf16* __restrict__ W, int N, int K, RowMap map,
                                                              Epi epi) {
  __shared__ uint4 smem[2 * BG_STAGE_U4];  // 128 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nt16 = N / 16;
  const int ntn = (nt16 + 15) / 16;
  const int ntm = (M + BG_BM - 1) / BG_BM;
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int GROUP = 8;
  const int per_group = GROUP * ntn;
  const int first_m = (bid / per_group) * GROUP;
  const int gsz = min(GROUP, ntm - first_m);
  const int bm = first_m + (bid % per_group) % gsz;
  const int bn = (bid % per_group) / gsz;
  const int nchunks = K / 32;

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-thread global sources.  A: element e = tid + 256 j is row e/8 =
  // tid/8 + 32 j, 16-byte segment tid%8 of the 64-wide k step; its LDS slot
  // advances by 256 per j.  B: element e is fragment e/64 (n-tile
  // tid/128 + 2 j, k-chunk (tid/64)%2), lane tid%64.
  const int ar0 = tid >> 3, as = tid & 7;
  const int arow0 = bm * BG_BM + ar0;
  const bf16* abase = A + (size_t)arow0 * lda + 8 * as;
  const int adst0 = (((ar0 >> 4) * 2 + (as >> 2)) << 6) + bg_swz((ar0 & 15) + 16 * (as & 3), as >> 2);
  const int bt0 = bn * 16 + (tid >> 7), bcc = (tid >> 6) & 1, bl = tid & 63;
  const bf16* bbase = W + (((size_t)bt0 * nchunks + bcc) * 64 + bl) * 8;  // packed
  const size_t bstep = (size_t)2 * nchunks * 512;                         // packed, per j

  uint4 ra[8], rb[8];
  auto load_stage = [&](int ks) {
    const int k0 = ks * BG_BK;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ra[j] = arow0 + 32 * j < M ? *(const uint4*)(abase + (size_t)32 * j * lda + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int nt = bt0 + 2 * j;
      if (nt >= nt16) {
        rb[j] = make_uint4(0, 0, 0, 0);
      } else if (PACKED) {
        rb[j] = ld_stream(bbase + j * bstep + (size_t)(k0 / 32) * 512);
      } else {
        rb[j] = *(const uint4*)(W + (size_t)map(nt, bl & 15) * K + k0 + bcc * 32 + 8 * (bl >> 4));
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint4* sa = smem + (size_t)buf * BG_STAGE_U4;
    uint4* sb = sa + BG_FRAGS * 64;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sa[adst0 + 256 * j] = ra[j];
      sb[tid + BG_THREADS * j] = rb[j];
    }
  };

  const int nk = K / BG_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) load_stage(ks + 1);
    const uint4* sa = smem + (size_t)(ks & 1) * BG_STAGE_U4;
    const uint4* sb = sa + BG_FRAGS * 64;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      U4 a[8], b[8];
      const int aslot = bg_swz(lane, cc);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i].u = sa[(((wm * 8 + i) * 2 + cc) << 6) + aslot];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j].u = sb[(((wn * 8 + j) * 2 + cc) << 6) + lane];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i].v, b[j].v, acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) store_stage((ks + 1) & 1);
    __syncthreads();
  }
  // lane l holds C[rowbase + 16 i + 4(l/16) + e][n of column tile colbase16 + j, slot l%16]
  epi(acc, bm * BG_BM + wm * 128, bn * 16 + wn * 8, lane, M, nt16);
}

// Lane l receives lane l^8 of its 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float xor8(float v) { return dpp_f<0x128>(v); }

// Reductions over the 16 lanes of a DPP row (the 16 columns of one C row).
__device__ __forceinline__ void row16_argmax(float& v, int& id) {
#define E3_ROW_STEP(CTRL)              \
  {                                    \
    const float ov = dpp_f<CTRL>(v);   \
    const int oi = dpp_i<CTRL>(id);    \
    if (better(ov, oi, v, id)) {       \
      v = ov;                          \
      id = oi;                         \
    }                                  \
  }
  E3_ROW_STEP(DPP_QUAD_1032)
  E3_ROW_STEP(DPP_QUAD_2301)
  E3_ROW_STEP(DPP_ROW_HALF_MIRROR)
  E3_ROW_STEP(DPP_ROW_MIRROR)
#undef E3_ROW_STEP
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  return v + dpp_f<DPP_ROW_MIRROR>(v);
}

typedef f32x4 BGAcc[8][8];

// --------------------------------------------------------------------------- epilogues
// C (plain map) -> float buffer, rounded to bf16 values when `round` is set.
struct BEpiStoreF {
  float* out;
  int ldo;
  bool round;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col16 = colbase16 + j;
        if (col16 >= nt16) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row0 + e < M) {
            const float v = acc[i][j][e];
            out[(size_t)(row0 + e) * ldo + col16 * 16 + m] = round ? round_bf(v) : v;
          }
      }
    }
  }
};

// out = out + C (fp32, plain map): the residual update of the state stream.
struct BEpiResid {
  float* out;
  int ld;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col16 = colbase16 + j;
        if (col16 >= nt16) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row0 + e < M) {
            const size_t o = (size_t)(row0 + e) * ld + col16 * 16 + m;
            out[o] = out[o] + acc[i][j][e];
          }
      }
    }
  }
};

// SwiGLU on MAP_PAIR_FFN tiles: slot m < 8 is gate column 8t+m, slot m+8
// the matching up column.  z = silu(gate) * up, rounded to bf16.
struct BEpiSwiGLU {
  bf16* z;
  int ffn;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f32x4 up;
#pragma unroll
        for (int e = 0; e < 4; ++e) up[e] = xor8(acc[i][j][e]);
        const int col16 = colbase16 + j;
        if (col16 < nt16 && m < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (row0 + e < M) {
              const float g = acc[i][j][e];
              z[(size_t)(row0 + e) * ffn + col16 * 8 + m] = f2bf(g / (1.f + expf(-g)) * up[e]);
            }
        }
      }
    }
  }
};

}  // namespace e3
