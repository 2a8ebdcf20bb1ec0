// Tiled MFMA GEMM for many rows (the training-time-test forward):
//   C[r, n] = sum_k A[r, k] * W[n, k]
// A: activations [M][K] bf16 row-major; W: weights in packed fragment order
// (eagle3_pack_weights) or row-major read through a row map.  fp32
// accumulation on v_mfma_f32_16x16x32_bf16.
//
// Workgroup tile 256 x 256, eight waves in a 2 x 4 grid (wave tile 128 x 64
// = 8 x 4 MFMA tiles, 128 accumulator registers, two waves per SIMD), K
// step 32.  Both operands are staged in LDS in MFMA fragment order (a 16 x
// 32 fragment is 64 lanes x 16 bytes; lane l holds row l%16, k-slice
// 8(l/16)) by direct global -> LDS copies (no VGPR staging), so an MFMA
// operand is one linear, conflict-free 16-byte LDS read per lane.  Four
// stages of LDS (128 KB) keep three k steps of copies in flight.  The k loop
// is a ping-pong of two wave groups one phase apart (see k_loop), and the
// launch is persistent: one block per compute unit walks its tiles, copying
// the next tile's first stages while the current tile's epilogue runs.
//
// Tile order: 8 row tiles share a column tile (grouped order), and tiles
// are dealt so that consecutive logical tiles run on the same XCD
// (hardware dispatch places block b on XCD b % 8) and share its L2.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "gemm_rows.hpp"
#include "timing.hpp"

namespace e3 {

#ifndef E3_BG_PERSIST
#define E3_BG_PERSIST 1
#endif

constexpr int BG_BM = 256, BG_BN = 256, BG_BK = 32;
constexpr int BG_THREADS = 512;                   // 8 waves: 2 (rows) x 4 (columns)
constexpr int BG_NJ = 4;                          // 16-column tiles per wave (64 columns)
constexpr int BG_FRAGS = BG_BM / 16;              // 16 fragments per operand per stage
constexpr int BG_STAGE_U4 = 2 * BG_FRAGS * 64;    // A + B of one stage, in uint4 (32 KB)
constexpr int BG_NSTAGE = 4;                      // 128 KB of LDS, three stages in flight

static inline int bg_grid(int M, int N) { return ((M + BG_BM - 1) / BG_BM) * ((N / 16 + 15) / 16); }

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l
// of the wave lands at LDS byte address lds + 16 l (lds wave-uniform, in
// M0, restored afterwards).  Issued from inline assembly so that the
// compiler does not insert conservative vmcnt waits before unrelated LDS
// reads; completion is awaited explicitly (bg_wait_copies), and extra copies
// in flight only make the compiler's own vmcnt waits stricter.  The
// instruction has no register results.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))  // wave-uniform by contract
      : "memory");
}
template <int N>
__device__ __forceinline__ void bg_wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Every LDS read of this wave has completed, then the workgroup barrier.
__device__ __forceinline__ void bg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef f32x4 BGAcc[8][BG_NJ];

// Element offset of (r, k) in a fragment-ordered [M][K] bf16 matrix (nkc =
// K/32): fragment (r/16, k/32) is 512 contiguous elements, lane slot
// (r%16) + 16*((k%32)/8) holds 8 consecutive k.  Used for activations that
// feed the A operand, so A copies read whole kilobytes like packed weights.
__device__ __forceinline__ size_t frag_off(int r, int k, int nkc) {
  return ((size_t)(r >> 4) * nkc + (k >> 5)) * 512 + ((((r & 15) + 16 * ((k & 31) >> 3))) << 3) + (k & 7);
}

// APACK: A in fragment order (frag_off) instead of row-major with stride lda.
// Optional epilogue hook run before the k loop (e.g. loading per-row data
// whose latency would otherwise sit in the epilogue): an epilogue that
// defines `Pre` and `pre(rowbase, lane, M)` receives the value as its second
// argument.
template <class E, class = void>
struct EpiHook {
  struct T {};
  static __device__ __forceinline__ T pre(const E&, int, int, int) { return T{}; }
  static __device__ __forceinline__ void run(const E& e, const BGAcc& acc, const T&, int r, int c, int l, int M,
                                             int n) {
    e(acc, r, c, l, M, n);
  }
};
template <class E>
struct EpiHook<E, std::void_t<typename E::Pre>> {
  using T = typename E::Pre;
  static __device__ __forceinline__ T pre(const E& e, int r, int l, int M) { return e.pre(r, l, M); }
  static __device__ __forceinline__ void run(const E& e, const BGAcc& acc, const T& p, int r, int c, int l, int M,
                                             int n) {
    e(acc, p, r, c, l, M, n);
  }
};

template <bool PACKED, bool APACK, class Epi>
__global__ __launch_bounds__(BG_THREADS) void big_gemm_kernel(const bf16* __restrict__ A, int lda, int M,
                                                              const bf16* __restrict__ W, int N, int K, RowMap map,
                                                              Epi epi) {
  __shared__ uint4 smem[BG_NSTAGE * BG_STAGE_U4];  // 128 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int nt16 = N / 16;
  const int ntn = (nt16 + 15) / 16;
  const int ntm = (M + BG_BM - 1) / BG_BM;
  // Tiles: ntm x ntn of 256 x 256.  Virtual block vb (the launch's block id,
  // or with a persistent launch every gridDim.x-th one from it) -> tile.
  const int ntiles = ntm * ntn;
  const int nchunks = K / 32;
  auto tile_of = [&](int vb, int& bm, int& bn) {
    int bid = vb;
#ifndef E3_BG_MAP
#define E3_BG_MAP 0
#endif
#if E3_BG_MAP != 3
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
#endif
#if E3_BG_MAP == 1
    const int GROUP = 16;
#elif E3_BG_MAP == 2
    const int GROUP = 4;
#elif E3_BG_MAP == 5
    const int GROUP = 32;
#else
    const int GROUP = 8;
#endif
    const int per_group = GROUP * ntn;
    const int first_m = (bid / per_group) * GROUP;
    const int gsz = min(GROUP, ntm - first_m);
    bm = first_m + (bid % per_group) % gsz;
    bn = (bid % per_group) / gsz;
  };

  f32x4 acc[8][BG_NJ];

  // Copy sources.  Per stage (32 k) wave w copies A fragments (m-tiles 2w,
  // 2w+1) and B fragments (n-tiles 2w, 2w+1); lane l of a fragment is row
  // (or weight row) l%16, k-slice 8(l/16).  Rows past M and n-tiles past N
  // read the last valid ones (their results are dropped by the epilogue).
  const bf16* asrc[2];
  const bf16* bsrc[2];
  auto set_sources = [&](int bm, int bn) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mt = wave * 2 + h;
      if (APACK) {
        const int mtc = min(bm * (BG_BM / 16) + mt, (M - 1) >> 4);
        asrc[h] = A + ((size_t)mtc * nchunks * 64 + lane) * 8;
      } else {
        const int row = min(bm * BG_BM + mt * 16 + (lane & 15), M - 1);
        asrc[h] = A + (size_t)row * lda + 8 * (lane >> 4);
      }
      const int ntile = min(bn * 16 + wave * 2 + h, nt16 - 1);
      if (PACKED)
        bsrc[h] = W + ((size_t)ntile * nchunks * 64 + lane) * 8;
      else
        bsrc[h] = W + (size_t)map(ntile, lane & 15) * K + 8 * (lane >> 4);
    }
  };
  int vb = blockIdx.x, bm, bn;
  tile_of(vb, bm, bn);
  set_sources(bm, bn);
  const uint32_t lds0 = lds_addr(smem);
  auto issue_stage = [&](int ks) {
    const uint32_t sa = lds0 + (uint32_t)((ks % BG_NSTAGE) * BG_STAGE_U4 * 16);
    const uint32_t sb = sa + BG_FRAGS * 64 * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t f = (uint32_t)(wave * 2 + h) * 1024u;
      dma16(asrc[h] + (APACK ? (size_t)ks * 512 : (size_t)ks * BG_BK), sa + f);
      if (PACKED)
        dma16(bsrc[h] + (size_t)ks * 512, sb + f);
      else
        dma16(bsrc[h] + ks * BG_BK, sb + f);
    }
  };
  // The k loop.  Two wave groups, waves 0-3 and 4-7 (the hardware places
  // waves w and w+4 on one SIMD), run one phase apart: while one group
  // multiplies its k-step from registers at raised priority, the other reads
  // its next k-step's operands from LDS into registers and issues its
  // copies, so each SIMD always has a wave feeding the matrix pipe.  Every
  // wave passes the same number of barriers (the lagging group's extra one
  // first, the leading group's last).  Four LDS stages: stages s+1..s+3 are
  // being copied while stage s is read; before the barrier that ends its
  // read phase a wave waits until its copies of stage s+1 have landed.
  const int nk = K / BG_BK;
  const int npre = nk < BG_NSTAGE - 1 ? nk : BG_NSTAGE - 1;
  const int grp = wave >> 2;
  auto k_loop = [&]() {
    if (grp == 1) bg_barrier();
    for (int ks = 0; ks < nk; ++ks) {
      U4 b[BG_NJ], a[8];
      {
        const uint4* sa = smem + (size_t)(ks % BG_NSTAGE) * BG_STAGE_U4 + lane;
        const uint4* sb = sa + BG_FRAGS * 64;
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j) b[j].u = sb[(wn * BG_NJ + j) << 6];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i].u = sa[(wm * 8 + i) << 6];
      }
      if (ks + BG_NSTAGE - 1 < nk) {
        issue_stage(ks + BG_NSTAGE - 1);
        bg_wait_copies<8>();  // stages ks+2, ks+3 may still be in flight
      } else {
        bg_wait_copies<0>();
      }
      bg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i].v, b[j].v, acc[i][j], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      bg_barrier();
    }
    if (grp == 0) bg_barrier();
  };

  typename EpiHook<Epi>::T pre = EpiHook<Epi>::pre(epi, bm * BG_BM + wm * 128, lane, M);
  for (int ks = 0; ks < npre; ++ks) issue_stage(ks);
  if (npre >= 3) bg_wait_copies<8>();
  else bg_wait_copies<0>();
  bg_barrier();
  // One tile per block, or (persistent launch) every gridDim.x-th tile: the
  // next tile's first stages are copied while this tile's epilogue runs.
  for (;;) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    k_loop();
    const int bm_c = bm, bn_c = bn;
    vb += E3_BG_PERSIST ? (int)gridDim.x : ntiles;
    const bool more = vb < ntiles;
    if (more) {
      tile_of(vb, bm, bn);
      set_sources(bm, bn);
      for (int ks = 0; ks < npre; ++ks) issue_stage(ks);
    }
    // lane l holds C[rowbase + 16 i + 4(l/16) + e][n of column tile colbase16 + j, slot l%16]
    EpiHook<Epi>::run(epi, acc, pre, bm_c * BG_BM + wm * 128, bn_c * 16 + wn * BG_NJ, lane, M, nt16);
    if (!more) break;
    pre = EpiHook<Epi>::pre(epi, bm * BG_BM + wm * 128, lane, M);
    bg_wait_copies<0>();
    bg_barrier();
  }
}

// Launch C = A . W^T on `st`.  apack: A in fragment order (frag_off) instead
// of row-major with stride lda; packed: W in packed fragment order (else
// row-major through `map`).  kc >= 0: timed as that class's principal kernel.
// Compute units of the current device (queried once per process).
inline int bg_cus() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return v;
  }();
  return n;
}

template <class Epi>
inline hipError_t bg_launch(const bf16* A, int lda, bool apack, int M, const void* W, bool packed, int N, int K,
                            RowMap map, Epi epi, hipStream_t st, int kc = -1) {
  int grid = bg_grid(M, N);
  // persistent: one block per compute unit (a multiple of the 8 XCDs keeps
  // each block on the XCD its tiles are mapped to)
  if (E3_BG_PERSIST && grid > bg_cus() && bg_cus() % 8 == 0) grid = bg_cus();
  const bf16* Wb = (const bf16*)W;
  const dim3 g(grid), b(BG_THREADS);
  if (packed && apack) launch_timed(kc, big_gemm_kernel<true, true, Epi>, g, b, 0, st, A, lda, M, Wb, N, K, map, epi);
  else if (packed) launch_timed(kc, big_gemm_kernel<true, false, Epi>, g, b, 0, st, A, lda, M, Wb, N, K, map, epi);
  else if (apack) launch_timed(kc, big_gemm_kernel<false, true, Epi>, g, b, 0, st, A, lda, M, Wb, N, K, map, epi);
  else launch_timed(kc, big_gemm_kernel<false, false, Epi>, g, b, 0, st, A, lda, M, Wb, N, K, map, epi);
  return hipGetLastError();
}

// Lane l receives lane l^8 of its 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float xor8(float v) { return dpp_f<0x128>(v); }

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
      for (int j = 0; j < BG_NJ; ++j) {
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

// out = in + C (fp32, plain map): the residual update of the state stream
// (in == out updates it in place).  A tile that lies wholly inside the matrix
// takes branch-free code that loads the residual values of row group i + 1
// before it stores group i: out may be in itself, so the compiler keeps a
// load behind the previous store, and guarded load, wait and store per
// element cost a memory round trip each (128 per lane and tile).  Each element
// is still read before it is written, so the in-place case holds.
struct BEpiAdd {
  const float* in;
  float* out;
  int ld;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
    if (rowbase + 128 <= M && colbase16 + BG_NJ <= nt16) {
      const float* ip = in + (size_t)(rowbase + 4 * (lane >> 4)) * ld + colbase16 * 16 + m;
      float* op = out + (size_t)(rowbase + 4 * (lane >> 4)) * ld + colbase16 * 16 + m;
      float cur[BG_NJ][4], nxt[BG_NJ][4];
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[j][e] = ip[(size_t)e * ld + 16 * j];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + 1 < 8) {
#pragma unroll
          for (int j = 0; j < BG_NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) nxt[j][e] = ip[(size_t)(16 * (i + 1) + e) * ld + 16 * j];
        }
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) op[(size_t)(16 * i + e) * ld + 16 * j] = cur[j][e] + acc[i][j][e];
        if (i + 1 < 8) {
#pragma unroll
          for (int j = 0; j < BG_NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) cur[j][e] = nxt[j][e];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j) {
        const int col16 = colbase16 + j;
        if (col16 >= nt16) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row0 + e < M) {
            const size_t o = (size_t)(row0 + e) * ld + col16 * 16 + m;
            out[o] = in[o] + acc[i][j][e];
          }
      }
    }
  }
};

// C (plain map) -> bf16, row-major with stride ldo.
struct BEpiStoreBF {
  bf16* out;
  int ldo;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j) {
        const int col16 = colbase16 + j;
        if (col16 >= nt16) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row0 + e < M) out[(size_t)(row0 + e) * ldo + col16 * 16 + m] = f2bf(acc[i][j][e]);
      }
    }
  }
};

// SwiGLU on MAP_PAIR_FFN tiles: slot m < 8 is gate column 8t+m, slot m+8
// the matching up column.  z = silu(gate) * up, rounded to bf16, written in
// fragment order for the down projection's A operand; with gu set, the fp32
// (gate, up) pair is kept as well ([M][ffn], for the backward).
struct BEpiSwiGLU {
  bf16* z;  // fragment order [M][ffn] (frag_off)
  int ffn;
  float2* gu = nullptr;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j) {
        f32x4 up;
#pragma unroll
        for (int e = 0; e < 4; ++e) up[e] = xor8(acc[i][j][e]);
        const int col16 = colbase16 + j;
        if (col16 < nt16 && m < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (row0 + e < M) {
              const float g = acc[i][j][e];
              z[frag_off(row0 + e, col16 * 8 + m, ffn >> 5)] = f2bf(g / (1.f + expf(-g)) * up[e]);
              if (gu) gu[(size_t)(row0 + e) * ffn + col16 * 8 + m] = make_float2(g, up[e]);
            }
        }
      }
    }
  }
};

}  // namespace e3
