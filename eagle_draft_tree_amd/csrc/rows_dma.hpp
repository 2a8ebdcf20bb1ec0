// Skinny GEMM for 17..64 rows (batch-64 drafting): Y[r, n] = sum_k X[r, k] W[n, k]
// with X [R <= 64][K] bf16 row-major and W in packed fragment order
// (eagle3_pack_weights).  Bound by the weight stream from HBM.
//
// Workgroup: 64 rows x BN weight rows (BN = 64 or 128), four waves
// splitting the weight tiles, K step 32 per stage.  Both operands reach LDS
// through direct global -> LDS copies (global_load_lds_dwordx4, issued from
// inline assembly with explicit waits, see bigemm.hpp): the X fragments
// (4 x 1 KB) and the weight fragments (BN/16 x 1 KB, each one contiguous
// kilobyte of the packed layout).  Six stages keep five k-steps of copies in
// flight.  Split-K partitions K per workgroup as in the rows plan; the
// epilogue interface is the rows GEMM's ([16][RP] fp32 tiles of weight rows
// x X rows, RP = 65 with one float of padding).
#pragma once
#include <type_traits>

#include "bigemm.hpp"
#include "gemm_rows.hpp"

namespace e3 {

constexpr int SK_NSTAGE = 6;

// An epilogue that defines kWhole = true receives the workgroup's whole tile
// (whole(wg, tile, RP, R, NB, ntiles16, scratch, split)) instead of one call
// per 16-row weight tile.
template <class E, class = void>
struct EpiWhole {
  static constexpr bool value = false;
};
template <class E>
struct EpiWhole<E, std::void_t<decltype(E::kWhole)>> {
  static constexpr bool value = E::kWhole;
};

static inline bool sk_ok(int R, int K, bool packed) { return packed && R > 16 && R <= 64 && K % 32 == 0; }

// Epilogues that can run on a row chunk of a larger call define
// rebase(r0): from then on their row r is row r0 + r of the call.
template <class E, class = void>
struct EpiRebase {
  static constexpr bool value = false;
  static __device__ __forceinline__ void run(E&, int) {}
};
template <class E>
struct EpiRebase<E, std::void_t<decltype(&E::rebase)>> {
  static constexpr bool value = true;
  static __device__ __forceinline__ void run(E& e, int r0) { e.rebase(r0); }
};

// More than 64 rows in one launch (a verification forward over a batch of
// chains): workgroup -> (unit, row chunk of 64), unit = weight-tile group *
// splits + split.  Workgroups are dealt round-robin over the eight XCDs, so
// the nchunk workgroups of a unit take consecutive slots of one XCD: they
// stream the same weights at about the same time, and the chunks after the
// first find them in that XCD's L2 instead of reading HBM again.  The grid
// is padded to whole rounds of 8 units; unit >= units marks a padding
// workgroup.  nchunk = 1: the plain mapping.
struct ChunkIdx {
  int unit, chunk;
};
__device__ __forceinline__ ChunkIdx chunk_of_block(int nchunk) {
  if (nchunk == 1) return {(int)blockIdx.x, 0};
  const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
  return {(s / nchunk) * 8 + x, s % nchunk};
}
static inline int chunked_grid(int units, int nchunk) {
  return nchunk == 1 ? units : (units + 7) / 8 * 8 * nchunk;
}
// weight rows per workgroup: 64 for split-K matrices up to 6144 rows (QKV and
// O of the 8B drafter), else 128 unless that leaves fewer than 192
// workgroups (measured on the 8B batch-64 shapes)
static inline int sk_bn(int ntiles16, int splits) {
  if (splits > 1 && ntiles16 <= 384) return 64;
  return (long)((ntiles16 + 7) / 8) * splits >= 192 ? 128 : 64;
}

template <int BN, class Epi>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(const bf16* __restrict__ X, int ldx, int R,
                                                          const bf16* __restrict__ W, int K, int ntiles16,
                                                          int splits, Epi epi) {
  constexpr int NB = BN / 16;              // weight tiles per workgroup
  constexpr int WT = NB / 4;               // weight tiles per wave
  constexpr int NF = 4 + NB;               // fragments per stage: 4 of X, NB of W
  constexpr int ND = NF / 4;               // copies per wave per stage
  static_assert(NF % 4 == 0, "fragments split evenly over the waves");
  constexpr int STAGE_U4 = NF * 64;
  constexpr int RP = 65;  // padded tile rows (conflict-free column reads in the epilogue)
  __shared__ uint4 smem[SK_NSTAGE * STAGE_U4];
  static_assert(NB * 16 * RP * 4 + 4096 <= SK_NSTAGE * STAGE_U4 * 16, "epilogue tile and 4 KB scratch fit");
  float* tile = (float*)smem;  // after the k loop: [NB*16][RP]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wgt = blockIdx.x / splits, split = blockIdx.x - wgt * splits;
  const int nsteps = K / 32;
  const int s0 = (int)((long)nsteps * split / splits), s1 = (int)((long)nsteps * (split + 1) / splits);

  // copy sources: fragment f = wave + 4 j; f < 4: X row group f; else W tile f - 4
  const bf16* src[ND];
  size_t step_stride[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int f = wave + 4 * j;
    if (f < 4) {
      const int row = min(f * 16 + (lane & 15), R - 1);
      src[j] = X + (size_t)row * ldx + 8 * (lane >> 4);
      step_stride[j] = 32;
    } else {
      const int t16 = min(wgt * NB + f - 4, ntiles16 - 1);
      src[j] = W + ((size_t)t16 * nsteps * 64 + lane) * 8;
      step_stride[j] = 512;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  // Each workgroup starts its k range at its own offset and wraps around, so
  // that concurrent workgroups do not all copy the same X fragments at the
  // same time (unsplit gate/up, 8B batch 64: 8-10 % faster, measured).  The
  // accumulation order is fixed per workgroup: results stay deterministic.
  const int span = s1 - s0;
  const int rot = span > 0 ? (int)((blockIdx.x * 37u) % (unsigned)span) : 0;
  auto issue = [&](int ks) {
    const uint32_t base = lds0 + (uint32_t)((ks % SK_NSTAGE) * STAGE_U4 * 16);
    int kr = ks + rot;
    if (kr >= s1) kr -= span;
#pragma unroll
    for (int j = 0; j < ND; ++j) dma16(src[j] + (size_t)kr * step_stride[j], base + (uint32_t)((wave + 4 * j) * 1024));
  };

  f32x4 acc[4][WT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npre = min(s1 - s0, SK_NSTAGE - 1);
  for (int i = 0; i < npre; ++i) issue(s0 + i);
  if (s0 + SK_NSTAGE - 1 <= s1) bg_wait_copies<(SK_NSTAGE - 2) * ND>();
  else bg_wait_copies<0>();
  bg_barrier();
  for (int ks = s0; ks < s1; ++ks) {
    const bool more = ks + SK_NSTAGE - 1 < s1;
    if (more) issue(ks + SK_NSTAGE - 1);
    const uint4* st = smem + (size_t)(ks % SK_NSTAGE) * STAGE_U4 + lane;
    U4 a[4], b[WT];
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c].u = st[c * 64];
#pragma unroll
    for (int j = 0; j < WT; ++j) b[j].u = st[(4 + wave * WT + j) * 64];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < WT; ++j)
        acc[c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c].v, b[j].v, acc[c][j], 0, 0, 0);
    if (more) bg_wait_copies<(SK_NSTAGE - 2) * ND>();  // stage ks+1 has landed
    else bg_wait_copies<0>();
    bg_barrier();
  }
  // D[x row][weight row]: lane l holds x rows c*16 + 4(l/16) + e of weight row l%16
  const int m = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[((wave * WT + j) * 16 + m) * RP + c * 16 + q4 * 4 + e] = acc[c][j][e];
  __syncthreads();
  if constexpr (EpiWhole<Epi>::value) {
    // whole-workgroup epilogue: all NB*16 weight rows at once, with the LDS
    // past the tile as scratch
    epi.whole(wgt, tile, RP, R, NB, ntiles16, tile + NB * 16 * RP, split);
  } else {
    for (int t = 0; t < NB; ++t) {
      const int t16 = wgt * NB + t;
      if (t16 < ntiles16) epi(t16, tile + t * 16 * RP, RP, R, split);
    }
  }
}

}  // namespace e3
