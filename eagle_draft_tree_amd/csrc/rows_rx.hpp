// GEMM for 17..64 rows (batch-64 drafting) with the weights in registers:
// Y[r, n] = sum_k X[r, k] W[n, k], X [R <= 64][K] bf16 row-major, W in
// packed fragment order (eagle3_pack_weights).  Bound by the weight stream.
//
// Workgroup: 64 X rows x 16*WT*WAVES weight rows, WAVES waves, each owning
// WT weight tiles of 16 rows.  Every weight fragment is read once, straight
// from HBM into the MFMA operand registers (nontemporal loads: the path
// that streams fastest); only the X operand, which every workgroup shares,
// goes through LDS.  X is staged per chunk of KU k-steps (32 k each) by
// global -> LDS copies in fragment order, double-buffered: a wave issues
// the copies of chunk c+1 after computing chunk c, and they land (L2 hits)
// while the weight loads of chunk c+1 are in flight.  Split-K partitions
// the k-steps per workgroup as in the rows plan.  The epilogue interface is
// the skinny kernel's: [16][RP] fp32 tiles (RP = 65), or the whole
// workgroup tile (EpiWhole, with 1 KB of LDS scratch per wave).
//
// nchunk > 1: one launch covers R > 64 rows as row chunks of 64, a
// workgroup per (unit, chunk) placed by chunk_of_block, the epilogue rebased
// to its chunk's rows; NTW = false then loads the weights through the cache,
// so that the chunks of a unit share them in L2.
#pragma once
#include "rows_dma.hpp"

namespace e3 {

template <int WT, int KU, class Epi, int WAVES = 4, bool NTW = true>
__global__ __launch_bounds__(WAVES * 64) void rx_gemm_kernel(const bf16* __restrict__ X, int ldx, int R,
                                                      const bf16* __restrict__ W, int K, int ntiles16,
                                                      int splits, Epi epi_in, int nchunk) {
  constexpr int NB = WAVES * WT;            // weight tiles per workgroup
  constexpr int XCH_U4 = KU * 4 * 64;       // one X chunk: KU steps x 4 row groups x 1 KB
  constexpr int RP = 65;                    // padded epilogue tile rows
  constexpr int TILE_U4 = (NB * 16 * RP * 4 + WAVES * 1024 + 15) / 16;  // tile + 1 KB of scratch per wave
  constexpr int SMEM_U4 = 2 * XCH_U4 > TILE_U4 ? 2 * XCH_U4 : TILE_U4;
  __shared__ uint4 smem[SMEM_U4];
  float* tile = (float*)smem;  // after the k loop: [NB*16][RP]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkIdx ci = chunk_of_block(nchunk);
  if (ci.unit >= (ntiles16 + NB - 1) / NB * splits) return;  // padding of a chunked grid (whole workgroup)
  Epi epi = epi_in;
  if (nchunk > 1) {
    X += (size_t)ci.chunk * 64 * ldx;
    R = min(64, R - ci.chunk * 64);
    EpiRebase<Epi>::run(epi, ci.chunk * 64);
  }
  const int wgt = ci.unit / splits, split = ci.unit - wgt * splits;
  const int nsteps = K / 32;
  const int s0 = (int)((long)nsteps * split / splits), s1 = (int)((long)nsteps * (split + 1) / splits);
  const int nch = (s1 - s0) / KU;  // the host guarantees (s1 - s0) % KU == 0

  // X copies: fragment f = s * 4 + g (step s, row group g) of a chunk is
  // copied by wave f % WAVES
  const uint32_t lds0 = lds_addr(smem);
  auto issue_x = [&](int c) {
    const uint32_t base = lds0 + (uint32_t)((c & 1) * XCH_U4 * 16);
    for (int f = wave; f < KU * 4; f += WAVES) {
      const int s = f >> 2, g = f & 3;
      const int xrow = min(g * 16 + (lane & 15), R - 1);
      dma16(X + (size_t)xrow * ldx + 8 * (lane >> 4) + (size_t)(s0 + c * KU + s) * 32, base + (uint32_t)(f * 1024));
    }
  };
  // weight fragments: tile t16 = wgt*NB + wave*WT + j, lane's 16 bytes
  const bf16* wsrc[WT];
#pragma unroll
  for (int j = 0; j < WT; ++j) {
    const int t16 = min(wgt * NB + wave * WT + j, ntiles16 - 1);
    wsrc[j] = W + ((size_t)t16 * nsteps * 64 + lane) * 8;
  }

  f32x4 acc[4][WT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](int c, U4 (&wf)[KU][WT]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KU; ++s)
#pragma unroll
      for (int j = 0; j < WT; ++j) {
        const bf16* p = wsrc[j] + (size_t)(s0 + c * KU + s) * 512;
        wf[s][j].u = NTW ? ld_stream(p) : *(const uint4*)p;
      }
  };
  auto compute = [&](int c, const U4 (&wf)[KU][WT]) __attribute__((always_inline)) {
    const uint4* xb = smem + (size_t)(c & 1) * XCH_U4 + lane;
#pragma unroll
    for (int s = 0; s < KU; ++s) {
      U4 xa[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) xa[g].u = xb[(s * 4 + g) * 64];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < WT; ++j)
          acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[g].v, wf[s][j].v, acc[g][j], 0, 0, 0);
    }
  };
  if constexpr (WAVES >= 8) {
    // Long k ranges (the unsplit LM head): weights one chunk ahead, chunk
    // c+1's weight loads in flight while chunk c is computed (two register
    // buffers, so the loop runs in pairs; measured about 5 % faster on the
    // 8B batch-64 LM head).  Issue order per chunk: w(c+1), compute(c),
    // x(c+1); at the top of chunk c the only loads issued after w(c) and
    // x(c) are those of w(c+1), so vmcnt(KU*WT) means chunk c's weights and
    // X have landed.  The short split-K ranges keep the single buffer: its
    // doubled registers halve their occupancy, which costs more than the
    // overlap gains there (measured).
    U4 wa[KU][WT], wb[KU][WT];
    if (nch > 0) {
      issue_x(0);
      load_w(0, wa);
    }
    for (int c = 0; c < nch; c += 2) {
      if (c + 1 < nch) {
        load_w(c + 1, wb);
        bg_wait_copies<KU * WT>();
      } else {
        bg_wait_copies<0>();
      }
      bg_barrier();  // chunk c is in LDS for every wave; chunk c-1 is no longer read
      compute(c, wa);
      if (c + 1 >= nch) break;
      // next chunk's X, into the buffer every wave left before the barrier above
      issue_x(c + 1);
      if (c + 2 < nch) {
        load_w(c + 2, wa);
        bg_wait_copies<KU * WT>();
      } else {
        bg_wait_copies<0>();
      }
      bg_barrier();
      compute(c + 1, wb);
      if (c + 2 < nch) issue_x(c + 2);
    }
  } else {
    if (nch > 0) issue_x(0);
    for (int c = 0; c < nch; ++c) {
      U4 wf[KU][WT];
      load_w(c, wf);
      // the X copies of chunk c were issued before these weight loads
      bg_wait_copies<KU * WT>();
      bg_barrier();  // chunk c is in LDS for every wave; chunk c-1 is no longer read
      compute(c, wf);
      // next chunk's X, into the buffer every wave left before the barrier
      // above; issued after this chunk's weight waits so that the compiler's
      // vmcnt counts for its own loads stay exact
      if (c + 1 < nch) issue_x(c + 1);
    }
  }
  bg_wait_copies<0>();
  __syncthreads();  // every wave is done with the X buffers
  // D[x row][weight row]: lane l holds x rows g*16 + 4(l/16) + e of weight row l%16
  const int m = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[((wave * WT + j) * 16 + m) * RP + g * 16 + q4 * 4 + e] = acc[g][j][e];
  __syncthreads();
  if constexpr (EpiWhole<Epi>::value) {
    epi.whole(wgt, tile, RP, R, NB, ntiles16, tile + NB * 16 * RP, split);
  } else {
    for (int t = 0; t < NB; ++t) {
      const int t16 = wgt * NB + t;
      if (t16 < ntiles16) epi(t16, tile + t * 16 * RP, RP, R, split);
    }
  }
}

}  // namespace e3
