// Row helpers shared by the training-time-test forward and backward: bf16
// packing of eight values and the 16-row block layout of the row kernels.
#pragma once
#include "common.hpp"
#include "gemm_rows.hpp"

namespace e3 {

__device__ __forceinline__ void unpack8(uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f[2 * c] = __uint_as_float(w[c] << 16);
    f[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = (uint32_t)f2bf(f[2 * c]) | ((uint32_t)f2bf(f[2 * c + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Row kernels over 16-row blocks (one MFMA m-tile): 256 threads, the 16
// threads of a DPP row own one matrix row for the sums of squares, then every
// thread writes whole 16-byte slots of the block's fragments (consecutive
// threads -> consecutive slots, 1 KB per fragment).
constexpr int TR = 256;

// Chunk j of a fragment-order bf16 matrix with nkc = K / 32 fragment
// columns: the calling lane's slot (row of its wave, columns 512 j + 8 l ..)
// goes through stage[j % 2]; one barrier per chunk (a buffer is written again
// two chunks later, after every thread has passed the barrier in between).
template <int RB>
__device__ __forceinline__ void put_chunk(uint4 (*stage)[64 * RB], bf16* __restrict__ out, int row0, int nkc, int j,
                                          uint4 slot) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint4* buf = stage[j & 1];
  buf[(l >> 2) * (4 * RB) + (l & 3) * RB + w] = slot;
  __syncthreads();
  const int t = threadIdx.x, q = t / (4 * RB), g = (t / RB) & 3, ww = t % RB;
  if (16 * j + q < nkc)
    ((uint4*)out)[((size_t)(row0 >> 4) * nkc + 16 * j + q) * 64 + (row0 & 15) + ww + 16 * g] = buf[t];
}

// sum of squares of row r0 + (tid/16) over n elements of src (fp32 or bf16),
// reduced over the 16 threads of the DPP row
template <typename TS>
__device__ __forceinline__ float row_ss(const TS* src, size_t ld, int r, int n) {
  const int c = threadIdx.x & 15;
  const TS* p = src + (size_t)r * ld;
  float ss = 0.f;
  for (int k = c * 8; k < n; k += 128) {
    float v[8];
    if (sizeof(TS) == 4) {
      const float4 a = *(const float4*)((const float*)p + k), b = *(const float4*)((const float*)p + k + 4);
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    } else {
      unpack8(*(const uint4*)((const bf16*)p + k), v);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
  return row16_sum(ss);
}

// The rollout-mask attention kernels: LDS blocks of K/V (or Q/dO) rows,
// row-major [rows][hd] bf16 with 16-byte chunk c of row r at slot
// c ^ (r % chunks-per-row), so the 16 rows an MFMA fragment reads sit in
// distinct banks.  A query-block kernel takes ta_waves(G, W) waves per
// workgroup (G query heads per kv head): W, or G when a group has more
// heads.  The forward takes W = 4, one wave per SIMD, so that two workgroups
// share a compute unit and the barrier after every key block does not hold
// all of its waves in step (their MFMA and softmax phases then overlap); the
// dQ kernel keeps W = 8, since with half the waves each wave's share of the
// copies no longer fits its registers.
constexpr int ta_waves(int G, int W) { return G > W ? G : W; }
constexpr int TA_FWD_WAVES = 4, TA_DQ_WAVES = 8;
constexpr float LOG2EF = 1.44269504088896340736f, LN2F = 0.69314718055994530942f;
// The forward's online softmax runs in base 2 with the scale folded into one
// FMA per score; its running maximum (log2 units) moves only when a key
// block's maximum exceeds it by more than TA_RESCALE, so most blocks skip
// rescaling the output, and the unnormalised probabilities stay below 2^8
// (the final division by their sum is unchanged).
constexpr float TA_RESCALE = 8.f;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* tta_lds_s16x4;

// Row-operand fragment from such a block: row r, 16-byte chunk ch (dims 8ch..+8).
template <int CPR>
__device__ __forceinline__ uint4 lds_chunk(const uint4* blk, int r, int ch) {
  return blk[r * CPR + (ch ^ (r % CPR))];
}

// Transposed-operand fragment from such a block (ds_read_tr16_b64): lane
// (ml, q4) gets column 16t + ml of the block with k-slots 8 q4 + j <- row
// base + 4 q4 + j and 8 q4 + 4 + j <- row base + 16 + 4 q4 + j (j < 4).
// Each of the 16 lanes of a group points at 4 consecutive columns of one
// row (row base + 4 q4 + s/4, columns 16t + 4 (s % 4)); the read hands lane
// s column s of the 4 rows.
template <int CPR>
__device__ __forceinline__ U4 lds_tr_frag(const bf16* blk, int base, int t, int ml, int q4) {
  const int r0 = base + 4 * q4 + (ml >> 2), r1 = r0 + 16;
  const int dim = 16 * t + 4 * (ml & 3), ch = dim >> 3, off = dim & 7;
  const s16x4 va =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((tta_lds_s16x4)(blk + (r0 * CPR + (ch ^ (r0 % CPR))) * 8 + off));
  const s16x4 vb =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((tta_lds_s16x4)(blk + (r1 * CPR + (ch ^ (r1 % CPR))) * 8 + off));
  U4 f;
  __builtin_memcpy(&f.u.x, &va, 8);
  __builtin_memcpy(&f.u.z, &vb, 8);
  return f;
}

// B operand of 32 k-slots from two 16 x 16 accumulator tiles x0 (k rows
// 0..15) and x1 (rows 16..31) in the MFMA output layout (lane holds rows
// 4 q4 + e of column ml): slots 8 q4 + e <- x0[e], 8 q4 + 4 + e <- x1[e],
// the k order lds_tr_frag produces.
__device__ __forceinline__ U4 pack_b_from_acc(const f32x4& x0, const f32x4& x1) {
  U4 f;
  f.u = make_uint4(f2bf2(x0[0], x0[1]), f2bf2(x0[2], x0[3]), f2bf2(x1[0], x1[1]), f2bf2(x1[2], x1[3]));
  return f;
}

}  // namespace e3
