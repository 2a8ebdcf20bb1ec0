// Device helpers shared by the gfx950 kernels of the EAGLE-3 library.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "eagle3.h"

namespace e3 {

typedef uint16_t bf16;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN): the gfx950
// conversion instruction v_cvt_pk_bf16_f32, which gives the same bits as
// adding 0x7fff + lsb and truncating for every non-NaN float (checked
// exhaustively over all 2^32 inputs on MI355X).
__device__ __forceinline__ bf16 f2bf(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 in one word (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round a float to the nearest bf16 value and return it as float.
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float rnd(float v) { return v; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p, size_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void st(bf16* p, size_t i, float v) { p[i] = f2bf(v); }
  static __device__ __forceinline__ float rnd(float v) { return round_bf(v); }
};

// ---------------------------------------------------------------------------
// Wave64 reductions on the ALU path: DPP exchanges inside each 16-lane row
// (quad_perm 1032, quad_perm 2301, row_half_mirror, row_mirror), then the
// four row results are read with v_readlane and combined.  The result is
// uniform across the wave and the combination order is fixed.
constexpr int DPP_QUAD_1032 = 0xB1;
constexpr int DPP_QUAD_2301 = 0x4E;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = dpp_i<CTRL>((int)(u & 0xffffffffu)), hi = dpp_i<CTRL>((int)(u >> 32));
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float rdl_f(float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); }
__device__ __forceinline__ double rdl_d(double x, int l) {
  const unsigned long long u = __double_as_longlong(x);
  const unsigned lo = __builtin_amdgcn_readlane((int)(u & 0xffffffffu), l);
  const unsigned hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
  return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);
  return (rdl_f(v, 0) + rdl_f(v, 16)) + (rdl_f(v, 32) + rdl_f(v, 48));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<DPP_QUAD_1032>(v);
  v += dpp_d<DPP_QUAD_2301>(v);
  v += dpp_d<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_d<DPP_ROW_MIRROR>(v);
  return (rdl_d(v, 0) + rdl_d(v, 16)) + (rdl_d(v, 32) + rdl_d(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  return fmaxf(fmaxf(rdl_f(v, 0), rdl_f(v, 16)), fmaxf(rdl_f(v, 32), rdl_f(v, 48)));
}

// Block-wide sum in a fixed order (deterministic).  `red` holds >= nwaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// (value, id) ordering used by every top-k / argmax: larger value first,
// then lower id.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Reductions over the 16 lanes of a DPP row (lanes 16q..16q+15);
// every lane of the row gets the same, bit-identical result.
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
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_i<DPP_QUAD_1032>(v));
  v = min(v, dpp_i<DPP_QUAD_2301>(v));
  v = min(v, dpp_i<DPP_ROW_HALF_MIRROR>(v));
  return min(v, dpp_i<DPP_ROW_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  return v + dpp_f<DPP_ROW_MIRROR>(v);
}

// Wave argmax of (value, id) under `better`; uniform result.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#define E3_ARG_STEP(CTRL)                              \
  {                                                    \
    const float ov = dpp_f<CTRL>(v);                   \
    const int oi = dpp_i<CTRL>(id);                    \
    if (better(ov, oi, v, id)) {                       \
      v = ov;                                          \
      id = oi;                                         \
    }                                                  \
  }
  E3_ARG_STEP(DPP_QUAD_1032)
  E3_ARG_STEP(DPP_QUAD_2301)
  E3_ARG_STEP(DPP_ROW_HALF_MIRROR)
  E3_ARG_STEP(DPP_ROW_MIRROR)
#undef E3_ARG_STEP
  float bv = rdl_f(v, 0);
  int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) {
    const float ov = rdl_f(v, l);
    const int oi = __builtin_amdgcn_readlane(id, l);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  v = bv;
  id = bi;
}

// Wave minimum of a 64-bit key with a payload; uniform result.
__device__ __forceinline__ void wave_argmin_u64(unsigned long long& key, int& pay) {
#define E3_MIN_STEP(CTRL)                                                                       \
  {                                                                                             \
    const unsigned lo = dpp_i<CTRL>((int)(key & 0xffffffffu)), hi = dpp_i<CTRL>((int)(key >> 32)); \
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;                          \
    const int op = dpp_i<CTRL>(pay);                                                            \
    if (o < key) {                                                                              \
      key = o;                                                                                  \
      pay = op;                                                                                 \
    }                                                                                           \
  }
  E3_MIN_STEP(DPP_QUAD_1032)
  E3_MIN_STEP(DPP_QUAD_2301)
  E3_MIN_STEP(DPP_ROW_HALF_MIRROR)
  E3_MIN_STEP(DPP_ROW_MIRROR)
#undef E3_MIN_STEP
  unsigned long long bk = ~0ull;
  int bp = 0;
#pragma unroll
  for (int l = 0; l < 64; l += 16) {
    const unsigned lo = __builtin_amdgcn_readlane((int)(key & 0xffffffffu), l);
    const unsigned hi = __builtin_amdgcn_readlane((int)(key >> 32), l);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    const int op = __builtin_amdgcn_readlane(pay, l);
    if (o < bk) {
      bk = o;
      bp = op;
    }
  }
  key = bk;
  pay = bp;
}

}  // namespace e3
