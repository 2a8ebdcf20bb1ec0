// The efficient draft LM head (EAGLE-4 blog: the paragraph "EAGLE Efficient
// LM Head" and the section 关于 Efficient LM Head).  Stage 1 scores the whole
// vocabulary with a low-rank head (two rows GEMMs in draft.hip: z = B y,
// s = A z, the second with per-16-column-tile {max, sum exp} statistics) and
// keeps the c best scores as candidates; stage 2 computes the full LM head's
// exact logits of the candidates only.  The top-k are the best candidates,
// their log-probabilities normalised over the candidate set.
//
// Kernels here, per row of the LM head:
//   topc_tiles_kernel  the c best scores (value desc, id asc) -> candidate ids
//   cand_logits_kernel exact logits W_lm[cand] . y, one wave per candidate
//   cand_topk_kernel   top-k among the candidates and their log-sum-exp
#include <limits.h>

#include "common.hpp"
#include "gemm_rows.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace e3 {

namespace {

constexpr int TC_THREADS = 512;
constexpr int TC_WAVES = TC_THREADS / 64;
constexpr int TC_TPT = 33;     // tile slots per thread: vocab <= 262144 plus slot padding
constexpr int TC_CMAX = 4096;  // collected scores (fallback: scores above T, fewer than 16 * LOWRANK_MAX_CAND)
constexpr int TC_EQT = 1024;   // fallback: tiles whose maximum reaches T, kept for the tie scan
constexpr int TC_LIST = 1024;  // slots reaching T0

// order-preserving map of float32 onto uint32 (and back)
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float kfloat(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ unsigned wave_incl_scan(unsigned v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Candidates of one row: the c best low-rank scores by (value desc, id asc).
//
// T0 is the smallest over the waves of each wave's ceil(c/w)-th largest
// thread maximum (a thread's maximum over its tiles; w = the waves whose
// lanes hold slots; every lane counts, through lane reads, the wave's maxima
// that reach its own).  The tiles reaching T0 are counted: when there are at
// least c of them (and T0 is a real score), every one of the c best scores
// is >= T0 and lies in a tile whose maximum reaches T0, and so does every
// score tied with the c-th best.  Those tiles (a small multiple of c) are
// listed, their scores >= T0 collected in LDS in one pass of 16-byte
// quarters, and ranked by counting: the first c are the candidates.
//
// Fallback, when fewer than c or more than TC_LIST tiles reach T0, or more
// than TC_CMAX scores are >= T0 (many equal scores): T, the c-th largest
// tile maximum, by
// a radix select over all tile maxima (four 8-bit passes, histogram in LDS);
// the scores above T (fewer than c tiles hold them) ranked; the remaining
// places filled with the lowest-id scores equal to T by an ordered scan of
// the tiles reaching T (sorted by tile id), or of the whole row when more
// than TC_EQT tiles reach T.
__global__ __launch_bounds__(TC_THREADS) void topc_tiles_kernel(const float* __restrict__ scores,
                                                                const float2* __restrict__ part, TileSlots sl,
                                                                int V, int c, int32_t* __restrict__ cand) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* x = scores + (size_t)row * V;
  const int ns = sl.count();
  const float2* p = part + (size_t)row * ns;
  int32_t* out = cand + (size_t)row * c;
  __shared__ unsigned hist[256];
  __shared__ unsigned wtot[TC_WAVES];
  __shared__ uint32_t sel_prefix;
  __shared__ int sel_need;
  __shared__ float2 cl[TC_CMAX + 8];
  __shared__ __attribute__((aligned(16))) int eqt[TC_EQT + 8];  // fallback: tiles reaching T
  __shared__ int eqs[TC_EQT];                                    // fallback: the same, by tile id
  __shared__ int slist[TC_LIST];                                 // slots reaching T0; fallback: tiles above T
  __shared__ int ngt, neqt, nlist;

  // every place starts as "no candidate" (-1): a row whose scores hold NaN
  // may leave places unfilled, and the gather below skips them
  for (int i = tid; i < c; i += TC_THREADS) out[i] = -1;
  // all loads issued before any is used (a load under a branch costs one
  // round trip each): slots past the end read the last slot and are dropped
  float mv[TC_TPT];
#pragma unroll
  for (int j = 0; j < TC_TPT; ++j) mv[j] = p[min(tid + TC_THREADS * j, ns - 1)].x;
  uint32_t key[TC_TPT];
#pragma unroll
  for (int j = 0; j < TC_TPT; ++j) key[j] = tid + TC_THREADS * j < ns ? fkey(mv[j]) : 0u;  // 0: below every float

  // ---- T0 and the slots reaching it
  uint32_t T0;
  {
    uint32_t mk = 0u;
#pragma unroll
    for (int j = 0; j < TC_TPT; ++j) mk = max(mk, key[j]);
    if (tid == 0) {
      nlist = 0;
      ngt = 0;
    }
    // waves whose lanes hold slots share the c tiles: ceil(c / nvw) each
    const int nvw = min(TC_WAVES, (min(ns, TC_THREADS) + 63) / 64);
    const int jw = (c + nvw - 1) / nvw;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) cnt += (uint32_t)__builtin_amdgcn_readlane((int)mk, i) >= mk ? 1 : 0;
    uint32_t tw = cnt >= jw ? mk : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tw = max(tw, (uint32_t)__shfl_xor((int)tw, o, 64));
    if (lane == 0) wtot[w] = tw;
    __syncthreads();
    // the smallest over the waves that have one (0: a wave with fewer than jw
    // slots, which must not pull T0 below every real key)
    T0 = 0xffffffffu;
    for (int i = 0; i < TC_WAVES; ++i)
      if (wtot[i] > 0u) T0 = min(T0, wtot[i]);
    // (the unrolled loop only compares and appends slot indices: the tile of
    // a slot, two integer divisions, is taken in a rolled loop below, which
    // keeps the kernel's code small)
#pragma unroll
    for (int j = 0; j < TC_TPT; ++j) {
      const int s = tid + TC_THREADS * j;
      if (s < ns && key[j] >= T0) {
        const int pos = atomicAdd(&nlist, 1);
        if (pos < TC_LIST) slist[pos] = s;
      }
    }
    __syncthreads();
  }
  const int n1 = nlist;
  // the fast path needs at least c real tiles reaching T0 (which also keeps
  // T0 above the key of -inf: no padding slot and no missing slot is listed)
  if (T0 > fkey(-INFINITY) && T0 != 0xffffffffu && n1 >= c && n1 <= TC_LIST) {
    // ---- the scores >= T0 of the listed tiles, one 16-byte quarter per task
    const float T0f = kfloat(T0);
    for (int e = tid; e < 4 * n1; e += TC_THREADS) {
      const int t = sl.tile(slist[e >> 2]), q = e & 3;
      if (t < 0) continue;  // a padding slot (T0 = -inf)
      const float4 f = *(const float4*)(x + t * 16 + 4 * q);
      const float v4[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v4[u] >= T0f) {
          const int pos = atomicAdd(&ngt, 1);
          if (pos < TC_CMAX) cl[pos] = make_float2(v4[u], __int_as_float(t * 16 + 4 * q + u));
        }
    }
    __syncthreads();
    const int C = ngt;
    if (C <= TC_CMAX) {
      const int C8 = (C + 7) & ~7;  // padded with (-inf, INT_MAX), which ranks last
      for (int i = C + tid; i < C8; i += TC_THREADS) cl[i] = make_float2(-INFINITY, __int_as_float(INT_MAX));
      __syncthreads();
      for (int i = tid; i < C; i += TC_THREADS) {
        const float2 me = cl[i];
        const int id = __float_as_int(me.y);
        int r = 0;
#pragma unroll 1
        for (int j0 = 0; j0 < C8; j0 += 8) {
          float2 o[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] = cl[j0 + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) r += better(o[u].x, __float_as_int(o[u].y), me.x, id) ? 1 : 0;
        }
        if (r < c) out[r] = id;
      }
      return;
    }
  }

  // ---- fallback (many equal scores): radix select of T, the c-th largest tile maximum
  uint32_t prefix = 0;
  int need = c;
#pragma unroll 1
  for (int pass = 3; pass >= 0; --pass) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const int shift = pass * 8;
#pragma unroll
    for (int j = 0; j < TC_TPT; ++j) {
      const int s = tid + TC_THREADS * j;
      if (s < ns && (pass == 3 || (key[j] >> (shift + 8)) == prefix)) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // descending bins: thread t < 256 holds bin 255 - t; inclusive scan
    const unsigned h = tid < 256 ? hist[255 - tid] : 0u;
    unsigned incl = wave_incl_scan(h, lane);
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    for (int i = 0; i < w; ++i) incl += wtot[i];
    if (tid < 256 && incl >= (unsigned)need && incl - h < (unsigned)need) {
      sel_prefix = (prefix << 8) | (uint32_t)(255 - tid);
      sel_need = need - (int)(incl - h);
    }
    __syncthreads();
    prefix = sel_prefix;
    need = sel_need;
    __syncthreads();
  }
  const uint32_t tkey = prefix;
  const float T = kfloat(tkey);

  // every tile reaching T (for the tie scan); the tiles above T (fewer than c)
  if (tid == 0) {
    ngt = 0;
    neqt = 0;
    nlist = 0;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TC_TPT; ++j) {
    const int s = tid + TC_THREADS * j;
    if (s < ns && key[j] >= tkey) {
      const int pos = atomicAdd(&neqt, 1);
      if (pos < TC_EQT) eqt[pos] = key[j] > tkey ? -1 - s : s;  // slots above T marked negative
    }
  }
  __syncthreads();
  const int NEs = neqt;
  for (int i = tid; i < min(NEs, TC_EQT); i += TC_THREADS) {
    const int e = eqt[i], sl_i = e < 0 ? -1 - e : e;
    const int t = sl.tile(sl_i);
    eqt[i] = t;  // -1 for a padding slot (only when T is -inf)
    if (e < 0 && t >= 0) slist[atomicAdd(&nlist, 1)] = t;  // fewer than c <= TC_LIST
  }
  __syncthreads();
  const int NG = nlist;
  for (int e = tid; e < 4 * NG; e += TC_THREADS) {
    const int t = slist[e >> 2], q = e & 3;
    const float4 f = *(const float4*)(x + t * 16 + 4 * q);
    const float v4[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (v4[u] > T) {
        const int pos = atomicAdd(&ngt, 1);
        if (pos < TC_CMAX) cl[pos] = make_float2(v4[u], __int_as_float(t * 16 + 4 * q + u));
      }
  }
  __syncthreads();
  const int G = min(ngt, TC_CMAX);  // never clipped: fewer than c tiles of 16 scores
  const int G8 = (G + 7) & ~7;
  for (int i = G + tid; i < G8; i += TC_THREADS) cl[i] = make_float2(-INFINITY, __int_as_float(INT_MAX));
  __syncthreads();
  for (int i = tid; i < G; i += TC_THREADS) {
    const float2 me = cl[i];
    const int id = __float_as_int(me.y);
    int r = 0;
#pragma unroll 1
    for (int j0 = 0; j0 < G8; j0 += 8) {
      float2 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = cl[j0 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += better(o[u].x, __float_as_int(o[u].y), me.x, id) ? 1 : 0;
    }
    if (r < c) out[r] = id;
  }
  if (G >= c) return;

  // the lowest-id scores equal to T fill the remaining c - G places
  const int need_eq = c - G;
  const int NE = neqt;
  const bool by_tiles = NE <= TC_EQT && T > -INFINITY;  // (T = -inf: padding slots listed; scan the row)
  if (by_tiles) {
    const int NE8 = (NE + 7) & ~7;  // padded with INT_MAX, larger than every tile id
    for (int i = NE + tid; i < NE8; i += TC_THREADS) eqt[i] = INT_MAX;
    __syncthreads();
    for (int i = tid; i < NE; i += TC_THREADS) {  // tile ids are distinct: rank = count of smaller ids
      const int me = eqt[i];
      int r = 0;
#pragma unroll 1
      for (int j0 = 0; j0 < NE8; j0 += 8) {
        const int4 a = *(const int4*)(eqt + j0), b = *(const int4*)(eqt + j0 + 4);
        r += (a.x < me) + (a.y < me) + (a.z < me) + (a.w < me) + (b.x < me) + (b.y < me) + (b.z < me) + (b.w < me);
      }
      eqs[r] = me;
    }
    __syncthreads();
  }
  const int n_elem = by_tiles ? NE * 16 : V;
  int base = 0;
  for (int e0 = 0; e0 < n_elem && base < need_eq; e0 += TC_THREADS) {
    const int e = e0 + tid;
    int id = -1;
    if (e < n_elem) id = by_tiles ? eqs[e >> 4] * 16 + (e & 15) : e;
    const unsigned f = (id >= 0 && x[id] == T) ? 1u : 0u;
    unsigned incl = wave_incl_scan(f, lane);
    __syncthreads();  // the previous chunk's reads of wtot are done
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    unsigned wb = 0, tot = 0;
    for (int i = 0; i < TC_WAVES; ++i) {
      if (i < w) wb += wtot[i];
      tot += wtot[i];
    }
    const int pos = base + (int)(wb + incl - f);
    if (f && pos < need_eq) out[G + pos] = id;
    base += (int)tot;
  }
}

// Stage-1 scores of up to 16 rows, s[n][v] = sum_k A[v][k] z[n][k], with A
// [V][rank] in packed fragment order and z [R][rank] bf16 row-major.  The
// rank is short (64..256), so a workgroup-tile GEMM would spend most of its
// time reducing partial tiles across waves; here each wave owns SC_TPW
// 16-row tiles over the whole rank: z's fragments stay in registers, the
// next tile's A fragments load while the current tile's MFMAs run, and the
// scores and each tile's per-row maximum leave straight from the
// accumulators (the pair's second half, a sum of exponentials, is not
// needed for the selection and is written as 0).
constexpr int SC_WAVES = 4, SC_TPW = 4;  // 16 tiles per workgroup

template <int NCH>
__global__ __launch_bounds__(SC_WAVES * 64) void lowrank_scores_kernel(const bf16* __restrict__ A,
                                                                       const bf16* __restrict__ z, int R, int nt16,
                                                                       int V, float* __restrict__ out,
                                                                       float2* __restrict__ part, TileSlots sl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, q4 = lane >> 4;
  U4 xf[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (m < R) xf[c].u = *(const uint4*)(z + (size_t)m * (NCH * 32) + 32 * c + 8 * q4);
    else xf[c].u = make_uint4(0u, 0u, 0u, 0u);
  }
  const int t0 = (blockIdx.x * SC_WAVES + wave) * SC_TPW;
  U4 af[2][NCH];
  auto load = [&](int t, U4 (&dst)[NCH]) __attribute__((always_inline)) {
    const bf16* src = A + ((size_t)min(t, nt16 - 1) * NCH * 64 + lane) * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c) dst[c].u = ld_stream(src + c * 512);
  };
  load(t0, af[0]);
#pragma unroll
  for (int i = 0; i < SC_TPW; ++i) {
    const int t = t0 + i;
    if (i + 1 < SC_TPW) load(t + 1, af[(i + 1) & 1]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i & 1][c].v, xf[c].v, acc, 0, 0, 0);
    if (t >= nt16) continue;  // uniform over the wave
    // lane l holds weight rows 4(l/16)+e of z row l%16
    if (m < R) *(float4*)(out + (size_t)m * V + t * 16 + 4 * q4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (q4 == 0 && m < R) part[(size_t)m * sl.count() + sl.slot(t)] = make_float2(mx, 0.f);
    if (t == nt16 - 1) {  // slots no tile fills: -inf
      const int npad = sl.count() - nt16;
      for (int e = lane; e < npad * R; e += 64) {
        const int j = e / R, r = e - j * R;
        part[(size_t)r * sl.count() + sl.slot(nt16 + j)] = make_float2(-INFINITY, 0.f);
      }
    }
  }
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
    acc = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), acc);
  }
  return acc;
}

// Exact logits of the candidates: wave (row, j) takes candidate j of the row
// and forms W_lm[id] . y in fp32.  Packed W_lm (MFMA fragment order): row id
// lives in 16-row tile id/16 at lane id%16 of each 32-wide k chunk, the four
// 16-byte pieces of a chunk 256 bytes apart; row-major: one contiguous row.
template <bool PACKED>
__global__ __launch_bounds__(256) void cand_logits_kernel(const bf16* __restrict__ W, const bf16* __restrict__ y,
                                                          int d, int V, int c, const int32_t* __restrict__ cand,
                                                          float* __restrict__ out) {
  const int row = blockIdx.x, j = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (j >= c) return;  // whole waves only
  const int id = cand[(size_t)row * c + j];
  if ((unsigned)id >= (unsigned)V) {  // an unfilled place: no load
    if (lane == 0) out[(size_t)row * c + j] = -INFINITY;
    return;
  }
  const bf16* yr = y + (size_t)row * d;
  float acc = 0.f;
  const int nch = d / 32;
  if (PACKED) {
    const size_t t = (size_t)(id >> 4);
    const int m = id & 15;
    for (int cc = lane; cc < nch; cc += 64) {
      const uint4* blk = (const uint4*)W + (t * nch + cc) * 64;
      uint4 wv[4], yv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wv[q] = blk[m + 16 * q];
        yv[q] = *(const uint4*)(yr + 32 * cc + 8 * q);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = dot8(wv[q], yv[q], acc);
    }
  } else {
    const bf16* wr = W + (size_t)id * d;
    for (int e = lane * 8; e < d; e += 512) acc = dot8(*(const uint4*)(wr + e), *(const uint4*)(yr + e), acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) out[(size_t)row * c + j] = acc;
}

// Top-k of the candidates by (exact logit desc, id asc) and lp = logit -
// logsumexp over the c candidates: one workgroup per row, thread i holds
// candidate i (c <= 256).
__global__ __launch_bounds__(256) void cand_topk_kernel(const int32_t* __restrict__ cand,
                                                        const float* __restrict__ cl, int c, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ lp) {
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // an unfilled candidate place (-1, only for rows whose scores hold NaN)
  // ranks last, and is emitted as token 0 if it has to be
  const int raw = tid < c ? cand[(size_t)row * c + tid] : -1;
  const float v = raw >= 0 ? cl[(size_t)row * c + tid] : -INFINITY;
  const int id = raw >= 0 ? raw : INT_MAX;
  sv[tid] = v;
  si[tid] = id;
  float m = wave_max(v);
  if (lane == 0) red[w] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float s = wave_sum(tid < c ? expf(v - M) : 0.f);
  if (lane == 0) red[w] = s;
  __syncthreads();
  const float L = M + logf((red[0] + red[1]) + (red[2] + red[3]));
  if (tid < c) {
    int r = 0;
    const int c8 = (c + 7) & ~7;  // places c..c8-1 hold (-inf, INT_MAX): they rank last
    for (int j0 = 0; j0 < c8; j0 += 8) {
      float ov[8];
      int oi[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ov[u] = sv[j0 + u];
        oi[u] = si[j0 + u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) r += better(ov[u], oi[u], v, id) ? 1 : 0;
    }
    if (r < k) {
      ids[(size_t)row * k + r] = id == INT_MAX ? 0 : id;
      lp[(size_t)row * k + r] = v - L;
    }
  }
}

}  // namespace

int lowrank_scores_tpw() { return SC_WAVES * SC_TPW; }

hipError_t launch_lowrank_scores(const void* A, const void* z, int rows, int rank, int V, float* scores,
                                 float2* part, hipStream_t st) {
  const int nt16 = V / 16;
  const TileSlots sl = tile_slots(nt16, SC_WAVES * SC_TPW);
  const int grid = (nt16 + SC_WAVES * SC_TPW - 1) / (SC_WAVES * SC_TPW);
  if (rows > 16) return hipErrorInvalidValue;
  switch (rank) {
    case 64:
      launch_timed(EAGLE3_KC_LR_SCORES, lowrank_scores_kernel<2>, dim3(grid), dim3(SC_WAVES * 64), 0, st,
                   (const bf16*)A, (const bf16*)z, rows, nt16, V, scores, part, sl);
      break;
    case 128:
      launch_timed(EAGLE3_KC_LR_SCORES, lowrank_scores_kernel<4>, dim3(grid), dim3(SC_WAVES * 64), 0, st,
                   (const bf16*)A, (const bf16*)z, rows, nt16, V, scores, part, sl);
      break;
    case 256:
      launch_timed(EAGLE3_KC_LR_SCORES, lowrank_scores_kernel<8>, dim3(grid), dim3(SC_WAVES * 64), 0, st,
                   (const bf16*)A, (const bf16*)z, rows, nt16, V, scores, part, sl);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lowrank_select(const float* scores, const float2* part, int tiles_per_wg, int rows, int V, int c,
                                 int32_t* cand, hipStream_t st) {
  const TileSlots sl = tile_slots(V / 16, tiles_per_wg);
  if (rows > 64 || c > LOWRANK_MAX_CAND || c > V / 16 || sl.count() > TC_THREADS * TC_TPT)
    return hipErrorInvalidValue;
  topc_tiles_kernel<<<rows, TC_THREADS, 0, st>>>(scores, part, sl, V, c, cand);
  return hipGetLastError();
}

hipError_t launch_lowrank_exact(const void* W_lm, bool packed, const void* y, int rows, int d, int V, int c, int k,
                                const int32_t* cand, float* cand_logits, int32_t* ids, float* lp, hipStream_t st) {
  if (c > LOWRANK_MAX_CAND || k > c || d % 32 != 0) return hipErrorInvalidValue;
  dim3 g(rows, (c + 3) / 4);
  if (packed)
    cand_logits_kernel<true><<<g, 256, 0, st>>>((const bf16*)W_lm, (const bf16*)y, d, V, c, cand, cand_logits);
  else
    cand_logits_kernel<false><<<g, 256, 0, st>>>((const bf16*)W_lm, (const bf16*)y, d, V, c, cand, cand_logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  cand_topk_kernel<<<rows, 256, 0, st>>>(cand, cand_logits, c, k, ids, lp);
  return hipGetLastError();
}

}  // namespace e3
