// Training-time-test forward ("EAGLE-3 精读" §2 Training-Time Test and §5
// 正确性、复现与风险): R self-fed rollout steps of the drafter over B
// sequences of S tokens, evaluated as R passes over all M = B*S rows.
//
// Step j (1..R) on row (b, i):
//   input state  s = g_i (j = 1) or h2 of (j-1, i)
//   input token  t = x_i (j = 1) or the argmax of (j-1, i) (or a forced token)
//   position     i + j - 1
//   attention    step-1 keys i' <= i and the chain keys (j', i), 2 <= j' <= j
//   target       x_{i+j} when i + j <= S-1; CE = logsumexp(logits) - logit[target]
//
// Kernels: one tiled MFMA GEMM (bigemm.hpp) per projection with fused
// epilogues (bf16 store, RoPE + KV scatter, residual, SwiGLU, and the LM head's
// per-128-column log-sum-exp / argmax / target pick-up, so the [M x V] logits
// never reach memory), an MFMA flash-attention kernel for the rollout mask,
// and row kernels for the RMSNorms and the CE merge.
#include <math.h>

#include "bigemm.hpp"
#include "timing.hpp"
#include "ttt.hpp"

namespace e3 {

namespace {

struct Carve {
  size_t off = 0;
  unsigned char* base = nullptr;
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

struct TLayout {
  float* hs;     // [M][d] state stream s -> h1 -> h2 (fp32)
  bf16* x;       // [M][2d] decoder input; reused as u [M][d] and y [M][d]
  bf16* a;       // [M][hq*hd] attention output
  bf16* z;       // [M][F] silu(gate) * up
  bf16* q;       // [M][hq][hd]
  bf16* k1;      // [M][hkv][hd] step-1 keys
  bf16* v1t;     // [B][hkv][hd][S] step-1 values, transposed
  bf16* kc;      // [R-1][M][hkv][hd] chain keys of steps 2..R
  bf16* vc;      // [R-1][M][hkv][hd] chain values
  float4* part;  // [M][nblk] LM-head partials per 64 columns {max, sum exp, argmax id, 0}
  float* lab;    // [M] target logit
  int32_t* tok;  // [M] input tokens of the next step
  float2* rope;  // [S+R][hd/2] (cos, sin)
  size_t bytes;
};

inline int ce_blocks(int V) { return (V / 16 + BG_NJ - 1) / BG_NJ; }

TLayout layout_of(const eagle3_dims& dm, int B, int S, int R, void* base) {
  Carve c;
  c.base = (unsigned char*)base;
  const size_t M = (size_t)B * S;
  const size_t d = dm.d, qd = (size_t)dm.n_q_heads * dm.head_dim, kvd = (size_t)dm.n_kv_heads * dm.head_dim;
  TLayout L;
  L.hs = (float*)c.take(M * d * 4);
  L.x = (bf16*)c.take(M * 2 * d * 2);
  L.a = (bf16*)c.take(M * qd * 2);
  L.z = (bf16*)c.take(M * dm.ffn * 2);
  L.q = (bf16*)c.take(M * qd * 2);
  L.k1 = (bf16*)c.take(M * kvd * 2);
  L.v1t = (bf16*)c.take(M * kvd * 2);
  const size_t nch = R > 1 ? R - 1 : 1;
  L.kc = (bf16*)c.take(nch * M * kvd * 2);
  L.vc = (bf16*)c.take(nch * M * kvd * 2);
  L.part = (float4*)c.take(M * ce_blocks(dm.vocab) * sizeof(float4));
  L.lab = (float*)c.take(M * 4);
  L.tok = (int32_t*)c.take(M * 4);
  L.rope = (float2*)c.take((size_t)(S + R) * (dm.head_dim / 2) * sizeof(float2));
  L.bytes = c.off;
  return L;
}

// ------------------------------------------------------------------ small kernels
// RoPE table: angle p * theta^(-2i/hd) in double, stored as float (cos, sin),
// the same rounding as the draft path's QKV epilogue.
__global__ void rope_table_kernel(float2* tab, int npos, int hd, float theta) {
  const int half = hd >> 1;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= npos * half) return;
  const int p = e / half, i = e - p * half;
  const double inv = pow((double)theta, -(2.0 * i) / (double)hd);
  const double ang = (double)p * inv;
  tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

constexpr int TR = 512;  // row-kernel threads; 8 elements per thread per pass, d <= 8192

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

// x = [rms(emb[t]) * norm_e ; rms(s) * norm_s] (bf16)
__global__ __launch_bounds__(TR) void ttt_prologue_kernel(const bf16* __restrict__ emb, const int32_t* __restrict__ tok,
                                                          const float* __restrict__ hs, int d,
                                                          const float* __restrict__ ge, const float* __restrict__ gs,
                                                          float eps, bf16* __restrict__ x) {
  __shared__ float red[TR / 64];
  const size_t r = blockIdx.x;
  const bf16* e = emb + (size_t)tok[r] * d;
  const float* s = hs + r * d;
  float ev[2][8], sv[2][8];
  float se = 0.f, ss = 0.f;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (threadIdx.x + TR * it) * 8;
    if (i < d) {
      unpack8(*(const uint4*)(e + i), ev[it]);
      const float4 s0 = *(const float4*)(s + i), s1 = *(const float4*)(s + i + 4);
      sv[it][0] = s0.x, sv[it][1] = s0.y, sv[it][2] = s0.z, sv[it][3] = s0.w;
      sv[it][4] = s1.x, sv[it][5] = s1.y, sv[it][6] = s1.z, sv[it][7] = s1.w;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) ev[it][c] = sv[it][c] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      se = fmaf(ev[it][c], ev[it][c], se);
      ss = fmaf(sv[it][c], sv[it][c], ss);
    }
  }
  se = block_sum(se, red);
  ss = block_sum(ss, red);
  const float ie = (float)(1.0 / sqrt((double)se / d + (double)eps));
  const float is = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  bf16* xr = x + r * 2 * d;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (threadIdx.x + TR * it) * 8;
    if (i < d) {
      float o1[8], o2[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        o1[c] = ev[it][c] * ie * ge[i + c];
        o2[c] = sv[it][c] * is * gs[i + c];
      }
      *(uint4*)(xr + i) = pack8(o1);
      *(uint4*)(xr + d + i) = pack8(o2);
    }
  }
}

// y = rms(h) * gain (bf16, [M][d])
__global__ __launch_bounds__(TR) void ttt_norm_kernel(const float* __restrict__ hs, int d,
                                                      const float* __restrict__ gain, float eps,
                                                      bf16* __restrict__ y) {
  __shared__ float red[TR / 64];
  const size_t r = blockIdx.x;
  const float* s = hs + r * d;
  float v[2][8];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (threadIdx.x + TR * it) * 8;
    if (i < d) {
      const float4 s0 = *(const float4*)(s + i), s1 = *(const float4*)(s + i + 4);
      v[it][0] = s0.x, v[it][1] = s0.y, v[it][2] = s0.z, v[it][3] = s0.w;
      v[it][4] = s1.x, v[it][5] = s1.y, v[it][6] = s1.z, v[it][7] = s1.w;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[it][c] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(v[it][c], v[it][c], ss);
  }
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (threadIdx.x + TR * it) * 8;
    if (i < d) {
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = v[it][c] * inv * gain[i + c];
      *(uint4*)(y + r * d + i) = pack8(o);
    }
  }
}

// ------------------------------------------------------------------ GEMM epilogues
// QKV on MAP_PAIR_HEAD tiles (slots m, m+8 = RoPE pair (p, p + hd/2) of one
// head, p = 8t + m): RoPE at position (row % S) + pos_off on q and k, then
// bf16 stores.  Values go row-major [M][hkv][hd], or, when vt is set,
// transposed [B][hkv][hd][S] (the attention kernel's operand layout).
struct TEpiQKV {
  bf16* q;
  bf16* k;
  bf16* v;
  int vt;
  const float2* rope;
  int hq, hkv, hd, S, pos_off;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15, tph = hd >> 4, half = hd >> 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row0 = rowbase + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < BG_NJ; ++j) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = xor8(acc[i][j][e]);
        const int col16 = colbase16 + j;
        if (col16 >= nt16 || m >= 8 || row0 >= M) continue;
        const int head = col16 / tph, t = col16 - head * tph, p = t * 8 + m;
        float av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          av[e] = acc[i][j][e];
          bv[e] = o[e];
        }
        if (head < hq + hkv) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 cs = rope[(size_t)((row0 + e) % S + pos_off) * half + p];
            const float a2 = av[e] * cs.x - bv[e] * cs.y, b2 = bv[e] * cs.x + av[e] * cs.y;
            av[e] = a2;
            bv[e] = b2;
          }
        }
        if (head < hq || head < hq + hkv || !vt) {
          bf16* base;
          int H, hh;
          if (head < hq) {
            base = q, H = hq, hh = head;
          } else if (head < hq + hkv) {
            base = k, H = hkv, hh = head - hq;
          } else {
            base = v, H = hkv, hh = head - hq - hkv;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const size_t off = ((size_t)(row0 + e) * H + hh) * hd;
            base[off + p] = f2bf(av[e]);
            base[off + p + half] = f2bf(bv[e]);
          }
        } else {
          const int g = head - hq - hkv, b = row0 / S, i0 = row0 - b * S;
          bf16* base = v + ((size_t)(b * hkv + g) * hd) * S + i0;
          const uint2 lo = make_uint2((uint32_t)f2bf(av[0]) | ((uint32_t)f2bf(av[1]) << 16),
                                      (uint32_t)f2bf(av[2]) | ((uint32_t)f2bf(av[3]) << 16));
          const uint2 hi = make_uint2((uint32_t)f2bf(bv[0]) | ((uint32_t)f2bf(bv[1]) << 16),
                                      (uint32_t)f2bf(bv[2]) | ((uint32_t)f2bf(bv[3]) << 16));
          *(uint2*)(base + (size_t)p * S) = lo;
          *(uint2*)(base + (size_t)(p + half) * S) = hi;
        }
      }
    }
  }
};

// LM head with the cross entropy folded in: for every row and each 64-column
// block (one wave's tile width) write {max, sum exp(x - max), argmax id};
// the lane that owns a row's target column writes the target logit.
struct TEpiCE {
  float4* part;
  float* lab;
  const int32_t* tokens;  // [M], targets are tokens[row + step] inside the sequence
  int S, step, nblk;
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15, blk = colbase16 / BG_NJ;
    if (blk >= nblk) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rowbase + 16 * i + 4 * (lane >> 4) + e;
        int target = -1;
        if (row < M && (row % S) + step <= S - 1) target = tokens[row + step];
        float mx = -INFINITY;
        int id = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j) {
          const int col16 = colbase16 + j, n = col16 * 16 + m;
          if (col16 < nt16) {
            const float xv = acc[i][j][e];
            if (xv > mx) {
              mx = xv;
              id = n;
            }
            if (n == target) lab[row] = xv;
          }
        }
        row16_argmax(mx, id);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j)
          if (colbase16 + j < nt16) s += __expf(acc[i][j][e] - mx);
        s = row16_sum(s);
        if (m == 0 && row < M) part[(size_t)row * nblk + blk] = make_float4(mx, s, __int_as_float(id), 0.f);
      }
    }
  }
};

// Per row: merge the partials into logsumexp and argmax; CE, prediction and
// the next step's input token.
__global__ __launch_bounds__(256) void ce_merge_kernel(const float4* __restrict__ part, int nblk,
                                                       const float* __restrict__ lab, const int32_t* __restrict__ forced,
                                                       int S, int R, int step, int32_t* __restrict__ pred,
                                                       float* __restrict__ ce, int32_t* __restrict__ tok_next) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  __shared__ double ws[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float4* p = part + (size_t)row * nblk;
  float4 loc[16];  // nblk <= 4096 (vocab <= 262144 in 64-column blocks)
  int nl = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int k = tid + 256 * c;
    loc[c] = k < nblk ? p[k] : make_float4(-INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f);
    if (k < nblk) nl = c + 1;
    const int id = __float_as_int(loc[c].z);
    if (better(loc[c].x, id, bv, bi)) {
      bv = loc[c].x;
      bi = id;
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    wv[w] = bv;
    wi[w] = bi;
  }
  __syncthreads();
  float gv = wv[0];
  int gi = wi[0];
  for (int c = 1; c < 4; ++c)
    if (better(wv[c], wi[c], gv, gi)) {
      gv = wv[c];
      gi = wi[c];
    }
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (c < nl) s += (double)loc[c].y * exp((double)loc[c].x - (double)gv);
  s = wave_sum_d(s);
  if (lane == 0) ws[w] = s;
  __syncthreads();
  if (tid == 0) {
    const double tot = (ws[0] + ws[1]) + (ws[2] + ws[3]);
    const double lse = (double)gv + log(tot);
    const int b = row / S, i = row - b * S;
    const size_t o = ((size_t)b * R + (step - 1)) * S + i;
    pred[o] = gi;
    ce[o] = i + step <= S - 1 ? (float)(lse - (double)lab[row]) : 0.f;
    if (tok_next) tok_next[row] = forced ? forced[((size_t)b * (R - 1) + (step - 1)) * S + i] : gi;
  }
}

// loss = sum of ce / count, fixed summation order.
__global__ __launch_bounds__(1024) void ttt_loss_kernel(const float* __restrict__ ce, size_t n, double count,
                                                        float* __restrict__ loss) {
  __shared__ double red[16];
  double s = 0.0;
  for (size_t k = threadIdx.x; k < n; k += 1024) s += ce[k];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int c = 0; c < 16; ++c) t += red[c];
    loss[0] = count > 0 ? (float)(t / count) : 0.f;
  }
}

// ------------------------------------------------------------------ attention
// Rollout-mask attention.  Block (query block of 32 positions, group of
// `wpb` query heads that share one kv head, sequence b); wave w takes query
// head blockIdx.y * wpb + w.  Scores are computed
// transposed, S^T = K Q^T, so that the probabilities come out of the MFMA in
// the B-operand layout of O^T = V^T P^T; P is split into bf16 hi + lo parts
// (two MFMAs) so that P.V keeps about 16 bits of the probabilities.  Causal
// blocks of 64 step-1 keys use online softmax; afterwards each query folds
// in its own chain keys (j', i) with plain FMAs.
template <int HD>
__global__ __launch_bounds__(256) void ttt_attn_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K1,
                                                        const bf16* __restrict__ V1T, const bf16* __restrict__ KC,
                                                        const bf16* __restrict__ VC, int nchain, size_t chain_stride,
                                                        bf16* __restrict__ out, int S, int hq, int hkv, float scale) {
  constexpr int NC = HD / 32, NT = HD / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nqb = S / 32;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
  const int h = blockIdx.y * (int)(blockDim.x >> 6) + w, b = blockIdx.z;
  const int g = h / (hq / hkv);
  const int i0 = qb * 32;
  const int ml = lane & 15, q4 = lane >> 4;
  const size_t kstride = (size_t)hkv * HD;  // between consecutive positions of K1
  const bf16* kbase = K1 + (size_t)b * S * kstride + (size_t)g * HD;
  const bf16* vbase = V1T + (size_t)(b * hkv + g) * HD * S;

  U4 qf[2][NC];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = i0 + 16 * nt + ml;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[nt][c].u = *(const uint4*)(Q + ((size_t)(b * S + i) * hq + h) * HD + 32 * c + 8 * q4);
  }
  f32x4 o[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  const int nkb = (i0 + 32 + 63) / 64;
  for (int kb = 0; kb < nkb; ++kb) {
    f32x4 st[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) st[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      U4 kf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        kf[mt].u = *(const uint4*)(kbase + (size_t)(kb * 64 + 16 * mt + ml) * kstride + 32 * c + 8 * q4);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          st[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt].v, qf[nt][c].v, st[mt][nt], 0, 0, 0);
    }
    const bool diag = kb * 64 + 63 > i0;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = i0 + 16 * nt + ml;
      float bm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = st[mt][nt][e] * scale;
          if (diag && kb * 64 + 16 * mt + 4 * q4 + e > qi) s = -INFINITY;
          st[mt][nt][e] = s;
          bm = fmaxf(bm, s);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mnew = fmaxf(mrun[nt], bm);
      const float alpha = __expf(mrun[nt] - mnew);
      mrun[nt] = mnew;
      lsum[nt] *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t][nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = __expf(st[mt][nt][e] - mnew);
          st[mt][nt][e] = pv;
          lsum[nt] += pv;
        }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // B operand P^T: k-slots 8 q4 + e <- key 32kc + 4 q4 + e, slots 8 q4 + 4 + e <- key 32kc + 16 + 4 q4 + e
      U4 phi[2], plo[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const float p0 = st[2 * kc + hh][nt][2 * e2], p1 = st[2 * kc + hh][nt][2 * e2 + 1];
            const bf16 h0 = f2bf(p0), h1 = f2bf(p1);
            const bf16 l0 = f2bf(p0 - bf2f(h0)), l1 = f2bf(p1 - bf2f(h1));
            hw[2 * hh + e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[2 * hh + e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
          }
        }
        phi[nt].u = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        plo[nt].u = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16* vp = vbase + (size_t)(16 * t + ml) * S + kb * 64 + 32 * kc + 4 * q4;
        const uint2 v0 = *(const uint2*)vp, v1 = *(const uint2*)(vp + 16);
        U4 vf;
        vf.u = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, phi[nt].v, o[t][nt], 0, 0, 0);
          o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, plo[nt].v, o[t][nt], 0, 0, 0);
        }
      }
    }
  }
  // chain keys (j', i), j' = 2..j: lane holds dims 16t + 4 q4 + e of its query
  for (int c = 0; c < nchain; ++c) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const size_t row = (size_t)b * S + i0 + 16 * nt + ml;
      const bf16* qp = Q + (row * hq + h) * HD + 4 * q4;
      const bf16* kp = KC + c * chain_stride + (row * hkv + g) * HD + 4 * q4;
      const bf16* vp = VC + c * chain_stride + (row * hkv + g) * HD + 4 * q4;
      float dot = 0.f;
      float vv[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint2 qa = *(const uint2*)(qp + 16 * t), ka = *(const uint2*)(kp + 16 * t), va = *(const uint2*)(vp + 16 * t);
        const uint32_t qw[2] = {qa.x, qa.y}, kw[2] = {ka.x, ka.y}, vw[2] = {va.x, va.y};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          dot = fmaf(__uint_as_float(qw[u] << 16), __uint_as_float(kw[u] << 16), dot);
          dot = fmaf(__uint_as_float(qw[u] & 0xffff0000u), __uint_as_float(kw[u] & 0xffff0000u), dot);
          vv[t][2 * u] = __uint_as_float(vw[u] << 16);
          vv[t][2 * u + 1] = __uint_as_float(vw[u] & 0xffff0000u);
        }
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      const float s = dot * scale;
      const float mnew = fmaxf(mrun[nt], s);
      const float alpha = __expf(mrun[nt] - mnew), pv = __expf(s - mnew);
      mrun[nt] = mnew;
      lsum[nt] = lsum[nt] * alpha + (q4 == 0 ? pv : 0.f);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[t][nt][e] = fmaf(pv, vv[t][e], o[t][nt][e] * alpha);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float L = lsum[nt];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const float inv = 1.f / L;
    const size_t row = (size_t)b * S + i0 + 16 * nt + ml;
    bf16* op = out + (row * hq + h) * HD + 4 * q4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 r = o[t][nt] * inv;
      *(uint2*)(op + 16 * t) = make_uint2((uint32_t)f2bf(r[0]) | ((uint32_t)f2bf(r[1]) << 16),
                                          (uint32_t)f2bf(r[2]) | ((uint32_t)f2bf(r[3]) << 16));
    }
  }
}

template <class Epi>
hipError_t bg_launch(const bf16* A, int lda, int M, const void* W, bool packed, int N, int K, RowMap map, Epi epi,
                     hipStream_t st) {
  const int grid = bg_grid(M, N);
  if (packed)
    big_gemm_kernel<true, Epi><<<grid, BG_THREADS, 0, st>>>(A, lda, M, (const bf16*)W, N, K, map, epi);
  else
    big_gemm_kernel<false, Epi><<<grid, BG_THREADS, 0, st>>>(A, lda, M, (const bf16*)W, N, K, map, epi);
  return hipGetLastError();
}

}  // namespace

size_t ttt_ws_bytes(const eagle3_dims& dm, int B, int S, int R) { return layout_of(dm, B, S, R, nullptr).bytes; }

int ttt_forward(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, const int32_t* tokens, int B, int S,
                int R, const int32_t* forced, int32_t* pred, float* ce, float* loss, void* wsp, hipStream_t st) {
  const int d = dm.d, hq = dm.n_q_heads, hkv = dm.n_kv_heads, hd = dm.head_dim, F = dm.ffn, V = dm.vocab;
  const int qd = hq * hd, kvd = hkv * hd;
  if (dm.dtype != EAGLE3_BF16 || (hd != 64 && hd != 128) || S % 64 != 0) return 1;
  if (d % 64 || F % 64 || qd % 64 || d > 8192 || hq % hkv) return 1;
  const int M = B * S;
  const TLayout L = layout_of(dm, B, S, R, wsp);
  const bool pk = w.layout == EAGLE3_LAYOUT_PACKED;
  const float eps = dm.rms_eps;
  const int nblk = ce_blocks(V);
  const RowMap plain{MAP_PLAIN, hd, F}, pair_head{MAP_PAIR_HEAD, hd, F}, pair_ffn{MAP_PAIR_FFN, hd, F};
  hipError_t e;
#define E3_CHECK(x) \
  if ((e = (x)) != hipSuccess) return -1;

  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    const int n = (S + R) * (hd / 2);
    rope_table_kernel<<<(n + 255) / 256, 256, 0, st>>>(L.rope, S + R, hd, dm.rope_theta);
    E3_CHECK(hipGetLastError());
  }
  {
    TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
    E3_CHECK(bg_launch((const bf16*)feats, 3 * d, M, w.fc, pk, d, 3 * d, plain, BEpiStoreF{L.hs, d, true}, st));
  }
  for (int j = 1; j <= R; ++j) {
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_prologue_kernel<<<M, TR, 0, st>>>((const bf16*)w.emb, j == 1 ? tokens : L.tok, L.hs, d, w.norm_e, w.norm_s,
                                            eps, L.x);
      E3_CHECK(hipGetLastError());
    }
    bf16* kdst = j == 1 ? L.k1 : L.kc + (size_t)(j - 2) * M * kvd;
    bf16* vdst = j == 1 ? L.v1t : L.vc + (size_t)(j - 2) * M * kvd;
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      TEpiQKV epi{L.q, kdst, vdst, j == 1, L.rope, hq, hkv, hd, S, j - 1};
      E3_CHECK(bg_launch(L.x, 2 * d, M, w.qkv, pk, qd + 2 * kvd, 2 * d, pair_head, epi, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_ATTN, st);
      const int gq = hq / hkv, wpb = gq % 4 == 0 ? 4 : (gq % 2 == 0 ? 2 : 1);
      const dim3 grid(S / 32, hq / wpb, B);
      const int threads = 64 * wpb;
      const float scale = (float)(1.0 / sqrt((double)hd));
      if (hd == 128)
        ttt_attn_kernel<128><<<grid, threads, 0, st>>>(L.q, L.k1, L.v1t, L.kc, L.vc, j - 1, (size_t)M * kvd, L.a, S,
                                                       hq, hkv, scale);
      else
        ttt_attn_kernel<64><<<grid, threads, 0, st>>>(L.q, L.k1, L.v1t, L.kc, L.vc, j - 1, (size_t)M * kvd, L.a, S,
                                                      hq, hkv, scale);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      E3_CHECK(bg_launch(L.a, qd, M, w.o, pk, d, qd, plain, BEpiResid{L.hs, d}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_norm_kernel<<<M, TR, 0, st>>>(L.hs, d, w.norm_ffn, eps, L.x);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      E3_CHECK(bg_launch(L.x, d, M, w.gate_up, pk, 2 * F, d, pair_ffn, BEpiSwiGLU{L.z, F}, st));
      E3_CHECK(bg_launch(L.z, F, M, w.down, pk, d, F, plain, BEpiResid{L.hs, d}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_norm_kernel<<<M, TR, 0, st>>>(L.hs, d, w.norm_out, eps, L.x);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_CE, st);
      E3_CHECK(bg_launch(L.x, d, M, w.lm, pk, V, d, plain, TEpiCE{L.part, L.lab, tokens, S, j, nblk}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ce_merge_kernel<<<M, 256, 0, st>>>(L.part, nblk, L.lab, forced, S, R, j, pred, ce, j < R ? L.tok : nullptr);
      E3_CHECK(hipGetLastError());
    }
  }
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    double count = 0;
    for (int j = 1; j <= R; ++j) count += (double)B * (S - j > 0 ? S - j : 0);
    ttt_loss_kernel<<<1, 1024, 0, st>>>(ce, (size_t)B * R * S, count, loss);
    E3_CHECK(hipGetLastError());
  }
#undef E3_CHECK
  return 0;
}

}  // namespace e3
