// Training-time-test backward ("EAGLE-3 精读" §1: target and LM head
// frozen, the light decoder trained; §2: CE at every rollout step under the
// training-time-test mask).  Gradients of the mean CE with respect to the
// fusion FC, the layer's four matrices and its four RMSNorm gains.
//
// The forward keeps every step's activations (ttt_forward with a TttSave:
// about 3.8 GB a step at the 8B shape with 16384 rows, cheap next to 288 GB
// of HBM) and already turns each step's logits into dy, the gradient at the
// LM head's input.  The backward then walks the steps in reverse, j = R..1,
// carrying the fp32 gradient of the state s_{j+1} = h2_j into step j:
//   dh2  = carry + rms'(h2, norm_out) dy
//   dz   = dh2 . W_down             -> SwiGLU backward -> d(gate, up)
//   du   = d(gate, up) . W_gate_up  -> dh1 = dh2 + rms'(h1, norm_ffn) du
//   da   = dh1 . W_o                -> attention backward -> dq, and the key/
//          value gradients of step-1 keys (every later step's queries see
//          them) and of the chain keys (j', i), completed by step j'
//   dx   = dqkv . W_qkv             -> carry = dh1 + rms'(s_j, norm_s) dx_s
// and finally dW_fc from the carry of step 1 (d g).  Data gradients run on
// the tiled MFMA GEMM with the weights transposed and packed once per call;
// every weight gradient is one GEMM over all R*B*S rows, its two operands
// transposed into fragment order (tokens along k) as the steps produce them.
// Gain gradients are column sums of gy * v * inv, reduced in a fixed order.
#include <math.h>

#include "bigemm.hpp"
#include "timing.hpp"
#include "ttt.hpp"
#include "ttt_common.hpp"

namespace e3 {

namespace {

// ------------------------------------------------------------------ transposes
// Logical row r of a weight stored in packed fragment order under `map`:
// (16-row tile, row slot).  Inverse of RowMap.
__device__ __forceinline__ void map_inv(const RowMap& mp, int n, int& t, int& m) {
  if (mp.kind == MAP_PLAIN) {
    t = n >> 4;
    m = n & 15;
  } else if (mp.kind == MAP_PAIR_HEAD) {
    const int half = mp.hd >> 1, h = n / mp.hd, i = n - h * mp.hd, hi = i >= half ? 1 : 0, ii = i - hi * half;
    t = h * (mp.hd >> 4) + (ii >> 3);
    m = (ii & 7) + 8 * hi;
  } else {
    const int up = n >= mp.ffn ? 1 : 0, f = n - up * mp.ffn;
    t = f >> 3;
    m = (f & 7) + 8 * up;
  }
}

// Sources of the transposes: address of X[r][k..k+8) (k a multiple of 8).
struct SrcRowMajor {
  const bf16* p;
  size_t ld;
  __device__ __forceinline__ const bf16* at(int r, int k) const { return p + (size_t)r * ld + k; }
};
struct SrcFrag {
  const bf16* p;
  int nkc;
  __device__ __forceinline__ const bf16* at(int r, int k) const { return p + frag_off(r, k, nkc); }
};
struct SrcPacked {
  const bf16* p;
  int nkc;
  RowMap map;
  __device__ __forceinline__ const bf16* at(int r, int k) const {
    int t, m;
    map_inv(map, r, t, m);
    return p + (((size_t)t * nkc + (k >> 5)) * 64 + m + 16 * ((k & 31) >> 3)) * 8;
  }
};

// out = X^T in fragment order: X [rows][K] (rows >= nrows read as zero), out
// [K][nkc_out * 32] with X's row r in column col0 + r.  One 64 x 64 tile per
// workgroup: 16-byte row reads into LDS, then each thread gathers 8 rows of
// one column into a 16-byte fragment slot (consecutive threads, consecutive
// slots).
constexpr int TP_PITCH = 64 + 8;  // LDS row pitch (elements)
template <class Src>
__global__ __launch_bounds__(256) void transpose_kernel(Src src, int nrows, bf16* __restrict__ out, int nkc_out,
                                                        int col0) {
  __shared__ __align__(16) bf16 t[64 * TP_PITCH];
  const int k0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int s = threadIdx.x; s < 512; s += 256) {
    const int r = s >> 3, kk = (s & 7) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + r < nrows) v = *(const uint4*)src.at(r0 + r, k0 + kk);
    *(uint4*)&t[r * TP_PITCH + kk] = v;
  }
  __syncthreads();
#pragma unroll
  for (int s = threadIdx.x; s < 512; s += 256) {
    const int f = s >> 6, l = s & 63, kt = f & 3, rc = f >> 2;
    const int kk = 16 * kt + (l & 15), rr = 32 * rc + 8 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(rr + 2 * e) * TP_PITCH + kk] | ((uint32_t)t[(rr + 2 * e + 1) * TP_PITCH + kk] << 16);
    *(uint4*)(out + frag_off(k0 + kk, col0 + r0 + rr, nkc_out)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <class Src>
hipError_t transpose(Src src, int nrows, int K, bf16* out, int nkc_out, int col0, hipStream_t st) {
  const dim3 grid(K / 64, (nrows + 63) / 64);
  transpose_kernel<Src><<<grid, 256, 0, st>>>(src, nrows, out, nkc_out, col0);
  return hipGetLastError();
}

// W [N][K] (row-major, or packed under map) -> W^T [K][np] packed, np = N
// rounded up to 64 (columns N..np-1 zero).
hipError_t transpose_weight(const void* W, bool packed, int N, int K, RowMap map, bf16* out, int np, hipStream_t st) {
  if (packed) return transpose(SrcPacked{(const bf16*)W, K / 32, map}, N, K, out, np / 32, 0, st);
  return transpose(SrcRowMajor{(const bf16*)W, (size_t)K}, N, K, out, np / 32, 0, st);
}

__global__ void fill_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ------------------------------------------------------------------ RMSNorm backward
// y = rms(v) * gain, inv = (mean(v^2) + eps)^-1/2 (the forward's rounding):
//   dv = inv * gain * gy - v * inv^3 / n * sum_k(gain_k gy_k v_k)
// Per 16-row block (the forward's row layout): carry = (add ? carry : 0) +
// dv in fp32, and optionally bf16(carry) in fragment order; inv_out[row] =
// inv.  With emb: inv_e[row] = inv of the embedding row of tok[row] (for
// the embedding norm's gain gradient).
__global__ __launch_bounds__(TR) void rms_bwd_kernel(const float* __restrict__ v, const float* __restrict__ gy,
                                                     int ldg, const float* __restrict__ gain, float eps, int d,
                                                     float* __restrict__ carry, int add, bf16* __restrict__ frag,
                                                     float* __restrict__ inv_out, const bf16* __restrict__ emb,
                                                     const int32_t* __restrict__ tok, float* __restrict__ inv_e) {
  __shared__ float inv_s[16], coef_s[16];
  const int mt = blockIdx.x, r0 = mt * 16, rr = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int row = r0 + rr;
  float ss = 0.f, dot = 0.f;
  for (int k = c * 8; k < d; k += 128) {
    const float* pv = v + (size_t)row * d + k;
    const float* pg = gy + (size_t)row * ldg + k;
    const float4 a0 = *(const float4*)pv, a1 = *(const float4*)(pv + 4);
    const float4 b0 = *(const float4*)pg, b1 = *(const float4*)(pg + 4);
    const float4 g0 = *(const float4*)(gain + k), g1 = *(const float4*)(gain + k + 4);
    const float vv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float gg[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const float ga[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss = fmaf(vv[i], vv[i], ss);
      dot = fmaf(ga[i] * gg[i], vv[i], dot);
    }
  }
  ss = row16_sum(ss);
  dot = row16_sum(dot);
  float se = 0.f;
  if (emb) se = row_ss(emb, (size_t)d, tok[row], d);
  if (c == 0) {
    const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
    inv_s[rr] = inv;
    coef_s[rr] = inv * inv * inv / (float)d * dot;
    inv_out[row] = inv;
    if (emb) inv_e[row] = (float)(1.0 / sqrt((double)se / d + (double)eps));
  }
  __syncthreads();
  const int nkc = d >> 5;
  for (int sl = threadIdx.x; sl < nkc * 64; sl += TR) {
    const int kc = sl >> 6, l = sl & 63, r = l & 15, k = kc * 32 + 8 * (l >> 4);
    const size_t o = (size_t)(r0 + r) * d + k;
    const float* pv = v + o;
    const float* pg = gy + (size_t)(r0 + r) * ldg + k;
    const float4 a0 = *(const float4*)pv, a1 = *(const float4*)(pv + 4);
    const float4 b0 = *(const float4*)pg, b1 = *(const float4*)(pg + 4);
    const float4 g0 = *(const float4*)(gain + k), g1 = *(const float4*)(gain + k + 4);
    float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0;
    if (add) {
      c0 = *(const float4*)(carry + o);
      c1 = *(const float4*)(carry + o + 4);
    }
    const float vv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float gg[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const float ga[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float inv = inv_s[r], coef = coef_s[r];
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = cc[i] + (inv * ga[i] * gg[i] - coef * vv[i]);
    *(float4*)(carry + o) = make_float4(out[0], out[1], out[2], out[3]);
    *(float4*)(carry + o + 4) = make_float4(out[4], out[5], out[6], out[7]);
    if (frag) *(uint4*)(frag + ((size_t)mt * nkc * 64 + sl) * 8) = pack8(out);
  }
}

// The same for d = 512 NJ (NJ <= 8) in one pass: a workgroup of RB_BWD waves
// takes as many rows, wave w row RB_BWD blockIdx.x + w with lane l holding
// columns 512 j + 8 l .. + 8 of v and gy in registers (read once; the
// two-pass kernel above reads both twice); carry is read, updated and written
// in the same pass, and the optional bf16 copy goes out through LDS in
// fragment order.  v and gy take about 150 VGPRs, so four rows per workgroup
// let three workgroups share a compute unit.
constexpr int RB_BWD = 4;
template <int NJ>
__global__ __launch_bounds__(64 * RB_BWD) void rms_bwd1_kernel(
    const float* __restrict__ v, const float* __restrict__ gy, int ldg, const float* __restrict__ gain, float eps,
    int d, float* __restrict__ carry, int add, bf16* __restrict__ frag, float* __restrict__ inv_out,
    const bf16* __restrict__ emb, const int32_t* __restrict__ tok, float* __restrict__ inv_e) {
  __shared__ uint4 stage[2][64 * RB_BWD];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, row0 = blockIdx.x * RB_BWD, row = row0 + w;
  const float* pv = v + (size_t)row * d + 8 * l;
  const float* pg = gy + (size_t)row * ldg + 8 * l;
  float vv[NJ][8], gg[NJ][8];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float4 a0 = *(const float4*)(pv + 512 * j), a1 = *(const float4*)(pv + 512 * j + 4);
    const float4 b0 = *(const float4*)(pg + 512 * j), b1 = *(const float4*)(pg + 512 * j + 4);
    vv[j][0] = a0.x, vv[j][1] = a0.y, vv[j][2] = a0.z, vv[j][3] = a0.w;
    vv[j][4] = a1.x, vv[j][5] = a1.y, vv[j][6] = a1.z, vv[j][7] = a1.w;
    gg[j][0] = b0.x, gg[j][1] = b0.y, gg[j][2] = b0.z, gg[j][3] = b0.w;
    gg[j][4] = b1.x, gg[j][5] = b1.y, gg[j][6] = b1.z, gg[j][7] = b1.w;
  }
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      ss = fmaf(vv[j][c], vv[j][c], ss);
      dot = fmaf(gain[512 * j + 8 * l + c] * gg[j][c], vv[j][c], dot);
    }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  const float coef = inv * inv * inv / (float)d * dot;
  if (emb) {
    const bf16* pe = emb + (size_t)__builtin_amdgcn_readfirstlane(tok[row]) * d + 8 * l;
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float f[8];
      unpack8(*(const uint4*)(pe + 512 * j), f);
#pragma unroll
      for (int c = 0; c < 8; ++c) se = fmaf(f[c], f[c], se);
    }
    se = wave_sum(se);
    if (l == 0) inv_e[row] = (float)(1.0 / sqrt((double)se / d + (double)eps));
  }
  if (l == 0) inv_out[row] = inv;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float* pc = carry + (size_t)row * d + 512 * j + 8 * l;
    float cc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (add) {
      const float4 c0 = *(const float4*)pc, c1 = *(const float4*)(pc + 4);
      cc[0] = c0.x, cc[1] = c0.y, cc[2] = c0.z, cc[3] = c0.w, cc[4] = c1.x, cc[5] = c1.y, cc[6] = c1.z, cc[7] = c1.w;
    }
    float out[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      out[c] = cc[c] + (inv * gain[512 * j + 8 * l + c] * gg[j][c] - coef * vv[j][c]);
    *(float4*)pc = make_float4(out[0], out[1], out[2], out[3]);
    *(float4*)(pc + 4) = make_float4(out[4], out[5], out[6], out[7]);
    if (frag) put_chunk<RB_BWD>(stage, frag, row0, d >> 5, j, pack8(out));
  }
}

// rms_bwd_kernel's operation: the one-pass kernel when d is 512, 1024, 2048
// or 4096 (rows: a multiple of 16), else the two-pass one.
inline void rms_bwd(const float* v, const float* gy, int ldg, const float* gain, float eps, int M, int d, float* carry,
                    int add, bf16* frag, float* inv_out, const bf16* emb, const int32_t* tok, float* inv_e,
                    hipStream_t st) {
  const dim3 g1(M / RB_BWD), b1(64 * RB_BWD);
  if (d == 512)
    rms_bwd1_kernel<1><<<g1, b1, 0, st>>>(v, gy, ldg, gain, eps, d, carry, add, frag, inv_out, emb, tok, inv_e);
  else if (d == 1024)
    rms_bwd1_kernel<2><<<g1, b1, 0, st>>>(v, gy, ldg, gain, eps, d, carry, add, frag, inv_out, emb, tok, inv_e);
  else if (d == 2048)
    rms_bwd1_kernel<4><<<g1, b1, 0, st>>>(v, gy, ldg, gain, eps, d, carry, add, frag, inv_out, emb, tok, inv_e);
  else if (d == 4096)
    rms_bwd1_kernel<8><<<g1, b1, 0, st>>>(v, gy, ldg, gain, eps, d, carry, add, frag, inv_out, emb, tok, inv_e);
  else
    rms_bwd_kernel<<<M / 16, TR, 0, st>>>(v, gy, ldg, gain, eps, d, carry, add, frag, inv_out, emb, tok, inv_e);
}

// Gain gradient partials: part[c][k] (+)= sum over the rows r of chunk c of
// gy[r][k] * v[r][k] * inv[r], rows in order; v is fp32 [M][d] or, with emb,
// the bf16 embedding row of tok[r].
constexpr int GG_ROWS = 64;
__global__ __launch_bounds__(256) void gain_grad_kernel(const float* __restrict__ gy, int ldg,
                                                        const float* __restrict__ v, const bf16* __restrict__ emb,
                                                        const int32_t* __restrict__ tok, const float* __restrict__ inv,
                                                        int d, float* __restrict__ part, int add) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d) return;
  const int r0 = blockIdx.y * GG_ROWS;
  float s = 0.f;
#pragma unroll 8
  for (int r = r0; r < r0 + GG_ROWS; ++r) {
    const float vv = emb ? bf2f(emb[(size_t)tok[r] * d + k]) : v[(size_t)r * d + k];
    s = fmaf(gy[(size_t)r * ldg + k] * vv, inv[r], s);
  }
  float* o = part + (size_t)blockIdx.y * d + k;
  *o = add ? *o + s : s;
}

// out[k] = sum over chunks c (in order) of part[c][k]
__global__ __launch_bounds__(256) void gain_final_kernel(const float* __restrict__ part, int nch, int d,
                                                         float* __restrict__ out) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d) return;
  float s = 0.f;
  for (int c = 0; c < nch; ++c) s += part[(size_t)c * d + k];
  out[k] = s;
}

// ------------------------------------------------------------------ GEMM epilogues
// SwiGLU backward on dz = dh2 . W_down (plain map, column f < F): with the
// forward's fp32 (gate g, up u), z = silu(g) u gives
//   d gate = dz u silu'(g),  d up = dz silu(g),  silu'(g) = sg (1 + g (1 - sg))
// stored bf16 in fragment order [M][2F] (gate columns, then up columns).
struct BEpiSwiGLUBwd {
  const float2* gu;  // [M][F]
  bf16* dgu;         // fragment order [M][2F]
  int F;
  // d gate at g[0], d up at g[up]
  __device__ __forceinline__ static void put(float dz, float2 p, bf16* g, size_t up) {
    const float sg = 1.f / (1.f + expf(-p.x));
    g[0] = f2bf(dz * p.y * sg * (1.f + p.x * (1.f - sg)));
    g[up] = f2bf(dz * p.x * sg);
  }
  __device__ __forceinline__ void operator()(const BGAcc& acc, int rowbase, int colbase16, int lane, int M,
                                             int nt16) const {
    const int m = lane & 15, nkc = (2 * F) >> 5;
    const size_t up = (size_t)(F >> 5) * 512;  // F % 32 == 0: the up half starts a fragment column
    if (rowbase + 128 <= M && colbase16 + BG_NJ <= nt16 && !(rowbase & 15) && !(colbase16 & 1)) {
      // A tile wholly inside the matrix: branch-free, the (gate, up) pairs of
      // the next half row group (two column tiles) load while this one is
      // stored, so the loads are not each waited for behind a store.  Row
      // group i is fragment band rowbase / 16 + i; column tile j is fragment
      // column colbase16 / 2 + j / 2, 8-column half j % 2 at +256.
      const float2* gp = gu + (size_t)(rowbase + 4 * (lane >> 4)) * F + colbase16 * 16 + m;
      bf16* dp = dgu + ((size_t)(rowbase >> 4) * nkc + (colbase16 >> 1)) * 512 +
                 (4 * (lane >> 4) + 16 * (m >> 3)) * 8 + (m & 7);
      const size_t band = (size_t)nkc * 512;
      float2 cur[2][4], nxt[2][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[jj][e] = gp[(size_t)e * F + 16 * jj];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 1, j0 = 2 * (q & 1);
        if (q + 1 < 16) {
          const int i1 = (q + 1) >> 1, j1 = 2 * ((q + 1) & 1);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) nxt[jj][e] = gp[(size_t)(16 * i1 + e) * F + 16 * (j1 + jj)];
          __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this group's stores
        }
        bf16* di = dp + i * band;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = j0 + jj;
#pragma unroll
          for (int e = 0; e < 4; ++e) put(acc[i][j][e], cur[jj][e], di + (j >> 1) * 512 + (j & 1) * 256 + e * 8, up);
        }
        if (q + 1 < 16) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) cur[jj][e] = nxt[jj][e];
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
        const int f = col16 * 16 + m;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + e;
          if (row >= M) continue;
          put(acc[i][j][e], gu[(size_t)row * F + f], dgu + frag_off(row, f, nkc), up);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ attention backward
// Softmax backward with the forward's log-sum-exp L per query row and head:
//   P = exp(s - L),  dP = dO . V^T,  dS = P (dP - D),  D = sum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// over the rollout mask: query (j, i) sees the step-1 keys i' <= i and the
// chain keys (j', i), 2 <= j' <= j.

// Per (row, kv head g), one wave: D ([hq][M]) for the g's query heads; then the chain
// keys of this row: dQ's chain part (unscaled, dq_chain [M][hq][hd]) and
// the chain keys' dK (scaled) and dV, summed over the group's heads in head
// order and added to the fp32 accumulators [R-1][M][hkv][hd].
template <int HD, int G>
__global__ __launch_bounds__(256) void attn_prep_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ dO,
                                                        const bf16* __restrict__ O, const float* __restrict__ lse,
                                                        const bf16* __restrict__ KC, const bf16* __restrict__ VC,
                                                        int nchain, size_t chain_stride, int M, int hq, int hkv,
                                                        float scale, float* __restrict__ Dout,
                                                        float* __restrict__ dq_chain, float* __restrict__ dKC,
                                                        float* __restrict__ dVC) {
  constexpr int EPL = HD / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= M * hkv) return;
  const int row = wid / hkv, g = wid - row * hkv;
  const int nkc = (hq * HD) >> 5, d0 = lane * EPL;
  float q[G][EPL], go[G][EPL], D[G], L[G];
#pragma unroll
  for (int hl = 0; hl < G; ++hl) {
    const int h = g * G + hl;
    const size_t o = ((size_t)row * hq + h) * HD + d0;
    float ov[EPL];
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      q[hl][u] = bf2f(Q[o + u]);
      go[hl][u] = bf2f(dO[o + u]);
      ov[u] = bf2f(O[frag_off(row, h * HD + d0 + u, nkc)]);
    }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < EPL; ++u) s = fmaf(go[hl][u], ov[u], s);
    D[hl] = wave_sum(s);
    L[hl] = lse[(size_t)h * M + row];
    if (lane == 0) Dout[(size_t)h * M + row] = D[hl];
  }
  if (nchain == 0) return;
  float dqc[G][EPL];
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
#pragma unroll
    for (int u = 0; u < EPL; ++u) dqc[hl][u] = 0.f;
  for (int c = 0; c < nchain; ++c) {
    const size_t ko = c * chain_stride + ((size_t)row * hkv + g) * HD + d0;
    float kc[EPL], vc[EPL], dk[EPL], dv[EPL];
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      kc[u] = bf2f(KC[ko + u]);
      vc[u] = bf2f(VC[ko + u]);
      dk[u] = dv[u] = 0.f;
    }
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int u = 0; u < EPL; ++u) {
        sd = fmaf(q[hl][u], kc[u], sd);
        pd = fmaf(go[hl][u], vc[u], pd);
      }
      const float p = __expf(wave_sum(sd) * scale - L[hl]);
      const float ds = p * (wave_sum(pd) - D[hl]);
#pragma unroll
      for (int u = 0; u < EPL; ++u) {
        dqc[hl][u] = fmaf(ds, kc[u], dqc[hl][u]);
        dk[u] = fmaf(ds, q[hl][u], dk[u]);
        dv[u] = fmaf(p, go[hl][u], dv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      dKC[ko + u] += scale * dk[u];
      dVC[ko + u] += dv[u];
    }
  }
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
#pragma unroll
    for (int u = 0; u < EPL; ++u) dq_chain[((size_t)row * hq + g * G + hl) * HD + d0 + u] = dqc[hl][u];
}

// dQ over the step-1 keys, the forward kernel's layout: workgroup = (block
// of QB query rows, kv head g, sequence b), ta_waves(G, TA_DQ_WAVES) waves
// (head g*G + w%G, 32 rows each); K and V blocks of 64 keys staged in LDS by direct copies (two
// stages).  Per key block: S^T = K Q^T and dP^T = V dO^T (keys x queries),
// dS^T = P^T (dP^T - D); dQ^T += K^T dS^T with K^T read transposed from LDS.
// Then the chain part (dq_chain), the scale, the inverse RoPE at position
// i + pos_off, and bf16 stores into dqkv's q columns (fragment order).
template <int HD, int G>
__global__ __launch_bounds__(ta_waves(G, TA_DQ_WAVES) * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ Dd, const bf16* __restrict__ K1, const bf16* __restrict__ V1,
    const float* __restrict__ dq_chain, const float2* __restrict__ rope, int pos_off, bf16* __restrict__ dqkv,
    int nkc_qkv, int S, int hq, int hkv, float scale) {
  constexpr int NC = HD / 32, NT = HD / 16, CPR = HD / 8;
  constexpr int W = ta_waves(G, TA_DQ_WAVES), RG = W / G, QB = 32 * RG, KB = 64;
  constexpr int BLK = KB * CPR;
  constexpr int NDMA = 2 * BLK / 64 / W;
  static_assert(W % G == 0 && NDMA * 64 * W == 2 * BLK, "whole row groups; copies split evenly over the waves");
  __shared__ uint4 sm[2][2][BLK];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = w % G, rg = w / G;
  const int nqb = (S + QB - 1) / QB;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
  const int g = blockIdx.y, b = blockIdx.z;
  const int h = g * G + hl;
  const int i0 = qb * QB + 32 * rg;
  const bool active = i0 < S;
  const int nkb = (min(qb * QB + QB, S) + KB - 1) / KB;
  const int ml = lane & 15, q4 = lane >> 4;
  const size_t kstride = (size_t)hkv * HD;

  const uint32_t lds0 = lds_addr(&sm[0][0][0]);
  auto issue = [&](int kb) {
    const uint32_t st_base = lds0 + (uint32_t)((kb & 1) * 2 * BLK * 16);
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const int dd = w * NDMA + u;
      const int kv = dd / (BLK / 64), part = dd - kv * (BLK / 64);
      const int e = part * 64 + lane;
      const int r = e / CPR, slot = e - r * CPR;
      const int key = min(kb * KB + r, S - 1);
      const bf16* src = (kv ? V1 : K1) + ((size_t)b * S + key) * kstride + (size_t)g * HD + 8 * (slot ^ (r % CPR));
      dma16(src, st_base + (uint32_t)(kv * BLK * 16 + part * 1024));
    }
  };

  U4 qf[2][NC], df[2][NC];
  float Ln[2], Dn[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = min(i0 + 16 * nt + ml, S - 1);
    const size_t o = ((size_t)(b * S + i) * hq + h);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[nt][c].u = *(const uint4*)(Q + o * HD + 32 * c + 8 * q4);
      df[nt][c].u = *(const uint4*)(dO + o * HD + 32 * c + 8 * q4);
    }
    const size_t ho = (size_t)h * gridDim.z * S + b * S + i;  // [hq][M]
    Ln[nt] = lse[ho];
    Dn[nt] = Dd[ho];
  }
  f32x4 dq[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) dq[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  bg_wait_copies<0>();
  bg_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) issue(kb + 1);
    if (active && kb * KB <= i0 + 31) {
      const uint4* ks = &sm[kb & 1][0][0];
      const uint4* vs = &sm[kb & 1][1][0];
      f32x4 st[4][2], dp[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) st[mt][nt] = dp[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        U4 kf[4], vf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          kf[mt].u = lds_chunk<CPR>(ks, 16 * mt + ml, 4 * c + q4);
          vf[mt].u = lds_chunk<CPR>(vs, 16 * mt + ml, 4 * c + q4);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            st[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt].v, qf[nt][c].v, st[mt][nt], 0, 0, 0);
            dp[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[mt].v, df[nt][c].v, dp[mt][nt], 0, 0, 0);
          }
      }
      const bool diag = kb * KB + 63 > i0;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int qi = i0 + 16 * nt + ml;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool masked = diag && kb * KB + 16 * mt + 4 * q4 + e > qi;
            const float p = masked ? 0.f : __expf(st[mt][nt][e] * scale - Ln[nt]);
            st[mt][nt][e] = p * (dp[mt][nt][e] - Dn[nt]);
          }
      }
      const bf16* kb16 = (const bf16*)ks;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        U4 bs[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bs[nt] = pack_b_from_acc(st[2 * kc][nt], st[2 * kc + 1][nt]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const U4 kt = lds_tr_frag<CPR>(kb16, 32 * kc, t, ml, q4);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            dq[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt.v, bs[nt].v, dq[t][nt], 0, 0, 0);
        }
      }
    }
    bg_wait_copies<0>();
    bg_barrier();
  }
  if (!active) return;
  // lane holds dQ^T[dim 16t + 4 q4 + e][query i0 + 16 nt + ml]
  const int half = HD / 2;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = i0 + 16 * nt + ml;
    const size_t row = (size_t)b * S + i;
    if (dq_chain) {
      const float* pc = dq_chain + (row * hq + h) * HD + 4 * q4;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 c4 = *(const float4*)(pc + 16 * t);
        dq[t][nt][0] += c4.x;
        dq[t][nt][1] += c4.y;
        dq[t][nt][2] += c4.z;
        dq[t][nt][3] += c4.w;
      }
    }
#pragma unroll
    for (int t = 0; t < NT / 2; ++t) {
      float a[4], bb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = 16 * t + 4 * q4 + e;
        const float2 cs = rope[(size_t)(i + pos_off) * half + p];
        const float x = dq[t][nt][e] * scale, y = dq[t + NT / 2][nt][e] * scale;
        a[e] = x * cs.x + y * cs.y;
        bb[e] = y * cs.x - x * cs.y;
      }
      *(uint2*)(dqkv + frag_off((int)row, h * HD + 16 * t + 4 * q4, nkc_qkv)) =
          make_uint2(f2bf2(a[0], a[1]), f2bf2(a[2], a[3]));
      *(uint2*)(dqkv + frag_off((int)row, h * HD + half + 16 * t + 4 * q4, nkc_qkv)) =
          make_uint2(f2bf2(bb[0], bb[1]), f2bf2(bb[2], bb[3]));
    }
  }
}

// dK and dV of the step-1 keys from one step's queries: workgroup = (block
// of 128 keys, kv head g, sequence b), four waves of 32 keys; the keys' K and
// V operands stay in registers.  For every query head of the group and every
// block of 32 queries at or after the workgroup's first key, the Q and dO
// rows and the rows' L and D ([hq][M], contiguous per head) are copied into
// LDS by direct global -> LDS copies (two stages: the next block's copies
// are in flight while this one is computed); each wave computes S = Q K^T
// and dP = dO V^T (queries x keys), P and dS, then dV^T += dO^T P and dK^T +=
// Q^T dS with dO^T and Q^T read transposed from LDS.  The results are added
// to the fp32 accumulators [M][hkv][hd] (each element owned by one lane:
// deterministic).
constexpr int DKV_KEYS = 128;
template <int HD, int G>
__global__ __launch_bounds__(256) void attn_dkv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ dO,
                                                       const float* __restrict__ lse, const float* __restrict__ Dd,
                                                       const bf16* __restrict__ K1, const bf16* __restrict__ V1,
                                                       float* __restrict__ dK, float* __restrict__ dV, int S, int hq,
                                                       int hkv, float scale) {
  constexpr int NC = HD / 32, NT = HD / 16, CPR = HD / 8;
  constexpr int CH = 32 * CPR;            // 16-byte chunks of a 32-row block
  constexpr int CPW = 2 * CH / 64 / 4;    // 64-lane copies per wave per stage (Q and dO)
  static_assert(CPW * 64 * 4 == 2 * CH, "copies split evenly over the waves");
  // one stage: Q rows, dO rows, then L[32] and D[32]
  constexpr int STAGE = 2 * CH + 16;      // in 16-byte units
  __shared__ uint4 sm[2][STAGE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ml = lane & 15, q4 = lane >> 4;
  const int g = blockIdx.y, b = blockIdx.z;
  const int M = gridDim.z * S;
  const int kblk = blockIdx.x * DKV_KEYS;
  const int k0 = kblk + 32 * w;  // the wave's first key
  const bool kact = k0 < S;      // S % 64 == 0: a wave's 32 keys are all inside or all outside
  const size_t kstride = (size_t)hkv * HD;

  U4 kf[2][NC], vf[2][NC];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const size_t o = ((size_t)b * S + min(k0 + 16 * bb + ml, S - 1)) * kstride + (size_t)g * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[bb][c].u = *(const uint4*)(K1 + o + 32 * c + 8 * q4);
      vf[bb][c].u = *(const uint4*)(V1 + o + 32 * c + 8 * q4);
    }
  }
  f32x4 dkT[NT][2], dvT[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) dkT[t][bb] = dvT[t][bb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qb0 = kblk / 32, nqb = S / 32;
  const int per_head = nqb - qb0, n_it = G * per_head;
  const uint32_t lds0 = lds_addr(&sm[0][0]);
  auto issue = [&](int it) {
    const int hl = it / per_head, qb = qb0 + it - hl * per_head;
    const int h = g * G + hl;
    const uint32_t st_base = lds0 + (uint32_t)((it & 1) * STAGE * 16);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int dd = w * CPW + u;              // copy index within the stage
      const int which = dd / (CH / 64), part = dd - which * (CH / 64);
      const int e = part * 64 + lane;          // chunk index within the block
      const int r = e / CPR, slot = e - r * CPR;
      const size_t o = ((size_t)(b * S + qb * 32 + r) * hq + h) * HD + 8 * (slot ^ (r % CPR));
      dma16((which ? dO : Q) + o, st_base + (uint32_t)((which * CH + part * 64) * 16));
    }
    if (w == 0 && lane < 16) {                 // L then D: 32 floats each
      const float* src = (lane < 8 ? lse : Dd) + (size_t)h * M + b * S + qb * 32 + 4 * (lane & 7);
      dma16(src, st_base + (uint32_t)(2 * CH * 16));
    }
  };

  issue(0);
  bg_wait_copies<0>();
  bg_barrier();
  for (int it = 0; it < n_it; ++it) {
    if (it + 1 < n_it) issue(it + 1);
    const int hl = it / per_head, qb = qb0 + it - hl * per_head;
    const int q0 = qb * 32;
    const uint4* qs = &sm[it & 1][0];
    const uint4* gs = qs + CH;
    const float* ls = (const float*)(qs + 2 * CH);  // L[32], then D[32]
    (void)hl;
    if (kact && k0 <= q0 + 31) {
      f32x4 st[2][2], dp[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) st[a][bb] = dp[a][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        U4 qa[2], ga[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          qa[a].u = lds_chunk<CPR>(qs, 16 * a + ml, 4 * c + q4);
          ga[a].u = lds_chunk<CPR>(gs, 16 * a + ml, 4 * c + q4);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            st[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[a].v, kf[bb][c].v, st[a][bb], 0, 0, 0);
            dp[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[a].v, vf[bb][c].v, dp[a][bb], 0, 0, 0);
          }
      }
      // lane holds (query q0 + 16 a + 4 q4 + e, key k0 + 16 bb + ml)
      const bool diag = k0 + 31 > q0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qr = 16 * a + 4 * q4 + e;
          const float L = ls[qr], D = ls[32 + qr];
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const bool masked = diag && k0 + 16 * bb + ml > q0 + qr;
            const float p = masked ? 0.f : __expf(st[a][bb][e] * scale - L);
            st[a][bb][e] = p;
            dp[a][bb][e] = p * (dp[a][bb][e] - D);
          }
        }
      U4 pb[2], sb[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        pb[bb] = pack_b_from_acc(st[0][bb], st[1][bb]);
        sb[bb] = pack_b_from_acc(dp[0][bb], dp[1][bb]);
      }
      const bf16* q16 = (const bf16*)qs;
      const bf16* g16 = (const bf16*)gs;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const U4 gt = lds_tr_frag<CPR>(g16, 0, t, ml, q4);
        const U4 qt = lds_tr_frag<CPR>(q16, 0, t, ml, q4);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          dvT[t][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gt.v, pb[bb].v, dvT[t][bb], 0, 0, 0);
          dkT[t][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt.v, sb[bb].v, dkT[t][bb], 0, 0, 0);
        }
      }
    }
    bg_wait_copies<0>();
    bg_barrier();
  }
  // lane holds dK^T[dim 16t + 4 q4 + e][key k0 + 16 bb + ml]
  if (!kact) return;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const size_t o = ((size_t)b * S + k0 + 16 * bb + ml) * kstride + (size_t)g * HD + 4 * q4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float4* pk = (float4*)(dK + o + 16 * t);
      float4* pv = (float4*)(dV + o + 16 * t);
      float4 a = *pk, c = *pv;
      a.x += scale * dkT[t][bb][0];
      a.y += scale * dkT[t][bb][1];
      a.z += scale * dkT[t][bb][2];
      a.w += scale * dkT[t][bb][3];
      c.x += dvT[t][bb][0];
      c.y += dvT[t][bb][1];
      c.z += dvT[t][bb][2];
      c.w += dvT[t][bb][3];
      *pk = a;
      *pv = c;
    }
  }
}

// One step's key and value gradients (fp32 [M][hkv][hd], after RoPE) into
// dqkv's k and v columns (bf16, fragment order): k gets the inverse RoPE at
// position (row % S) + pos_off.  One thread per (row, kv head, pair p).
__global__ __launch_bounds__(256) void kv_final_kernel(const float* __restrict__ dK, const float* __restrict__ dV,
                                                       const float2* __restrict__ rope, int S, int pos_off, int M,
                                                       int hq, int hkv, int hd, bf16* __restrict__ dqkv, int nkc) {
  const int half = hd >> 1;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)M * hkv * half) return;
  const int p = (int)(e % half);
  const size_t rg = e / half;
  const int g = (int)(rg % hkv), row = (int)(rg / hkv);
  const size_t o = ((size_t)row * hkv + g) * hd;
  const float2 cs = rope[(size_t)(row % S + pos_off) * half + p];
  const float x = dK[o + p], y = dK[o + p + half];
  const int kc = hq * hd + g * hd, vc = (hq + hkv) * hd + g * hd;
  dqkv[frag_off(row, kc + p, nkc)] = f2bf(x * cs.x + y * cs.y);
  dqkv[frag_off(row, kc + p + half, nkc)] = f2bf(y * cs.x - x * cs.y);
  dqkv[frag_off(row, vc + p, nkc)] = f2bf(dV[o + p]);
  dqkv[frag_off(row, vc + p + half, nkc)] = f2bf(dV[o + p + half]);
}

// ------------------------------------------------------------------ workspace
struct Carve {
  size_t off = 0;
  unsigned char* base = nullptr;
  template <typename T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

inline int vocab_pad(int V) { return (V + 63) / 64 * 64; }

struct TrainLayout {
  void* fwd;  // the forward's own workspace (ttt_ws_bytes)
  TttSave sv;
  bf16 *qkv_t, *o_t, *gu_t, *down_t;                       // W^T packed
  float* carry;                                           // [M][d]
  bf16 *dh2f, *dh1f, *dguf, *dqkvf, *dgf;                 // fragment order [M][*]
  float *du, *dx;                                         // [M][d], [M][2d]
  bf16* da;                                               // [M][hq*hd] row-major
  float *Dd, *dqc;                                        // [hq][M], [M][hq][hd]
  float *dk1, *dv1, *dkc, *dvc;                           // [M][kvd], [R-1][M][kvd]
  bf16 *dqkvT, *xT, *dh1T, *aT, *dguT, *uT, *dh2T, *zT;  // [N][R*M] fragment order
  bf16 *dgT, *featsT;                                     // [d][M], [3d][M]
  float *inv_a, *inv_b;                                   // [M]
  float* gpart;                                           // [4][M/64][d]
  size_t bytes;
};

TrainLayout train_layout(const eagle3_dims& dm, int B, int S, int R, void* base) {
  Carve c;
  c.base = (unsigned char*)base;
  const size_t M = (size_t)B * S, MT = M * R, d = dm.d, F = dm.ffn;
  const size_t qd = (size_t)dm.n_q_heads * dm.head_dim, kvd = (size_t)dm.n_kv_heads * dm.head_dim;
  const size_t nqkv = qd + 2 * kvd, vp = vocab_pad(dm.vocab), nch = R > 1 ? R - 1 : 1;
  TrainLayout L;
  L.fwd = c.take<unsigned char>(ttt_ws_bytes(dm, B, S, R));
  TttSave& s = L.sv;
  s.s = c.take<float>((R + 1) * M * d);
  s.h1 = c.take<float>(R * M * d);
  s.x = c.take<bf16>(R * M * 2 * d);
  s.q = c.take<bf16>(R * M * qd);
  s.lse = c.take<float>(R * M * dm.n_q_heads);
  s.a = c.take<bf16>(R * M * qd);
  s.u = c.take<bf16>(R * M * d);
  s.gu = c.take<float2>(R * M * F);
  s.z = c.take<bf16>(R * M * F);
  s.dy = c.take<float>(R * M * d);
  s.tok = c.take<int32_t>(R * M);
  s.dlogits = c.take<bf16>(M * vp);
  s.exm = c.take<float>(M * (vp / 64));
  s.lse_ce = c.take<float>(M);
  bf16* lm_t = c.take<bf16>(d * vp);
  s.lm_t = lm_t;
  s.vp = (int)vp;
  s.count = 0;
  for (int j = 1; j <= R; ++j) s.count += (double)B * (S - j > 0 ? S - j : 0);
  L.qkv_t = c.take<bf16>(2 * d * nqkv);
  L.o_t = c.take<bf16>(qd * d);
  L.gu_t = c.take<bf16>(d * 2 * F);
  L.down_t = c.take<bf16>(F * d);
  L.carry = c.take<float>(M * d);
  L.dh2f = c.take<bf16>(M * d);
  L.dh1f = c.take<bf16>(M * d);
  L.dguf = c.take<bf16>(M * 2 * F);
  L.dqkvf = c.take<bf16>(M * nqkv);
  L.dgf = c.take<bf16>(M * d);
  L.du = c.take<float>(M * d);
  L.dx = c.take<float>(M * 2 * d);
  L.da = c.take<bf16>(M * qd);
  L.Dd = c.take<float>(M * dm.n_q_heads);
  L.dqc = c.take<float>(M * qd);
  L.dk1 = c.take<float>(M * kvd);
  L.dv1 = c.take<float>(M * kvd);
  L.dkc = c.take<float>(nch * M * kvd);
  L.dvc = c.take<float>(nch * M * kvd);
  L.dqkvT = c.take<bf16>(nqkv * MT);
  L.xT = c.take<bf16>(2 * d * MT);
  L.dh1T = c.take<bf16>(d * MT);
  L.aT = c.take<bf16>(qd * MT);
  L.dguT = c.take<bf16>(2 * F * MT);
  L.uT = c.take<bf16>(d * MT);
  L.dh2T = c.take<bf16>(d * MT);
  L.zT = c.take<bf16>(F * MT);
  L.dgT = c.take<bf16>(d * M);
  L.featsT = c.take<bf16>(3 * d * M);
  L.inv_a = c.take<float>(M);
  L.inv_b = c.take<float>(M);
  L.gpart = c.take<float>(4 * (M / GG_ROWS) * d);
  L.bytes = c.off;
  return L;
}

}  // namespace

size_t ttt_train_ws_bytes(const eagle3_dims& dm, int B, int S, int R) {
  return train_layout(dm, B, S, R, nullptr).bytes;
}

int ttt_train(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, const int32_t* tokens, int B, int S,
              int R, const int32_t* forced, int32_t* pred, float* ce, float* loss, const eagle3_grads& gr, void* wsp,
              hipStream_t st) {
  const int d = dm.d, hq = dm.n_q_heads, hkv = dm.n_kv_heads, hd = dm.head_dim, F = dm.ffn, V = dm.vocab;
  const int qd = hq * hd, kvd = hkv * hd, nqkv = qd + 2 * kvd, G = hq / hkv;
  if (dm.dtype != EAGLE3_BF16 || (hd != 64 && hd != 128) || S % 64 != 0 || V % 16 != 0) return 1;
  if (d % 64 || F % 64 || qd % 64 || d > 8192 || hq % hkv || 8 % G) return 1;
  const int M = B * S, MT = M * R;
  TrainLayout L = train_layout(dm, B, S, R, wsp);
  TttSave& sv = L.sv;
  const bool pk = w.layout == EAGLE3_LAYOUT_PACKED;
  const float eps = dm.rms_eps;
  const float scale = (float)(1.0 / sqrt((double)hd));
  const RowMap plain{MAP_PLAIN, hd, F}, pair_head{MAP_PAIR_HEAD, hd, F}, pair_ffn{MAP_PAIR_FFN, hd, F};
  const size_t Md = (size_t)M * d;
  const int nch = M / GG_ROWS;
  hipError_t e;
#define E3_CHECK(x) \
  if ((e = (x)) != hipSuccess) return -1;

  {
    // W^T of every matrix the backward multiplies by, packed in fragment order
    TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
    E3_CHECK(transpose_weight(w.lm, pk, V, d, plain, (bf16*)sv.lm_t, sv.vp, st));
    E3_CHECK(transpose_weight(w.qkv, pk, nqkv, 2 * d, pair_head, L.qkv_t, nqkv, st));
    E3_CHECK(transpose_weight(w.o, pk, d, qd, plain, L.o_t, d, st));
    E3_CHECK(transpose_weight(w.gate_up, pk, 2 * F, d, pair_ffn, L.gu_t, 2 * F, st));
    E3_CHECK(transpose_weight(w.down, pk, d, F, plain, L.down_t, d, st));
  }
  int rc = ttt_forward(dm, w, feats, tokens, B, S, R, forced, pred, ce, loss, L.fwd, st, &sv);
  if (rc) return rc;
  {
    TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
    const size_t n1 = (size_t)M * kvd, nc = (size_t)(R > 1 ? R - 1 : 1) * M * kvd;
    fill_kernel<<<1024, 256, 0, st>>>(L.dk1, n1);
    fill_kernel<<<1024, 256, 0, st>>>(L.dv1, n1);
    fill_kernel<<<1024, 256, 0, st>>>(L.dkc, nc);
    fill_kernel<<<1024, 256, 0, st>>>(L.dvc, nc);
    E3_CHECK(hipGetLastError());
  }
  float* gp_out = L.gpart;
  float* gp_ffn = L.gpart + (size_t)nch * d;
  float* gp_s = L.gpart + (size_t)2 * nch * d;
  float* gp_e = L.gpart + (size_t)3 * nch * d;
  const dim3 gg_grid((d + 255) / 256, nch);

  for (int j = R; j >= 1; --j) {
    const size_t js = (size_t)(j - 1);
    const int col0 = (int)(js * M);  // the step's token columns in the transposed operands
    const float* s_in = sv.s + js * Md;
    const float* h1 = sv.h1 + js * Md;
    const float* h2 = sv.s + (js + 1) * Md;
    const int32_t* tok = j == 1 ? tokens : sv.tok + js * M;
    const int add = j < R;
    {
      // dh2 = carry + rms'(h2, norm_out) dy
      TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
      rms_bwd(h2, sv.dy + js * Md, d, w.norm_out, eps, M, d, L.carry, add, L.dh2f, L.inv_a, nullptr, nullptr, nullptr,
              st);
      gain_grad_kernel<<<gg_grid, 256, 0, st>>>(sv.dy + js * Md, d, h2, nullptr, nullptr, L.inv_a, d, gp_out, add);
      E3_CHECK(hipGetLastError());
      E3_CHECK(transpose(SrcFrag{L.dh2f, d / 32}, M, d, L.dh2T, MT / 32, col0, st));
      E3_CHECK(transpose(SrcFrag{sv.z + js * M * F, F / 32}, M, F, L.zT, MT / 32, col0, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_GEMM, st);
      E3_CHECK(bg_launch(L.dh2f, d, true, M, L.down_t, true, F, d, plain,
                         BEpiSwiGLUBwd{sv.gu + js * M * F, L.dguf, F}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
      E3_CHECK(transpose(SrcFrag{L.dguf, 2 * F / 32}, M, 2 * F, L.dguT, MT / 32, col0, st));
      E3_CHECK(transpose(SrcFrag{sv.u + js * Md, d / 32}, M, d, L.uT, MT / 32, col0, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_GEMM, st);
      E3_CHECK(bg_launch(L.dguf, 2 * F, true, M, L.gu_t, true, d, 2 * F, plain, BEpiStoreF{L.du, d, false}, st));
    }
    {
      // dh1 = dh2 + rms'(h1, norm_ffn) du
      TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
      rms_bwd(h1, L.du, d, w.norm_ffn, eps, M, d, L.carry, 1, L.dh1f, L.inv_a, nullptr, nullptr, nullptr, st);
      gain_grad_kernel<<<gg_grid, 256, 0, st>>>(L.du, d, h1, nullptr, nullptr, L.inv_a, d, gp_ffn, add);
      E3_CHECK(hipGetLastError());
      E3_CHECK(transpose(SrcFrag{L.dh1f, d / 32}, M, d, L.dh1T, MT / 32, col0, st));
      E3_CHECK(transpose(SrcFrag{sv.a + js * M * qd, qd / 32}, M, qd, L.aT, MT / 32, col0, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_GEMM, st);
      E3_CHECK(bg_launch(L.dh1f, d, true, M, L.o_t, true, qd, d, plain, BEpiStoreBF{L.da, qd}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_ATTN, st);
      const int nchain = j - 1;
      const bf16* q = sv.q + js * M * qd;
      const float* lse = sv.lse + js * M * hq;
      const size_t cstride = (size_t)M * kvd;
#define E3_BWD_ATTN(HDV, GV)                                                                                          \
  {                                                                                                                   \
    attn_prep_kernel<HDV, GV><<<(M * hkv + 3) / 4, 256, 0, st>>>(q, L.da, sv.a + js * M * qd, lse, sv.kc, sv.vc,      \
                                                                 nchain, cstride, M, hq, hkv, scale, L.Dd, L.dqc,     \
                                                                 L.dkc, L.dvc);                                       \
    constexpr int QB = 32 * (ta_waves(GV, TA_DQ_WAVES) / GV);                                                                      \
    attn_dq_kernel<HDV, GV><<<dim3((S + QB - 1) / QB, hkv, B), ta_waves(GV, TA_DQ_WAVES) * 64, 0, st>>>(                          \
        q, L.da, lse, L.Dd, sv.k1, sv.v1, nchain ? L.dqc : nullptr, sv.rope, j - 1, L.dqkvf, nqkv / 32, S, hq, hkv,    \
        scale);                                                                                                       \
    attn_dkv_kernel<HDV, GV><<<dim3((S + DKV_KEYS - 1) / DKV_KEYS, hkv, B), 256, 0, st>>>(q, L.da, lse, L.Dd, sv.k1, sv.v1, L.dk1,    \
                                                                         L.dv1, S, hq, hkv, scale);                   \
  }
      if (hd == 128) {
        if (G == 1) E3_BWD_ATTN(128, 1) else if (G == 2) E3_BWD_ATTN(128, 2) else if (G == 4) E3_BWD_ATTN(128, 4)
        else E3_BWD_ATTN(128, 8)
      } else {
        if (G == 1) E3_BWD_ATTN(64, 1) else if (G == 2) E3_BWD_ATTN(64, 2) else if (G == 4) E3_BWD_ATTN(64, 4)
        else E3_BWD_ATTN(64, 8)
      }
#undef E3_BWD_ATTN
      E3_CHECK(hipGetLastError());
      // this step's keys are complete: step 1's from every step, chain keys (j, i) from steps j..R
      const float* dk = j == 1 ? L.dk1 : L.dkc + (size_t)(j - 2) * cstride;
      const float* dv = j == 1 ? L.dv1 : L.dvc + (size_t)(j - 2) * cstride;
      const size_t n = (size_t)M * hkv * (hd / 2);
      kv_final_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dk, dv, sv.rope, S, j - 1, M, hq, hkv, hd, L.dqkvf,
                                                                  nqkv / 32);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
      E3_CHECK(transpose(SrcFrag{L.dqkvf, nqkv / 32}, M, nqkv, L.dqkvT, MT / 32, col0, st));
      E3_CHECK(transpose(SrcFrag{sv.x + js * 2 * Md, 2 * d / 32}, M, 2 * d, L.xT, MT / 32, col0, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_BWD_GEMM, st);
      E3_CHECK(bg_launch(L.dqkvf, nqkv, true, M, L.qkv_t, true, 2 * d, nqkv, plain, BEpiStoreF{L.dx, 2 * d, false},
                         st));
    }
    {
      // carry = ds_j = dh1 + rms'(s_j, norm_s) dx_s; the embedding half only trains norm_e
      TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
      rms_bwd(s_in, L.dx + d, 2 * d, w.norm_s, eps, M, d, L.carry, 1, j == 1 ? L.dgf : nullptr, L.inv_a,
              (const bf16*)w.emb, tok, L.inv_b, st);
      gain_grad_kernel<<<gg_grid, 256, 0, st>>>(L.dx + d, 2 * d, s_in, nullptr, nullptr, L.inv_a, d, gp_s, add);
      gain_grad_kernel<<<gg_grid, 256, 0, st>>>(L.dx, 2 * d, nullptr, (const bf16*)w.emb, tok, L.inv_b, d, gp_e, add);
      E3_CHECK(hipGetLastError());
    }
  }
  {
    TimedScope ts(EAGLE3_KC_TTT_BWD_ROWS, st);
    E3_CHECK(transpose(SrcFrag{L.dgf, d / 32}, M, d, L.dgT, M / 32, 0, st));
    E3_CHECK(transpose(SrcRowMajor{(const bf16*)feats, (size_t)3 * d}, M, 3 * d, L.featsT, M / 32, 0, st));
    const dim3 fg((d + 255) / 256);
    gain_final_kernel<<<fg, 256, 0, st>>>(gp_out, nch, d, gr.norm_out);
    gain_final_kernel<<<fg, 256, 0, st>>>(gp_ffn, nch, d, gr.norm_ffn);
    gain_final_kernel<<<fg, 256, 0, st>>>(gp_s, nch, d, gr.norm_s);
    gain_final_kernel<<<fg, 256, 0, st>>>(gp_e, nch, d, gr.norm_e);
    E3_CHECK(hipGetLastError());
  }
  {
    // weight gradients: dW = dY^T X over all steps' rows, one GEMM each
    TimedScope ts(EAGLE3_KC_TTT_WGRAD, st);
    E3_CHECK(bg_launch(L.dqkvT, MT, true, nqkv, L.xT, true, 2 * d, MT, plain, BEpiStoreF{gr.qkv, 2 * d, false}, st,
                       EAGLE3_KC_TTT_WGRAD));
    E3_CHECK(bg_launch(L.dh1T, MT, true, d, L.aT, true, qd, MT, plain, BEpiStoreF{gr.o, qd, false}, st,
                       EAGLE3_KC_TTT_WGRAD));
    E3_CHECK(bg_launch(L.dguT, MT, true, 2 * F, L.uT, true, d, MT, plain, BEpiStoreF{gr.gate_up, d, false}, st,
                       EAGLE3_KC_TTT_WGRAD));
    E3_CHECK(bg_launch(L.dh2T, MT, true, d, L.zT, true, F, MT, plain, BEpiStoreF{gr.down, F, false}, st,
                       EAGLE3_KC_TTT_WGRAD));
    E3_CHECK(bg_launch(L.dgT, M, true, d, L.featsT, true, 3 * d, M, plain, BEpiStoreF{gr.fc, 3 * d, false}, st,
                       EAGLE3_KC_TTT_WGRAD));
  }
#undef E3_CHECK
  return 0;
}

}  // namespace e3
