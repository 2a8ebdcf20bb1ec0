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
#include "ttt_common.hpp"

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
  bf16* x;       // [M][2d] decoder input; reused as u [M][d] and y [M][d] (fragment order)
  bf16* a;       // [M][hq*hd] attention output (fragment order)
  bf16* z;       // [M][F] silu(gate) * up (fragment order)
  bf16* q;       // [M][hq][hd]
  bf16* k1;      // [M][hkv][hd] step-1 keys
  bf16* v1t;     // step-1 values: [M][hkv][hd] (LDS attention kernel) or [B][hkv][hd][S] (transposed)
  bf16* kc;      // [R-1][M][hkv][hd] chain keys of steps 2..R
  bf16* vc;      // [R-1][M][hkv][hd] chain values
  float4* part;  // [M][nblk] LM-head partials per 256 columns {max, sum exp, argmax id, 0}
  float* lab;    // [M] target logit
  int32_t* tok;  // [M] input tokens of the next step
  float2* rope;  // [S+R][hd/2] (cos, sin)
  size_t bytes;
};

inline int ce_blocks(int V) { return (V / 16 + 15) / 16; }  // 256-column blocks

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

// x = [rms(emb[t]) * norm_e ; rms(s) * norm_s] (bf16, fragment order, K = 2d)
__global__ __launch_bounds__(TR) void ttt_prologue_kernel(const bf16* __restrict__ emb, const int32_t* __restrict__ tok,
                                                          const float* __restrict__ hs, int d,
                                                          const float* __restrict__ ge, const float* __restrict__ gs,
                                                          float eps, bf16* __restrict__ x) {
  __shared__ float ie_s[16], is_s[16];
  __shared__ int tok_s[16];
  const int mt = blockIdx.x, r0 = mt * 16, rr = threadIdx.x >> 4;
  const int t = tok[r0 + rr];
  const float se = row_ss(emb, (size_t)d, t, d);
  const float ss = row_ss(hs, (size_t)d, r0 + rr, d);
  if ((threadIdx.x & 15) == 0) {
    ie_s[rr] = (float)(1.0 / sqrt((double)se / d + (double)eps));
    is_s[rr] = (float)(1.0 / sqrt((double)ss / d + (double)eps));
    tok_s[rr] = t;
  }
  __syncthreads();
  const int nkc = (2 * d) >> 5;
  for (int sl = threadIdx.x; sl < nkc * 64; sl += TR) {
    const int kc = sl >> 6, l = sl & 63, r = l & 15, k = kc * 32 + 8 * (l >> 4);
    float v[8], o[8];
    if (k < d) {
      unpack8(*(const uint4*)(emb + (size_t)tok_s[r] * d + k), v);
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = v[c] * ie_s[r] * ge[k + c];
    } else {
      const float* p = hs + (size_t)(r0 + r) * d + (k - d);
      const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = v[c] * is_s[r] * gs[k - d + c];
    }
    *(uint4*)(x + ((size_t)mt * nkc * 64 + sl) * 8) = pack8(o);
  }
}

// y = rms(h) * gain (bf16, [M][d] in fragment order)
__global__ __launch_bounds__(TR) void ttt_norm_kernel(const float* __restrict__ hs, int d,
                                                      const float* __restrict__ gain, float eps,
                                                      bf16* __restrict__ y) {
  __shared__ float inv_s[16];
  const int mt = blockIdx.x, r0 = mt * 16, rr = threadIdx.x >> 4;
  const float ss = row_ss(hs, (size_t)d, r0 + rr, d);
  if ((threadIdx.x & 15) == 0) inv_s[rr] = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  __syncthreads();
  const int nkc = d >> 5;
  for (int sl = threadIdx.x; sl < nkc * 64; sl += TR) {
    const int kc = sl >> 6, l = sl & 63, r = l & 15, k = kc * 32 + 8 * (l >> 4);
    const float* p = hs + (size_t)(r0 + r) * d + k;
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = v[c] * inv_s[r] * gain[k + c];
    *(uint4*)(y + ((size_t)mt * nkc * 64 + sl) * 8) = pack8(o);
  }
}

// One-pass row kernels for d = 512 NJ (NJ <= 8): a workgroup of RB waves
// takes RB rows (RB = 8 for the norm; 4 for the prologue, whose two rows per
// wave hold 164 VGPRs, so that three workgroups share a compute unit), wave
// w row RB blockIdx.x + w, lane l columns 512 j + 8 l .. + 8 of each
// 512-column chunk j: a row is read from memory once and kept in registers
// (the two-pass kernels above read it twice).  Each output chunk (16
// fragments of the 16-row tile, the block's RB rows of their slots) is
// assembled in LDS and leaves as runs of RB 16-byte slots.
constexpr int RB_NORM = 8, RB_PRO = 4;

// y = rms(h) * gain, one pass (see above)
template <int NJ>
__global__ __launch_bounds__(64 * RB_NORM) void ttt_norm1_kernel(const float* __restrict__ hs, int d,
                                                             const float* __restrict__ gain, float eps,
                                                             bf16* __restrict__ y) {
  __shared__ uint4 stage[2][64 * RB_NORM];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, row0 = blockIdx.x * RB_NORM;
  const float* p = hs + (size_t)(row0 + w) * d + 8 * l;
  float v[NJ][8];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float4 a = *(const float4*)(p + 512 * j), b = *(const float4*)(p + 512 * j + 4);
    v[j][0] = a.x, v[j][1] = a.y, v[j][2] = a.z, v[j][3] = a.w, v[j][4] = b.x, v[j][5] = b.y, v[j][6] = b.z,
    v[j][7] = b.w;
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(v[j][c], v[j][c], ss);
  const float inv = (float)(1.0 / sqrt((double)wave_sum(ss) / d + (double)eps));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = v[j][c] * inv * gain[512 * j + 8 * l + c];
    put_chunk<RB_NORM>(stage, y, row0, d >> 5, j, pack8(o));
  }
}

// x = [rms(emb[t]) * norm_e ; rms(s) * norm_s], one pass (see above)
template <int NJ>
__global__ __launch_bounds__(64 * RB_PRO) void ttt_prologue1_kernel(
    const bf16* __restrict__ emb, const int32_t* __restrict__ tok, const float* __restrict__ hs, int d,
    const float* __restrict__ ge, const float* __restrict__ gs, float eps, bf16* __restrict__ x) {
  __shared__ uint4 stage[2][64 * RB_PRO];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, row0 = blockIdx.x * RB_PRO;
  const int t = __builtin_amdgcn_readfirstlane(tok[row0 + w]);
  const bf16* pe = emb + (size_t)t * d + 8 * l;
  const float* ps = hs + (size_t)(row0 + w) * d + 8 * l;
  uint4 e[NJ];
  float v[NJ][8];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    e[j] = *(const uint4*)(pe + 512 * j);
    const float4 a = *(const float4*)(ps + 512 * j), b = *(const float4*)(ps + 512 * j + 4);
    v[j][0] = a.x, v[j][1] = a.y, v[j][2] = a.z, v[j][3] = a.w, v[j][4] = b.x, v[j][5] = b.y, v[j][6] = b.z,
    v[j][7] = b.w;
  }
  float se = 0.f, ss = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float f[8];
    unpack8(e[j], f);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      se = fmaf(f[c], f[c], se);
      ss = fmaf(v[j][c], v[j][c], ss);
    }
  }
  const float ie = (float)(1.0 / sqrt((double)wave_sum(se) / d + (double)eps));
  const float is = (float)(1.0 / sqrt((double)wave_sum(ss) / d + (double)eps));
  const int nkc = (2 * d) >> 5;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float f[8], o[8];
    unpack8(e[j], f);
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = f[c] * ie * ge[512 * j + 8 * l + c];
    put_chunk<RB_PRO>(stage, x, row0, nkc, j, pack8(o));
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = v[j][c] * is * gs[512 * j + 8 * l + c];
    put_chunk<RB_PRO>(stage, x, row0, nkc, NJ + j, pack8(o));
  }
}

// Launch the one-pass kernel when d is 512, 1024, 2048 or 4096 (rows: a
// multiple of 8), else the two-pass one.
inline void ttt_norm(const float* hs, int M, int d, const float* gain, float eps, bf16* y, hipStream_t st) {
  switch (d) {
    case 512: ttt_norm1_kernel<1><<<M / RB_NORM, 64 * RB_NORM, 0, st>>>(hs, d, gain, eps, y); break;
    case 1024: ttt_norm1_kernel<2><<<M / RB_NORM, 64 * RB_NORM, 0, st>>>(hs, d, gain, eps, y); break;
    case 2048: ttt_norm1_kernel<4><<<M / RB_NORM, 64 * RB_NORM, 0, st>>>(hs, d, gain, eps, y); break;
    case 4096: ttt_norm1_kernel<8><<<M / RB_NORM, 64 * RB_NORM, 0, st>>>(hs, d, gain, eps, y); break;
    default: ttt_norm_kernel<<<M / 16, TR, 0, st>>>(hs, d, gain, eps, y);
  }
}
inline void ttt_prologue(const bf16* emb, const int32_t* tok, const float* hs, int M, int d, const float* ge,
                         const float* gs, float eps, bf16* x, hipStream_t st) {
  switch (d) {
    case 512: ttt_prologue1_kernel<1><<<M / RB_PRO, 64 * RB_PRO, 0, st>>>(emb, tok, hs, d, ge, gs, eps, x); break;
    case 1024: ttt_prologue1_kernel<2><<<M / RB_PRO, 64 * RB_PRO, 0, st>>>(emb, tok, hs, d, ge, gs, eps, x); break;
    case 2048: ttt_prologue1_kernel<4><<<M / RB_PRO, 64 * RB_PRO, 0, st>>>(emb, tok, hs, d, ge, gs, eps, x); break;
    case 4096: ttt_prologue1_kernel<8><<<M / RB_PRO, 64 * RB_PRO, 0, st>>>(emb, tok, hs, d, ge, gs, eps, x); break;
    default: ttt_prologue_kernel<<<M / 16, TR, 0, st>>>(emb, tok, hs, d, ge, gs, eps, x);
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

// LM head with the cross entropy folded in: for every row and each
// 256-column block (one workgroup tile) write {max, sum exp(x - max), argmax
// id}; the lane that owns a row's target column writes the target logit.
// Each wave reduces its 64 columns per row (maximum, then the lowest column
// holding it, then the sum of exponentials, each a 16-lane DPP reduction),
// then the four column waves' results meet in LDS and are combined in wave
// order.  The targets of the lane's 32 rows are loaded before the k loop.
struct TEpiCE {
  float4* part;
  float* lab;
  const int32_t* tokens;  // [M], targets are tokens[row + step] inside the sequence
  int S, step, nblk;
  // optional, for the backward: bf16 exp(logit - m) [M][ldl] with m the row's
  // maximum over this wave's 64 columns, and those maxima [M][ldl / 64]
  bf16* ex = nullptr;
  float* exm = nullptr;
  int ldl = 0;
  struct Pre {
    int tg[8][4];
  };
  __device__ __forceinline__ Pre pre(int rowbase, int lane, int M) const {
    // one division per lane; S >= 64, so a row offset of at most 115 wraps a
    // sequence at most once
    Pre p;
    const int r0 = rowbase + 4 * (lane >> 4);
    const int p0 = r0 % S;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 16 * i + e;
        int pos = p0 + 16 * i + e;
        if (pos >= S) pos -= S;
        if (pos >= S) pos -= S;
        p.tg[i][e] = row < M && pos + step <= S - 1 ? tokens[row + step] : -1;
      }
    return p;
  }
  __device__ __forceinline__ void operator()(const BGAcc& acc, const Pre& pr, int rowbase, int colbase16, int lane,
                                             int M, int nt16) const {
    __shared__ float4 cs[BG_BM][4];  // [row in tile][column wave]
    const int m = lane & 15, wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
    const int r0 = rowbase + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 16 * i + e;
        const int target = pr.tg[i][e];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < BG_NJ; ++j) {
          const int col16 = colbase16 + j, n = col16 * 16 + m;
          if (col16 < nt16) {
            const float xv = acc[i][j][e];
            mx = fmaxf(mx, xv);
            if (n == target) lab[row] = xv;
          }
        }
        mx = row16_max(mx);
        int id = 0x7fffffff;
        float s = 0.f;
        if (mx > -INFINITY) {
#pragma unroll
          for (int j = BG_NJ - 1; j >= 0; --j)  // lowest column of this lane holding the maximum
            if (colbase16 + j < nt16 && acc[i][j][e] == mx) id = (colbase16 + j) * 16 + m;
#pragma unroll
          for (int j = 0; j < BG_NJ; ++j)
            if (colbase16 + j < nt16) {
              const float ev = __expf(acc[i][j][e] - mx);
              s += ev;
              if (ex && row < M) ex[(size_t)row * ldl + (colbase16 + j) * 16 + m] = f2bf(ev);
            }
          if (exm && m == 0 && row < M) exm[(size_t)row * (ldl >> 6) + (colbase16 >> 2)] = mx;
        }
        id = row16_min(id);
        s = row16_sum(s);
        if (m == 0) cs[wm * 128 + 16 * i + 4 * (lane >> 4) + e][wn] = make_float4(mx, s, __int_as_float(id), 0.f);
      }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < BG_BM) {
      const int row = rowbase - wm * 128 + t, blk = colbase16 / 16;
      if (row < M && blk < nblk) {
        float gm = -INFINITY;
        int gi = 0x7fffffff;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 c = cs[t][w];
          if (better(c.x, __float_as_int(c.z), gm, gi)) {
            gm = c.x;
            gi = __float_as_int(c.z);
          }
        }
        float gs = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 c = cs[t][w];
          if (c.x > -INFINITY) gs += c.y * __expf(c.x - gm);
        }
        part[(size_t)row * nblk + blk] = make_float4(gm, gs, __int_as_float(gi), 0.f);
      }
    }
  }
};

// Per row: merge the partials into logsumexp and argmax; CE, prediction and
// the next step's input token.
__global__ __launch_bounds__(256) void ce_merge_kernel(const float4* __restrict__ part, int nblk,
                                                       const float* __restrict__ lab, const int32_t* __restrict__ forced,
                                                       int S, int R, int step, int32_t* __restrict__ pred,
                                                       float* __restrict__ ce, int32_t* __restrict__ tok_next,
                                                       float* __restrict__ lse_out) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  __shared__ double ws[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float4* p = part + (size_t)row * nblk;
  float4 loc[4];  // nblk <= 1024 (vocab <= 262144 in 256-column blocks)
  int nl = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
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
  for (int c = 0; c < 4; ++c)
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
    if (lse_out) lse_out[row] = (float)lse;
  }
}

// Gradient of the mean CE at one step's logits, bf16 row-major [M][ldl],
// written in place over the CE epilogue's e = exp(logit - m) (m the row's
// maximum over each 64 columns, exm): (softmax - onehot(target)) / count on
// rows with a target (i + step <= S-1), zero on the others and in the
// padding columns V..ldl-1.  softmax = e exp(m - lse); the target column
// takes exp(target logit - lse) - 1 from the fp32 target logit, so that the
// cancellation near p = 1 keeps float precision.
__global__ __launch_bounds__(256) void dlogits_kernel(bf16* __restrict__ e, const float* __restrict__ exm, int V,
                                                      int ldl, const float* __restrict__ lse,
                                                      const float* __restrict__ lab, const int32_t* __restrict__ tokens,
                                                      int S, int step, float inv_count) {
  const int row = blockIdx.x;
  const bool valid = row % S + step <= S - 1;
  const int target = valid ? tokens[row + step] : -1;
  const float l = lse[row];
  const float pt = valid ? __expf(lab[row] - l) - 1.f : 0.f;
  const float* mrow = exm + (size_t)row * (ldl >> 6);
  bf16* p = e + (size_t)row * ldl;
  for (int k = threadIdx.x * 4; k < ldl; k += 256 * 4) {
    float g[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid && k < V) {  // V % 16 == 0: a group of four is inside or outside, within one 64-column group
      const float sc = __expf(mrow[k >> 6] - l) * inv_count;
      const uint2 u = *(const uint2*)(p + k);
      const uint32_t w[2] = {u.x, u.y};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        g[2 * c] = __uint_as_float(w[c] << 16) * sc;
        g[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u) * sc;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (k + c == target) g[c] = pt * inv_count;
    }
    *(uint2*)(p + k) = make_uint2(f2bf2(g[0], g[1]), f2bf2(g[2], g[3]));
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
// the B-operand layout of O^T = V^T P^T; P enters as bf16 (the output is
// rounded to bf16 next, which dominates the error of P's rounding).  Causal
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
      U4 pb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) pb[nt] = pack_b_from_acc(st[2 * kc][nt], st[2 * kc + 1][nt]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16* vp = vbase + (size_t)(16 * t + ml) * S + kb * 64 + 32 * kc + 4 * q4;
        const uint2 v0 = *(const uint2*)vp, v1 = *(const uint2*)(vp + 16);
        U4 vf;
        vf.u = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pb[nt].v, o[t][nt], 0, 0, 0);
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
    const int row = b * S + i0 + 16 * nt + ml;
    const int nkc = (hq * HD) >> 5;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 r = o[t][nt] * inv;
      *(uint2*)(out + frag_off(row, h * HD + 16 * t + 4 * q4, nkc)) =
          make_uint2((uint32_t)f2bf(r[0]) | ((uint32_t)f2bf(r[1]) << 16), (uint32_t)f2bf(r[2]) | ((uint32_t)f2bf(r[3]) << 16));
    }
  }
}

// Step-1 causal attention with the K/V blocks shared through LDS: workgroup
// = (sequence b, KV head g, block of QB query rows) with all G query heads of
// the group, ta_waves(G, TA_FWD_WAVES) waves (head g*G + w%G, 32 rows of the
// block each).  Keys come in blocks of 64; the block's K and V rows
// ([M][Hkv][hd] row-major) are copied once into LDS by direct global -> LDS
// copies (two stages, the next block in flight while this one is computed)
// and read by every wave:
// K fragments with ds_read_b128, V^T fragments with the transpose read
// ds_read_b64_tr_b16.  16-byte chunk c of key row r sits at slot
// c ^ (r % chunks-per-row), so the 16 rows of a fragment read distinct
// banks.  The per-wave MFMA operands, P packing and chain keys are those of
// ttt_attn_kernel; the online softmax runs in base 2 with a lazily moved
// maximum (TA_RESCALE).

template <int HD, int G>
__global__ __launch_bounds__(ta_waves(G, TA_FWD_WAVES) * 64) __attribute__((amdgpu_waves_per_eu(2))) void ttt_attn_lds_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K1, const bf16* __restrict__ V1,
    const bf16* __restrict__ KC, const bf16* __restrict__ VC, int nchain, size_t chain_stride,
    bf16* __restrict__ out, int S, int hq, int hkv, float scale, float* __restrict__ lse) {
  constexpr int NC = HD / 32, NT = HD / 16, CPR = HD / 8;  // 16-byte chunks per row
  constexpr int W = ta_waves(G, TA_FWD_WAVES), RG = W / G, QB = 32 * RG, KB = 64;
  constexpr int BLK = KB * CPR;                    // 16-byte chunks per K (or V) block
  constexpr int NDMA = 2 * BLK / 64 / W;           // copies per wave per stage
  static_assert(W % G == 0 && NDMA * 64 * W == 2 * BLK, "whole row groups; copies split evenly over the waves");
  __shared__ uint4 sm[2][2][BLK];  // [stage][K, V][row * CPR + slot]
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = w % G, rg = w / G;
  const int nqb = (S + QB - 1) / QB;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
  const int g = blockIdx.y, b = blockIdx.z;
  const int h = g * G + hl;
  const int i0 = qb * QB + 32 * rg;  // the wave's first row
  const bool active = i0 < S;
  const int nkb = (min(qb * QB + QB, S) + KB - 1) / KB;
  const int ml = lane & 15, q4 = lane >> 4;
  const size_t kstride = (size_t)hkv * HD;

  const uint32_t lds0 = lds_addr(&sm[0][0][0]);
  auto issue = [&](int kb) {
    const uint32_t st_base = lds0 + (uint32_t)((kb & 1) * 2 * BLK * 16);
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const int d = w * NDMA + u;               // copy index within the stage
      const int kv = d / (BLK / 64), part = d - kv * (BLK / 64);
      const int e = part * 64 + lane;           // chunk index within the block
      const int r = e / CPR, slot = e - r * CPR;
      const int key = min(kb * KB + r, S - 1);  // rows past S are masked by causality
      const bf16* src = (kv ? V1 : K1) + ((size_t)b * S + key) * kstride + (size_t)g * HD + 8 * (slot ^ (r % CPR));
      dma16(src, st_base + (uint32_t)(kv * BLK * 16 + part * 1024));
    }
  };

  U4 qf[2][NC];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = min(i0 + 16 * nt + ml, S - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[nt][c].u = *(const uint4*)(Q + ((size_t)(b * S + i) * hq + h) * HD + 32 * c + 8 * q4);
  }
  f32x4 o[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // softmax in base 2: p = 2^(s c2 - mrun) with c2 = scale log2(e), mrun the
  // running maximum of s c2
  const float c2 = scale * LOG2EF;
  float mrun[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  issue(0);
  bg_wait_copies<0>();
  bg_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) issue(kb + 1);
    if (active && kb * KB <= i0 + 31) {
      const uint4* ks = &sm[kb & 1][0][0];
      const bf16* vs = (const bf16*)&sm[kb & 1][1][0];
      f32x4 st[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) st[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        U4 kf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int r = 16 * mt + ml, ch = 4 * c + q4;
          kf[mt].u = ks[r * CPR + (ch ^ (r % CPR))];
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            st[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt].v, qf[nt][c].v, st[mt][nt], 0, 0, 0);
      }
      const bool diag = kb * KB + 63 > i0;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int qi = i0 + 16 * nt + ml;
        float bm = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (diag && kb * KB + 16 * mt + 4 * q4 + e > qi) st[mt][nt][e] = -INFINITY;
            bm = fmaxf(bm, st[mt][nt][e]);
          }
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        // mrun (log2 units) moves only when the block's maximum exceeds it by
        // more than TA_RESCALE, so most blocks skip the rescale of o
        const float bmc = bm * c2;
        const bool upd = bmc > mrun[nt] + TA_RESCALE;
        if (__any(upd)) {
          const float mnew = upd ? bmc : mrun[nt];
          const float alpha = __builtin_amdgcn_exp2f(mrun[nt] - mnew);
          mrun[nt] = mnew;
          lsum[nt] *= alpha;
#pragma unroll
          for (int t = 0; t < NT; ++t) o[t][nt] *= alpha;
        }
        const float mneg = -mrun[nt];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(st[mt][nt][e], c2, mneg));
            st[mt][nt][e] = pv;
            lsum[nt] += pv;
          }
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        // B operand P^T: k-slots 8 q4 + e <- key 32kc + 4 q4 + e, slots 8 q4 + 4 + e <- key 32kc + 16 + 4 q4 + e
        U4 pb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) pb[nt] = pack_b_from_acc(st[2 * kc][nt], st[2 * kc + 1][nt]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // V^T fragment: dim 16t + ml, keys 32kc + 4q4 + j and 32kc + 16 + 4q4 + j (j < 4): source lane
          // s = ml of this lane group points at key 32kc + 4q4 + s/4, dims 16t + 4(s%4) .. +4
          const int r0 = 32 * kc + 4 * q4 + (ml >> 2), r1 = r0 + 16;
          const int dim = 16 * t + 4 * (ml & 3), ch = dim >> 3, off = dim & 7;
          const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (tta_lds_s16x4)(vs + (r0 * CPR + (ch ^ (r0 % CPR))) * 8 + off));
          const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (tta_lds_s16x4)(vs + (r1 * CPR + (ch ^ (r1 % CPR))) * 8 + off));
          U4 vf;
          __builtin_memcpy(&vf.u.x, &va, 8);
          __builtin_memcpy(&vf.u.z, &vb, 8);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pb[nt].v, o[t][nt], 0, 0, 0);
        }
      }
    }
    bg_wait_copies<0>();
    bg_barrier();
  }
  if (!active) return;
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
      const float sv = dot * c2;
      const float mnew = fmaxf(mrun[nt], sv);
      const float alpha = __builtin_amdgcn_exp2f(mrun[nt] - mnew), pv = __builtin_amdgcn_exp2f(sv - mnew);
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
    const int row = b * S + i0 + 16 * nt + ml;
    const int nkc = (hq * HD) >> 5;
    if (lse && q4 == 0) lse[(size_t)h * gridDim.z * S + row] = mrun[nt] * LN2F + logf(L);  // [hq][M], natural log
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 r = o[t][nt] * inv;
      *(uint2*)(out + frag_off(row, h * HD + 16 * t + 4 * q4, nkc)) =
          make_uint2((uint32_t)f2bf(r[0]) | ((uint32_t)f2bf(r[1]) << 16), (uint32_t)f2bf(r[2]) | ((uint32_t)f2bf(r[3]) << 16));
    }
  }
}

}  // namespace

size_t ttt_ws_bytes(const eagle3_dims& dm, int B, int S, int R) { return layout_of(dm, B, S, R, nullptr).bytes; }

int ttt_forward(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, const int32_t* tokens, int B, int S,
                int R, const int32_t* forced, int32_t* pred, float* ce, float* loss, void* wsp, hipStream_t st,
                TttSave* sv) {
  const int d = dm.d, hq = dm.n_q_heads, hkv = dm.n_kv_heads, hd = dm.head_dim, F = dm.ffn, V = dm.vocab;
  const int qd = hq * hd, kvd = hkv * hd;
  if (dm.dtype != EAGLE3_BF16 || (hd != 64 && hd != 128) || S % 64 != 0) return 1;
  if (d % 64 || F % 64 || qd % 64 || d > 8192 || hq % hkv) return 1;
  const int M = B * S;
  const size_t Md = (size_t)M * d;
  const TLayout L = layout_of(dm, B, S, R, wsp);
  const bool pk = w.layout == EAGLE3_LAYOUT_PACKED;
  const float eps = dm.rms_eps;
  const int nblk = ce_blocks(V);
  const RowMap plain{MAP_PLAIN, hd, F}, pair_head{MAP_PAIR_HEAD, hd, F}, pair_ffn{MAP_PAIR_FFN, hd, F};
  const int gq = hq / hkv;
  const bool lds_attn = 8 % gq == 0;  // step-1 values stay row-major for the LDS kernel
  if (sv && !lds_attn) return 1;      // the backward reads row-major step-1 values
  if (sv) {
    sv->k1 = L.k1;
    sv->v1 = L.v1t;
    sv->kc = L.kc;
    sv->vc = L.vc;
    sv->rope = L.rope;
  }
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
    E3_CHECK(bg_launch((const bf16*)feats, 3 * d, false, M, w.fc, pk, d, 3 * d, plain,
                       BEpiStoreF{sv ? sv->s : L.hs, d, true}, st));
  }
  for (int j = 1; j <= R; ++j) {
    // state buffers: in place without sv; kept per step with it
    float* s_in = sv ? sv->s + (size_t)(j - 1) * Md : L.hs;
    float* h1 = sv ? sv->h1 + (size_t)(j - 1) * Md : L.hs;
    float* s_out = sv ? sv->s + (size_t)j * Md : L.hs;
    bf16* x = sv ? sv->x + (size_t)(j - 1) * 2 * Md : L.x;
    bf16* q = sv ? sv->q + (size_t)(j - 1) * M * qd : L.q;
    bf16* a = sv ? sv->a + (size_t)(j - 1) * M * qd : L.a;
    bf16* u = sv ? sv->u + (size_t)(j - 1) * Md : L.x;
    bf16* z = sv ? sv->z + (size_t)(j - 1) * M * F : L.z;
    const int32_t* tok_in = j == 1 ? tokens : (sv ? sv->tok + (size_t)(j - 1) * M : L.tok);
    int32_t* tok_out = j == R ? nullptr : (sv ? sv->tok + (size_t)j * M : L.tok);
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_prologue((const bf16*)w.emb, tok_in, s_in, M, d, w.norm_e, w.norm_s, eps, x, st);
      E3_CHECK(hipGetLastError());
    }
    bf16* kdst = j == 1 ? L.k1 : L.kc + (size_t)(j - 2) * M * kvd;
    bf16* vdst = j == 1 ? L.v1t : L.vc + (size_t)(j - 2) * M * kvd;
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      TEpiQKV epi{q, kdst, vdst, j == 1 && !lds_attn, L.rope, hq, hkv, hd, S, j - 1};
      E3_CHECK(bg_launch(x, 2 * d, true, M, w.qkv, pk, qd + 2 * kvd, 2 * d, pair_head, epi, st));
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_ATTN, st);
      const float scale = (float)(1.0 / sqrt((double)hd));
      float* lse = sv ? sv->lse + (size_t)(j - 1) * M * hq : nullptr;
      if (lds_attn) {
        const int qbr = 32 * (ta_waves(gq, TA_FWD_WAVES) / gq);
        const dim3 grid((S + qbr - 1) / qbr, hkv, B);
#define E3_TTA(HDV, GV)                                                                     \
  ttt_attn_lds_kernel<HDV, GV><<<grid, ta_waves(GV, TA_FWD_WAVES) * 64, 0, st>>>(q, L.k1, L.v1t, L.kc, L.vc, j - 1, \
                                                                  (size_t)M * kvd, a, S, hq, hkv, scale, lse)
        if (hd == 128) {
          if (gq == 1) E3_TTA(128, 1);
          else if (gq == 2) E3_TTA(128, 2);
          else if (gq == 4) E3_TTA(128, 4);
          else E3_TTA(128, 8);
        } else {
          if (gq == 1) E3_TTA(64, 1);
          else if (gq == 2) E3_TTA(64, 2);
          else if (gq == 4) E3_TTA(64, 4);
          else E3_TTA(64, 8);
        }
#undef E3_TTA
        E3_CHECK(hipGetLastError());
      } else {
        const int wpb = gq % 4 == 0 ? 4 : (gq % 2 == 0 ? 2 : 1);
        const dim3 grid(S / 32, hq / wpb, B);
        const int threads = 64 * wpb;
        if (hd == 128)
          ttt_attn_kernel<128><<<grid, threads, 0, st>>>(q, L.k1, L.v1t, L.kc, L.vc, j - 1, (size_t)M * kvd, a, S,
                                                         hq, hkv, scale);
        else
          ttt_attn_kernel<64><<<grid, threads, 0, st>>>(q, L.k1, L.v1t, L.kc, L.vc, j - 1, (size_t)M * kvd, a, S,
                                                        hq, hkv, scale);
        E3_CHECK(hipGetLastError());
      }
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      E3_CHECK(bg_launch(a, qd, true, M, w.o, pk, d, qd, plain, BEpiAdd{s_in, h1, d}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_norm(h1, M, d, w.norm_ffn, eps, u, st);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_GEMM, st);
      BEpiSwiGLU swi{z, F, sv ? sv->gu + (size_t)(j - 1) * M * F : nullptr};
      E3_CHECK(bg_launch(u, d, true, M, w.gate_up, pk, 2 * F, d, pair_ffn, swi, st));
      E3_CHECK(bg_launch(z, F, true, M, w.down, pk, d, F, plain, BEpiAdd{h1, s_out, d}, st));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ttt_norm(s_out, M, d, w.norm_out, eps, L.x, st);
      E3_CHECK(hipGetLastError());
    }
    {
      TimedScope ts(EAGLE3_KC_TTT_CE, st);
      TEpiCE epi{L.part, L.lab, tokens, S, j, nblk};
      if (sv) {
        epi.ex = sv->dlogits;
        epi.exm = sv->exm;
        epi.ldl = sv->vp;
      }
      E3_CHECK(bg_launch(L.x, d, true, M, w.lm, pk, V, d, plain, epi, st, EAGLE3_KC_TTT_CE));
    }
    {
      TimedScope ts(EAGLE3_KC_ROWOPS, st);
      ce_merge_kernel<<<M, 256, 0, st>>>(L.part, nblk, L.lab, forced, S, R, j, pred, ce, tok_out,
                                         sv ? sv->lse_ce : nullptr);
      E3_CHECK(hipGetLastError());
    }
    if (sv) {
      // dy = dlogits . W_lm: the LM head's backward, done while the logits are at hand
      {
        TimedScope ts(EAGLE3_KC_ROWOPS, st);
        dlogits_kernel<<<M, 256, 0, st>>>(sv->dlogits, sv->exm, V, sv->vp, sv->lse_ce, L.lab, tokens, S, j,
                                          (float)(1.0 / sv->count));
        E3_CHECK(hipGetLastError());
      }
      TimedScope ts(EAGLE3_KC_TTT_BWD_GEMM, st);
      E3_CHECK(bg_launch(sv->dlogits, sv->vp, false, M, sv->lm_t, true, d, sv->vp, plain,
                         BEpiStoreF{sv->dy + (size_t)(j - 1) * Md, d, false}, st, EAGLE3_KC_TTT_BWD_GEMM));
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
