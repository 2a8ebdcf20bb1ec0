// One drafter round (fusion, decoder layer, LM head + top-k) as a sequence
// of gfx950 kernels ("EAGLE-3 精读" §1: g = FC([f_low; f_mid; f_high]); the
// one-layer draft decoder combines g or its own state with the token
// embedding; the frozen LM head gives the draft distribution).
//
// Kernel sequence of eagle3_draft_step (R = B*rows query rows):
//   prologue    x = [rms(emb[t]); rms(s)] (dtype), S = s (fp32)
//   qkv         rows GEMM (split-K partials) + qkv_finish: sum, RoPE, q -> ws,
//               k/v -> cache or tree slots   (unsplit: fused paired-RoPE epilogue)
//   attention   split-K partials + ordered merge -> a (dtype)
//   o           rows GEMM (split-K partials)
//   norm        h1 = S + sum(o partials); u = rms(h1) (dtype)
//   gate/up     rows GEMM, paired SwiGLU epilogue: z = silu(gate.u)*(up.u)
//   down        rows GEMM (split-K partials)
//   final norm  h2 = h1 + sum(down partials) -> h_tree; y = rms(h2) (dtype)
//   lm head     rows GEMM -> fp32 logits
//   top-k       partition top-k + LSE, ordered merge -> ids, lp
// Split-K partials are added in split order by the consumer, so every
// result is deterministic.
#include <string.h>

#include "common.hpp"
#include "draft.hpp"
#include "gemm_rows.hpp"
#include "rows_dma.hpp"
#include "rows_rx.hpp"
#include "kernels.hpp"
#include "layer_ops.hpp"
#include "timing.hpp"

namespace e3 {

// x = [rms(emb[t]) * ge ; rms(s) * gs], S = s.  Workgroup (row, half):
// half 0 normalises the token embedding, half 1 the state (and keeps its
// fp32 copy); the two norms are independent, so each workgroup streams half
// of the row's bytes.
template <typename T>
__global__ __launch_bounds__(RT) void prologue_kernel(
    const T* __restrict__ emb, const int32_t* __restrict__ tokens, const T* __restrict__ state,
    const float* __restrict__ h_tree, const int32_t* __restrict__ parent_slot, int mode, int rows,
    int d, const float* __restrict__ ge, const float* __restrict__ gs, float eps,
    float* __restrict__ S, T* __restrict__ x) {
  __shared__ float red[RT / 64];
  const int r = blockIdx.x, half = blockIdx.y;
  const int b = r / rows;
  float v[EPT_MAX];
  if (half == 0) {
    const T* e = emb + (size_t)tokens[r] * d;
#pragma unroll
    for (int j = 0; j < EPT_MAX; ++j) {
      const int i = threadIdx.x + RT * j;
      v[j] = i < d ? Elem<T>::ld(e, i) : 0.f;
    }
  } else {
    const float* hs = nullptr;
    if (mode == EAGLE3_TREE) hs = h_tree + ((size_t)b * (EAGLE3_MAX_TREE_SLOTS + 1) + parent_slot[r]) * d;
#pragma unroll
    for (int j = 0; j < EPT_MAX; ++j) {
      const int i = threadIdx.x + RT * j;
      v[j] = i < d ? (mode == EAGLE3_TREE ? hs[i] : Elem<T>::ld(state, (size_t)r * d + i)) : 0.f;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) ss = fmaf(v[j], v[j], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  const float* g = half == 0 ? ge : gs;
  T* xo = x + (size_t)r * 2 * d + (size_t)half * d;
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    if (i < d) {
      if (half == 1) S[(size_t)r * d + i] = v[j];
      Elem<T>::st(xo, i, v[j] * inv * g[i]);
    }
  }
}

// h2 = h1 + sum of down partials (splits > 0), or h2 already complete;
// post-norm (post_gain not NULL): h2 = rms(h2) * post_gain; h2 rows ->
// h_tree (COMMIT: last row of each request -> slot 0; TREE: row rr -> 1 +
// slot_base + rr); y = rms(h2)*gain for the rows whose top-k is taken (all
// rows, or the last row of each request), packed.
template <typename T>
__global__ __launch_bounds__(RT) void final_norm_kernel(
    const float* __restrict__ h1, const float* __restrict__ part, int splits, int R, const float* __restrict__ h2buf,
    int d, const float* __restrict__ gain, float eps, int mode, int rows, int slot_base, int topk_last,
    float* __restrict__ h_tree, T* __restrict__ y, const float* __restrict__ post_gain = nullptr) {
  __shared__ float red[RT / 64];
  const int r = blockIdx.x;
  const int b = r / rows, rr = r - b * rows;
  const bool last = rr == rows - 1;
  int hslot = -1;
  if (mode == EAGLE3_TREE) hslot = 1 + slot_base + rr;
  else if (last) hslot = 0;
  if (hslot < 0 && topk_last && !last) return;
  float v[EPT_MAX];
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    v[j] = i < d ? (splits > 0 ? h1[(size_t)r * d + i] : h2buf[(size_t)r * d + i]) : 0.f;
  }
  if (splits > 0) add_partials(v, part, splits, (size_t)R * d, (size_t)r * d, d);
  if (post_gain) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < EPT_MAX; ++j) ss = fmaf(v[j], v[j], ss);
    ss = block_sum(ss, red);
    const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
#pragma unroll
    for (int j = 0; j < EPT_MAX; ++j) {
      const int i = threadIdx.x + RT * j;
      v[j] = i < d ? v[j] * inv * post_gain[i] : 0.f;
    }
  }
  if (hslot >= 0) {
    float* dst = h_tree + ((size_t)b * (EAGLE3_MAX_TREE_SLOTS + 1) + hslot) * d;
#pragma unroll
    for (int j = 0; j < EPT_MAX; ++j) {
      const int i = threadIdx.x + RT * j;
      if (i < d) dst[i] = v[j];
    }
  }
  if (topk_last && !last) return;
  const int yr = topk_last ? b : r;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) ss = fmaf(v[j], v[j], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    if (i < d) Elem<T>::st(y, (size_t)yr * d + i, v[j] * inv * gain[i]);
  }
}

// FC norm: g = rms(sum of fusion partials) * gain, rounded once; one
// workgroup per row (partials [splits][n][d])
template <typename T>
__global__ __launch_bounds__(RT) void fuse_norm_kernel(const float* __restrict__ part, int splits, int n, int d,
                                                       const float* __restrict__ gain, float eps, T* __restrict__ g) {
  __shared__ float red[RT / 64];
  const int r = blockIdx.x;
  float v[EPT_MAX];
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) v[j] = 0.f;
  add_partials(v, part, splits, (size_t)n * d, (size_t)r * d, d);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) ss = fmaf(v[j], v[j], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
#pragma unroll
  for (int j = 0; j < EPT_MAX; ++j) {
    const int i = threadIdx.x + RT * j;
    if (i < d) Elem<T>::st(g, (size_t)r * d + i, v[j] * inv * gain[i]);
  }
}

// g = round(sum of fusion partials)
template <typename T>
__global__ __launch_bounds__(256) void fuse_finish_kernel(const float* __restrict__ part, int splits, int n, int d,
                                                          T* __restrict__ g) {
  const size_t total = (size_t)n * d;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    float p[16];
    float acc = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 16) {
      const int ns = min(16, splits - s0);
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < ns) p[s] = part[(size_t)(s0 + s) * total + e];
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < ns) acc += p[s];
    }
    Elem<T>::st(g, e, acc);
  }
}

// ---------------------------------------------------------------------------
// LM head with top-1 folded in (no split-K, logits not kept): per X row and
// workgroup (its NB*16 vocabulary columns) write {max, sum exp(x - max),
// lowest column holding the max}.  Thread t takes row t%64 and column part
// t/64 of blockDim/64 equal parts (a wave reads one LDS column slice of all
// rows: conflict-free); the parts meet in LDS and are combined in order.
struct EpiTop1Part {
  static constexpr bool kWhole = true;
  float4* part;  // [R][nwg]
  int nwg;
  __device__ void whole(int wg, const float* tile, int RP, int R, int NB, int ntiles16, float* scratch,
                        int) const {
    float4* red = (float4*)scratch;  // [blockDim/64][64]
    const int t = threadIdx.x, r = t & 63, q = t >> 6, nq = blockDim.x >> 6;
    const int qw = NB * 16 / nq;  // columns per part
    float mx = -INFINITY;
    int id = 0x7fffffff;
    float s = 0.f;
    if (r < R) {
      // columns past the vocabulary exist only in the last workgroup
      const int c0 = q * qw, c1 = min((q + 1) * qw, (ntiles16 - wg * NB) * 16);
      const float* col = tile + r;
      if (c1 - c0 == qw && (qw & 7) == 0) {
        for (int c = c0; c < c1; c += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = col[(c + u) * RP];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (v[u] > mx) {
              mx = v[u];
              id = (wg * NB) * 16 + c + u;
            }
        }
        if (mx > -INFINITY)
          for (int c = c0; c < c1; c += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = col[(c + u) * RP];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += __expf(v[u] - mx);
          }
      } else {
        for (int c = c0; c < c1; ++c) {
          const float v = col[c * RP];
          if (v > mx) {
            mx = v;
            id = (wg * NB) * 16 + c;
          }
        }
        if (mx > -INFINITY)
          for (int c = c0; c < c1; ++c) s += __expf(col[c * RP] - mx);
      }
    }
    red[q * 64 + r] = make_float4(mx, s, __int_as_float(id), 0.f);
    __syncthreads();
    if (q == 0 && r < R) {
      float gm = -INFINITY;
      int gi = 0x7fffffff;
      for (int u = 0; u < nq; ++u) {
        const float4 c = red[u * 64 + r];
        if (better(c.x, __float_as_int(c.z), gm, gi)) {
          gm = c.x;
          gi = __float_as_int(c.z);
        }
      }
      float gs = 0.f;
      for (int u = 0; u < nq; ++u) {
        const float4 c = red[u * 64 + r];
        if (c.x > -INFINITY) gs += c.y * __expf(c.x - gm);
      }
      part[(size_t)r * nwg + wg] = make_float4(gm, gs, __int_as_float(gi), 0.f);
    }
  }
};

// GEMM shapes of a draft step: qkv, o, gate_up, down, lm, and the fusion fc.
struct Shapes {
  int n[6], k[6];
  bool split[6];
};
static Shapes shapes_of(const eagle3_dims& dm) {
  const int d = dm.d, F = dm.ffn, qd = dm.n_q_heads * dm.head_dim;
  const int nqkv = (dm.n_q_heads + 2 * dm.n_kv_heads) * dm.head_dim;
  Shapes s{{nqkv, d, 2 * F, d, dm.vocab, d}, {2 * d, qd, d, F, d, 3 * d}, {true, true, false, true, false, true}};
  return s;
}

static size_t max_partials(const eagle3_dims& dm, int R) {
  const bool bf = dm.dtype == EAGLE3_BF16;
  const Shapes sh = shapes_of(dm);
  size_t m = 0;
  for (int i = 0; i < 6; ++i) {
    for (int pk = 0; pk < 2; ++pk) {
      const size_t f = rows_partial_floats(plan_rows(R, sh.n[i], sh.k[i], bf, sh.split[i], pk), R, sh.n[i]);
      if (f > m) m = f;
    }
  }
  return m;
}

struct DraftWS {
  float* part;
  float* S;
  void* x;
  void* q;
  float* part_o;
  float* part_ml;
  void* a;
  float* h1;
  void* u;
  void* z;
  float* h2;
  void* y;
  float* logits;
  void* topk;  // not used by the draft step: keeps eagle3_topk covered for R rows
  void* lmpart;  // LM-head partials: top-1 float4 [R][V/128 or V/512], or tile float2 [R][V/16 + pad]
  void* lrz;     // efficient head: z = B y [R][rank <= d] (dtype)
  int32_t* cand;  // efficient head: candidate ids [R][c <= 256]
  float* cand_l;  // efficient head: their exact logits [R][c]
};

static size_t layout_draft(const eagle3_dims& dm, int R, int cap_rows, void* base, DraftWS* w) {
  const size_t es = dm.dtype == EAGLE3_BF16 ? 2 : 4;
  const int qd = dm.n_q_heads * dm.head_dim;
  const int nch = attn_num_chunks(cap_rows);
  Bump bp;
  bp.base = (unsigned char*)base;
  DraftWS t;
  t.part = (float*)bp.take(max_partials(dm, R) * 4);
  t.S = (float*)bp.take((size_t)R * dm.d * 4);
  t.x = bp.take((size_t)R * 2 * dm.d * es);
  t.q = bp.take((size_t)R * qd * es);
  t.part_o = (float*)bp.take((size_t)R * dm.n_q_heads * nch * dm.head_dim * 4);
  t.part_ml = (float*)bp.take((size_t)R * dm.n_q_heads * nch * 2 * 4);
  t.a = bp.take((size_t)R * qd * es);
  t.h1 = (float*)bp.take((size_t)R * dm.d * 4);
  t.u = bp.take((size_t)R * dm.d * es);
  t.z = bp.take((size_t)R * dm.ffn * es);
  t.h2 = (float*)bp.take((size_t)R * dm.d * 4);
  t.y = bp.take((size_t)R * dm.d * es);
  t.logits = (float*)bp.take((size_t)R * dm.vocab * 4);
  t.topk = bp.take(topk_ws_bytes(R, dm.vocab));
  // top-1 float4 [R][one per workgroup of 8 or 32 tiles] or tile pairs
  // float2 [R][V/16 + up to 8*tpw - 1 slots of padding, tpw <= 32]
  t.lmpart = bp.take((size_t)R * (dm.vocab / 16 + 256) * sizeof(float2));
  t.lrz = bp.take((size_t)R * dm.d * es);
  t.cand = (int32_t*)bp.take((size_t)R * LOWRANK_MAX_CAND * 4);
  t.cand_l = (float*)bp.take((size_t)R * LOWRANK_MAX_CAND * 4);
  if (w) *w = t;
  return bp.off + 256;
}

size_t draft_ws_bytes(const eagle3_dims& dm, int B, int max_rows, int max_ctx) {
  const size_t a = layout_draft(dm, B * max_rows, max_ctx + max_rows, nullptr, nullptr);
  const size_t f = fuse_ws_bytes(dm, B * max_rows);
  return a > f ? a : f;
}

// split-K partials, or (FC norm without a split) the float32 projection [n][d]
size_t fuse_ws_bytes(const eagle3_dims& dm, int n) {
  const size_t p = max_partials(dm, n), f = (size_t)n * dm.d;
  return (p > f ? p : f) * 4 + 512;
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t fuse_impl(const eagle3_dims& dm, const eagle3_weights& w, const void* feats,
                            int n, void* g, void* ws, hipStream_t st) {
  const int K = 3 * dm.d;
  RowMap map{MAP_PLAIN, dm.head_dim, dm.ffn};
  const bool pk = w.layout == EAGLE3_LAYOUT_PACKED;
  TimedScope ts(EAGLE3_KC_FUSE, st);
  const RowsPlan p = plan_rows(n, dm.d, K, sizeof(T) == 2, true, pk);
  if (p.splits > 1) {  // n <= 64
    EpiPartial epi{(float*)ws, dm.d, map};
    hipError_t e = rows_gemm<T>((const T*)feats, K, n, (const T*)w.fc, K, dm.d, map, epi, p, pk, st);
    if (e != hipSuccess) return e;
    if (w.norm_fc) {
      fuse_norm_kernel<T><<<n, RT, 0, st>>>((const float*)ws, p.splits, n, dm.d, w.norm_fc, dm.rms_eps, (T*)g);
      return hipGetLastError();
    }
    int blocks = (int)(((size_t)n * dm.d + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    fuse_finish_kernel<T><<<blocks, 256, 0, st>>>((const float*)ws, p.splits, n, dm.d, (T*)g);
    return hipGetLastError();
  }
  for (int r0 = 0; r0 < n; r0 += 64) {
    const int R = n - r0 < 64 ? n - r0 : 64;
    const RowsPlan pc = plan_rows(R, dm.d, K, sizeof(T) == 2, false);
    hipError_t e;
    if (w.norm_fc) {  // float32 projection into the workspace, normalised below
      EpiStore<float> epi{(float*)ws + (size_t)r0 * dm.d, dm.d, map};
      e = rows_gemm<T>((const T*)feats + (size_t)r0 * K, K, R, (const T*)w.fc, K, dm.d, map, epi, pc, pk, st);
    } else {
      EpiStore<T> epi{(T*)g + (size_t)r0 * dm.d, dm.d, map};
      e = rows_gemm<T>((const T*)feats + (size_t)r0 * K, K, R, (const T*)w.fc, K, dm.d, map, epi, pc, pk, st);
    }
    if (e != hipSuccess) return e;
  }
  if (w.norm_fc) {
    fuse_norm_kernel<T><<<n, RT, 0, st>>>((const float*)ws, 1, n, dm.d, w.norm_fc, dm.rms_eps, (T*)g);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t fuse_rows(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, int n,
                     void* g, void* ws, hipStream_t st) {
  return dm.dtype == EAGLE3_BF16 ? fuse_impl<bf16>(dm, w, feats, n, g, ws, st)
                                 : fuse_impl<float>(dm, w, feats, n, g, ws, st);
}

template <typename T>
static hipError_t draft_impl(const DraftCall& c, hipStream_t st) {
  const eagle3_dims& dm = *c.dims;
  const eagle3_weights& w = *c.w;
  const eagle3_kv& kv = *c.kv;
  const bool bf = sizeof(T) == 2;
  const int d = dm.d, hd = dm.head_dim, hq = dm.n_q_heads, hkv = dm.n_kv_heads, F = dm.ffn;
  const int V = dm.vocab;
  const int R = c.B * c.rows;
  const int qd = hq * hd;
  const int cap_rows = kv.block_table ? kv.max_blocks * kv.block_size : kv.cap;
  DraftWS ws;
  layout_draft(dm, R, cap_rows, c.ws, &ws);
  hipError_t e;
  const RowMap plain{MAP_PLAIN, hd, F};
  const RowMap pair_head{MAP_PAIR_HEAD, hd, F};
  const bool pk = w.layout == EAGLE3_LAYOUT_PACKED;

  const int topk_last = c.topk_rows == EAGLE3_TOPK_LAST;
  const int Rl = topk_last ? c.B : R;  // rows through the LM head and top-k
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    prologue_kernel<T><<<dim3(R, 2), RT, 0, st>>>((const T*)w.emb, c.tokens, (const T*)c.state, c.h_tree,
                                                  c.parent_slot, c.mode, c.rows, d, w.norm_e, w.norm_s, dm.rms_eps,
                                                  ws.S, (T*)ws.x);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // ---- QKV + RoPE + KV write
  const int nqkv = (hq + 2 * hkv) * hd;
  KVDest dst{kv.k, kv.v, kv.tk, kv.tv, kv.ctx_len, kv.block_table, kv.cap, kv.max_blocks, kv.block_size,
             c.rows, c.mode, c.slot_base, hkv, hd, 0};
  {
    TimedScope ts(EAGLE3_KC_QKV, st);
    const RowsPlan p = plan_rows(R, nqkv, 2 * d, bf, true, pk);
    if (p.splits > 1) {
      EpiPartial epi{ws.part, nqkv, pair_head};
      if ((e = rows_gemm<T>((const T*)ws.x, 2 * d, R, (const T*)w.qkv, 2 * d, nqkv, pair_head, epi, p, pk, st)) !=
          hipSuccess)
        return e;
      qkv_finish_kernel<T><<<dim3(R, hq + 2 * hkv), 64, 0, st>>>(ws.part, p.splits, R, nqkv, c.pos, dst, (T*)ws.q,
                                                                 hq, dm.rope_theta);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      for (int r0 = 0; r0 < R; r0 += 64) {
        const int Rc = R - r0 < 64 ? R - r0 : 64;
        RowMap map{MAP_PAIR_HEAD, hd, F};
        EpiQKV<T> epi;
        epi.q_out = (T*)ws.q + (size_t)r0 * qd;
        epi.pos = c.pos + r0;
        epi.dst = dst;
        epi.dst.row0 = r0;
        epi.hq = hq;
        epi.theta = dm.rope_theta;
        const RowsPlan pc = plan_rows(Rc, nqkv, 2 * d, bf, false);
        if ((e = rows_gemm<T>((const T*)ws.x + (size_t)r0 * 2 * d, 2 * d, Rc, (const T*)w.qkv, 2 * d, nqkv, map, epi,
                              pc, pk, st)) != hipSuccess)
          return e;
      }
    }
  }
  // ---- attention
  AttnLaunch al;
  al.q = ws.q;
  al.kc = kv.k;
  al.vc = kv.v;
  al.tk = kv.tk;
  al.tv = kv.tv;
  al.ctx_len = kv.ctx_len;
  al.block_table = kv.block_table;
  al.anc = c.anc;
  al.cap = kv.cap;
  al.max_blocks = kv.max_blocks;
  al.block_size = kv.block_size;
  al.cap_rows = cap_rows;
  al.B = c.B;
  al.rows = c.rows;
  al.hq = hq;
  al.hkv = hkv;
  al.hd = hd;
  al.mode = c.mode;
  al.bf16 = bf;
  al.part_o = ws.part_o;
  al.part_ml = ws.part_ml;
  al.out = ws.a;
  {
    TimedScope ts(EAGLE3_KC_ATTN, st);
    if ((e = launch_attention(al, st)) != hipSuccess) return e;
  }
  // ---- O projection (+ residual in the FFN norm)
  int o_splits = 0;
  {
    TimedScope ts(EAGLE3_KC_O, st);
    const RowsPlan p = plan_rows(R, d, qd, bf, true, pk);
    if (p.splits > 1) {
      EpiPartial epi{ws.part, d, plain};
      if ((e = rows_gemm<T>((const T*)ws.a, qd, R, (const T*)w.o, qd, d, plain, epi, p, pk, st)) != hipSuccess) return e;
      o_splits = p.splits;
    } else {
      for (int r0 = 0; r0 < R; r0 += 64) {
        const int Rc = R - r0 < 64 ? R - r0 : 64;
        EpiResidual epi{ws.h1 + (size_t)r0 * d, ws.S + (size_t)r0 * d, d};
        const RowsPlan pc = plan_rows(Rc, d, qd, bf, false);
        if ((e = rows_gemm<T>((const T*)ws.a + (size_t)r0 * qd, qd, Rc, (const T*)w.o, qd, d, plain, epi, pc, pk, st)) !=
            hipSuccess)
          return e;
      }
    }
  }
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    const bool post = w.norm_post_attn != nullptr;
    ffn_norm_kernel<T><<<R, RT, 0, st>>>(ws.S, ws.part, o_splits, R, d, post ? w.norm_post_attn : w.norm_ffn,
                                         dm.rms_eps, ws.h1, (T*)ws.u, post);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // ---- gate/up + SwiGLU
  {
    TimedScope ts(EAGLE3_KC_GATEUP, st);
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int Rc = R - r0 < 64 ? R - r0 : 64;
      RowMap pf{MAP_PAIR_FFN, hd, F};
      EpiSwiGLU<T> epi{(T*)ws.z + (size_t)r0 * F, F};
      const RowsPlan pc = plan_rows(Rc, 2 * F, d, bf, false);
      if ((e = rows_gemm_gate_up<T>((const T*)ws.u + (size_t)r0 * d, d, Rc, (const T*)w.gate_up, d, 2 * F, pf, epi, pc,
                                    pk, st)) != hipSuccess)
        return e;
    }
  }
  // ---- down (+ residual in the final norm)
  int down_splits = 0;
  {
    TimedScope ts(EAGLE3_KC_DOWN, st);
    const RowsPlan p = plan_rows(R, d, F, bf, true, pk);
    if (p.splits > 1) {
      EpiPartial epi{ws.part, d, plain};
      if ((e = rows_gemm<T>((const T*)ws.z, F, R, (const T*)w.down, F, d, plain, epi, p, pk, st)) != hipSuccess) return e;
      down_splits = p.splits;
    } else {
      for (int r0 = 0; r0 < R; r0 += 64) {
        const int Rc = R - r0 < 64 ? R - r0 : 64;
        EpiResidual epi{ws.h2 + (size_t)r0 * d, ws.h1 + (size_t)r0 * d, d};
        const RowsPlan pc = plan_rows(Rc, d, F, bf, false);
        if ((e = rows_gemm<T>((const T*)ws.z + (size_t)r0 * F, F, Rc, (const T*)w.down, F, d, plain, epi, pc, pk, st)) !=
            hipSuccess)
          return e;
      }
    }
  }
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    final_norm_kernel<T><<<R, RT, 0, st>>>(ws.h1, ws.part, down_splits, R, ws.h2, d, w.norm_out, dm.rms_eps, c.mode,
                                           c.rows, c.slot_base, topk_last, c.h_tree, (T*)ws.y, w.norm_post_ffn);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // ---- LM head + top-k
  float* logits = c.logits_out ? c.logits_out : ws.logits;
  if (c.lr) {
    // efficient head: z = B y, scores = A z with tile statistics, the c best
    // scores as candidates, exact logits of the candidates, their top-k
    const eagle3_lowrank_head& lr = *c.lr;
    const bool lpk = lr.layout == EAGLE3_LAYOUT_PACKED;
    const int r = lr.rank, nt16 = V / 16;
    int32_t* cand = c.cand_out ? c.cand_out : ws.cand;
    float* cand_l = c.cand_logits_out ? c.cand_logits_out : ws.cand_l;
    {
      TimedScope ts(EAGLE3_KC_LMHEAD, st);
      const RowsPlan pz = plan_rows(Rl, r, d, bf, false);
      EpiStore<T> ez{(T*)ws.lrz, r, plain};
      if ((e = rows_gemm<T>((const T*)ws.y, d, Rl, (const T*)lr.b, d, r, plain, ez, pz, lpk, st)) != hipSuccess)
        return e;
      RowsPlan ps = plan_rows(Rl, V, r, bf, false);
      // packed factors, up to 16 rows, rank 64/128/256: wave-owned tiles over
      // the short K (the rank), no cross-wave reduction (lowrank.hip)
      const bool own = bf && lpk && Rl <= 16 && (r == 64 || r == 128 || r == 256);
      // packed factors, 17..64 rows: the register-weight kernel
      const bool rx = !own && bf && lpk && Rl <= 64 && r % (32 * LM_RX_KU) == 0;
      // row-major factors up to 16 rows: eight tiles per workgroup, one 32-wide
      // k-group per wave, so that all eight waves stream
      const bool small_k = !own && !rx && bf && Rl <= 16;
      if (small_k) {
        ps.t = 8;
        ps.u = 1;
        ps.waves = 8;
        ps.splits = 1;
        ps.tiles = (nt16 + 7) / 8;
      }
      const int tpw = own ? lowrank_scores_tpw() : rx ? LM_RX_TPW : bf && sk_ok(Rl, r, lpk) ? sk_bn(nt16, 1) / 16
                                                                                              : ps.t;
      float2* tpart = (float2*)ws.lmpart;
      EpiLogitsTiles es{logits, V, tpart, tile_slots(nt16, tpw)};
      if (own) {
        TimedScope ts2(EAGLE3_KC_LR_SCORES, st);
        if ((e = launch_lowrank_scores(lr.a, ws.lrz, Rl, r, V, logits, tpart, st)) != hipSuccess) return e;
      } else if (rx) {
        rx_gemm_kernel<LM_RX_WT, LM_RX_KU, EpiLogitsTiles, LM_RX_WAVES>
            <<<(nt16 + tpw - 1) / tpw, LM_RX_WAVES * 64, 0, st>>>((const bf16*)ws.lrz, r, Rl, (const bf16*)lr.a, r,
                                                                   nt16, 1, es, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      } else if (small_k) {
        if constexpr (sizeof(T) == 2) {
          if ((e = rows_gemm_launch<T, 8, 1, 1, 8>((const T*)ws.lrz, r, Rl, (const T*)lr.a, r, V, plain, es, ps, lpk,
                                                   st)) != hipSuccess)
            return e;
        }
      } else if ((e = rows_gemm<T>((const T*)ws.lrz, r, Rl, (const T*)lr.a, r, V, plain, es, ps, lpk, st)) !=
                 hipSuccess) {
        return e;
      }
      if ((e = launch_lowrank_select(logits, tpart, tpw, Rl, V, lr.candidates, cand, st)) != hipSuccess) return e;
    }
    TimedScope ts(EAGLE3_KC_TOPK, st);
    return launch_lowrank_exact(w.lm, pk, ws.y, Rl, d, V, lr.candidates, c.k, cand, cand_l, c.topk_id, c.topk_lp,
                                st);
  }
  // top-1 without kept logits on the skinny GEMM: the LM head writes per-
  // workgroup (max, sum exp, argmax) partials instead of the logits
  if (c.k == 1 && !c.logits_out && bf && Rl <= 64 && sk_ok(Rl, d, pk)) {
    const int nt16 = V / 16;
    const bool rx = lm_rx_ok(Rl, d, pk);
    const int tpw = rx ? LM_RX_TPW : sk_bn(nt16, 1) / 16;
    const int nwg = (nt16 + tpw - 1) / tpw;
    {
      TimedScope ts(EAGLE3_KC_LMHEAD, st);
      EpiTop1Part epi{(float4*)ws.lmpart, nwg};
      const bf16* Xb = (const bf16*)ws.y;
      const bf16* Wb = (const bf16*)w.lm;
      constexpr int KL = EAGLE3_KC_LMHEAD;
      if (rx)
        launch_timed(KL, rx_gemm_kernel<LM_RX_WT, LM_RX_KU, EpiTop1Part, LM_RX_WAVES>, dim3(nwg),
                     dim3(LM_RX_WAVES * 64), 0, st, Xb, d, Rl, Wb, d, nt16, 1, epi, 1);
      else if (tpw == 8)
        launch_timed(KL, skinny_gemm_kernel<128, EpiTop1Part>, dim3(nwg), dim3(256), 0, st, Xb, d, Rl, Wb, d, nt16, 1,
                     epi);
      else
        launch_timed(KL, skinny_gemm_kernel<64, EpiTop1Part>, dim3(nwg), dim3(256), 0, st, Xb, d, Rl, Wb, d, nt16, 1,
                     epi);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    TimedScope ts(EAGLE3_KC_TOPK, st);
    return launch_top1_merge((const float4*)ws.lmpart, Rl, nwg, c.topk_id, c.topk_lp, st);
  }
  // up to 64 rows: the LM head writes the logits and each 16-column tile's
  // {max, sum exp} per row; the top-k reads the pairs and only the logits of
  // the tiles that can hold one of the k best
  if (Rl <= 64) {
    const int nt16 = V / 16;
    const RowsPlan pc = plan_rows(Rl, V, d, bf, false);
    const bool rx = bf && lm_rx_ok(Rl, d, pk);
    // tiles per workgroup, as dispatched
    const int tpw = rx ? LM_RX_TPW : bf && sk_ok(Rl, d, pk) ? sk_bn(nt16, 1) / 16 : pc.t;
    float2* tpart = (float2*)ws.lmpart;
    {
      TimedScope ts(EAGLE3_KC_LMHEAD, st);
      EpiLogitsTiles epi{logits, V, tpart, tile_slots(nt16, tpw)};
      if (rx) {
        launch_timed(EAGLE3_KC_LMHEAD, rx_gemm_kernel<LM_RX_WT, LM_RX_KU, EpiLogitsTiles, LM_RX_WAVES>,
                     dim3((nt16 + tpw - 1) / tpw), dim3(LM_RX_WAVES * 64), 0, st, (const bf16*)ws.y, d, Rl,
                     (const bf16*)w.lm, d, nt16, 1, epi, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      } else if ((e = rows_gemm<T>((const T*)ws.y, d, Rl, (const T*)w.lm, d, V, plain, epi, pc, pk, st,
                                   EAGLE3_KC_LMHEAD)) != hipSuccess) {
        return e;
      }
    }
    TimedScope ts(EAGLE3_KC_TOPK, st);
    return launch_topk_tiles(logits, tpart, tpw, Rl, V, c.k, c.topk_id, c.topk_lp, st);
  }
  {
    TimedScope ts(EAGLE3_KC_LMHEAD, st);
    for (int r0 = 0; r0 < Rl; r0 += 64) {
      const int Rc = Rl - r0 < 64 ? Rl - r0 : 64;
      EpiStore<float> epi{logits + (size_t)r0 * V, V, plain};
      const RowsPlan pc = plan_rows(Rc, V, d, bf, false);
      if ((e = rows_gemm<T>((const T*)ws.y + (size_t)r0 * d, d, Rc, (const T*)w.lm, d, V, plain, epi, pc, pk, st,
                            EAGLE3_KC_LMHEAD)) != hipSuccess)
        return e;
    }
  }
  TimedScope ts(EAGLE3_KC_TOPK, st);
  return launch_topk(logits, Rl, V, c.k, c.topk_id, c.topk_lp, nullptr, ws.topk, st);
}

hipError_t draft_step(const DraftCall& c, hipStream_t st) {
  return c.dims->dtype == EAGLE3_BF16 ? draft_impl<bf16>(c, st) : draft_impl<float>(c, st);
}

}  // namespace e3
