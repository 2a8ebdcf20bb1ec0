// One drafter round (fusion, decoder layer, LM head + top-k) as a sequence
// of gfx950 kernels ("EAGLE-3 精读" §1: g = FC([f_low; f_mid; f_high]); the
// one-layer draft decoder combines g or its own state with the token
// embedding; the frozen LM head gives the draft distribution).
//
// Kernel sequence of eagle3_draft_step (R = B*rows query rows):
//   prologue   x = [rms(emb[t]); rms(s)] (dtype), S = s (fp32)
//   qkv        rows GEMM, paired-RoPE epilogue; q -> ws, k/v -> cache/slots
//   attention  split-K partials + ordered merge -> a (dtype)
//   o          rows GEMM, residual epilogue: h1 = S + o.a
//   norm       u = rms(h1) (dtype)
//   gate/up    rows GEMM, paired SwiGLU epilogue: z = silu(gate.u)*(up.u)
//   down       rows GEMM, residual epilogue: h2 = h1 + down.z
//   final norm h2 -> h_tree slots; y = rms(h2) of the top-k rows (dtype)
//   lm head    rows GEMM -> fp32 logits
//   top-k      partition top-k + LSE, ordered merge -> ids, lp
#include <string.h>

#include "common.hpp"
#include "draft.hpp"
#include "gemm_rows.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace e3 {

constexpr int ROW_THREADS = 256;

// ---------------------------------------------------------------------------
// row kernels
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void prologue_kernel(
    const T* __restrict__ emb, const int32_t* __restrict__ tokens, const T* __restrict__ state,
    const float* __restrict__ h_tree, const int32_t* __restrict__ parent_slot, int mode, int rows,
    int d, const float* __restrict__ ge, const float* __restrict__ gs, float eps,
    float* __restrict__ S, T* __restrict__ x) {
  __shared__ float red[ROW_THREADS / 64];
  const int r = blockIdx.x;
  const int b = r / rows;
  const T* e = emb + (size_t)tokens[r] * d;
  const float* hs = nullptr;
  if (mode == EAGLE3_TREE) hs = h_tree + ((size_t)b * (EAGLE3_MAX_TREE_SLOTS + 1) + parent_slot[r]) * d;
  float se = 0.f, ss = 0.f;
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) {
    const float ev = Elem<T>::ld(e, i);
    const float sv = mode == EAGLE3_TREE ? hs[i] : Elem<T>::ld(state, (size_t)r * d + i);
    se = fmaf(ev, ev, se);
    ss = fmaf(sv, sv, ss);
    S[(size_t)r * d + i] = sv;
  }
  se = block_sum(se, red);
  ss = block_sum(ss, red);
  const float ie = (float)(1.0 / sqrt((double)se / d + (double)eps));
  const float is = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) {
    const float ev = Elem<T>::ld(e, i);
    const float sv = mode == EAGLE3_TREE ? hs[i] : Elem<T>::ld(state, (size_t)r * d + i);
    Elem<T>::st(x, (size_t)r * 2 * d + i, ev * ie * ge[i]);
    Elem<T>::st(x, (size_t)r * 2 * d + d + i, sv * is * gs[i]);
  }
}

// out[r] = rms(in[r]) * gain (dtype)
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void rms_rows_kernel(const float* __restrict__ in, int d,
                                                               const float* __restrict__ gain,
                                                               float eps, T* __restrict__ out) {
  __shared__ float red[ROW_THREADS / 64];
  const int r = blockIdx.x;
  const float* v = in + (size_t)r * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) ss = fmaf(v[i], v[i], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) Elem<T>::st(out, (size_t)r * d + i, v[i] * inv * gain[i]);
}

// h2 rows -> h_tree (COMMIT: last row of each request -> slot 0; TREE: row
// rr -> 1 + slot_base + rr) and y = rms(h2)*gain for the rows whose top-k is
// taken (all rows, or the last row of each request), packed.
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void final_rows_kernel(
    const float* __restrict__ h2, int d, const float* __restrict__ gain, float eps, int mode,
    int rows, int slot_base, int topk_last, float* __restrict__ h_tree, T* __restrict__ y) {
  __shared__ float red[ROW_THREADS / 64];
  const int r = blockIdx.x;
  const int b = r / rows, rr = r - b * rows;
  const float* v = h2 + (size_t)r * d;
  const bool last = rr == rows - 1;
  int hslot = -1;
  if (mode == EAGLE3_TREE) hslot = 1 + slot_base + rr;
  else if (last) hslot = 0;
  if (hslot >= 0) {
    float* dst = h_tree + ((size_t)b * (EAGLE3_MAX_TREE_SLOTS + 1) + hslot) * d;
    for (int i = threadIdx.x; i < d; i += ROW_THREADS) dst[i] = v[i];
  }
  if (topk_last && !last) return;
  const int yr = topk_last ? b : r;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) ss = fmaf(v[i], v[i], ss);
  ss = block_sum(ss, red);
  const float inv = (float)(1.0 / sqrt((double)ss / d + (double)eps));
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) Elem<T>::st(y, (size_t)yr * d + i, v[i] * inv * gain[i]);
}

// ---------------------------------------------------------------------------
// rows-GEMM dispatch.  The epilogue sees rows 0..R-1 of one launch; row
// chunks beyond 64 are launched separately with shifted pointers.
template <typename TW, int T, int NT, int U, int WAVES, class Epi>
static hipError_t rows_gemm_launch(const TW* X, int ldx, int R, const TW* W, int K, int N,
                                   RowMap map, const Epi& epi, hipStream_t st) {
  const int nt16 = N / 16;
  const int grid = (nt16 + T - 1) / T;
  const size_t lds = sizeof(TW) == 2 ? (size_t)WAVES * T * NT * 256 * sizeof(float) : 0;
  rows_gemm_kernel<TW, T, NT, U, WAVES, Epi><<<grid, WAVES * 64, lds, st>>>(X, ldx, R, W, K, K, nt16, map, epi);
  return hipGetLastError();
}

template <typename TW, class Epi>
static hipError_t rows_gemm(const TW* X, int ldx, int R, const TW* W, int K, int N, RowMap map,
                            const Epi& epi, hipStream_t st) {
  if (sizeof(TW) == 2) {
    if (R <= 16) return rows_gemm_launch<TW, 2, 1, 8, 4>(X, ldx, R, W, K, N, map, epi, st);
    if (R <= 32) return rows_gemm_launch<TW, 1, 2, 8, 4>(X, ldx, R, W, K, N, map, epi, st);
    if (R <= 48) return rows_gemm_launch<TW, 1, 3, 8, 4>(X, ldx, R, W, K, N, map, epi, st);
    return rows_gemm_launch<TW, 1, 4, 8, 4>(X, ldx, R, W, K, N, map, epi, st);
  }
  if (R <= 16) return rows_gemm_launch<TW, 1, 1, 1, 4>(X, ldx, R, W, K, N, map, epi, st);
  return rows_gemm_launch<TW, 1, 4, 1, 4>(X, ldx, R, W, K, N, map, epi, st);
}

// ---------------------------------------------------------------------------
// Workspace layout (shared by the size query and the calls).
struct Bump {
  size_t off = 0;
  unsigned char* base = nullptr;
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

struct DraftWS {
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
  void* topk;
};

static size_t layout_draft(const eagle3_dims& dm, int R, int cap_rows, void* base, DraftWS* w) {
  const size_t es = dm.dtype == EAGLE3_BF16 ? 2 : 4;
  const int qd = dm.n_q_heads * dm.head_dim;
  const int nch = attn_num_chunks(cap_rows);
  Bump bp;
  bp.base = (unsigned char*)base;
  DraftWS t;
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
  // fusion reuses the same memory: g needs nothing beyond the GEMM itself
  if (w) *w = t;
  return bp.off + 256;
}

size_t draft_ws_bytes(const eagle3_dims& dm, int B, int max_rows, int max_ctx) {
  return layout_draft(dm, B * max_rows, max_ctx + max_rows, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t fuse_impl(const eagle3_dims& dm, const eagle3_weights& w, const void* feats,
                            int n, void* g, hipStream_t st) {
  const int K = 3 * dm.d;
  RowMap map{MAP_PLAIN, dm.head_dim, dm.ffn};
  TimedScope ts(EAGLE3_KC_FUSE, st);
  for (int r0 = 0; r0 < n; r0 += 64) {
    const int R = n - r0 < 64 ? n - r0 : 64;
    EpiStore<T> epi{(T*)g + (size_t)r0 * dm.d, dm.d, map};
    hipError_t e = rows_gemm<T>((const T*)feats + (size_t)r0 * K, K, R, (const T*)w.fc, K, dm.d, map, epi, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t fuse_rows(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, int n,
                     void* g, hipStream_t st) {
  return dm.dtype == EAGLE3_BF16 ? fuse_impl<bf16>(dm, w, feats, n, g, st)
                                 : fuse_impl<float>(dm, w, feats, n, g, st);
}

template <typename T>
static hipError_t draft_impl(const DraftCall& c, hipStream_t st) {
  const eagle3_dims& dm = *c.dims;
  const eagle3_weights& w = *c.w;
  const eagle3_kv& kv = *c.kv;
  const int d = dm.d, hd = dm.head_dim, hq = dm.n_q_heads, hkv = dm.n_kv_heads, F = dm.ffn;
  const int V = dm.vocab;
  const int R = c.B * c.rows;
  const int qd = hq * hd;
  const int cap_rows = kv.block_table ? kv.max_blocks * kv.block_size : kv.cap;
  DraftWS ws;
  layout_draft(dm, R, cap_rows, c.ws, &ws);
  hipError_t e;

  {
  TimedScope ts(EAGLE3_KC_ROWOPS, st);
  prologue_kernel<T><<<R, ROW_THREADS, 0, st>>>((const T*)w.emb, c.tokens, (const T*)c.state, c.h_tree,
                                                c.parent_slot, c.mode, c.rows, d, w.norm_e, w.norm_s,
                                                dm.rms_eps, ws.S, (T*)ws.x);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // QKV + RoPE + KV write, in chunks of <= 64 rows
  const int nqkv = (hq + 2 * hkv) * hd;
  {
  TimedScope ts(EAGLE3_KC_QKV, st);
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int Rc = R - r0 < 64 ? R - r0 : 64;
    RowMap map{MAP_PAIR_HEAD, hd, F};
    EpiQKV<T> epi;
    epi.q_out = (T*)ws.q + (size_t)r0 * qd;
    epi.pos = c.pos + r0;
    epi.dst = KVDest{kv.k, kv.v, kv.tk, kv.tv, kv.ctx_len, kv.block_table, kv.cap, kv.max_blocks,
                     kv.block_size, c.rows, c.mode, c.slot_base, hkv, hd};
    epi.dst.row0 = r0;
    epi.hq = hq;
    epi.theta = dm.rope_theta;
    if ((e = rows_gemm<T>((const T*)ws.x + (size_t)r0 * 2 * d, 2 * d, Rc, (const T*)w.qkv, 2 * d, nqkv,
                          map, epi, st)) != hipSuccess)
      return e;
  }
  }
  // attention
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
  al.bf16 = sizeof(T) == 2;
  al.part_o = ws.part_o;
  al.part_ml = ws.part_ml;
  al.out = ws.a;
  {
    TimedScope ts(EAGLE3_KC_ATTN, st);
    if ((e = launch_attention(al, st)) != hipSuccess) return e;
  }
  {
  TimedScope ts(EAGLE3_KC_O, st);
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int Rc = R - r0 < 64 ? R - r0 : 64;
    RowMap plain{MAP_PLAIN, hd, F};
    EpiResidual epi{ws.h1 + (size_t)r0 * d, ws.S + (size_t)r0 * d, d};
    if ((e = rows_gemm<T>((const T*)ws.a + (size_t)r0 * qd, qd, Rc, (const T*)w.o, qd, d, plain, epi, st)) !=
        hipSuccess)
      return e;
  }
  }
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    rms_rows_kernel<T><<<R, ROW_THREADS, 0, st>>>(ws.h1, d, w.norm_ffn, dm.rms_eps, (T*)ws.u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
  TimedScope ts(EAGLE3_KC_GATEUP, st);
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int Rc = R - r0 < 64 ? R - r0 : 64;
    RowMap pf{MAP_PAIR_FFN, hd, F};
    EpiSwiGLU<T> epi{(T*)ws.z + (size_t)r0 * F, F};
    if ((e = rows_gemm<T>((const T*)ws.u + (size_t)r0 * d, d, Rc, (const T*)w.gate_up, d, 2 * F, pf, epi,
                          st)) != hipSuccess)
      return e;
  }
  }
  {
  TimedScope ts(EAGLE3_KC_DOWN, st);
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int Rc = R - r0 < 64 ? R - r0 : 64;
    RowMap plain{MAP_PLAIN, hd, F};
    EpiResidual epi{ws.h2 + (size_t)r0 * d, ws.h1 + (size_t)r0 * d, d};
    if ((e = rows_gemm<T>((const T*)ws.z + (size_t)r0 * F, F, Rc, (const T*)w.down, F, d, plain, epi, st)) !=
        hipSuccess)
      return e;
  }
  }
  const int topk_last = c.topk_rows == EAGLE3_TOPK_LAST;
  {
    TimedScope ts(EAGLE3_KC_ROWOPS, st);
    final_rows_kernel<T><<<R, ROW_THREADS, 0, st>>>(ws.h2, d, w.norm_out, dm.rms_eps, c.mode, c.rows,
                                                    c.slot_base, topk_last, c.h_tree, (T*)ws.y);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int Rl = topk_last ? c.B : R;
  float* logits = c.logits_out ? c.logits_out : ws.logits;
  {
  TimedScope ts(EAGLE3_KC_LMHEAD, st);
  for (int r0 = 0; r0 < Rl; r0 += 64) {
    const int Rc = Rl - r0 < 64 ? Rl - r0 : 64;
    RowMap plain{MAP_PLAIN, hd, F};
    EpiStore<float> epi{logits + (size_t)r0 * V, V, plain};
    if ((e = rows_gemm<T>((const T*)ws.y + (size_t)r0 * d, d, Rc, (const T*)w.lm, d, V, plain, epi, st)) !=
        hipSuccess)
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
