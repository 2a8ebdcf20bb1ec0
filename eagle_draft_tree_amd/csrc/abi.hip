// C ABI of the library: argument validation (before anything is launched),
// workspace sizing, error codes and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "draft.hpp"
#include "eagle3.h"
#include "kernels.hpp"
#include "pack.hpp"
#include "timing.hpp"
#include "ttt.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = 0;
  return EAGLE3_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(EAGLE3_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_dims(const eagle3_dims* dm) {
  REQUIRE(dm, EAGLE3_EINVAL, "dims is NULL");
  REQUIRE(dm->dtype == EAGLE3_F32 || dm->dtype == EAGLE3_BF16, EAGLE3_EINVAL, "dtype %d unknown", dm->dtype);
  REQUIRE(dm->d > 0 && dm->n_q_heads > 0 && dm->n_kv_heads > 0 && dm->ffn > 0 && dm->vocab > 0,
          EAGLE3_EINVAL, "non-positive dimension");
  REQUIRE(dm->n_q_heads % dm->n_kv_heads == 0, EAGLE3_EINVAL, "n_q_heads %% n_kv_heads != 0");
  REQUIRE(dm->head_dim == 64 || dm->head_dim == 128, EAGLE3_EUNSUPPORTED, "head_dim %d (64 or 128)",
          dm->head_dim);
  REQUIRE(dm->dtype == EAGLE3_BF16 || dm->head_dim == 64, EAGLE3_EUNSUPPORTED,
          "fp32 drafters need head_dim 64");
  REQUIRE(dm->d % 32 == 0 && dm->ffn % 32 == 0 && dm->vocab % 16 == 0, EAGLE3_EUNSUPPORTED,
          "d and ffn must be multiples of 32, vocab of 16");
  REQUIRE(dm->rms_eps >= 0.f && dm->rope_theta > 0.f, EAGLE3_EINVAL, "rms_eps/rope_theta");
  REQUIRE(dm->vocab <= 262144, EAGLE3_EUNSUPPORTED, "vocab %d > 262144", dm->vocab);
  return EAGLE3_OK;
}

int check_weights(const eagle3_weights* w) {
  REQUIRE(w, EAGLE3_EINVAL, "weights is NULL");
  REQUIRE(w->fc && w->emb && w->qkv && w->o && w->gate_up && w->down && w->lm, EAGLE3_EINVAL,
          "a weight pointer is NULL");
  REQUIRE(w->norm_e && w->norm_s && w->norm_ffn && w->norm_out, EAGLE3_EINVAL, "a norm gain is NULL");
  REQUIRE(w->layout == EAGLE3_LAYOUT_ROWMAJOR || w->layout == EAGLE3_LAYOUT_PACKED, EAGLE3_EINVAL, "layout %d",
          w->layout);
  return EAGLE3_OK;
}

}  // namespace

extern "C" {

const char* eagle3_strerror(int code) {
  switch (code) {
    case EAGLE3_OK: return "ok";
    case EAGLE3_EINVAL: return "invalid argument";
    case EAGLE3_ECAPACITY: return "capacity exceeded";
    case EAGLE3_EUNSUPPORTED: return "unsupported shape";
    case EAGLE3_EWORKSPACE: return "workspace too small";
    case EAGLE3_EHIP: return "HIP error";
    case EAGLE3_ENUMERIC: return "NaN in target logits";
    default: return "unknown error";
  }
}

const char* eagle3_last_error(void) { return g_last_error; }

const char* eagle3_version(void) { return "eagle3-gfx950 0.1"; }

int eagle3_packed_weights_size(const eagle3_dims* dims, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  REQUIRE(bytes, EAGLE3_EINVAL, "bytes is NULL");
  REQUIRE(dims->dtype == EAGLE3_BF16, EAGLE3_EUNSUPPORTED, "packing needs bf16 weights");
  *bytes = e3::packed_bytes(*dims);
  return ok();
}

int eagle3_pack_weights(const eagle3_dims* dims, const eagle3_weights* src, void* dst, size_t dst_bytes,
                        eagle3_weights* packed, eagle3_stream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(src))) return rc;
  REQUIRE(dims->dtype == EAGLE3_BF16, EAGLE3_EUNSUPPORTED, "packing needs bf16 weights");
  REQUIRE(src->layout == EAGLE3_LAYOUT_ROWMAJOR, EAGLE3_EINVAL, "src must be row-major");
  REQUIRE(dst && packed, EAGLE3_EINVAL, "dst/packed is NULL");
  REQUIRE(dst_bytes >= e3::packed_bytes(*dims), EAGLE3_EWORKSPACE, "dst %zu < %zu bytes", dst_bytes,
          e3::packed_bytes(*dims));
  return hip_status(e3::pack_weights(*dims, *src, dst, packed, (hipStream_t)stream), "eagle3_pack_weights");
}

int eagle3_workspace_size(const eagle3_dims* dims, int B, int max_rows, int max_ctx, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  REQUIRE(bytes, EAGLE3_EINVAL, "bytes is NULL");
  REQUIRE(B >= 1 && max_rows >= 1 && max_ctx >= 0, EAGLE3_EINVAL, "B/max_rows/max_ctx");
  *bytes = e3::draft_ws_bytes(*dims, B, max_rows, max_ctx);
  return ok();
}

int eagle3_tree_state_size(int B, int k, int D, size_t* bytes) {
  REQUIRE(bytes, EAGLE3_EINVAL, "bytes is NULL");
  REQUIRE(B >= 1 && k >= 1 && D >= 1, EAGLE3_EINVAL, "B/k/D");
  REQUIRE(k <= EAGLE3_MAX_TOPK && (D - 1) * k <= EAGLE3_MAX_TREE_SLOTS, EAGLE3_ECAPACITY,
          "k=%d D=%d exceeds the tree limits", k, D);
  *bytes = (size_t)B * e3::tree_state_bytes_per_req(k, D);
  return ok();
}

int eagle3_ttt_workspace_size(const eagle3_dims* dims, int B, int S, int R, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  REQUIRE(bytes, EAGLE3_EINVAL, "bytes is NULL");
  REQUIRE(B >= 1 && S >= 1 && R >= 1, EAGLE3_EINVAL, "B/S/R");
  *bytes = e3::ttt_ws_bytes(*dims, B, S, R);
  return ok();
}

int eagle3_fuse(const eagle3_dims* dims, const eagle3_weights* w, const void* feats, int n, void* g,
                void* ws, size_t ws_bytes, eagle3_stream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  REQUIRE(w->layout == EAGLE3_LAYOUT_ROWMAJOR || dims->dtype == EAGLE3_BF16, EAGLE3_EINVAL, "packed fp32");
  REQUIRE(feats && g, EAGLE3_EINVAL, "feats/g is NULL");
  REQUIRE(n >= 1, EAGLE3_EINVAL, "n=%d", n);
  REQUIRE(ws, EAGLE3_EINVAL, "workspace is NULL");
  const size_t need = e3::fuse_ws_bytes(*dims, n);
  REQUIRE(ws_bytes >= need, EAGLE3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(e3::fuse_rows(*dims, *w, feats, n, g, ws, (hipStream_t)stream), "eagle3_fuse");
}

int eagle3_draft_step(const eagle3_dims* dims, const eagle3_weights* w, const eagle3_kv* kv, int mode,
                      int B, int rows, const void* state, const int32_t* parent_slot,
                      const int32_t* tokens, const int32_t* pos, const uint64_t* anc, int slot_base,
                      int k, int topk_rows, float* h_tree, int32_t* topk_id, float* topk_lp,
                      float* logits_out, void* ws, size_t ws_bytes, eagle3_stream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  REQUIRE(w->layout == EAGLE3_LAYOUT_ROWMAJOR || dims->dtype == EAGLE3_BF16, EAGLE3_EINVAL, "packed fp32");
  REQUIRE(kv && kv->k && kv->v && kv->ctx_len, EAGLE3_EINVAL, "kv/k/v/ctx_len is NULL");
  REQUIRE(mode == EAGLE3_COMMIT || mode == EAGLE3_TREE, EAGLE3_EINVAL, "mode %d", mode);
  REQUIRE(B >= 1, EAGLE3_EINVAL, "B=%d", B);
  REQUIRE(rows >= 1, EAGLE3_EINVAL, "rows=%d", rows);
  REQUIRE(rows <= EAGLE3_MAX_ROWS, EAGLE3_ECAPACITY, "rows=%d > %d", rows, EAGLE3_MAX_ROWS);
  REQUIRE(tokens && pos && h_tree && topk_id && topk_lp, EAGLE3_EINVAL, "a required pointer is NULL");
  REQUIRE(k >= 1 && k <= dims->vocab, EAGLE3_EINVAL, "k=%d", k);
  REQUIRE(k <= EAGLE3_MAX_TOPK, EAGLE3_ECAPACITY, "k=%d > %d", k, EAGLE3_MAX_TOPK);
  REQUIRE(topk_rows == EAGLE3_TOPK_ALL || topk_rows == EAGLE3_TOPK_LAST, EAGLE3_EINVAL, "topk_rows");
  if (mode == EAGLE3_COMMIT) {
    REQUIRE(state, EAGLE3_EINVAL, "COMMIT needs state");
  } else {
    REQUIRE(parent_slot && anc && kv->tk && kv->tv, EAGLE3_EINVAL, "TREE needs parent_slot, anc, tk, tv");
    REQUIRE(slot_base >= 0, EAGLE3_EINVAL, "slot_base=%d", slot_base);
    REQUIRE(slot_base + rows <= EAGLE3_MAX_TREE_SLOTS, EAGLE3_ECAPACITY, "slot_base+rows=%d > %d",
            slot_base + rows, EAGLE3_MAX_TREE_SLOTS);
  }
  int cap_rows;
  if (kv->block_table) {
    REQUIRE(dims->dtype == EAGLE3_BF16, EAGLE3_EUNSUPPORTED, "paged KV needs bf16");
    REQUIRE(kv->block_size >= 1 && kv->max_blocks >= 1, EAGLE3_EINVAL, "block_size/max_blocks");
    cap_rows = kv->max_blocks * kv->block_size;
  } else {
    REQUIRE(kv->cap >= 1, EAGLE3_EINVAL, "cap=%d", kv->cap);
    cap_rows = kv->cap;
  }
  REQUIRE(cap_rows <= 32000, EAGLE3_EUNSUPPORTED, "KV capacity %d rows > 32000", cap_rows);
  const size_t need = e3::draft_ws_bytes(*dims, B, rows, cap_rows - rows > 0 ? cap_rows - rows : 0);
  REQUIRE(ws, EAGLE3_EINVAL, "workspace is NULL");
  REQUIRE(ws_bytes >= need, EAGLE3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  e3::DraftCall c{dims, w, kv, mode, B, rows, state, parent_slot, tokens, pos, anc, slot_base, k,
                  topk_rows, h_tree, topk_id, topk_lp, logits_out, ws};
  return hip_status(e3::draft_step(c, (hipStream_t)stream), "eagle3_draft_step");
}

int eagle3_tree_expand(int phase, int B, int k, int D, int m, const int32_t* root_tok,
                       const int32_t* root_pos, void* tree_state, const int32_t* topk_id,
                       const float* topk_lp, int32_t* next_tok, int32_t* next_parent_slot,
                       int32_t* next_pos, uint64_t* next_anc, int32_t* v_tok, int32_t* v_parent,
                       int32_t* v_depth, int32_t* v_pos, uint64_t* v_anc, eagle3_stream_t stream) {
  REQUIRE(phase == EAGLE3_INIT || phase == EAGLE3_STEP || phase == EAGLE3_FINAL, EAGLE3_EINVAL,
          "phase %d", phase);
  REQUIRE(B >= 1 && k >= 1 && D >= 1 && m >= 1, EAGLE3_EINVAL, "B/k/D/m");
  REQUIRE(k <= EAGLE3_MAX_TOPK, EAGLE3_ECAPACITY, "k=%d > %d", k, EAGLE3_MAX_TOPK);
  REQUIRE((D - 1) * k <= EAGLE3_MAX_TREE_SLOTS, EAGLE3_ECAPACITY, "(D-1)k=%d > 64", (D - 1) * k);
  REQUIRE(m + 1 <= EAGLE3_MAX_TREE_SLOTS, EAGLE3_ECAPACITY, "m+1=%d > 64", m + 1);
  REQUIRE(m <= k + (D - 1) * k * k, EAGLE3_EINVAL, "m=%d exceeds the pool", m);
  REQUIRE(tree_state, EAGLE3_EINVAL, "tree_state is NULL");
  if (phase == EAGLE3_INIT) {
    REQUIRE(root_tok && root_pos, EAGLE3_EINVAL, "INIT needs root_tok/root_pos");
  }
  if (phase != EAGLE3_FINAL) {
    REQUIRE(topk_id && topk_lp, EAGLE3_EINVAL, "topk_id/topk_lp is NULL");
    REQUIRE(next_tok && next_parent_slot && next_pos && next_anc, EAGLE3_EINVAL, "next_* is NULL");
  } else {
    REQUIRE(v_tok && v_parent && v_depth && v_pos && v_anc, EAGLE3_EINVAL, "v_* is NULL");
  }
  e3::TimedScope ts(EAGLE3_KC_TREE, (hipStream_t)stream);
  return hip_status(e3::launch_tree_expand(phase, B, k, D, m, root_tok, root_pos, tree_state, topk_id,
                                           topk_lp, next_tok, next_parent_slot, next_pos, next_anc,
                                           v_tok, v_parent, v_depth, v_pos, v_anc, (hipStream_t)stream),
                    "eagle3_tree_expand");
}

int eagle3_verify_workspace_size(int B, int m, int V, size_t* bytes) {
  REQUIRE(bytes, EAGLE3_EINVAL, "bytes is NULL");
  REQUIRE(B >= 1 && m >= 0 && V >= 1, EAGLE3_EINVAL, "B/m/V");
  *bytes = e3::verify_ws_bytes(B, m, V);
  return ok();
}

int eagle3_verify(int B, int m, int V, int Dmax, const int32_t* v_tok, const int32_t* v_parent,
                  const float* target_logits, int mode, float temperature, const double* u_try,
                  const double* u_res, int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                  int32_t* status, void* ws, size_t ws_bytes, eagle3_stream_t stream) {
  REQUIRE(B >= 1 && m >= 0 && V >= 1 && Dmax >= 1, EAGLE3_EINVAL, "B/m/V/Dmax");
  REQUIRE(m + 1 <= EAGLE3_MAX_TREE_SLOTS, EAGLE3_ECAPACITY, "m+1=%d > 64", m + 1);
  REQUIRE(v_tok && v_parent && target_logits && accept_len && accepted && bonus && status, EAGLE3_EINVAL,
          "a required pointer is NULL");
  REQUIRE(mode == EAGLE3_GREEDY || mode == EAGLE3_SAMPLE, EAGLE3_EINVAL, "mode %d", mode);
  if (mode == EAGLE3_SAMPLE) {
    REQUIRE(temperature > 0.f, EAGLE3_EINVAL, "temperature must be > 0 for sampling");
    REQUIRE(u_try && u_res, EAGLE3_EINVAL, "sampling needs u_try/u_res");
  }
  REQUIRE(ws, EAGLE3_EINVAL, "workspace is NULL");
  REQUIRE(ws_bytes >= e3::verify_ws_bytes(B, m, V), EAGLE3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
          e3::verify_ws_bytes(B, m, V));
  e3::TimedScope ts(EAGLE3_KC_VERIFY, (hipStream_t)stream);
  return hip_status(e3::launch_verify(B, m, V, Dmax, v_tok, v_parent, target_logits, mode, temperature,
                                      u_try, u_res, accept_len, accepted, bonus, status, ws,
                                      ws_bytes, (hipStream_t)stream),
                    "eagle3_verify");
}

int eagle3_topk(const float* logits, int rows, int V, int k, int32_t* ids, float* lp, float* lse,
                void* ws, size_t ws_bytes, eagle3_stream_t stream) {
  REQUIRE(logits && ids && lp && ws, EAGLE3_EINVAL, "a required pointer is NULL");
  REQUIRE(rows >= 1 && V >= 1 && k >= 1 && k <= V, EAGLE3_EINVAL, "rows/V/k");
  REQUIRE(V <= 262144, EAGLE3_EUNSUPPORTED, "V %d > 262144", V);
  REQUIRE(k <= EAGLE3_MAX_TOPK, EAGLE3_ECAPACITY, "k=%d > %d", k, EAGLE3_MAX_TOPK);
  const size_t need = e3::topk_ws_bytes(rows, V);
  REQUIRE(ws_bytes >= need, EAGLE3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(e3::launch_topk(logits, rows, V, k, ids, lp, lse, ws, (hipStream_t)stream), "eagle3_topk");
}

int eagle3_ttt_forward(const eagle3_dims* dims, const eagle3_weights* w, const void* feats,
                       const int32_t* tokens, int B, int S, int R, const int32_t* forced_tokens,
                       int32_t* pred, float* ce, float* loss, void* ws, size_t ws_bytes,
                       eagle3_stream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  REQUIRE(dims->dtype == EAGLE3_BF16, EAGLE3_EUNSUPPORTED, "TTT needs bf16");
  REQUIRE(feats && tokens && pred && ce && loss && ws, EAGLE3_EINVAL, "a required pointer is NULL");
  REQUIRE(B >= 1 && S >= 1 && R >= 1, EAGLE3_EINVAL, "B/S/R");
  REQUIRE(S % 64 == 0, EAGLE3_EUNSUPPORTED, "S=%d must be a multiple of 64", S);
  REQUIRE(dims->d % 64 == 0 && dims->ffn % 64 == 0 && dims->d <= 8192, EAGLE3_EUNSUPPORTED,
          "TTT needs d and ffn multiples of 64 and d <= 8192");
  const size_t need = e3::ttt_ws_bytes(*dims, B, S, R);
  REQUIRE(ws_bytes >= need, EAGLE3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rc = e3::ttt_forward(*dims, *w, feats, tokens, B, S, R, forced_tokens, pred, ce, loss, ws,
                       (hipStream_t)stream);
  if (rc == 1) return fail(EAGLE3_EUNSUPPORTED, "TTT forward: shape not supported");
  if (rc < 0) return fail(EAGLE3_EHIP, "eagle3_ttt_forward: HIP launch failed");
  return ok();
}

}  // extern "C"
