// Host-side launchers of the library's kernels (internal interface between
// the C ABI layer and the kernel translation units).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e3 {

// ---- decode attention (attention.hip)
struct AttnLaunch {
  const void* q;
  const void *kc, *vc, *tk, *tv;
  const int32_t* ctx_len;
  const int32_t* block_table;
  const uint64_t* anc;
  int cap, max_blocks, block_size, cap_rows;
  int B, rows, hq, hkv, hd, mode;
  bool bf16;
  float* part_o;
  float* part_ml;
  void* out;  // [B*rows][hq*hd] dtype
};
int attn_num_chunks(int cap_rows);
hipError_t launch_attention(const AttnLaunch& L, hipStream_t st);

// ---- top-k + log-probs over vocab rows (topk.hip)
size_t topk_ws_bytes(int rows, int V);
hipError_t launch_topk(const float* logits, int rows, int V, int k, int32_t* ids, float* lp, float* lse, void* ws,
                       hipStream_t st);
// top-1 and log-probability from per-workgroup (max, sum exp, argmax) partials [rows][nparts]
hipError_t launch_top1_merge(const float4* part, int rows, int nparts, int32_t* ids, float* lp, hipStream_t st);
// top-k from fp32 logits [rows][V] (rows <= 64, V a multiple of 16) and the
// per-16-column-tile {max, sum exp} pairs EpiLogitsTiles wrote with
// `tiles_per_wg` tiles per LM-head workgroup
hipError_t launch_topk_tiles(const float* logits, const float2* part, int tiles_per_wg, int rows, int V, int k,
                             int32_t* ids, float* lp, hipStream_t st);

// ---- efficient LM head (lowrank.hip)
constexpr int LOWRANK_MAX_CAND = 256;
// stage-1 scores of up to 16 rows from packed A [V][rank] (rank 64, 128 or
// 256) and z [rows][rank], with per-tile row maxima in the slots of
// tile_slots(V/16, lowrank_scores_tpw())
int lowrank_scores_tpw();
hipError_t launch_lowrank_scores(const void* A, const void* z, int rows, int rank, int V, float* scores,
                                 float2* part, hipStream_t st);
// candidates [rows][c]: the c best low-rank scores [rows][V] by (value desc,
// id asc), from the scores and the per-tile pairs EpiLogitsTiles wrote
hipError_t launch_lowrank_select(const float* scores, const float2* part, int tiles_per_wg, int rows, int V, int c,
                                 int32_t* cand, hipStream_t st);
// exact logits of the candidates (bf16 LM head, packed or row-major, and
// bf16 y [rows][d]) -> cand_logits [rows][c]; then the top-k of the
// candidates and lp normalised over them -> ids/lp [rows][k]
hipError_t launch_lowrank_exact(const void* W_lm, bool packed, const void* y, int rows, int d, int V, int c, int k,
                                const int32_t* cand, float* cand_logits, int32_t* ids, float* lp, hipStream_t st);

// ---- dynamic tree (tree.hip)
size_t tree_state_bytes_per_req(int k, int D);
hipError_t launch_tree_expand(int phase, int B, int k, int D, int m, const int32_t* root_tok,
                              const int32_t* root_pos, void* state, const int32_t* topk_id,
                              const float* topk_lp, int32_t* next_tok, int32_t* next_parent_slot,
                              int32_t* next_pos, uint64_t* next_anc, int32_t* v_tok,
                              int32_t* v_parent, int32_t* v_depth, int32_t* v_pos, uint64_t* v_anc,
                              hipStream_t st);

// ---- verification (verify.hip)
size_t verify_ws_bytes(int B, int m, int V);
// static per-device scratch of the allocation-free verify (noalloc.hip):
// its size, and its device address on the current device (set up on first use)
size_t static_scratch_bytes();
hipError_t static_scratch(hipStream_t st, void** out);
hipError_t launch_verify(int B, int m, int V, int Dmax, const int32_t* v_tok,
                         const int32_t* v_parent, const float* logits, int mode, float temperature,
                         const double* u_try, const double* u_res, int32_t* accept_len,
                         int32_t* accepted, int32_t* bonus, int32_t* status, void* ws,
                         size_t ws_bytes, hipStream_t st);

}  // namespace e3
