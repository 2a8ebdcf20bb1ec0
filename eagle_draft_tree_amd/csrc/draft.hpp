// Internal interface of the draft-step / fusion implementation.
#pragma once
#include <hip/hip_runtime.h>

#include "eagle3.h"

namespace e3 {

struct DraftCall {
  const eagle3_dims* dims;
  const eagle3_weights* w;
  const eagle3_kv* kv;
  int mode, B, rows;
  const void* state;
  const int32_t* parent_slot;
  const int32_t* tokens;
  const int32_t* pos;
  const uint64_t* anc;
  int slot_base, k, topk_rows;
  float* h_tree;
  int32_t* topk_id;
  float* topk_lp;
  float* logits_out;
  void* ws;
  // efficient LM head (NULL: the full head); optional candidate outputs
  const eagle3_lowrank_head* lr = nullptr;
  int32_t* cand_out = nullptr;
  float* cand_logits_out = nullptr;
};

size_t draft_ws_bytes(const eagle3_dims& dm, int B, int max_rows, int max_ctx);
hipError_t draft_step(const DraftCall& c, hipStream_t st);
size_t fuse_ws_bytes(const eagle3_dims& dm, int n);
hipError_t fuse_rows(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, int n,
                     void* g, void* ws, hipStream_t st);

}  // namespace e3
