// Internal interface of the target's verification forward and KV commit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "eagle3.h"

namespace e3 {

struct TargetCall {
  const eagle3_dims* dims;
  const eagle3_target* t;
  const eagle3_kv* kv;  // host array [n_layers]
  int B, rows;
  const int32_t* tokens;
  const int32_t* pos;
  const uint64_t* anc;
  int begin, end;
  float* hidden;  // [B*rows][d]
  void* feats;    // [B*rows][3][d] dtype, or NULL
  float* logits;  // [B*rows][V], or NULL
  void* ws;
};

// Workspace bytes for B*rows verify rows whose layers' key space holds at
// most cap_rows committed rows.
size_t target_ws_bytes(const eagle3_dims& dm, int B, int rows, int cap_rows);
hipError_t target_forward(const TargetCall& c, hipStream_t st);

hipError_t kv_commit(const eagle3_dims& dm, int n_layers, const eagle3_kv* kv, int B, int rows,
                     const int32_t* accept_len, const int32_t* accepted, int Dmax, const void* feats,
                     void* feats_next, int32_t* ctx_len_out, int32_t* status, hipStream_t st);

// packed copy of one target layer's four GEMM matrices
size_t target_layer_packed_bytes(const eagle3_dims& dm);
hipError_t pack_target_layer(const eagle3_dims& dm, const eagle3_target_layer& src, void* dst,
                             eagle3_target_layer* packed, hipStream_t st);

}  // namespace e3
