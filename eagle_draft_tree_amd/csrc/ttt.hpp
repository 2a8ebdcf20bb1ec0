// Internal interface of the training-time-test forward and backward.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "eagle3.h"

namespace e3 {

// Per-step state the forward keeps for the backward (M = B*S rows a step;
// step j = 1..R at index j-1).  All device memory inside the train workspace.
struct TttSave {
  float* s;          // [R+1][M][d]  state fed to step j (s_1 = g); s_{j+1} = h2 of step j
  float* h1;         // [R][M][d]    residual after attention
  bf16* x;           // [R][M][2d]   decoder input, fragment order
  bf16* q;           // [R][M][hq][hd] queries after RoPE
  float* lse;        // [R][hq][M]   attention log-sum-exp per query head and row
  bf16* a;           // [R][M][hq*hd] attention output, fragment order
  bf16* u;           // [R][M][d]    FFN input, fragment order
  float2* gu;        // [R][M][ffn]  (gate, up) before SwiGLU
  bf16* z;           // [R][M][ffn]  SwiGLU output, fragment order
  float* dy;         // [R][M][d]    gradient at the LM head input rms(h2)*norm_out
  int32_t* tok;      // [R][M]       tokens fed at step j >= 2 (index 0 unused)
  bf16* dlogits;     // [M][vp]      one step's exp(logit - m), then its gradient at the logits (scratch)
  float* exm;        // [M][vp/64]   the m of each 64 columns (scratch)
  float* lse_ce;     // [M]          one step's logits log-sum-exp (scratch)
  const bf16* lm_t;  // [d][vp]      LM head transposed, packed fragment order
  int vp;            // vocab rounded up to 64 (the backward's K padding)
  double count;      // valid rows of all steps (the loss's divisor)
  // set by the forward: its keys/values ([M][hkv][hd]; chain steps 2..R at
  // [R-1][M][hkv][hd]) and RoPE table ([S+R][hd/2] (cos, sin))
  const bf16 *k1, *v1, *kc, *vc;
  const float2* rope;
};

size_t ttt_ws_bytes(const eagle3_dims& dm, int B, int S, int R);
// 0 ok, 1 unsupported shape, -1 HIP error.  sv != nullptr keeps the
// backward's per-step state and computes dy of every step.
int ttt_forward(const eagle3_dims& dm, const eagle3_weights& w, const void* feats,
                const int32_t* tokens, int B, int S, int R, const int32_t* forced, int32_t* pred,
                float* ce, float* loss, void* ws, hipStream_t st, TttSave* sv = nullptr);

// Forward + backward: gradients of the mean CE w.r.t. the drafter's trained
// parameters.  ws: ttt_train_ws_bytes.  0 ok, 1 unsupported shape, -1 HIP error.
size_t ttt_train_ws_bytes(const eagle3_dims& dm, int B, int S, int R);
int ttt_train(const eagle3_dims& dm, const eagle3_weights& w, const void* feats, const int32_t* tokens, int B,
              int S, int R, const int32_t* forced, int32_t* pred, float* ce, float* loss, const eagle3_grads& g,
              void* ws, hipStream_t st);

}  // namespace e3
