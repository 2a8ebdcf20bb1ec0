// Internal interface of the training-time-test forward.
#pragma once
#include <hip/hip_runtime.h>

#include "eagle3.h"

namespace e3 {

size_t ttt_ws_bytes(const eagle3_dims& dm, int B, int S, int R);
// 0 ok, 1 unsupported shape, -1 HIP error
int ttt_forward(const eagle3_dims& dm, const eagle3_weights& w, const void* feats,
                const int32_t* tokens, int B, int S, int R, const int32_t* forced, int32_t* pred,
                float* ce, float* loss, void* ws, hipStream_t st);

}  // namespace e3
