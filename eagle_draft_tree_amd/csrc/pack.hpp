// Internal interface of the weight packer.
#pragma once
#include <hip/hip_runtime.h>

#include "eagle3.h"

namespace e3 {
size_t packed_bytes(const eagle3_dims& dm);
hipError_t pack_weights(const eagle3_dims& dm, const eagle3_weights& src, void* dst, eagle3_weights* packed,
                        hipStream_t st);
// one bf16 matrix [n][k] in plain row order (n % 16 == 0, k % 32 == 0)
hipError_t pack_matrix(const void* src, int n, int k, void* dst, hipStream_t st);
}  // namespace e3
