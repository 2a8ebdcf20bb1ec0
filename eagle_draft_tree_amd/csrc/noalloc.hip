// Static device scratch for the allocation-free verify entry point.
//
// Callers that cannot allocate (code under HIP graph capture, tight serving
// loops) get their verify workspace from a file-scope device array instead
// of a caller buffer.  Each GPU the library runs on holds its own copy of the
// array until the process ends.  Host code never passes the array's name to
// a kernel: its device address is looked up once per device with
// hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace e3 {

constexpr size_t kStaticScratchBytes = size_t(8) << 20;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void zero_words_kernel(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // The verify arrival counters must start at zero (each call leaves them
    // at zero); clear the whole array once, on the caller's stream, with a
    // kernel rather than a memset node.
    zero_words_kernel<<<256, 256, 0, st>>>((uint4*)p, kStaticScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace e3
