// Optional per-kernel-class HIP event timing (see eagle3_timing_enable).
#pragma once
#include <hip/hip_runtime.h>

#include <hip/hip_ext.h>

namespace e3 {
void timing_begin(int kc, hipStream_t st);
void timing_end(int kc, hipStream_t st);
// Kernel mode (eagle3_timing_mode 1): the event pair of the class's next
// launch, for a launch that records its own start and stop
// (hipExtLaunchKernel); false when the class is off or in scope mode.
bool timing_kernel_events(int kc, hipEvent_t* start, hipEvent_t* stop);

// Launch `kernel` on `st`; when class kc is timed in kernel mode, through
// hipExtLaunchKernelGGL with the class's next event pair, so that the pair
// holds the kernel's own start and end (the dispatch timestamps a profiler
// reads) rather than events enqueued around it.
template <typename... Args, typename F = void (*)(Args...)>
inline void launch_timed(int kc, F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (kc >= 0 && timing_kernel_events(kc, &a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, st, a, b, 0u, args...);
  else
    kernel<<<grid, block, shmem, st>>>(args...);
}

// RAII scope: events around every launch enqueued inside it.
struct TimedScope {
  int kc;
  hipStream_t st;
  TimedScope(int k, hipStream_t s) : kc(k), st(s) { timing_begin(kc, st); }
  ~TimedScope() { timing_end(kc, st); }
};
}  // namespace e3
