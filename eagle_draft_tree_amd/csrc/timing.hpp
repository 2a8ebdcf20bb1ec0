// Optional per-kernel-class HIP event timing (see eagle3_timing_enable).
#pragma once
#include <hip/hip_runtime.h>

namespace e3 {
void timing_begin(int kc, hipStream_t st);
void timing_end(int kc, hipStream_t st);

// RAII scope: events around every launch enqueued inside it.
struct TimedScope {
  int kc;
  hipStream_t st;
  TimedScope(int k, hipStream_t s) : kc(k), st(s) { timing_begin(kc, st); }
  ~TimedScope() { timing_end(kc, st); }
};
}  // namespace e3
