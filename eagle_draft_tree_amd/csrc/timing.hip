// Per-kernel-class HIP event timing for benchmarks (eagle3_timing_*).
#include <vector>

#include "eagle3.h"
#include "timing.hpp"

namespace e3 {
namespace {
struct ClassTiming {
  bool on = false;
  int mode = 0;  // 0: events around the class's scopes; 1: the principal kernel's own start/stop
  int n = 0;  // completed pairs
  bool open = false;
  std::vector<hipEvent_t> ev;  // 2 per launch
};
ClassTiming g_t[EAGLE3_KC_COUNT];
}  // namespace

void timing_begin(int kc, hipStream_t st) {
  ClassTiming& t = g_t[kc];
  if (!t.on || t.mode != 0 || 2 * t.n + 1 >= (int)t.ev.size()) return;
  (void)hipEventRecord(t.ev[2 * t.n], st);
  t.open = true;
}

void timing_end(int kc, hipStream_t st) {
  ClassTiming& t = g_t[kc];
  if (!t.on || t.mode != 0 || !t.open) return;
  (void)hipEventRecord(t.ev[2 * t.n + 1], st);
  t.open = false;
  ++t.n;
}
bool timing_kernel_events(int kc, hipEvent_t* start, hipEvent_t* stop) {
  if (kc < 0 || kc >= EAGLE3_KC_COUNT) return false;
  ClassTiming& t = g_t[kc];
  if (!t.on || t.mode != 1 || 2 * t.n + 1 >= (int)t.ev.size()) return false;
  *start = t.ev[2 * t.n];
  *stop = t.ev[2 * t.n + 1];
  ++t.n;
  return true;
}
}  // namespace e3

extern "C" {

int eagle3_timing_mode(int kc, int mode) {
  if (kc < 0 || kc >= EAGLE3_KC_COUNT || (mode != 0 && mode != 1)) return EAGLE3_EINVAL;
  e3::g_t[kc].mode = mode;
  return EAGLE3_OK;
}

int eagle3_timing_enable(int kc, int max_launches) {
  if (kc < 0 || kc >= EAGLE3_KC_COUNT || max_launches < 0) return EAGLE3_EINVAL;
  e3::ClassTiming& t = e3::g_t[kc];
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.n = 0;
  t.open = false;
  t.on = max_launches > 0;
  if (!t.on) return EAGLE3_OK;
  t.ev.resize(2 * (size_t)max_launches);
  for (auto& e : t.ev)
    if (hipEventCreate(&e) != hipSuccess) return EAGLE3_EHIP;
  return EAGLE3_OK;
}

int eagle3_timing_read(int kc, double* total_ms, int* launches) {
  if (kc < 0 || kc >= EAGLE3_KC_COUNT || !total_ms || !launches) return EAGLE3_EINVAL;
  e3::ClassTiming& t = e3::g_t[kc];
  double tot = 0.0;
  if (t.n > 0 && hipEventSynchronize(t.ev[2 * t.n - 1]) != hipSuccess) return EAGLE3_EHIP;
  for (int i = 0; i < t.n; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return EAGLE3_EHIP;
    tot += ms;
  }
  *total_ms = tot;
  *launches = t.n;
  return EAGLE3_OK;
}

}  // extern "C"
