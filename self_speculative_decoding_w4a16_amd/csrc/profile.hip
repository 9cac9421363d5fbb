// Launch profiler (see include/subspec.h, "Profiling").
#include <mutex>
#include <vector>

#include "../../include/subspec.h"
#include "profile.h"

namespace {
struct Rec {
  int cls;
  double bytes;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
size_t g_used = 0;
}  // namespace

namespace prof {
bool enabled() { return g_on; }

int begin(int cls, double bytes, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_used >= g_recs.size()) return -1;
  const int slot = (int)g_used++;
  g_recs[slot].cls = cls;
  g_recs[slot].bytes = bytes;
  if (hipEventRecord(g_recs[slot].a, s) != hipSuccess) return -1;
  return slot;
}

void end(int slot, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  (void)hipEventRecord(g_recs[slot].b, s);
}
}  // namespace prof

extern "C" {

int subspec_profile_start(int32_t max_records) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (max_records < 1) return SUBSPEC_EINVAL;
  while ((int32_t)g_recs.size() < max_records) {
    Rec r{0, 0.0, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return SUBSPEC_EHIP;
    g_recs.push_back(r);
  }
  g_used = 0;
  g_on = true;
  return SUBSPEC_OK;
}

int subspec_profile_stop(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  return SUBSPEC_OK;
}

int subspec_profile_read(int32_t cls, int64_t* launches, double* total_ms, double* bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (cls < 0 || cls >= SUBSPEC_K_CLASSES || !launches || !total_ms || !bytes) return SUBSPEC_EINVAL;
  int64_t n = 0;
  double ms = 0.0, by = 0.0;
  for (size_t i = 0; i < g_used; ++i) {
    Rec& r = g_recs[i];
    if (r.cls != cls) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return SUBSPEC_EHIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return SUBSPEC_EHIP;
    ++n;
    ms += t;
    by += r.bytes;
  }
  *launches = n;
  *total_ms = ms;
  *bytes = by;
  return SUBSPEC_OK;
}
}
