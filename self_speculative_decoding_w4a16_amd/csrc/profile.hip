// Launch profiler (declared in include/subspec.h, "Profiling"; mechanism in
// profile.h).
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/subspec.h"
#include "profile.h"

namespace {
struct Rec {
  int cls;
  double bytes;
  int prev;  // previous record on the same stream, or -1
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
size_t g_used = 0;
std::vector<std::pair<hipStream_t, int>> g_last;  // stream -> its last record
}  // namespace

namespace prof {
thread_local Current cur;

bool enabled() { return g_on; }

void on_launch(hipStream_t s, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  *start = *stop = nullptr;
  int slot = cur.slot;
  if (slot < 0) {
    if (!g_on || g_used >= g_recs.size()) return;
    slot = (int)g_used++;
    Rec& r = g_recs[slot];
    r.cls = cur.cls >= 0 ? cur.cls : SUBSPEC_K_MISC;
    r.bytes = cur.cls >= 0 ? cur.bytes : 0.0;
    r.prev = -1;
    for (auto& sl : g_last)
      if (sl.first == s) r.prev = sl.second;
    *start = r.a;
    if (cur.cls >= 0) cur.slot = slot;
  }
  *stop = g_recs[slot].b;
  bool found = false;
  for (auto& sl : g_last)
    if (sl.first == s) {
      sl.second = slot;
      found = true;
    }
  if (!found) g_last.push_back({s, slot});
}
}  // namespace prof

extern "C" {

int subspec_profile_start(int32_t max_records) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (max_records < 1) return SUBSPEC_EINVAL;
  while ((int32_t)g_recs.size() < max_records) {
    Rec r{0, 0.0, -1, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return SUBSPEC_EHIP;
    g_recs.push_back(r);
  }
  g_used = 0;
  g_last.clear();
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
    if (r.prev >= 0) {
      float tp = 0.0f;
      if (hipEventElapsedTime(&tp, g_recs[r.prev].b, r.b) != hipSuccess) return SUBSPEC_EHIP;
      if (tp < t) t = tp;
    }
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
