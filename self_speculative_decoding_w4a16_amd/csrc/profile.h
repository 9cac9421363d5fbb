// Launch profiler: brackets launches with HIP events on their own stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prof {
bool enabled();
// Records the start event for a launch of class `cls` moving `bytes`
// algorithmic bytes; returns a slot index or -1.
int begin(int cls, double bytes, hipStream_t s);
void end(int slot, hipStream_t s);

struct Scope {
  int slot;
  hipStream_t s;
  Scope(int cls, double bytes, hipStream_t st) : slot(enabled() ? begin(cls, bytes, st) : -1), s(st) {}
  ~Scope() {
    if (slot >= 0) end(slot, s);
  }
};
}  // namespace prof
