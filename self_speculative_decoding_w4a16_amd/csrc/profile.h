// Launch profiler.  While recording, every kernel the library launches goes
// through hipExtLaunchKernel with a pair of events, so the events take the
// kernel dispatch's own timestamps (no marker packets between kernels).  A
// launch's duration is taken from the end of the previous launch on the same
// stream (or from its own start stamp, if that is later, as after a host
// synchronisation) to its own end: for kernels queued back to back this is
// the time each kernel holds the stream.  A prof::Scope assigns its launches
// to a class and to one record, so a scope that makes several launches is
// timed as one unit.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prof {
bool enabled();

struct Current {
  int cls = -1;      // class of the enclosing scope, -1 outside scopes
  double bytes = 0;  // algorithmic bytes of the scope
  int slot = -1;     // record claimed by the scope's first launch
};
extern thread_local Current cur;

// Called by SS_LAUNCH while recording: returns the events for this launch
// (start is null for the second and later launches of a scope).
void on_launch(hipStream_t s, hipEvent_t* start, hipEvent_t* stop);

struct Scope {
  Scope(int cls, double bytes, hipStream_t) {
    cur = Current{};
    cur.cls = cls;
    cur.bytes = bytes;
  }
  ~Scope() { cur = Current{}; }
};
}  // namespace prof

// Kernel launch used throughout the library (see above).
#define SS_LAUNCH(kernel, grid, block, lds, stream, ...)                                     \
  do {                                                                                      \
    if (prof::enabled()) {                                                                  \
      hipEvent_t ss_e0 = nullptr, ss_e1 = nullptr;                                          \
      prof::on_launch(stream, &ss_e0, &ss_e1);                                              \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ss_e0, ss_e1, 0, __VA_ARGS__); \
    } else {                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                    \
    }                                                                                       \
  } while (0)
