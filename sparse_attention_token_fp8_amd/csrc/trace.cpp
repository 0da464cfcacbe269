// Per-kernel timing without a profiler (idx_trace_begin / idx_trace_end):
// every kernel the library enqueues from a tracing thread is bracketed by two
// of the caller's events, recorded on the kernel's stream.

#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr int kMaxTraced = 4096;                // kernels one trace can name

struct TraceState {
  hipEvent_t* events = nullptr;                 // null: not tracing
  int capacity = 0;
  int used = 0;                                 // events recorded
  bool skip = false;                            // the current kernel did not fit
  const char* names[kMaxTraced];
};

thread_local TraceState g_trace;

}  // namespace

namespace idx {

void trace_mark(hipStream_t stream, const char* name, bool after) {
  TraceState& t = g_trace;
  if (t.events == nullptr) return;
  // A failed launch leaves its error pending for the launcher to report: then
  // record nothing (the pair is dropped) and leave the error alone.
  if (hipPeekAtLastError() != hipSuccess) {
    if (after && !t.skip) t.used -= 1;
    t.skip = true;
    return;
  }
  if (!after) {
    t.skip = t.used + 2 > t.capacity || t.used / 2 >= kMaxTraced;
    if (t.skip) return;
    t.names[t.used / 2] = name;
  } else if (t.skip) {
    return;
  }
  if (hipEventRecord(t.events[t.used], stream) != hipSuccess) {
    // an unusable event: drop its error (no launch error was pending) and
    // stop tracing, keeping the kernels bracketed so far
    (void)hipGetLastError();
    if (after) t.used -= 1;
    t.capacity = t.used;
    t.skip = true;
    return;
  }
  t.used += 1;
}

}  // namespace idx

extern "C" {

idx_status_t idx_trace_begin(hipEvent_t* events, int32_t capacity) {
  if (events == nullptr || capacity < 2) return IDX_ERR_INVALID_ARG;
  g_trace.events = events;
  g_trace.capacity = capacity;
  g_trace.used = 0;
  g_trace.skip = false;
  return IDX_OK;
}

int32_t idx_trace_end(const char** names, int32_t max_names) {
  TraceState& t = g_trace;
  const int n = t.events ? t.used / 2 : 0;
  if (names != nullptr)
    for (int i = 0; i < n && i < max_names; ++i) names[i] = t.names[i];
  t.events = nullptr;
  t.capacity = t.used = 0;
  return n;
}

}  // extern "C"
