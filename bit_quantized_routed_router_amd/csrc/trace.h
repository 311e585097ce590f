// Opt-in per-kernel timing.  While enabled (ds4moe_trace_enable), every
// launch made through DS4_LAUNCH goes out through hipExtLaunchKernel with a
// start and a stop event, which the runtime attaches to the kernel's own
// dispatch on its stream (they time the kernel, not the gap between host
// calls); ds4moe_trace_read waits for them and returns the accumulated time
// and launch count per kernel.  Disabled, the cost is one relaxed atomic
// load per launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace ds4 {

// Takes an event pair at construction (none while tracing is off); the pair
// joins the pending list (under the lock) at destruction, after the launch
// that records them, so a concurrent ds4moe_trace_read never sees half an
// entry.
struct TraceScope {
  int id = -1;
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t st;
  TraceScope(const char* name, hipStream_t s);
  ~TraceScope();
};

}  // namespace ds4

#define DS4_LAUNCH(kernel, grid, block, shmem, stream, ...)                                          \
  do {                                                                                               \
    ::ds4::TraceScope ds4_trace_scope_(#kernel, stream);                                             \
    if (ds4_trace_scope_.a)                                                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ds4_trace_scope_.a, ds4_trace_scope_.b, \
                            0u, __VA_ARGS__);                                                        \
    else                                                                                             \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                           \
  } while (0)
