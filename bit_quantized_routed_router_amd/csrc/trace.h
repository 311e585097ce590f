// Opt-in per-kernel timing.  While enabled (ds4moe_trace_enable), every
// launch made through DS4_LAUNCH is bracketed by a pair of HIP events on its
// own stream; ds4moe_trace_read waits for the recorded events and returns
// the accumulated time and launch count per kernel.  Disabled, the cost is
// one relaxed atomic load per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace ds4 {

struct TraceScope {
  int slot = -1;
  hipStream_t st;
  TraceScope(const char* name, hipStream_t s);
  ~TraceScope();
};

}  // namespace ds4

#define DS4_LAUNCH(kernel, grid, block, shmem, stream, ...)                  \
  do {                                                                       \
    ::ds4::TraceScope ds4_trace_scope_(#kernel, stream);                     \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);     \
  } while (0)
