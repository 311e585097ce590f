// Chunk ring of the prefill GEMMs: activation (and weight) chunks copied
// straight into LDS (global_load_lds) a few chunks ahead of the compute, one
// workgroup barrier per chunk.
#pragma once

#include "common.h"

namespace ds4 {

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the chunk loop.  __syncthreads() carries a release
// fence, and the compiler meets it by waiting for every outstanding load --
// LDS-bound copies count as LDS stores -- which would drain the whole
// prefetch ring.  Here the loop orders memory itself: a wave has waited for
// its own copies into the slot it is about to read before this barrier, and
// its reads of a slot have returned (lgkmcnt) before the barrier after which
// that slot is refilled.  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ inline void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The chunk loop of a tile with R chunks in flight and one barrier per
// chunk.  issue(ch, u) starts loading chunk ch into ring slot u (B
// vector-memory instructions per lane); compute(u) consumes slot u.  At each
// step the wave waits for its copies of the chunk it is about to use, the
// barrier makes everyone's copies visible and shows that all waves are done
// with the previous chunk, whose slot is then refilled with the chunk R - 1
// ahead before computing.  Every step issues a batch -- past the last chunk
// it repeats the last one (cache hits, never read) -- so the loop has one
// shape and the compiler's own waits for the weight registers stay partial.
// Passes of R chunks run unrolled (static slot indices); steps past the last
// chunk keep the waits and issues and skip the compute.  The final wait
// drains every load before the block's LDS can be reused.
template <int R, int B, typename Issue, typename Compute>
__device__ __attribute__((always_inline)) inline void ring_loop(int nch, Issue issue, Compute compute) {
  static_assert(R >= 2 && (R - 1) * B <= 63, "ring depth");
#pragma unroll
  for (int u = 0; u < R - 1; ++u) issue(min(u, nch - 1), u);
  auto step = [&](int ch, int u) {
    pin();
    vm_wait<(R - 2) * B>();
    ring_barrier();
    pin();
    issue(min(ch + R - 1, nch - 1), (u + R - 1) % R);
    pin();
    if (ch < nch) compute(u);
  };
  for (int ch0 = 0; ch0 < nch; ch0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) step(ch0 + u, u);
  }
  vm_wait<0>();
}

}  // namespace ds4
