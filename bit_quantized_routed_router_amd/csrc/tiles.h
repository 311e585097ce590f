// Small helpers shared by the routing and decode kernels: a block reduction
// over waves, an even range split and the binary16 bit-pattern conversion.
#pragma once

#include "common.h"

namespace ds4 {

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Sum a per-lane float4 accumulator over the NW waves of a block through LDS;
// the result lands in wave 0.  red: NW*64*4 floats of LDS.
template <int NW>
__device__ inline float4_t block_reduce_waves(float4_t v, float* red, int wave, int lane) {
  if (NW == 1) return v;
  *(float4_t*)(red + (wave * 64 + lane) * 4) = v;
  __syncthreads();
  float4_t s = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w) s += *(const float4_t*)(red + (w * 64 + lane) * 4);
  }
  __syncthreads();
  return s;
}

// Even split of [0, n) into NW parts.
__device__ inline void split_range(int n, int parts, int i, int& b, int& e) {
  b = (int)(((int64_t)n * i) / parts);
  e = (int)(((int64_t)n * (i + 1)) / parts);
}

}  // namespace ds4
