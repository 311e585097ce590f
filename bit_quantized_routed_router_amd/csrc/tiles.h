// Small wave-level helpers shared by the routing and decode kernels: an F16
// MFMA row tile, a block reduction over waves, an even range split and the
// binary16 bit-pattern conversion.
//
// A "row tile" is 16 output rows of one weight matrix against 16 activation
// columns (tokens or slots).  Each wave walks a range of K-steps of 32 input
// elements; lane l feeds row (l & 15) of A and column (l & 15) of B with
// K-slots 8*(l>>4) .. +7, and holds D rows 4*(l>>4) .. +3 of column (l & 15).
// Activation columns are given per lane as a pointer to a binary16 vector of
// the K length (nullptr = zero column).
#pragma once

#include "common.h"

namespace ds4 {

__device__ inline half8_t load_b(const _Float16* col, int ks, int lane) {
  if (!col) return zero_half8();
  return *(const half8_t*)(col + ks * 32 + 8 * (lane >> 4));
}

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ------------------------------------------------------------------ F16 rows
// One F16 matrix (16 rows at rowp, lane row lane & 15) against 16 binary16
// columns (bcol, and bcol_lo for the lo half of a split fp32 input; NULL
// columns read as zero) over K-steps [ks0, ks1) of 32 inputs.  The loads of
// a batch of K-steps go out together before its MFMAs (constant-trip inner
// loops, so they unroll); the batch's tail past ks1 repeats the last step's
// address and is not multiplied.
template <bool LO>
__device__ inline void f16_tile(const uint16_t* __restrict__ rowp, const _Float16* bcol, const _Float16* bcol_lo,
                                int ks0, int ks1, int lane, float4_t& acc) {
  constexpr int kB = LO ? 4 : 8;
  const int ko = 8 * (lane >> 4);
  for (int k0 = ks0; k0 < ks1; k0 += kB) {
    half8_t a[kB], b[kB], bl[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int ks = min(k0 + u, ks1 - 1);
      a[u] = *(const half8_t*)(rowp + ks * 32 + ko);
      b[u] = load_b(bcol, ks, lane);
      if (LO) bl[u] = load_b(bcol_lo, ks, lane);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (k0 + u < ks1) {  // wave-uniform
        acc = mfma16x16x32(a[u], b[u], acc);
        if (LO) acc = mfma16x16x32(a[u], bl[u], acc);
      }
    }
  }
}

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
