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
// Two F16 matrices (e.g. gate and up) against the same columns.  W rows are
// row-major with row length K; rowp* point at row (row0 + (lane & 15)).
template <bool PAIR, bool LO>
__device__ inline void f16_tile(const uint16_t* __restrict__ rowp0, const uint16_t* __restrict__ rowp1,
                                const _Float16* bcol, const _Float16* bcol_lo, int ks0, int ks1, int lane,
                                float4_t& acc0, float4_t& acc1) {
  const int ko = 8 * (lane >> 4);
#pragma unroll 4
  for (int ks = ks0; ks < ks1; ++ks) {
    half8_t b = load_b(bcol, ks, lane);
    half8_t a0 = *(const half8_t*)(rowp0 + ks * 32 + ko);
    acc0 = mfma16x16x32(a0, b, acc0);
    half8_t a1;
    if (PAIR) {
      a1 = *(const half8_t*)(rowp1 + ks * 32 + ko);
      acc1 = mfma16x16x32(a1, b, acc1);
    }
    if (LO) {
      half8_t bl = load_b(bcol_lo, ks, lane);
      acc0 = mfma16x16x32(a0, bl, acc0);
      if (PAIR) acc1 = mfma16x16x32(a1, bl, acc1);
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
