// Wave-level MFMA tile loops shared by the decode and prefill kernels.
//
// A "row tile" is 16 output rows of one weight matrix against 16 activation
// columns (tokens or slots).  Each wave walks a range of K-steps of 32 input
// elements; lane l feeds row (l & 15) of A and column (l & 15) of B with
// K-slots 8*(l>>4) .. +7, and holds D rows 4*(l>>4) .. +3 of column (l & 15).
//
// Activation columns are given per lane as a pointer to a binary16 vector of
// the K length (nullptr = zero column).  Weights are dequantized in
// registers into exact small integers (CB2: sign*(2s+1)*m, Q2K: s*q), the
// MFMA accumulates one super-block in fp32, and the super-block scales are
// applied to that partial sum:  CB2 acc += d * P;  Q2K acc += d * P - dmin * M
// where M is a second MFMA of the sub-block mins m_j against per-sub-block
// column sums (hi and lo binary16 parts).
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

// ------------------------------------------------------------------ CB2 rows
// codes0/1: code plane of the matrix (or matrices), dpl0/1: its scale plane,
// nb blocks per row, row0: first row of the tile.
template <bool PAIR, bool LO>
__device__ inline void cb2_tile(const uint8_t* __restrict__ codes0, const uint16_t* __restrict__ dpl0,
                                const uint8_t* __restrict__ codes1, const uint16_t* __restrict__ dpl1, int nb,
                                int row0, const _Float16* bcol, const _Float16* bcol_lo, int ks0, int ks1,
                                int lane, const uint32_t* mag, const uint32_t* sgn, float4_t& acc0,
                                float4_t& acc1) {
  const int q = lane >> 4;
  const int arow = row0 + (lane & 15);
  const uint8_t* rp0 = codes0 + (int64_t)arow * nb * 64;
  const uint8_t* rp1 = PAIR ? codes1 + (int64_t)arow * nb * 64 : nullptr;
  const int orow = row0 + 4 * q;  // first of this lane's four output rows
  int ks = ks0;
  while (ks < ks1) {
    const int b = ks >> 3;
    const int kend = min(ks1, (b + 1) << 3);
    float4_t p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
    for (; ks < kend; ++ks) {
      const int off = b * 64 + 8 * (ks & 7);
      half8_t bv = load_b(bcol, ks, lane);
      u32x2_t c0 = *(const u32x2_t*)(rp0 + off);
      half8_t a0 = cb2_frag(c0.x, c0.y, q, mag, sgn);
      p0 = mfma16x16x32(a0, bv, p0);
      half8_t a1;
      if (PAIR) {
        u32x2_t c1 = *(const u32x2_t*)(rp1 + off);
        a1 = cb2_frag(c1.x, c1.y, q, mag, sgn);
        p1 = mfma16x16x32(a1, bv, p1);
      }
      if (LO) {
        half8_t bl = load_b(bcol_lo, ks, lane);
        p0 = mfma16x16x32(a0, bl, p0);
        if (PAIR) p1 = mfma16x16x32(a1, bl, p1);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc0[r] += h2f(dpl0[(int64_t)(orow + r) * nb + b]) * p0[r];
      if (PAIR) acc1[r] += h2f(dpl1[(int64_t)(orow + r) * nb + b]) * p1[r];
    }
  }
}

// ------------------------------------------------------------------ Q2K rows
// bcol: binary16 column of length K; csum: fp32 sums of that column over
// each 16-element sub-block (length K/16), nullptr with bcol == nullptr.
__device__ inline void q2k_tile(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sub,
                                const uint16_t* __restrict__ sup, int nb, int row0, const _Float16* bcol,
                                const float* csum, int ks0, int ks1, int lane, float4_t& acc) {
  const int q = lane >> 4;
  const int arow = row0 + (lane & 15);
  const uint8_t* rp = codes + (int64_t)arow * nb * 64;
  const uint8_t* sp = sub + (int64_t)arow * nb * 16;
  const int orow = row0 + 4 * q;
  int ks = ks0;
  while (ks < ks1) {
    const int b = ks >> 3;
    const int kend = min(ks1, (b + 1) << 3);
    const bool first = ks == (b << 3);
    float4_t p = {0.f, 0.f, 0.f, 0.f};
    for (; ks < kend; ++ks) {
      const int jsub = 2 * (ks & 7) + (q >> 1);  // Q2K sub-block of this lane's 8 codes
      const uint32_t u = *(const uint32_t*)(rp + b * 64 + 4 * jsub);
      const uint32_t s = sp[b * 16 + jsub] & 15u;
      half8_t a = q2k_frag(u, q & 1, s);
      p = mfma16x16x32(a, load_b(bcol, ks, lane), p);
    }
    // min term of super-block b: K'-slots = its 16 sub-blocks (lanes q = 0, 1).
    // Added once per super-block, by the wave whose range holds its first step.
    float4_t pm = {0.f, 0.f, 0.f, 0.f};
    if (first) {
      half8_t am = zero_half8(), bh = zero_half8(), bl = zero_half8();
      if (q < 2) {
        u32x2_t mb = *(const u32x2_t*)(sp + b * 16 + 8 * q);
        u32x4_t t;
        t.x = nib_hi_pair_f16(mb.x, 0);
        t.y = nib_hi_pair_f16(mb.x, 2);
        t.z = nib_hi_pair_f16(mb.y, 0);
        t.w = nib_hi_pair_f16(mb.y, 2);
        am = as_half8(t);
        if (csum) {
          const float* cs = csum + b * 16 + 8 * q;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = cs[e];
            _Float16 h = (_Float16)v;
            bh[e] = h;
            bl[e] = (_Float16)(v - (float)h);
          }
        }
      }
      pm = mfma16x16x32(am, bh, pm);
      pm = mfma16x16x32(am, bl, pm);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t* ss = sup + ((int64_t)(orow + r) * nb + b) * 2;
      acc[r] += h2f(ss[0]) * p[r] - h2f(ss[1]) * pm[r];
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

__device__ inline void stage_grid_tables(uint32_t* mag, uint32_t* sgn, const GridTables& t) {
  for (int i = threadIdx.x; i < 256 * 4; i += blockDim.x) mag[i] = (&t.mag[0][0])[i];
  for (int i = threadIdx.x; i < 128 * 4; i += blockDim.x) sgn[i] = (&t.sgn[0][0])[i];
}

}  // namespace ds4
