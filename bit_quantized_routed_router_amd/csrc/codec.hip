// CB2 / Q2K / MXFP4 / Q4K encoders and decoders (byte layouts in include/ds4moe.h).
//
// The pages name the formats only (DS4 (DwarfStar 4) wiki note, "Key
// Techniques": IQ2_XXS for gate/up, Q2_K for down); the quantizer steps are
// this library's own deterministic definition, reproduced bit for bit: every
// floating-point step is a single IEEE binary32 operation with
// round-to-nearest-even (explicit _rn intrinsics, file built with
// -ffp-contract=off), binary16 rounding is done in integer arithmetic, and
// every search breaks ties towards the lower index.
#include "common.h"
#include "internal.h"
#include "trace.h"

namespace ds4 {

__constant__ GridTables c_tables = make_grid_tables();

// ---------------------------------------------------------------------------
// CB2 quantizer.  32 lanes per 256-weight super-block, one lane per group of
// 8: lane g32 owns sub-block j = g32 / 4, group g = g32 % 4.
//  1. A_j = max|x| / 5 over the sub-block
//  2. d = half(min(max_j A_j / 31, 65504)); d == 0 -> all codes zero
//  3. s_j = clamp(rne((A_j / d - 1) * 0.5), 0, 15), a_j = d * (2 s_j + 1)
//  4. R_k = rne(min(|x_k| / a_j, 64) * 4096); entry score
//     sum_k 4096 m^2 - 2 R_k m, plus 4 min_k R_k m when the count of x_k < 0
//     is odd; lowest score wins (lower entry on ties), the flipped element is
//     the lowest k of minimal R_k m.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_cb2(const float* __restrict__ w, int64_t nblk,
                                                   uint8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ dplane) {
  __shared__ int32_t s_imag[256 * 8];
  __shared__ int32_t s_isq[256];
  for (int i = threadIdx.x; i < 256 * 8; i += blockDim.x) s_imag[i] = (&c_tables.imag[0][0])[i];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s_isq[i] = c_tables.isq[i];
  __syncthreads();

  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  const int g32 = threadIdx.x & 31;
  const int j = g32 >> 2, g = g32 & 3;
  const bool valid = blk < nblk;
  float v[8];
  if (valid) {
    const float4* src = (const float4*)(w + blk * QK + 8 * g32);
    float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.0f;
  }
  float gm = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) gm = fmaxf(gm, fabsf(v[k]));
  gm = fmaxf(gm, __shfl_xor(gm, 1, 32));
  gm = fmaxf(gm, __shfl_xor(gm, 2, 32));
  const float A = __fdiv_rn(gm, 5.0f);
  float amax = A;
  amax = fmaxf(amax, __shfl_xor(amax, 4, 32));
  amax = fmaxf(amax, __shfl_xor(amax, 8, 32));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 32));
  const uint32_t dbits = f32_to_f16_bits_rne(fminf(__fdiv_rn(amax, 31.0f), 65504.0f));
  const float d = f16_bits_to_f32(dbits);

  uint32_t best = 0, code = 0, s = 0;
  if (d != 0.0f) {
    float u = __fmul_rn(__fsub_rn(__fdiv_rn(A, d), 1.0f), 0.5f);
    float sr = __builtin_rintf(u);
    s = sr < 0.0f ? 0u : (sr > 15.0f ? 15u : (uint32_t)sr);
    const float a = __fmul_rn(d, (float)(2 * s + 1));
    int32_t R[8];
    uint32_t neg = 0;
    int nneg = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float r = fminf(__fdiv_rn(fabsf(v[k]), a), 64.0f);
      R[k] = (int32_t)__builtin_rintf(__fmul_rn(r, 4096.0f));
      if (v[k] < 0.0f) {
        neg |= 1u << k;
        ++nneg;
      }
    }
    const bool odd = nneg & 1;
    int32_t bscore = 0;
    for (int e = 0; e < 256; ++e) {
      const int32_t* m = s_imag + 8 * e;
      int32_t dot = 0, mn = 0x7FFFFFFF;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int32_t f = R[k] * m[k];
        dot += f;
        mn = f < mn ? f : mn;
      }
      int32_t sc = s_isq[e] - 2 * dot + (odd ? 4 * mn : 0);
      if (e == 0 || sc < bscore) {
        bscore = sc;
        best = (uint32_t)e;
      }
    }
    if (odd) {
      const int32_t* m = s_imag + 8 * best;
      int kf = 0;
      int32_t fmin = R[0] * m[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) {
        int32_t f = R[k] * m[k];
        if (f < fmin) {
          fmin = f;
          kf = k;
        }
      }
      neg ^= 1u << kf;
    }
    code = neg & 0x7Fu;
  }
  // gather the four sign codes of the sub-block into its aux word
  uint32_t c1 = __shfl_xor(code, 1, 32), c2 = __shfl_xor(code, 2, 32), c3 = __shfl_xor(code, 3, 32);
  if (valid) {
    uint8_t* blkp = codes + blk * 64;
    blkp[8 * j + g] = (uint8_t)best;
    if (g == 0) {
      uint32_t aux = code | (c1 << 7) | (c2 << 14) | (c3 << 21) | (s << 28);
      *(uint32_t*)(blkp + 8 * j + 4) = aux;
    }
    if (g32 == 0) dplane[blk] = (uint16_t)dbits;
  }
}

// ---------------------------------------------------------------------------
// Q2K quantizer.  16 lanes per super-block, one lane per sub-block of 16.
//  1. b_j = max(0, -min x), a_j = (max x + b_j) / 3
//  2. d = half(min(max a / 15, 65504)), dmin = half(min(max b / 15, 65504))
//  3. s_j = d > 0 ? clamp(rne(a_j / d), 0, 15) : 0; m_j likewise with dmin
//  4. q = argmin_q |((d*s)*q - dmin*m) - x|, lower q on ties.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_q2k(const float* __restrict__ w, int64_t nblk,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ sub,
                                                   uint16_t* __restrict__ sup) {
  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int j = threadIdx.x & 15;
  const bool valid = blk < nblk;
  float v[16];
  if (valid) {
    const float4* src = (const float4*)(w + blk * QK + 16 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 t = src[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }
  float mx = v[0], mn = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mx = fmaxf(mx, v[i]);
    mn = fminf(mn, v[i]);
  }
  const float b = mn < 0.0f ? -mn : 0.0f;
  const float a = __fdiv_rn(__fadd_rn(mx, b), 3.0f);
  float amax = a, bmax = b;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, o, 16));
  }
  const uint32_t dbits = f32_to_f16_bits_rne(fminf(__fdiv_rn(amax, 15.0f), 65504.0f));
  const uint32_t mbits = f32_to_f16_bits_rne(fminf(__fdiv_rn(bmax, 15.0f), 65504.0f));
  const float d = f16_bits_to_f32(dbits), dmin = f16_bits_to_f32(mbits);
  uint32_t s = 0, m = 0;
  if (d > 0.0f) {
    float t = __builtin_rintf(__fdiv_rn(a, d));
    s = t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
  }
  if (dmin > 0.0f) {
    float t = __builtin_rintf(__fdiv_rn(b, dmin));
    m = t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
  }
  const float ds = __fmul_rn(d, (float)s);
  const float dm = __fmul_rn(dmin, (float)m);
  float lvl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) lvl[q] = __fsub_rn(__fmul_rn(ds, (float)q), dm);
  uint32_t u = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t bq = 0;
    float berr = fabsf(__fsub_rn(lvl[0], v[i]));
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      float err = fabsf(__fsub_rn(lvl[q], v[i]));
      if (err < berr) {
        berr = err;
        bq = (uint32_t)q;
      }
    }
    u |= bq << (2 * i);
  }
  if (valid) {
    *(uint32_t*)(codes + blk * 64 + 4 * j) = u;
    sub[blk * 16 + j] = (uint8_t)(s | (m << 4));
    if (j == 0) {
      sup[2 * blk] = (uint16_t)dbits;
      sup[2 * blk + 1] = (uint16_t)mbits;
    }
  }
}

// ---------------------------------------------------------------------------
// Decoders (test export): one lane per CB2 group / Q2K sub-block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_cb2(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ dplane, int64_t ngroups,
                                                     float* __restrict__ out) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= ngroups) return;
  const int64_t blk = gi >> 5;
  const int j = (int)((gi >> 2) & 7), g = (int)(gi & 3);
  const uint8_t* bp = codes + blk * 64 + 8 * j;
  const uint32_t idx = bp[g];
  const uint32_t aux = *(const uint32_t*)(bp + 4);
  const uint32_t code = (aux >> (7 * g)) & 0x7Fu;
  const float d = f16_bits_to_f32(dplane[blk]);
  const float ds = __fmul_rn(d, (float)(2 * (aux >> 28) + 1));
  const uint32_t par = __builtin_popcount(code) & 1u;
  float r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float mag = __fmul_rn(ds, (float)c_tables.imag[idx][k]);
    uint32_t negk = k < 7 ? (code >> k) & 1u : par;
    r[k] = negk ? -mag : mag;
  }
  float4* dst = (float4*)(out + gi * 8);
  dst[0] = make_float4(r[0], r[1], r[2], r[3]);
  dst[1] = make_float4(r[4], r[5], r[6], r[7]);
}

__global__ __launch_bounds__(256) void k_dequant_q2k(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ sub,
                                                     const uint16_t* __restrict__ sup, int64_t nsub,
                                                     float* __restrict__ out) {
  const int64_t si = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= nsub) return;
  const int64_t blk = si >> 4;
  const int j = (int)(si & 15);
  const uint32_t u = *(const uint32_t*)(codes + blk * 64 + 4 * j);
  const uint32_t sm = sub[blk * 16 + j];
  const float d = f16_bits_to_f32(sup[2 * blk]), dmin = f16_bits_to_f32(sup[2 * blk + 1]);
  const float ds = __fmul_rn(d, (float)(sm & 15u));
  const float dm = __fmul_rn(dmin, (float)(sm >> 4));
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = __fsub_rn(__fmul_rn(ds, (float)((u >> (2 * i)) & 3u)), dm);
  float4* dst = (float4*)(out + si * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// MXFP4 (OCP MX: FP4 E2M1 elements, one E8M0 scale per 32), one lane per
// block of 32.  Quantizer:
//  1. amax = max |x|; zero blocks get scale 0 and zero codes;
//  2. scale code = clamp(floor(log2 amax) - 2 + 127, 0, 254), floor(log2)
//     read from amax's exponent bits (normal or subnormal);
//  3. r = |x| * 2^(127 - code) (exact wherever it can change the code:
//     results below 2^-126, the only ones rounded, all give code 0), then
//     the nearest E2M1 magnitude, ties to the even code, beyond 6 to 6;
//     the sign bit for negative x of non-zero magnitude.
// ---------------------------------------------------------------------------
__device__ inline int floor_log2_pos(float a) {  // a > 0, finite
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  const int e = (int)(u >> 23);
  if (e > 0) return e - 127;
  return (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;  // subnormal: mantissa * 2^-149
}
__device__ inline float pow2f(int k) {  // 2^k for -149 <= k <= 127, exact
  return k >= -126 ? __builtin_bit_cast(float, (uint32_t)(k + 127) << 23)
                   : __builtin_bit_cast(float, 1u << (k + 149));
}
// nearest E2M1 magnitude code of r >= 0, ties to the even code, saturating
__device__ inline uint32_t e2m1_code(float r) {
  if (r <= 0.25f) return 0;
  if (r < 0.75f) return 1;
  if (r <= 1.25f) return 2;
  if (r < 1.75f) return 3;
  if (r <= 2.5f) return 4;
  if (r < 3.5f) return 5;
  if (r <= 5.0f) return 6;
  return 7;
}
// E2M1 magnitude of a 3-bit code: exponent 0 subnormal (0, 0.5), else
// (1 + m/2) * 2^(e - 1)
__device__ inline float e2m1_mag(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  return e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * pow2f((int)e - 1);
}

__global__ __launch_bounds__(256) void k_quant_mx4(const float* __restrict__ w, int64_t nblk,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblk) return;
  float v[32];
  const float4* src = (const float4*)(w + blk * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 a = src[i];
    v[4 * i] = a.x;
    v[4 * i + 1] = a.y;
    v[4 * i + 2] = a.z;
    v[4 * i + 3] = a.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t out[4] = {0u, 0u, 0u, 0u};
  int sc = 0;
  if (amax > 0.0f) {
    sc = min(max(floor_log2_pos(amax) - 2 + 127, 0), 254);
    const float inv = pow2f(127 - sc);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t m = e2m1_code(__fmul_rn(fabsf(v[i]), inv));
      const uint32_t c = m | ((v[i] < 0.0f && m != 0u) ? 8u : 0u);
      out[i >> 3] |= c << (4 * (i & 7));
    }
  }
  *(u32x4_t*)(codes + blk * 16) = u32x4_t{out[0], out[1], out[2], out[3]};
  scales[blk] = (uint8_t)sc;
}

__global__ __launch_bounds__(256) void k_dequant_mx4(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t nblk,
                                                     float* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblk) return;
  const u32x4_t cw = *(const u32x4_t*)(codes + blk * 16);
  const int sc = scales[blk];
  const float x = sc == 255 ? __builtin_nanf("") : pow2f(sc - 127);
  float4* dst = (float4*)(out + blk * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c = (cw[i >> 1] >> (4 * (4 * (i & 1) + j))) & 15u;
      const float m = __fmul_rn(e2m1_mag(c & 7u), x);
      r[j] = (c & 8u) ? -m : m;
    }
    dst[i] = make_float4(r[0], r[1], r[2], r[3]);
  }
}

// ---------------------------------------------------------------------------
// Q4K quantizer.  8 lanes per super-block, one lane per sub-block of 32: the
// Q2K steps with 4-bit codes and 6-bit scales.
//  1. b_j = max(0, -min x), a_j = (max x + b_j) / 15
//  2. d = half(min(max a / 63, 65504)), dmin = half(min(max b / 63, 65504))
//  3. s_j = d > 0 ? clamp(rne(a_j / d), 0, 63) : 0; m_j likewise with dmin
//  4. q = argmin_q |((d*s)*q - dmin*m) - x|, lower q on ties.
// Code word k of sub-block j: element 8k + 2p at bits 4p, 8k + 2p + 1 at
// bits 16 + 4p; scale words: nibbles of s and m, then their high bits.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_q4k(const float* __restrict__ w, int64_t nblk,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scl,
                                                   uint16_t* __restrict__ sup) {
  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  const bool valid = blk < nblk;
  float v[32];
  if (valid) {
    const float4* src = (const float4*)(w + blk * QK + 32 * j);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 t = src[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  float mx = v[0], mn = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mx = fmaxf(mx, v[i]);
    mn = fminf(mn, v[i]);
  }
  const float b = mn < 0.0f ? -mn : 0.0f;
  const float a = __fdiv_rn(__fadd_rn(mx, b), 15.0f);
  float amax = a, bmax = b;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o, 8));
    bmax = fmaxf(bmax, __shfl_xor(bmax, o, 8));
  }
  const uint32_t dbits = f32_to_f16_bits_rne(fminf(__fdiv_rn(amax, 63.0f), 65504.0f));
  const uint32_t mbits = f32_to_f16_bits_rne(fminf(__fdiv_rn(bmax, 63.0f), 65504.0f));
  const float d = f16_bits_to_f32(dbits), dmin = f16_bits_to_f32(mbits);
  uint32_t s = 0, m = 0;
  if (d > 0.0f) {
    float t = __builtin_rintf(__fdiv_rn(a, d));
    s = t < 0.0f ? 0u : (t > 63.0f ? 63u : (uint32_t)t);
  }
  if (dmin > 0.0f) {
    float t = __builtin_rintf(__fdiv_rn(b, dmin));
    m = t < 0.0f ? 0u : (t > 63.0f ? 63u : (uint32_t)t);
  }
  const float ds = __fmul_rn(d, (float)s);
  const float dm = __fmul_rn(dmin, (float)m);
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t bq = 0;
    float berr = fabsf(__fsub_rn(__fsub_rn(0.0f, dm), v[i]));
    for (int q = 1; q < 16; ++q) {
      const float err = fabsf(__fsub_rn(__fsub_rn(__fmul_rn(ds, (float)q), dm), v[i]));
      if (err < berr) {
        berr = err;
        bq = (uint32_t)q;
      }
    }
    const int e = i & 7, p = e >> 1;
    cw[i >> 3] |= bq << ((e & 1) ? 16 + 4 * p : 4 * p);
  }
  // scale words of the block: each lane's fields, OR-reduced over the 8 lanes
  uint32_t w0 = (s & 15u) << (4 * j), w1 = (m & 15u) << (4 * j);
  uint32_t w2 = ((s >> 4) << (2 * j)) | ((m >> 4) << (16 + 2 * j));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    w0 |= __shfl_xor(w0, o, 8);
    w1 |= __shfl_xor(w1, o, 8);
    w2 |= __shfl_xor(w2, o, 8);
  }
  if (valid) {
    *(u32x4_t*)(codes + blk * 128 + 16 * j) = u32x4_t{cw[0], cw[1], cw[2], cw[3]};
    if (j == 0) {
      uint32_t* sw = (uint32_t*)(scl + blk * 12);
      sw[0] = w0;
      sw[1] = w1;
      sw[2] = w2;
      sup[2 * blk] = (uint16_t)dbits;
      sup[2 * blk + 1] = (uint16_t)mbits;
    }
  }
}

// One lane per Q4K sub-block of 32.
__global__ __launch_bounds__(256) void k_dequant_q4k(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scl,
                                                     const uint16_t* __restrict__ sup, int64_t nsub,
                                                     float* __restrict__ out) {
  const int64_t si = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= nsub) return;
  const int64_t blk = si >> 3;
  const int j = (int)(si & 7);
  const u32x4_t cw = *(const u32x4_t*)(codes + blk * 128 + 16 * j);
  const uint32_t* sw = (const uint32_t*)(scl + blk * 12);
  const uint32_t s = ((sw[0] >> (4 * j)) & 15u) | (((sw[2] >> (2 * j)) & 3u) << 4);
  const uint32_t m = ((sw[1] >> (4 * j)) & 15u) | (((sw[2] >> (16 + 2 * j)) & 3u) << 4);
  const float d = f16_bits_to_f32(sup[2 * blk]), dmin = f16_bits_to_f32(sup[2 * blk + 1]);
  const float ds = __fmul_rn(d, (float)s);
  const float dm = __fmul_rn(dmin, (float)m);
  float4* dst = (float4*)(out + si * 32);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = e >> 1;
      const uint32_t q = (cw[k] >> ((e & 1) ? 16 + 4 * p : 4 * p)) & 15u;
      r[e] = __fsub_rn(__fmul_rn(ds, (float)q), dm);
    }
    dst[2 * k] = make_float4(r[0], r[1], r[2], r[3]);
    dst[2 * k + 1] = make_float4(r[4], r[5], r[6], r[7]);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_cb2(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  uint8_t* codes = (uint8_t*)packed;
  uint16_t* dpl = (uint16_t*)(codes + nblk * 64);
  const int64_t threads = nblk * 32;
  if (threads == 0) return hipSuccess;
  DS4_LAUNCH(k_quant_cb2, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, w, nblk, codes, dpl);
  return hipGetLastError();
}

hipError_t launch_quant_q2k(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  uint8_t* codes = (uint8_t*)packed;
  uint8_t* sub = codes + nblk * 64;
  uint16_t* sup = (uint16_t*)(codes + nblk * 80);
  const int64_t threads = nblk * 16;
  if (threads == 0) return hipSuccess;
  DS4_LAUNCH(k_quant_q2k, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, w, nblk, codes, sub, sup);
  return hipGetLastError();
}

hipError_t launch_dequant_cb2(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  const uint8_t* codes = (const uint8_t*)packed;
  const uint16_t* dpl = (const uint16_t*)(codes + nblk * 64);
  const int64_t ng = nblk * 32;
  if (ng == 0) return hipSuccess;
  DS4_LAUNCH(k_dequant_cb2, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, codes, dpl, ng, out);
  return hipGetLastError();
}

hipError_t launch_dequant_q2k(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  const uint8_t* codes = (const uint8_t*)packed;
  const uint8_t* sub = codes + nblk * 64;
  const uint16_t* sup = (const uint16_t*)(codes + nblk * 80);
  const int64_t ns = nblk * 16;
  if (ns == 0) return hipSuccess;
  DS4_LAUNCH(k_dequant_q2k, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, codes, sub, sup, ns, out);
  return hipGetLastError();
}

hipError_t launch_quant_q4k(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  uint8_t* codes = (uint8_t*)packed;
  uint8_t* scl = codes + nblk * 128;
  uint16_t* sup = (uint16_t*)(codes + nblk * 140);
  const int64_t threads = nblk * 8;
  if (threads == 0) return hipSuccess;
  DS4_LAUNCH(k_quant_q4k, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, w, nblk, codes, scl, sup);
  return hipGetLastError();
}

hipError_t launch_dequant_q4k(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st) {
  const int64_t nblk = rows * (cols / QK);
  const uint8_t* codes = (const uint8_t*)packed;
  const uint8_t* scl = codes + nblk * 128;
  const uint16_t* sup = (const uint16_t*)(codes + nblk * 140);
  const int64_t ns = nblk * 8;
  if (ns == 0) return hipSuccess;
  DS4_LAUNCH(k_dequant_q4k, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, codes, scl, sup, ns, out);
  return hipGetLastError();
}

hipError_t launch_quant_mx4(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st) {
  const int64_t nblk = rows * (cols / 32);
  uint8_t* codes = (uint8_t*)packed;
  uint8_t* scales = codes + nblk * 16;
  if (nblk == 0) return hipSuccess;
  DS4_LAUNCH(k_quant_mx4, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st, w, nblk, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dequant_mx4(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st) {
  const int64_t nblk = rows * (cols / 32);
  const uint8_t* codes = (const uint8_t*)packed;
  const uint8_t* scales = codes + nblk * 16;
  if (nblk == 0) return hipSuccess;
  DS4_LAUNCH(k_dequant_mx4, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st, codes, scales, nblk, out);
  return hipGetLastError();
}

}  // namespace ds4
