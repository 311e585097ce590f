// Shared device helpers for the ds4moe kernels (gfx950 / CDNA4, wave64).
//
// The layer is the routed mixture-of-experts feed-forward block of DeepSeek V4
// Flash as DS4 runs it (DS4 (DwarfStar 4) wiki note, "Architecture" and "Key
// Techniques"): an F16 router picks the top-k of E experts, one F16 shared
// expert always runs, and the routed experts' gate/up weights are stored in a
// 2-bit codebook format (CB2, IQ2_XXS class) and their down weights in a
// 2-bit super-block format (Q2K, Q2_K class).  The byte layouts are the
// library's own (the pages only name the formats); they are written out in
// include/ds4moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// Three words at a 4-byte-aligned address (one global_load_dwordx3)
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef u32x3_t u32x3_a4_t __attribute__((aligned(4)));

constexpr int QK = 256;  // super-block length along K
constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// Codebook grid: 256 entries x 8 levels in {0,1,2} (magnitude 2*level+1),
// drawn with splitmix64 (Steele, Lea & Flood 2014) from a fixed seed, the
// high 32 bits of each draw taken modulo 3; an entry equal to an earlier one
// is drawn again.  Built at compile time, so no table is ever uploaded.
// ---------------------------------------------------------------------------
constexpr uint64_t kGridSeed = 0x44533447524944ULL;  // ASCII "DS4GRID"

constexpr uint64_t splitmix64_next(uint64_t& s) {
  s += 0x9E3779B97F4A7C15ULL;
  uint64_t z = s;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

struct GridLevels {
  uint8_t lv[256][8];
};

constexpr GridLevels make_grid_levels() {
  GridLevels g{};
  uint64_t st = kGridSeed;
  for (int i = 0; i < 256; ++i) {
    for (;;) {
      for (int k = 0; k < 8; ++k) g.lv[i][k] = (uint8_t)((splitmix64_next(st) >> 32) % 3);
      bool dup = false;
      for (int j = 0; j < i && !dup; ++j) {
        bool same = true;
        for (int k = 0; k < 8; ++k) same = same && (g.lv[j][k] == g.lv[i][k]);
        dup = same;
      }
      if (!dup) break;
    }
  }
  return g;
}

inline constexpr GridLevels kGridLevels = make_grid_levels();

// Tables the kernels stage into LDS:
//   mag[e][p]  : binary16 pair (m_{2p}, m_{2p+1}) of entry e (low, high half)
//   sgn[c][p]  : sign bits (bit 15 / bit 31) of elements 2p, 2p+1 for the
//                7-bit sign code c; element 7's sign is the parity of c
//   imag[e][k] : integer magnitudes for the quantizer's search
//   isq[e]     : sum_k 4096 * m_ek^2
//   mag8[e][w] : byte k of word w = high byte of binary16 m_{4w+k} (its low
//                byte is zero for m in {1, 3, 5})
//   sgn8[c][w] : byte k of word w = 0x80 if element 4w+k is negative
struct GridTables {
  uint32_t mag[256][4];
  uint32_t sgn[128][4];
  int32_t imag[256][8];
  int32_t isq[256];
  uint32_t mag8[256][2];
  uint32_t sgn8[128][2];
};

constexpr uint32_t f16_of_small_odd(int m) {  // 1 -> 0x3C00, 3 -> 0x4200, 5 -> 0x4500
  return m == 1 ? 0x3C00u : (m == 3 ? 0x4200u : 0x4500u);
}

constexpr GridTables make_grid_tables() {
  GridTables t{};
  for (int e = 0; e < 256; ++e) {
    int sq = 0;
    for (int k = 0; k < 8; ++k) {
      int m = 2 * kGridLevels.lv[e][k] + 1;
      t.imag[e][k] = m;
      sq += 4096 * m * m;
    }
    t.isq[e] = sq;
    for (int p = 0; p < 4; ++p)
      t.mag[e][p] = f16_of_small_odd(t.imag[e][2 * p]) | (f16_of_small_odd(t.imag[e][2 * p + 1]) << 16);
    for (int k = 0; k < 8; ++k) t.mag8[e][k >> 2] |= (f16_of_small_odd(t.imag[e][k]) >> 8) << (8 * (k & 3));
  }
  for (int c = 0; c < 128; ++c) {
    int par = 0;
    for (int k = 0; k < 7; ++k) par ^= (c >> k) & 1;
    for (int p = 0; p < 4; ++p) {
      int k0 = 2 * p, k1 = 2 * p + 1;
      uint32_t n0 = (uint32_t)((c >> k0) & 1);
      uint32_t n1 = k1 < 7 ? (uint32_t)((c >> k1) & 1) : (uint32_t)par;
      t.sgn[c][p] = (n0 << 15) | (n1 << 31);
      t.sgn8[c][p >> 1] |= ((n0 << 7) | (n1 << 15)) << (16 * (p & 1));
    }
  }
  return t;
}

// ---------------------------------------------------------------------------
// binary16 <-> binary32 in integer arithmetic (independent of mode bits)
// ---------------------------------------------------------------------------
__host__ __device__ inline float f16_bits_to_f32(uint32_t h) {
  uint32_t sign = (h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu;
  uint32_t m = h & 0x3FFu;
  uint32_t bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal: normalise
      int sh = 0;
      while (!(m & 0x400u)) {
        m <<= 1;
        ++sh;
      }
      m &= 0x3FFu;
      bits = sign | ((uint32_t)(113 - sh) << 23) | (m << 13);
    }
  } else if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112u) << 23) | (m << 13);
  }
  return __builtin_bit_cast(float, bits);
}

// Nearest binary16 to a finite, non-negative binary32 no larger than 65504,
// ties to even.
__host__ __device__ inline uint32_t f32_to_f16_bits_rne(float f) {
  uint32_t x = __builtin_bit_cast(uint32_t, f) & 0x7FFFFFFFu;
  int e = (int)(x >> 23) - 127;
  if (e < -25) return 0;  // below half of the smallest subnormal
  uint32_t mant = (x & 0x7FFFFFu) | 0x800000u;  // 24 significant bits
  if (e < -14) {  // subnormal result: quantum 2^-24
    int sh = -1 - e;  // value = mant * 2^(e-23); count of 2^-24 = mant >> (-e-1)
    uint32_t q = mant >> sh;
    uint32_t rem = mant & ((1u << sh) - 1);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    return q;  // may carry into 0x400 = smallest normal, still correct
  }
  uint32_t q = mant >> 13;  // 11 bits
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (q & 1))) ++q;
  uint32_t ex = (uint32_t)(e + 15);
  if (q == 0x800u) {
    q >>= 1;
    ++ex;
  }
  return (ex << 10) | (q & 0x3FFu);
}

// ---------------------------------------------------------------------------
// MFMA: v_mfma_f32_16x16x32_f16.  Lane l supplies row (l & 15) of A and
// column (l & 15) of B, each with the eight K-slots 8*(l>>4) .. +7, and
// receives D[rows 4*(l>>4) .. +3][column l & 15].
// ---------------------------------------------------------------------------
__device__ inline float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }
__device__ inline half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ inline uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// (1024 + q_a, 1024 + q_b) binary16 pairs of the 8 codes packed in v (code
// 2p at bits 4p, code 2p+1 at bits 16 + 4p): one shift and one three-input
// bit operation, (x & 0x00030003) | 0x64006400, per pair.
__device__ inline void q2k_pairs(uint32_t v, uint32_t (&pr)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) pr[p] = __builtin_amdgcn_bitop3_b32(v >> (4 * p), 0x00030003u, 0x64006400u, 0xEA);
}

// MXFP4 fragment: the 8 elements of one 32-bit code word (element 2i in the
// low nibble of byte i) as binary16 with the block scale folded in, by the
// FP4 conversion instruction; exact for scale codes 104..140 (every product
// then lies on the binary16 grid).
__device__ inline float e8m0_f32(uint32_t sc) {  // 2^(sc - 127); sc = 0 gives the subnormal 2^-127
  return sc ? __builtin_bit_cast(float, sc << 23) : __builtin_bit_cast(float, 0x00400000u);
}
__device__ inline half8_t mx4_frag(uint32_t w, float scale) {
  u32x4_t r;
  r.x = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
  r.y = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
  r.z = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
  r.w = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
  return as_half8(r);
}

// Q4K fragment: the 8 codes of one 32-bit word (element 2p at bits 4p,
// element 2p + 1 at bits 16 + 4p) as binary16 q * DS + NDM rounded once,
// with DS = binary16(d * s) and NDM = -binary16(dmin * m) in both halves:
// (x & 0x000F000F) | 0x64006400 reads 1024 + q in each half, exactly.
__device__ inline half8_t q4k_frag(uint32_t w, half2_t DS, half2_t NDM) {
  const half2_t k1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  u32x4_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t t = __builtin_amdgcn_bitop3_b32(w >> (4 * p), 0x000F000Fu, 0x64006400u, 0xEA);
    r[p] = as_u32(__builtin_elementwise_fma(as_half2(t) + k1024, DS, NDM));
  }
  return as_half8(r);
}
// DS and NDM of sub-block j of a Q4K super-block from its scale words
// (w0: s nibbles, w1: m nibbles, w2: high bits) and its (d, dmin) word.
__device__ inline void q4k_scales(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t sup, int j, half2_t& DS,
                                  half2_t& NDM) {
  const uint32_t s = ((w0 >> (4 * j)) & 15u) | (((w2 >> (2 * j)) & 3u) << 4);
  const uint32_t m = ((w1 >> (4 * j)) & 15u) | (((w2 >> (16 + 2 * j)) & 3u) << 4);
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(sup & 0xFFFFu));
  const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(sup >> 16));
  const _Float16 a = (_Float16)(d * (float)s), b = -(_Float16)(dmin * (float)m);
  DS = (half2_t){a, a};
  NDM = (half2_t){b, b};
}

__device__ inline half8_t zero_half8() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return as_half8(z);
}

// Keeps the scheduler from moving instructions across it: load phases are
// issued in program order, so a wait for an early phase never waits for the
// weight stream behind it (loads retire in issue order).
__device__ inline void pin() { __builtin_amdgcn_sched_barrier(0); }

// Load of a wave-uniform address through the scalar unit (constant address
// space): it is counted apart from vector loads, so waiting for it does not
// wait for the wave's vector loads or copies into LDS.  Only for data that no
// block of the running kernel writes.
// Coherent (device-scope) loads of data another block wrote in the same
// kernel, after observing its release.
__device__ inline int ld_acq_int(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ inline void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// Write-through (device-coherent) store for data handed to another block of
// the same kernel; a writer waits for its coherent stores to complete
// (wait_stores) before the counter that publishes them is incremented, so no
// L2 write-back is needed.
__device__ inline void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ inline int ld_uniform(const int32_t* p) { return *(const __attribute__((address_space(4))) int32_t*)p; }

// Raw buffer (stride 0) over n bytes at p, 32-bit data format.  The hardware
// range-checks each lane's offset: a load at an offset of n or more returns
// zeros and reads no memory, so a lane with nothing to load passes kOob and
// gets a zero operand without a branch or a register clear.  vo is the
// lane's byte offset, so a wave-uniform one (an SGPR) added to it; both stay
// below 2^31.
constexpr uint32_t kOob = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
constexpr int kBufNt = 2;  // cache policy: streamed once (non-temporal)
template <int AUX = 0>
__device__ inline u32x4_t buf_ld128(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, AUX));
}
__device__ inline u32x3_t buf_ld96(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, (int)vo, (int)so, 0));
}
__device__ inline u32x2_t buf_ld64(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)vo, (int)so, 0));
}
__device__ inline uint32_t buf_ld32(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, (int)so, 0));
}
__device__ inline uint32_t buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return (uint32_t)__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, (int)so, 0));
}

__device__ inline float silu(float g) { return g / (1.0f + __expf(-g)); }

// Work item of this block: blocks b < count are spread so that XCD x = b % 8
// (blocks are dealt to the 8 XCDs round-robin) runs the contiguous items
// [start_x, start_x + quota_x) in order, so neighbouring items share an L2;
// blocks >= count get none.
__device__ inline bool xcd_item(int count, int& item) {
  const int b = blockIdx.x;
  if (b >= count) return false;
  const int x = b & 7, i = b >> 3;
  const int base = count >> 3, rem = count & 7;
  item = x * base + min(x, rem) + i;
  return true;
}

}  // namespace ds4
