// Prefill (any T): grouped expert products over the work list of (expert,
// run of up to 128 of its slots) tiles built by the grouping kernels, plus
// the dense shared expert.
//
//   k_shared_gateup_prefill   hs16[t]  = silu(Wsg x_t) * (Wsu x_t)        (binary16)
//   k_pf_gateup               hw16[p]  = w_s * silu(G_e x_t) * (U_e x_t)  (binary16)
//   k_pf_down                 yp[s]    = D_e hw16[p]                       (fp32)
//   k_shared_down_prefill     y[t]     = Wsd hs16[t]                       (fp32)
//   k_combine                 y[t]    += sum_j yp[t*k + j], j ascending
// Slots s = t*k + j sit at position p of the expert-sorted list (perm[p] = s).
// The combine order is fixed, so results are deterministic.
//
// Routed products (grouped GEMM).  A block takes one work tile and a slice
// of output rows.  Each of its four waves owns four 16-row weight fragments
// and all of the tile's slots (up to eight 16-slot fragments), so a weight is
// decoded once per tile and a staged activation fragment feeds four MFMAs
// (v_mfma_f32_16x16x32_f16 with the slots as A rows and the weights as B
// columns: lane (c, q) holds slots 4q..4q+3 of weight row c).  Activation
// chunks of 128 inputs are copied straight into LDS (global_load_lds), double
// buffered, in a layout whose 16-byte pieces are XOR-swizzled by row so that
// the fragment reads of 16 rows hit distinct banks.  Inside a chunk the
// K-steps are permuted so that a lane's weight codes for the whole chunk are
// one 8-byte piece of its row (CB2: one sub-block; Q2K: two sub-blocks): at
// step j lane group q covers inputs 32q + 8j .. +7 of the chunk, and the
// activation fragments are read at the same offsets.  Weights are decoded to
// binary16 with the block scales folded in (one rounding of d*(2s+1) and one
// of the product, CB2; d*s*q - dmin*m rounded once, Q2K); the fp32 MFMA
// accumulates.  Work items are laid out so that each XCD takes a contiguous
// range (blocks are dealt to the 8 XCDs round-robin): the row slices of one
// tile and the tiles of one expert share that XCD's L2.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "trace.h"
#include "tiles.h"

namespace ds4 {

__constant__ GridTables c_pre_tables = make_grid_tables();

constexpr int kPW = 4;  // waves per block, splitting K

template <bool LO>
__global__ __launch_bounds__(kPW * 64) void k_shared_gateup_prefill(ds4moe_layer L, int64_t T,
                                                                    const _Float16* __restrict__ xh,
                                                                    const _Float16* __restrict__ xl,
                                                                    _Float16* __restrict__ hs16) {
  __shared__ float s_red[kPW * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, fs = L.d_ff_shared;
  const int row0 = blockIdx.x * 16;
  const int64_t t = (int64_t)blockIdx.y * 16 + c;
  const _Float16* bh = t < T ? xh + t * d : nullptr;
  const _Float16* bl = (LO && t < T) ? xl + t * d : nullptr;
  int ks0, ks1;
  split_range(d / 32, kPW, wave, ks0, ks1);
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  const int64_t ar = (int64_t)(row0 + c) * d;
  f16_tile<true, LO>(L.sh_gate + ar, L.sh_up + ar, bh, bl, ks0, ks1, lane, ag, au);
  ag = block_reduce_waves<kPW>(ag, s_red, wave, lane);
  au = block_reduce_waves<kPW>(au, s_red, wave, lane);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) hs16[t * fs + row0 + 4 * q + r] = (_Float16)(silu(ag[r]) * au[r]);
  }
}

constexpr int kTT = kPrefillTile;  // slots per work tile (128)
constexpr int kKC = 128;           // inputs per staged activation chunk
constexpr int kGW = 4;             // waves per block
constexpr int kChunk = kTT * kKC;  // halves per staged chunk (32 KB)

// Work item of this block: blocks b < count are spread so that XCD x = b % 8
// runs items [start_x, start_x + quota_x) in order; blocks >= count exit.
__device__ inline bool xcd_item(int count, int& item) {
  const int b = blockIdx.x;
  if (b >= count) return false;
  const int x = b & 7, i = b >> 3;
  const int base = count >> 3, rem = count & 7;
  item = x * base + min(x, rem) + i;
  return true;
}

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 128-input chunk of the tile's 128 activation rows into a swizzled LDS
// buffer: wave instruction m moves rows 4g .. 4g+3 (g = wave + 4m), lane l
// writing physical piece l & 15 of row 4g + l/16, which holds logical piece
// (l & 15) ^ (row & 15).  row_of(r): element offset of tile row r from src
// (src is the same for the whole block, offsets fit 32 bits).
template <bool LO, typename RowOf>
__device__ inline void stage_rows(const _Float16* __restrict__ src, const _Float16* __restrict__ src_lo, RowOf row_of,
                                  int ch, _Float16* dh, _Float16* dl, int wave, int lane) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int g = wave + kGW * m;
    const int r = 4 * g + (lane >> 4);
    const int u = (lane & 15) ^ (r & 15);
    const uint32_t off = 2u * ((uint32_t)row_of(r) + (uint32_t)(ch * kKC + 8 * u));
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)src + off),
                                     (__attribute__((address_space(3))) void*)(dh + g * 4 * kKC), 16, 0, 0);
    if (LO)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)src_lo + off),
                                       (__attribute__((address_space(3))) void*)(dl + g * 4 * kKC), 16, 0, 0);
  }
}

template <typename T>
__device__ inline T ld_at(const void* base, uint32_t byte_off) {
  return *(const T*)((const char*)base + byte_off);
}

// A fragment of slot fragment i at step j: row 16i + c, inputs 32q + 8j .. +7.
__device__ inline half8_t slot_frag(const _Float16* buf, int i, int c, int q, int j) {
  return *(const half8_t*)(buf + (16 * i + c) * kKC + 8 * ((4 * q + j) ^ c));
}

// CB2 group j of a sub-block (index word idxw, aux word aux) as binary16
// sign * m * D, with D = binary16(d * (2s+1)) in both halves of D2.
__device__ inline half8_t cb2_frag_scaled(uint32_t idxw, uint32_t aux, int j, const uint32_t* mag,
                                          const uint32_t* sgn, half2_t D2) {
  const uint32_t idx = (idxw >> (8 * j)) & 0xFFu;
  const uint32_t code = (aux >> (7 * j)) & 0x7Fu;
  const u32x4_t m = *(const u32x4_t*)(mag + 4 * idx);
  const u32x4_t s = *(const u32x4_t*)(sgn + 4 * code);
  u32x4_t r;
  r.x = as_u32(as_half2(m.x ^ s.x) * D2);
  r.y = as_u32(as_half2(m.y ^ s.y) * D2);
  r.z = as_u32(as_half2(m.z ^ s.z) * D2);
  r.w = as_u32(as_half2(m.w ^ s.w) * D2);
  return as_half8(r);
}

__device__ inline float f16f(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }
__device__ inline half2_t h2splat(float v) {
  const _Float16 h = (_Float16)v;
  return (half2_t){h, h};
}

template <bool LO>
struct GuLds {
  _Float16 xh[2][kChunk];
  _Float16 xl[LO ? 2 : 1][LO ? kChunk : 8];
  uint32_t mag[256 * 4];
  uint32_t sgn[128 * 4];
  int tok[kTT];
  float w[kTT];
};

// Gate/up of one work tile for a 128-row slice of h, NF slot fragments.
template <bool LO, int NF>
__device__ __attribute__((always_inline)) inline void gateup_tile(const ds4moe_layer& L, GuLds<LO>& s,
                                                                  const _Float16* __restrict__ xh,
                                                                  const _Float16* __restrict__ xl, int e, int rt,
                                                                  int pos0, int n, _Float16* __restrict__ hw16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, q = lane >> 4;
  const int d = L.d_model, fd = L.d_ff, nb = d / QK, nch = d / kKC;
  const size_t mb = (size_t)fd * nb;
  const uint8_t* gb = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* ub = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const int hr0 = rt * 128 + 32 * wave;
  // fragment f: rows hr0 + 16 (f & 1) + c of gate (f < 2) or up (f >= 2)
  const uint8_t* gd = gb + mb * 64;
  const uint8_t* ud = ub + mb * 64;
  uint32_t rowblk[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) rowblk[h] = (uint32_t)((hr0 + 16 * h + c) * nb);
  auto load_w = [&](int ch, u32x2_t (&cw)[4], uint32_t (&dv)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t blk = rowblk[f & 1] + (uint32_t)(ch >> 1);
      cw[f] = ld_at<u32x2_t>(f < 2 ? gb : ub, blk * 64u + (uint32_t)(32 * (ch & 1) + 8 * q));
      dv[f] = ld_at<uint16_t>(f < 2 ? gd : ud, blk * 2u);
    }
  };
  auto rows = [&](int r) { return s.tok[r] * d; };
  float4_t acc[4][NF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};

  constexpr int kBatch = 8 * (LO ? 2 : 1) + 8;  // vector-memory instructions per chunk and lane
  u32x2_t cw[4], cwn[4];
  uint32_t dv[4], dvn[4];
  stage_rows<LO>(xh, xl, rows, 0, s.xh[0], s.xl[0], wave, lane);
  load_w(0, cw, dv);
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nch) {
      pin();
      stage_rows<LO>(xh, xl, rows, ch + 1, s.xh[buf ^ 1], s.xl[LO ? buf ^ 1 : 0], wave, lane);
      load_w(ch + 1, cwn, dvn);
      pin();
      vm_wait<kBatch>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    half2_t D2[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) D2[f] = h2splat(f16f(dv[f]) * (float)(2 * (cw[f].y >> 28) + 1));
    const _Float16* bh = s.xh[buf];
    const _Float16* bl = s.xl[LO ? buf : 0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t wf[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) wf[f] = cb2_frag_scaled(cw[f].x, cw[f].y, j, s.mag, s.sgn, D2[f]);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const half8_t a = slot_frag(bh, i, c, q, j);
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(a, wf[f], acc[f][i]);
        if (LO) {
          const half8_t al = slot_frag(bl, i, c, q, j);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(al, wf[f], acc[f][i]);
        }
      }
    }
    __syncthreads();
    if (ch + 1 < nch) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        cw[f] = cwn[f];
        dv[f] = dvn[f];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NF; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * i + 4 * q + r;
      if (t < n) {
        const float wt = s.w[t];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          hw16[(int64_t)(pos0 + t) * fd + hr0 + 16 * h + c] =
              (_Float16)(wt * (silu(acc[h][i][r]) * acc[h + 2][i][r]));
      }
    }
  }
}

template <bool LO>
__global__ __launch_bounds__(kGW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_gateup(
    ds4moe_layer L, const _Float16* __restrict__ xh, const _Float16* __restrict__ xl,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, const float* __restrict__ topk_w,
    _Float16* __restrict__ hw16) {
  __shared__ GuLds<LO> s;
  const int rowtiles = L.d_ff / 128;
  int item;
  if (!xcd_item(*ntiles * rowtiles, item)) return;
  const int tile = item / rowtiles, rt = item - tile * rowtiles;
  const int e = tiles[2 * tile], g = tiles[2 * tile + 1];
  const int pos0 = offsets[e] + kTT * g;
  const int n = min(kTT, counts[e] - kTT * g);
  stage_grid_tables(s.mag, s.sgn, c_pre_tables);
  if ((int)threadIdx.x < kTT) {
    const int slot = perm[pos0 + min((int)threadIdx.x, n - 1)];
    s.tok[threadIdx.x] = slot / L.top_k;
    s.w[threadIdx.x] = topk_w[slot];
  }
  __syncthreads();
  switch ((n + 15) >> 4) {
    case 1: gateup_tile<LO, 1>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 2: gateup_tile<LO, 2>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 3: gateup_tile<LO, 3>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 4: gateup_tile<LO, 4>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 5: gateup_tile<LO, 5>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 6: gateup_tile<LO, 6>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    case 7: gateup_tile<LO, 7>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
    default: gateup_tile<LO, 8>(L, s, xh, xl, e, rt, pos0, n, hw16); break;
  }
}

struct DnLds {
  _Float16 xh[2][kChunk];
  int slot[kTT];
};

// Down product of one work tile for a 256-row slice of the output.
template <int NF>
__device__ __attribute__((always_inline)) inline void down_tile(const ds4moe_layer& L, DnLds& s,
                                                                const _Float16* __restrict__ hw16, int e, int rt,
                                                                int pos0, int n, float* __restrict__ yp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, q = lane >> 4;
  const int d = L.d_model, fd = L.d_ff, nb = fd / QK, nch = fd / kKC;
  const size_t mb = (size_t)d * nb;
  const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mb * 84;
  const uint8_t* sub = base + mb * 64;
  const uint8_t* sup = base + mb * 80;
  const int r0 = rt * 256 + 64 * wave;
  const uint32_t blk0 = (uint32_t)((r0 + c) * nb);  // fragment f: + 16 f nb
  auto load_w = [&](int ch, u32x2_t (&cw)[4], uint32_t (&sc)[4], uint32_t (&dd)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t blk = blk0 + (uint32_t)(16 * f * nb + (ch >> 1));
      cw[f] = ld_at<u32x2_t>(base, blk * 64u + (uint32_t)(32 * (ch & 1) + 8 * q));
      sc[f] = ld_at<uint16_t>(sub, blk * 16u + (uint32_t)(8 * (ch & 1) + 2 * q));
      dd[f] = ld_at<uint32_t>(sup, blk * 4u);
    }
  };
  const _Float16* hbase = hw16 + (int64_t)pos0 * fd;
  auto rows = [&](int r) { return min(r, n - 1) * fd; };
  float4_t acc[4][NF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};

  constexpr int kBatch = 8 + 12;
  u32x2_t cw[4], cwn[4];
  uint32_t sc[4], scn[4], dd[4], ddn[4];
  stage_rows<false>(hbase, nullptr, rows, 0, s.xh[0], nullptr, wave, lane);
  load_w(0, cw, sc, dd);
  const half2_t k1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nch) {
      pin();
      stage_rows<false>(hbase, nullptr, rows, ch + 1, s.xh[buf ^ 1], nullptr, wave, lane);
      load_w(ch + 1, cwn, scn, ddn);
      pin();
      vm_wait<kBatch>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    const _Float16* bh = s.xh[buf];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // sub-block 2q + h of the chunk: steps 2h, 2h+1
      half2_t A2[4], nB2[4];  // binary16 d * s and -(dmin * m) of the sub-block
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t sm = (sc[f] >> (8 * h)) & 0xFFu;
        A2[f] = h2splat(f16f(dd[f]) * (float)(sm & 15u));
        nB2[f] = h2splat(-f16f(dd[f] >> 16) * (float)(sm >> 4));
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {  // codes 8jj .. 8jj+7 of the sub-block
        const int j = 2 * h + jj;
        half8_t wf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint32_t fld = (cw[f][h] >> (16 * jj)) & 0xFFFFu;
          uint32_t pr[4];
          q2k_pairs(fld | (fld << 14), pr);
          u32x4_t a;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            a[p] = as_u32(__builtin_elementwise_fma(as_half2(pr[p]) + k1024, A2[f], nB2[f]));
          wf[f] = as_half8(a);
        }
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          const half8_t a = slot_frag(bh, i, c, q, j);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(a, wf[f], acc[f][i]);
        }
      }
    }
    __syncthreads();
    if (ch + 1 < nch) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        cw[f] = cwn[f];
        sc[f] = scn[f];
        dd[f] = ddn[f];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NF; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * i + 4 * q + r;
      if (t < n) {
        const int64_t row = (int64_t)s.slot[t] * d;
#pragma unroll
        for (int f = 0; f < 4; ++f) yp[row + r0 + 16 * f + c] = acc[f][i][r];
      }
    }
  }
}

__global__ __launch_bounds__(kGW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_down(
    ds4moe_layer L, const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const _Float16* __restrict__ hw16, float* __restrict__ yp) {
  __shared__ DnLds s;
  const int rowtiles = L.d_model / 256;
  int item;
  if (!xcd_item(*ntiles * rowtiles, item)) return;
  const int tile = item / rowtiles, rt = item - tile * rowtiles;
  const int e = tiles[2 * tile], g = tiles[2 * tile + 1];
  const int pos0 = offsets[e] + kTT * g;
  const int n = min(kTT, counts[e] - kTT * g);
  if ((int)threadIdx.x < kTT) s.slot[threadIdx.x] = perm[pos0 + min((int)threadIdx.x, n - 1)];
  __syncthreads();
  switch ((n + 15) >> 4) {
    case 1: down_tile<1>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 2: down_tile<2>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 3: down_tile<3>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 4: down_tile<4>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 5: down_tile<5>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 6: down_tile<6>(L, s, hw16, e, rt, pos0, n, yp); break;
    case 7: down_tile<7>(L, s, hw16, e, rt, pos0, n, yp); break;
    default: down_tile<8>(L, s, hw16, e, rt, pos0, n, yp); break;
  }
}

__global__ __launch_bounds__(kPW * 64) void k_shared_down_prefill(ds4moe_layer L, int64_t T,
                                                                  const _Float16* __restrict__ hs16,
                                                                  float* __restrict__ y) {
  __shared__ float s_red[kPW * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, fs = L.d_ff_shared;
  const int row0 = blockIdx.x * 16;
  const int64_t t = (int64_t)blockIdx.y * 16 + c;
  const _Float16* bcol = t < T ? hs16 + t * fs : nullptr;
  int ks0, ks1;
  split_range(fs / 32, kPW, wave, ks0, ks1);
  float4_t acc = {0.f, 0.f, 0.f, 0.f}, unused = acc;
  f16_tile<false, false>(L.sh_down + (int64_t)(row0 + c) * fs, nullptr, bcol, nullptr, ks0, ks1, lane, acc, unused);
  acc = block_reduce_waves<kPW>(acc, s_red, wave, lane);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[t * d + row0 + 4 * q + r] = acc[r];
  }
}

// y[t][i] += sum_j yp[t*k + j][i], four columns per lane.
__global__ __launch_bounds__(256) void k_combine(int64_t T, int d, int k, const float* __restrict__ yp,
                                                 float* __restrict__ y) {
  const int64_t n4 = T * d / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = (i * 4) / d;
    const int64_t col = (i * 4) % d;
    float4 a = ((float4*)y)[i];
    for (int j = 0; j < k; ++j) {
      const float4 b = *(const float4*)(yp + (t * k + j) * d + col);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    ((float4*)y)[i] = a;
  }
}

hipError_t launch_prefill_experts(const Fwd& f) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int64_t T = f.T;
  const int d = L.d_model, E = L.n_experts, k = L.top_k;
  const int64_t S = T * k;
  const int64_t maxtiles = (S + kTT - 1) / kTT + E;  // >= sum_e ceil(n_e / kTT)
  auto xh = (const _Float16*)(ws + y.x_hi);
  auto xl = f.lo ? (const _Float16*)(ws + y.x_lo) : nullptr;
  auto tiles = (const int32_t*)(ws + y.tiles);
  auto ntiles = (const int32_t*)(ws + y.ntiles);
  auto counts = (const int32_t*)(ws + y.counts);
  auto offsets = (const int32_t*)(ws + y.offsets);
  auto perm = (const int32_t*)(ws + y.perm);
  auto w = (const float*)(ws + y.topk_w);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto yp = (float*)(ws + y.yp);
  const unsigned tg = (unsigned)((T + 15) / 16);
  const dim3 blk(kPW * 64), gblk(kGW * 64);
  const dim3 ggu((unsigned)(maxtiles * (L.d_ff / 128))), gdn((unsigned)(maxtiles * (d / 256)));
  if (f.lo) {
    DS4_LAUNCH(k_shared_gateup_prefill<true>, dim3(L.d_ff_shared / 16, tg), blk, 0, f.st, L, T, xh, xl, hs16);
    DS4_LAUNCH(k_pf_gateup<true>, ggu, gblk, 0, f.st, L, xh, xl, tiles, ntiles, counts, offsets, perm, w, hw16);
  } else {
    DS4_LAUNCH(k_shared_gateup_prefill<false>, dim3(L.d_ff_shared / 16, tg), blk, 0, f.st, L, T, xh, xl, hs16);
    DS4_LAUNCH(k_pf_gateup<false>, ggu, gblk, 0, f.st, L, xh, xl, tiles, ntiles, counts, offsets, perm, w, hw16);
  }
  DS4_LAUNCH(k_pf_down, gdn, gblk, 0, f.st, L, tiles, ntiles, counts, offsets, perm, hw16, yp);
  DS4_LAUNCH(k_shared_down_prefill, dim3(d / 16, tg), blk, 0, f.st, L, T, hs16, f.y);
  const int64_t n4 = T * d / 4;
  const int cb = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  DS4_LAUNCH(k_combine, dim3(cb), dim3(256), 0, f.st, T, d, k, yp, f.y);
  return hipGetLastError();
}

}  // namespace ds4
