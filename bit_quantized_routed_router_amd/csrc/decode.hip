// Batched decode (T <= 16 tokens per group): the whole layer in three
// streaming kernels whose 16 MFMA columns are the group's tokens.
//
//   k_dec_stage1  router partial logits per input chunk, and the shared
//                 expert's gate and up products as half-K partial tiles;
//                 neither depends on routing.  The last router block to
//                 arrive finishes routing (sum of partials, top-k, gate
//                 weights, grouping); the last of the four blocks of a shared
//                 tile forms h = silu(g) * u.  x is read in its input type and
//                 converted in registers (the chunk owners of expert tile 0
//                 keep the binary16 copy for stage 2).
//   k_dec_stage2  the shared expert's down product, and for every distinct
//                 selected expert its gate/up tiles: w * silu(G x) * (U x) as
//                 binary16 plus fp32 sums over each 16 rows (one Q2K
//                 sub-block of the down input).
//   k_dec_stage3  one block per 16 output rows runs every distinct expert's
//                 down product for those rows, adds the shared expert's
//                 output, and writes y; waves take (expert, super-block)
//                 units round-robin and their partials are added in a fixed
//                 order.  It also clears stage 1's arrival counters.
// Each distinct expert is read once per call however many tokens chose it,
// and results do not depend on block scheduling.  Inside stage 1, blocks hand
// partials to the last arriver with device-coherent (sc1) stores and loads
// around an atomic counter, which needs no L2 write-back.
//
// Operands.  Packed weights: every lane owns a contiguous 16-byte piece of
// its row's super-block and feeds those weights to consecutive MFMA steps
// (CB2: lane group q holds sub-blocks 2q, 2q+1; Q2K: sub-blocks 4q..4q+3);
// the activation column is read at the matching K offsets.  F16 weights:
// K-step ks, lane group q -> K = 32 ks + 8 q.  Activation (B) columns at or
// beyond the group's T repeat its last token and their outputs are dropped,
// so no load is predicated.  When a block's activations are small (BL) they
// are staged once in LDS as binary16; otherwise each wave reads them from
// global memory.  Every wave issues the weight loads of its share before its
// first MFMA.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "routefin.h"
#include "tiles.h"
#include "trace.h"

namespace ds4 {

__constant__ GridTables c_dec_tables = make_grid_tables();

constexpr int kW = 4;           // waves per block, stages 1 and 2
constexpr int kW3 = 8;          // waves per block, stage 3
constexpr int kStageHalves = 4096;        // binary16 activations a stage-1/2 block may stage (per hi/lo part)
constexpr size_t kStage3Bytes = 36 * 1024;  // stage 3 LDS for staged activations
constexpr int kUnitsAhead = 8;  // stage 3 units whose weight loads a wave keeps in flight

// inputs per router partial: 512, or 256 when d is an odd multiple of 256
__host__ __device__ inline int router_chunk(int d) { return d % 512 == 0 ? 512 : 256; }

__device__ inline int cb2_boff(int q, int s) { return 32 * (2 * q + (s >> 2)) + 8 * (s & 3); }
__device__ inline int q2k_boff(int q, int s) { return 16 * (4 * q + (s >> 1)) + 8 * (s & 1); }
__device__ inline int clamp_index(int v, int n) { return (unsigned)v < (unsigned)n ? v : 0; }

// 8 activations x[t][k0 .. k0+7] (bf16 bits or fp32) as binary16 hi and lo parts.
template <bool LO>
__device__ inline void load_x8(const void* x, int d, int t, int k0, half8_t& h, half8_t& l) {
  float v[8];
  if (!LO) {
    const u32x4_t u = *(const u32x4_t*)((const uint16_t*)x + (int64_t)t * d + k0);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      v[2 * p] = __builtin_bit_cast(float, u[p] << 16);
      v[2 * p + 1] = __builtin_bit_cast(float, u[p] & 0xFFFF0000u);
    }
  } else {
    const float4* src = (const float4*)((const float*)x + (int64_t)t * d + k0);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (_Float16)v[e];
    l[e] = LO ? (_Float16)(v[e] - (float)h[e]) : (_Float16)0.0f;
  }
}

template <int NW>
__device__ inline float4_t reduce_waves(float4_t v, float4_t (*red)[64], int wave, int lane) {
  red[wave][lane] = v;
  __syncthreads();
  float4_t s = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][lane];
  return s;  // the same in every wave; callers use wave 0
}

// Row stride (halves) of staged activations: 8 extra halves shift the rows
// of consecutive tokens across LDS banks.
__host__ __device__ inline int stage_stride(int K) { return K + 8; }

// Keeps the scheduler from moving instructions across it: the load phases
// below are issued in program order, so a wait for an early phase never
// waits for the weight stream behind it (loads retire in issue order).
__device__ inline void pin() { __builtin_amdgcn_sched_barrier(0); }

// LDS staging of a small row set in two steps: load() issues up to M
// 16-byte pieces per thread into registers, store() writes them to LDS
// later.  The callers' launch conditions keep the row set within M pieces
// per thread.
template <int M>
struct F16Stage {  // binary16 rows [R][K] of a matrix with row stride ld -> LDS rows of stage_stride(K)
  u32x4_t r[M];
  __device__ inline void load(const _Float16* src, int ld, int R, int K) {
    const int n8 = K / 8, n = R * n8;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const int i = min((int)threadIdx.x + j * (int)blockDim.x, n - 1);
      r[j] = *(const u32x4_t*)(src + (int64_t)(i / n8) * ld + 8 * (i % n8));
    }
  }
  __device__ inline void store(_Float16* dst, int R, int K) const {
    const int n8 = K / 8, n = R * n8, st = stage_stride(K);
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const int i = (int)threadIdx.x + j * (int)blockDim.x;
      if (i < n) *(u32x4_t*)(dst + (i / n8) * st + 8 * (i % n8)) = r[j];
    }
  }
};

// Copy of rows [0, R) x [0, K) halves of a binary16 matrix (row stride ld)
// into LDS rows of stride st, straight from memory into LDS (no registers):
// one 1 KB chunk per wave instruction, chunks dealt round-robin to the
// block's waves.  The data is in LDS once the issuing wave has waited for
// its loads (wait_all) and the block has met a barrier.
__device__ inline void dma_rows(const _Float16* src, int ld, int R, int K, _Float16* dst, int st, int wave, int nw,
                                int lane) {
  const int per_row = (K + 511) / 512;
  for (int ch = wave; ch < R * per_row; ch += nw) {
    const int r = ch / per_row, j = ch % per_row;
    if (j * 512 + lane * 8 < K)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + (int64_t)r * ld + j * 512 + lane * 8),
          (__attribute__((address_space(3))) void*)(dst + r * st + j * 512), 16, 0, 0);
  }
}

// Same for a contiguous run of n 16-byte pieces.
__device__ inline void dma_pieces(const void* src, int n, void* dst, int wave, int nw, int lane) {
  for (int ch = wave; ch * 64 < n; ch += nw) {
    if (ch * 64 + lane < n)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)((const u32x4_t*)src + ch * 64 + lane),
          (__attribute__((address_space(3))) void*)((u32x4_t*)dst + ch * 64), 16, 0, 0);
  }
}

__device__ inline void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

template <bool LO>
struct XStage {  // activations x[T][k0 .. k0+K) in the input type -> binary16 hi/lo LDS rows, one piece per thread
  u32x4_t u;
  float4 a, b;
  __device__ inline void load(const void* x, int d, int T, int k0, int K) {
    const int n8 = K / 8;
    const int i = min((int)threadIdx.x, T * n8 - 1);
    const int64_t off = (int64_t)(i / n8) * d + k0 + 8 * (i % n8);
    if (!LO) {
      u = *(const u32x4_t*)((const uint16_t*)x + off);
    } else {
      const float4* src = (const float4*)((const float*)x + off);
      a = src[0];
      b = src[1];
    }
  }
  __device__ inline void store(_Float16* sh, _Float16* sl, int T, int K) const {
    const int n8 = K / 8, st = stage_stride(K);
    const int i = threadIdx.x;
    if (i >= T * n8) return;
    float v[8];
    if (!LO) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[2 * p] = __builtin_bit_cast(float, u[p] << 16);
        v[2 * p + 1] = __builtin_bit_cast(float, u[p] & 0xFFFF0000u);
      }
    } else {
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    half8_t h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (_Float16)v[e];
      l[e] = (_Float16)(v[e] - (float)h[e]);
    }
    *(half8_t*)(sh + (i / n8) * st + 8 * (i % n8)) = h;
    if (LO) *(half8_t*)(sl + (i / n8) * st + 8 * (i % n8)) = l;
  }
};

// ============================================================== stage 1
struct Stage1Lds {
  union {
    RouteLds route;
    struct {
      _Float16 bh[kStageHalves + 16 * 8];
      _Float16 bl[kStageHalves + 16 * 8];
      float4_t red[kW][64];
    } sh;
  };
  int last;
};

// blocks [0, rblocks): router (expert tile, input chunk), chunk-major;
// then 4 blocks per shared 16-row tile: (gate|up) x (K half).
template <bool LO, bool BL>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_stage1(ds4moe_layer L, int T, const void* __restrict__ x,
                                                        int rblocks, float* __restrict__ plog, RouteOut ro,
                                                        _Float16* __restrict__ xh, _Float16* __restrict__ xl,
                                                        float* __restrict__ gu_part, _Float16* __restrict__ hs16,
                                                        int32_t* __restrict__ ctrl) {
  __shared__ Stage1Lds lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);  // token feeding MFMA column c
  const int d = L.d_model, E = L.n_experts, fs = L.d_ff_shared;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  if ((int)blockIdx.x < rblocks) {  // ---------------- router partial logits
    const int ntile = (E + 15) / 16;
    const int et = blockIdx.x % ntile, kc = blockIdx.x / ntile;
    const int e0 = et * 16;
    const uint16_t* rp = L.router_w + (int64_t)min(e0 + c, E - 1) * d;
    const int ck = router_chunk(d), spw = ck / (32 * kW);  // K-steps per wave (4 or 2)
    half8_t a[4], bh[4], bl[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h < spw) {
        const int k0 = (kc * (ck / 32) + wave * spw + h) * 32 + 8 * q;
        a[h] = *(const half8_t*)(rp + k0);
        load_x8<LO>(x, d, tc, k0, bh[h], bl[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h < spw) {
        if (et == 0 && c < T) {
          const int k0 = (kc * (ck / 32) + wave * spw + h) * 32 + 8 * q;
          *(half8_t*)(xh + (int64_t)c * d + k0) = bh[h];
          if (LO) *(half8_t*)(xl + (int64_t)c * d + k0) = bl[h];
        }
        acc = mfma16x16x32(a[h], bh[h], acc);
        if (LO) acc = mfma16x16x32(a[h], bl[h], acc);
      }
    }
    acc = reduce_waves<kW>(acc, lds.sh.red, wave, lane);
    if (wave == 0) {
      if (c < T) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = e0 + 4 * q + r;
          if (e < E) st_coh(&plog[((int64_t)kc * T + c) * E + e], acc[r]);
        }
      }
      wait_stores();
    }
    __syncthreads();
    if (threadIdx.x == 0) lds.last = atomicAdd(&ctrl[0], 1) == rblocks - 1;
    __syncthreads();
    if (!lds.last) return;
    route_finish_block<true>(lds.route, plog, d / ck, L.router_bias, E, L.top_k, T, ro);
    if (threadIdx.x == 0) ctrl[0] = 0;
    return;
  }
  // ---------------- shared expert: (tile, gate|up, K half)
  const int sb = blockIdx.x - rblocks;
  const int tile = sb >> 2, part = sb & 3, mat = part >> 1, half = part & 1;
  const uint16_t* rp = (mat ? L.sh_up : L.sh_gate) + (int64_t)(tile * 16 + c) * d;
  const int nkh = d / 64;  // K-steps per half
  int ks0, ks1;
  split_range(nkh, kW, wave, ks0, ks1);
  const int kb = half * (d / 2);  // first input of this half
  const int st = stage_stride(d / 2);
  constexpr int kBatch = 16;
  XStage<LO> xs;
  if (BL) xs.load(x, d, T, kb, d / 2);  // one piece per thread: T * d / 2 <= 8 * blockDim
  pin();
  for (int ks = ks0; ks < ks1 || ks == ks0; ks += kBatch) {  // every wave runs the first batch (staging barrier)
    half8_t a[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) a[j] = *(const half8_t*)(rp + kb + max(min(ks + j, ks1 - 1), 0) * 32 + 8 * q);
    pin();
    if (BL && ks == ks0) {
      xs.store(lds.sh.bh, lds.sh.bl, T, d / 2);
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // steps past the range multiply a zero A fragment
      const int ksj = max(min(ks + j, ks1 - 1), 0);
      const half8_t aj = ks + j < ks1 ? a[j] : zero_half8();
      const int kk = ksj * 32 + 8 * q;  // within the half
      half8_t bh, bl;
      if (BL) {
        bh = *(const half8_t*)(lds.sh.bh + tc * st + kk);
        if (LO) bl = *(const half8_t*)(lds.sh.bl + tc * st + kk);
      } else {
        load_x8<LO>(x, d, tc, kb + kk, bh, bl);
      }
      acc = mfma16x16x32(aj, bh, acc);
      if (LO) acc = mfma16x16x32(aj, bl, acc);
    }
  }
  acc = reduce_waves<kW>(acc, lds.sh.red, wave, lane);
  float* tp = gu_part + (size_t)tile * 4 * 16 * T;  // [part][row][t]
  if (wave == 0) {
    if (c < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st_coh(&tp[((size_t)part * 16 + 4 * q + r) * T + c], acc[r]);
    }
    wait_stores();
  }
  __syncthreads();
  if (threadIdx.x == 0) lds.last = atomicAdd(&ctrl[1 + tile], 1) == 3;
  __syncthreads();
  if (!lds.last || wave != 0) return;
  if (c < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      const float g = ld_coh(&tp[((size_t)0 * 16 + row) * T + c]) + ld_coh(&tp[((size_t)1 * 16 + row) * T + c]);
      const float u = ld_coh(&tp[((size_t)2 * 16 + row) * T + c]) + ld_coh(&tp[((size_t)3 * 16 + row) * T + c]);
      hs16[(int64_t)c * fs + tile * 16 + row] = (_Float16)(silu(g) * u);
    }
  }
  if (lane == 0) ctrl[1 + tile] = 0;
}

// ============================================================== stage 2
struct Stage2Lds {
  uint32_t mag[256 * 4];
  uint32_t sgn[128 * 4];
  _Float16 bh[kStageHalves + 16 * 8];
  _Float16 bl[kStageHalves + 16 * 8];
  float4_t red[kW][64];
  float4_t red2[kW][64];
};

constexpr int kSb2 = 4;  // CB2 super-blocks a wave loads at once

template <bool LO, bool BL>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_stage2(ds4moe_layer L, int T, RouteOut ro,
                                                        const _Float16* __restrict__ xh,
                                                        const _Float16* __restrict__ xl,
                                                        const _Float16* __restrict__ hs16, float* __restrict__ ys,
                                                        _Float16* __restrict__ hw16, float* __restrict__ hsum) {
  __shared__ Stage2Lds lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);
  const int d = L.d_model, f = L.d_ff, fs = L.d_ff_shared, k = L.top_k;
  const int nr = f / 16, nb = d / QK, ndt = d / 16;
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  if ((int)blockIdx.x < ndt) {  // ---------------- shared expert down, 16 output rows
    const int row0 = blockIdx.x * 16;
    int ks0, ks1;
    split_range(fs / 32, kW, wave, ks0, ks1);
    const uint16_t* rp = L.sh_down + (int64_t)(row0 + c) * fs;
    const int st = stage_stride(fs);
    F16Stage<2> hs;  // T * fs <= 4096 halves: 512 pieces over 256 threads
    if (BL) hs.load(hs16, fs, T, fs);
    pin();
    constexpr int kBatch = 16;
    for (int ks = ks0; ks < ks1 || ks == ks0; ks += kBatch) {
      half8_t a[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) a[j] = *(const half8_t*)(rp + max(min(ks + j, ks1 - 1), 0) * 32 + 8 * q);
      pin();
      if (BL && ks == ks0) {
        hs.store(lds.bh, T, fs);
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // steps past the range multiply a zero A fragment
        const int ksj = max(min(ks + j, ks1 - 1), 0);
        const half8_t aj = ks + j < ks1 ? a[j] : zero_half8();
        const int kk = ksj * 32 + 8 * q;
        const half8_t b = BL ? *(const half8_t*)(lds.bh + tc * st + kk)
                             : *(const half8_t*)(hs16 + (int64_t)tc * fs + kk);
        ag = mfma16x16x32(aj, b, ag);
      }
    }
    ag = reduce_waves<kW>(ag, lds.red, wave, lane);
    if (wave == 0 && c < T) *(float4_t*)(ys + (int64_t)c * d + row0 + 4 * q) = ag;
    return;
  }
  // ---------------- routed gate/up: distinct expert i, 16-row tile
  const int rel = blockIdx.x - ndt;
  const int i = rel / nr, tile = rel % nr;
  const int row0 = tile * 16;
  // phase 1: copies into LDS (activations, grid tables), independent of routing
  const int st = stage_stride(d);
  if (BL) dma_rows(xh, d, T, d, lds.bh, st, wave, kW, lane);
  if (BL && LO) dma_rows(xl, d, T, d, lds.bl, st, wave, kW, lane);
  dma_pieces(&c_dec_tables.mag[0][0], 384, lds.mag, wave, kW, lane);  // mag (256 pieces), then sgn
  // phase 2: routing tables; waiting for them also completes the copies
  const int nd = *ro.ndist;
  const int e = clamp_index(ro.distinct[i], L.n_experts);
  int slot = ro.tok_slot[i * kDecodeGroup + c];
  wait_all();
  if (i >= nd) return;  // whole block; no copy is in flight
  __syncthreads();
  if (slot >= T * k) slot = -1;
  const int tb = slot >= 0 ? slot / k : 0;  // token feeding column c (any token when c has none)
  const size_t mb = (size_t)f * nb;  // blocks per matrix
  const uint8_t* gc = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* uc = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const uint16_t* gd = (const uint16_t*)(gc + mb * 64) + (size_t)(row0 + c) * nb;
  const uint16_t* ud = (const uint16_t*)(uc + mb * 64) + (size_t)(row0 + c) * nb;
  const uint8_t* grow = gc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  const uint8_t* urow = uc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  int sb0, sb1;
  split_range(nb, kW, wave, sb0, sb1);
  for (int b0 = sb0; b0 < sb1; b0 += kSb2) {
    // phase 3: weight loads, consumed as they arrive
    u32x4_t cg[kSb2], cu[kSb2];
    float dg[kSb2], du[kSb2];
#pragma unroll
    for (int j = 0; j < kSb2; ++j) {
      const int b = min(b0 + j, sb1 - 1);
      cg[j] = __builtin_nontemporal_load((const u32x4_t*)(grow + b * 64));
      cu[j] = __builtin_nontemporal_load((const u32x4_t*)(urow + b * 64));
      dg[j] = h2f(gd[b]);
      du[j] = h2f(ud[b]);
    }
#pragma unroll
    for (int j = 0; j < kSb2; ++j) {  // super-blocks past the range get a zero scale
      {
        const int kb = min(b0 + j, sb1 - 1) * QK;
        if (b0 + j >= sb1) {
          dg[j] = 0.0f;
          du[j] = 0.0f;
        }
        float4_t pg = {0.f, 0.f, 0.f, 0.f}, pu = pg;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int kk = kb + cb2_boff(q, s);
          half8_t bh, bl;
          if (BL) {
            bh = *(const half8_t*)(lds.bh + tb * st + kk);
            if (LO) bl = *(const half8_t*)(lds.bl + tb * st + kk);
          } else {
            bh = *(const half8_t*)(xh + (int64_t)tb * d + kk);
            if (LO) bl = *(const half8_t*)(xl + (int64_t)tb * d + kk);
          }
          const half8_t a0 = cb2_frag((s & 4) ? cg[j].z : cg[j].x, (s & 4) ? cg[j].w : cg[j].y, s & 3, lds.mag, lds.sgn);
          const half8_t a1 = cb2_frag((s & 4) ? cu[j].z : cu[j].x, (s & 4) ? cu[j].w : cu[j].y, s & 3, lds.mag, lds.sgn);
          pg = mfma16x16x32(a0, bh, pg);
          pu = mfma16x16x32(a1, bh, pu);
          if (LO) {
            pg = mfma16x16x32(a0, bl, pg);
            pu = mfma16x16x32(a1, bl, pu);
          }
        }
        // d of output row 4q + r is the A-row value of lane 4q + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ag[r] += __shfl(dg[j], 4 * q + r) * pg[r];
          au[r] += __shfl(du[j], 4 * q + r) * pu[r];
        }
      }
    }
  }
  lds.red[wave][lane] = ag;
  lds.red2[wave][lane] = au;
  __syncthreads();
  if (wave != 0) return;
  ag = lds.red[0][lane];
  au = lds.red2[0][lane];
#pragma unroll
  for (int w = 1; w < kW; ++w) {
    ag += lds.red[w][lane];
    au += lds.red2[w][lane];
  }
  float psum = 0.0f;
  if (slot >= 0) {
    const float wt = ro.w[slot];
    _Float16 hv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv[r] = (_Float16)(wt * (silu(ag[r]) * au[r]));
      psum += (float)hv[r];
    }
    u32x2_t pk;
    pk.x = (uint32_t)__builtin_bit_cast(uint16_t, hv[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, hv[1]) << 16);
    pk.y = (uint32_t)__builtin_bit_cast(uint16_t, hv[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, hv[3]) << 16);
    *(u32x2_t*)(hw16 + (int64_t)slot * f + row0 + 4 * q) = pk;
  }
  psum += __shfl_xor(psum, 16);
  psum += __shfl_xor(psum, 32);
  if (slot >= 0 && q == 0) hsum[(int64_t)slot * (f / 16) + tile] = psum;
}

// ============================================================== stage 3
// Weight operands of one (expert, super-block) Q2K unit for lane (c, q).
struct Q2kW {
  u32x4_t codes;    // sub-blocks 4q..4q+3 of the lane's row
  uint32_t sc4;     // their scale/min bytes
  u32x2_t mins;     // scale/min bytes 8(q&1)..+7 (min MFMA operand; used by lanes q < 2)
  uint32_t sup[4];  // (d, dmin) of the lane's four output rows
};

__device__ inline void q2k_wload(Q2kW& U, const uint8_t* base, size_t mb, int nb, int row0, int b, int c, int q) {
  const uint8_t* rc = base + (size_t)(row0 + c) * nb * 64 + b * 64;
  const uint8_t* rs = base + mb * 64 + (size_t)(row0 + c) * nb * 16 + b * 16;
  const uint16_t* sup = (const uint16_t*)(base + mb * 80);
  U.codes = __builtin_nontemporal_load((const u32x4_t*)(rc + 16 * q));
  U.sc4 = *(const uint32_t*)(rs + 4 * q);
  U.mins = *(const u32x2_t*)(rs + 8 * (q & 1));
#pragma unroll
  for (int r = 0; r < 4; ++r) U.sup[r] = *(const uint32_t*)(sup + ((size_t)(row0 + 4 * q + r) * nb + b) * 2);
}

// bcol: activation column of the unit's super-block (LDS or global);
// cs: its 16 sub-block sums.  valid: the column has a slot for this expert.
__device__ inline void q2k_unit(const Q2kW& U, const _Float16* bcol, const float* cs, bool valid, int q,
                                float4_t& acc) {
  half8_t b[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) b[s] = *(const half8_t*)(bcol + q2k_boff(q, s));
  half8_t bh, bl;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = cs[8 * (q & 1) + e];
    bh[e] = (_Float16)v;
    bl[e] = (_Float16)(v - (float)bh[e]);
  }
  float4_t p = {0.f, 0.f, 0.f, 0.f}, pm = p;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const half8_t a = q2k_frag(U.codes[s >> 1], s & 1, (U.sc4 >> (8 * (s >> 1))) & 15u);
    p = mfma16x16x32(a, b[s], p);
  }
  // min term: K-slots 0..15 are the 16 sub-blocks (lane groups q >= 2 add zeros)
  u32x4_t t;
  t.x = nib_hi_pair_f16(U.mins.x, 0);
  t.y = nib_hi_pair_f16(U.mins.x, 2);
  t.z = nib_hi_pair_f16(U.mins.y, 0);
  t.w = nib_hi_pair_f16(U.mins.y, 2);
  const half8_t am = q < 2 ? as_half8(t) : zero_half8();
  pm = mfma16x16x32(am, bh, pm);
  pm = mfma16x16x32(am, bl, pm);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float v = h2f((uint16_t)(U.sup[r] & 0xFFFFu)) * p[r] - h2f((uint16_t)(U.sup[r] >> 16)) * pm[r];
    acc[r] += valid ? v : 0.0f;
  }
}

template <bool BL>
__global__ __launch_bounds__(kW3 * 64) void k_dec_stage3(ds4moe_layer L, int T, const int32_t* __restrict__ ndist,
                                                         const int32_t* __restrict__ distinct,
                                                         const int32_t* __restrict__ tok_slot,
                                                         const _Float16* __restrict__ hw16,
                                                         const float* __restrict__ hsum,
                                                         const float* __restrict__ ys, int32_t* __restrict__ ctrl,
                                                         int nctrl, int maxd, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char s_dyn[];  // staged activations when BL
  __shared__ float4_t s_red[kW3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, k = L.top_k;
  const int row0 = blockIdx.x * 16;
  const int nb = f / QK;
  const size_t mb = (size_t)d * nb;
  const int S = T * k;
  const uint8_t* down = (const uint8_t*)L.down;
  _Float16* s_h = (_Float16*)s_dyn;                   // [S][f]
  float* s_cs = (float*)(s_dyn + (size_t)S * f * 2);  // [S][f/16]
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int maxunits = maxd * nb;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctrl; i += blockDim.x) ctrl[i] = 0;
  // copies of the activations into LDS, then the routing tables; waiting for
  // the tables also completes the copies, and one barrier publishes them
  if (BL) {
    dma_pieces(hw16, S * f / 8, s_h, wave, kW3, lane);
    dma_pieces(hsum, S * (f / 16) / 4, s_cs, wave, kW3, lane);
  }
  const int nunits = min(*ndist, maxd) * nb;
  // Units: u = (expert slot u / nb, super-block u % nb); wave w takes
  // u = w, w + kW3, ... in batches of kUnitsAhead whose weight loads are all
  // issued before the batch's first MFMA.
  int ej[kUnitsAhead], sj[kUnitsAhead];
#pragma unroll
  for (int j = 0; j < kUnitsAhead; ++j) {
    const int i = min((wave + j * kW3) / nb, maxd - 1);
    ej[j] = distinct[i];
    sj[j] = tok_slot[i * kDecodeGroup + c];
  }
  wait_all();
  __syncthreads();
  for (int u0 = wave; u0 < maxunits; u0 += kW3 * kUnitsAhead) {
    if (u0 != wave) {  // routing tables of later batches
#pragma unroll
      for (int j = 0; j < kUnitsAhead; ++j) {
        const int i = min((u0 + j * kW3) / nb, maxd - 1);
        ej[j] = distinct[i];
        sj[j] = tok_slot[i * kDecodeGroup + c];
      }
    }
    Q2kW W[kUnitsAhead];
#pragma unroll
    for (int j = 0; j < kUnitsAhead; ++j) {
      const int u = min(u0 + j * kW3, maxunits - 1);
      q2k_wload(W[j], down + (size_t)clamp_index(ej[j], L.n_experts) * mb * 84, mb, nb, row0, u % nb, c, q);
    }
    // units past the end and columns without a slot add nothing
#pragma unroll
    for (int j = 0; j < kUnitsAhead; ++j) {
      const int u = u0 + j * kW3;
      const int slot = sj[j];
      const bool valid = u < nunits && slot >= 0 && slot < S;
      const int row = valid ? slot : 0;
      const int b = min(u, maxunits - 1) % nb;
      if (BL)
        q2k_unit(W[j], s_h + (size_t)row * f + b * QK, s_cs + (size_t)row * (f / 16) + b * 16, valid, q, acc);
      else
        q2k_unit(W[j], hw16 + (size_t)row * f + b * QK, hsum + (size_t)row * (f / 16) + b * 16, valid, q, acc);
    }
  }
  acc = reduce_waves<kW3>(acc, s_red, wave, lane);
  if (wave == 0 && c < T) {
    const float4_t s = *(const float4_t*)(ys + (int64_t)c * d + row0 + 4 * q);
    *(float4_t*)(y + (int64_t)c * d + row0 + 4 * q) = acc + s;
  }
}

// ============================================================== launcher
template <bool LO, bool BL>
static void launch_stages12(const Fwd& f, int rblocks, int nsh, int ndt, int maxd, int nr, const RouteOut& ro) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  auto xh = (_Float16*)(ws + y.x_hi);
  auto xl = LO ? (_Float16*)(ws + y.x_lo) : nullptr;
  auto plog = (float*)(ws + y.plog);
  auto ctrl = (int32_t*)(ws + y.ctrl);
  auto gu = (float*)(ws + y.gu_part);
  auto ys = (float*)(ws + y.ys);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (float*)(ws + y.hsum);
  const dim3 blk(kW * 64);
  DS4_LAUNCH((k_dec_stage1<LO, BL>), dim3(rblocks + 4 * nsh), blk, 0, f.st, L, T, f.x, rblocks, plog, ro, xh, xl, gu,
             hs16, ctrl);
  DS4_LAUNCH((k_dec_stage2<LO, BL>), dim3(ndt + maxd * nr), blk, 0, f.st, L, T, ro, xh, xl, hs16, ys, hw16, hsum);
}

hipError_t launch_decode(const Fwd& f) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  const int d = L.d_model, E = L.n_experts;
  const int kr = d / router_chunk(d);
  const int rblocks = ((E + 15) / 16) * kr;
  const int nsh = L.d_ff_shared / 16, nr = L.d_ff / 16, ndt = d / 16;
  const int maxd = std::min(E, T * L.top_k);
  const RouteOut ro = route_out(f);
  // stage the activations in LDS when every staged row set fits:
  // x halves (stage 1), hs16 and x (stage 2)
  const bool bl = (int64_t)T * std::max(d, L.d_ff_shared) <= kStageHalves;
  if (f.lo) {
    if (bl) launch_stages12<true, true>(f, rblocks, nsh, ndt, maxd, nr, ro);
    else launch_stages12<true, false>(f, rblocks, nsh, ndt, maxd, nr, ro);
  } else {
    if (bl) launch_stages12<false, true>(f, rblocks, nsh, ndt, maxd, nr, ro);
    else launch_stages12<false, false>(f, rblocks, nsh, ndt, maxd, nr, ro);
  }
  auto ctrl = (int32_t*)(ws + y.ctrl);
  auto ys = (float*)(ws + y.ys);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (float*)(ws + y.hsum);
  const int S = T * L.top_k;
  const size_t stage_bytes = (size_t)S * L.d_ff * 2 + (size_t)S * (L.d_ff / 16) * 4;
  const dim3 blk3(kW3 * 64);
  if (stage_bytes <= kStage3Bytes)
    DS4_LAUNCH(k_dec_stage3<true>, dim3(ndt), blk3, stage_bytes, f.st, L, T, ro.ndist, ro.distinct, ro.tok_slot,
               hw16, hsum, ys, ctrl, ctrl_ints(L), maxd, f.y);
  else
    DS4_LAUNCH(k_dec_stage3<false>, dim3(ndt), blk3, 0, f.st, L, T, ro.ndist, ro.distinct, ro.tok_slot, hw16,
               hsum, ys, ctrl, ctrl_ints(L), maxd, f.y);
  return hipGetLastError();
}

}  // namespace ds4
