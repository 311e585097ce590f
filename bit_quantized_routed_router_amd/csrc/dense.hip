// Dense fp16 GEMMs of prefill and routing: the shared expert (F16, always
// on) and the F16 router (DS4 (DwarfStar 4) wiki note, "Key Techniques"):
//   k_pf_shared_gateup   hs16[t][r] = silu(Wsg[r] . x[t]) * (Wsu[r] . x[t])   (binary16)
//   k_pf_shared_down     y[t][o]    = Wsd[o] . hs16[t]                          (fp32)
//   k_router_gemm        logits[t][e] = Wr[e] . x[t] + bias[e]                 (fp32)
//                        (K split into parts when few tiles would fill the
//                        chip: fp32 partials, then k_router_reduce adds them
//                        in a fixed order)
// C[t][n] = sum_k A[t][k] B[n][k] with A the token rows (binary16; an fp32
// input as a hi + lo pair, both contracted) and B the weight rows.
//
// Block tile: 128 tokens x 256 weight rows (gate/up: 128 gate rows and the
// same 128 up rows), 8 waves of 64 x 64 (two along tokens, four along
// rows), K in chunks of 64 copied straight into LDS (global_load_lds)
// through a ring of chunks with one barrier per chunk (ring.h).  In LDS a
// row is 64 halves = 8 pieces of 16 bytes, piece p stored at p ^ (row & 7),
// so the 16 rows of an MFMA fragment read (v_mfma_f32_16x16x32_f16: lane
// (c, q) reads row c, K-slots 8q..8q+7) hit distinct banks in each group of
// 8 lanes.  Blocks take (row tile, token tile) items, row tile major, dealt
// so that each XCD runs a contiguous range: the blocks that share a weight
// tile share an L2.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "ring.h"
#include "trace.h"

namespace ds4 {

namespace dense {

constexpr int kBM = 128;  // tokens per block tile
constexpr int kBN = 256;  // weight rows per block tile
constexpr int kBK = 64;   // inputs per chunk (= halves per LDS row)
constexpr int kW = 8;     // waves per block

// A chunk in LDS: A rows (kBM), the lo rows of an fp32 input (kBM, LO
// only), then B rows (kBN), 64 halves each.
template <bool LO>
constexpr int slot_halves() { return ((LO ? 2 : 1) * kBM + kBN) * kBK; }
// Ring depth: three chunks (144 KB), two with the lo rows (128 KB).
template <bool LO>
constexpr int ring() { return LO ? 2 : 3; }
// Copies per wave and chunk: 8-row groups over the 8 waves.
template <bool LO>
constexpr int dma_per_wave() { return ((LO ? 2 : 1) * kBM + kBN) / 8 / kW; }

// MFMA operand fragment: rows row0 .. row0+15 of a region, K-step s (0, 1).
__device__ inline half8_t frag(const _Float16* region, int row0, int s, int c, int q) {
  const int r = row0 + c;
  return *(const half8_t*)(region + r * kBK + 8 * ((4 * s + q) ^ (r & 7)));
}

// The block's GEMM over K = nk inputs into acc[4 token fragments][4 row
// fragments] of wave (wm, wn).  arow(r) / brow(r): pointer to A row r
// (0..127, clamped into the input) / B row r (0..255).  bfrag_row(j): the
// B-tile row of the wave's row fragment j.
template <bool LO, typename ARow, typename BRow, typename BFragRow>
__device__ __attribute__((always_inline)) inline void gemm(int nk, const _Float16* __restrict__ a_hi,
                                                           const _Float16* __restrict__ a_lo, ARow arow, BRow brow,
                                                           BFragRow bfrag_row, _Float16* lds, float4_t (&acc)[4][4],
                                                           int wave, int lane) {
  constexpr int R = ring<LO>();
  constexpr int B = dma_per_wave<LO>();
  constexpr int kSlot = slot_halves<LO>();
  constexpr int kGA = kBM / 8, kGL = LO ? kBM / 8 : 0;
  const int c = lane & 15, q = lane >> 4, wm = wave >> 2;
  const int rr = lane >> 3, lp = (lane & 7) ^ rr;  // row in its group of 8, logical piece of the lane's copy
  // wave w copies 8-row groups w, w + 8, ...: A (kGA), A lo (kGL), then B
  auto issue = [&](int ch, int u) {
    _Float16* slot = lds + u * kSlot;
    const int k0 = ch * kBK + 8 * lp;
#pragma unroll
    for (int m = 0; m < B; ++m) {
      const int g = wave + kW * m;  // wave-uniform
      const _Float16* src;
      if (g < kGA) {
        src = a_hi + arow(8 * g + rr);
      } else if (LO && g < kGA + kGL) {
        src = a_lo + arow(8 * (g - kGA) + rr);
      } else {
        src = brow(8 * (g - kGA - kGL) + rr);
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + k0),
                                       (__attribute__((address_space(3))) void*)(slot + g * 8 * kBK), 16, 0, 0);
    }
  };
  auto compute = [&](int u) {
    const _Float16* sa = lds + u * kSlot;
    const _Float16* sl = sa + kBM * kBK;
    const _Float16* sb = sa + (LO ? 2 : 1) * kBM * kBK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8_t a[4], al[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = frag(sb, bfrag_row(j), s, c, q);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = frag(sa, 64 * wm + 16 * i, s, c, q);
        if (LO) al[i] = frag(sl, 64 * wm + 16 * i, s, c, q);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
          if (LO) acc[i][j] = mfma16x16x32(al[i], b[j], acc[i][j]);
        }
    }
  };
  ring_loop<R, B>(nk / kBK, issue, compute);
}

// Block -> (row tile, token tile); false for blocks without work.
__device__ inline bool item_of(int ntn, int ntt, int& nt, int& tt) {
  int item;
  if (!xcd_item(ntn * ntt, item)) return false;
  nt = item / ntt;
  tt = item - nt * ntt;
  return true;
}

}  // namespace dense

// K parts of the router GEMM: enough for about 256 blocks, each part a whole
// number of 64-input chunks.
int router_splits(int64_t T, int E, int d) {
  // (callers may size a workspace before rejecting T or E: at least one tile)
  const int64_t tiles =
      std::max<int64_t>(1, ((T + dense::kBM - 1) / dense::kBM) * ((E + dense::kBN - 1) / dense::kBN));
  int s = (int)std::max<int64_t>(1, std::min<int64_t>(256 / tiles, d / dense::kBK));
  while (s > 1 && (d / dense::kBK) % s) --s;
  return s;
}

// Shared gate/up: row tile nt = h-rows nt*128 .. +127 (B rows 0..127 its
// gate rows, 128..255 its up rows); wave wn owns h-rows 32 wn .. +31 (row
// fragments: gate 0/1, up 0/1).
template <bool LO>
__global__ __launch_bounds__(dense::kW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_shared_gateup(
    const _Float16* __restrict__ xh, const _Float16* __restrict__ xl, int64_t T, int d, int fs,
    const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu, int ntt, _Float16* __restrict__ hs16) {
  using namespace dense;
  __shared__ __align__(16) _Float16 s_ring[ring<LO>() * slot_halves<LO>()];
  int nt, tt;
  if (!item_of(fs / 128, ntt, nt, tt)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
  const int c = lane & 15, q = lane >> 4;
  const int64_t t0 = (int64_t)tt * kBM;
  const int r0 = nt * 128;
  auto arow = [&](int r) { return (int64_t)min(t0 + r, T - 1) * d; };
  auto brow = [&](int r) {
    return (const _Float16*)(r < 128 ? wg : wu) + (int64_t)(r0 + (r & 127)) * d;
  };
  auto bfrag = [&](int j) { return (j >> 1) * 128 + 32 * wn + 16 * (j & 1); };
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  gemm<LO>(d, xh, xl, arow, brow, bfrag, s_ring, acc, wave, lane);
  // lane (c, q): tokens 16 i + 4 q + r of the wave's 64, h-row 32 wn + 16 h + c
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 64 * wm + 16 * i + 4 * q + r;
      if (t < T) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          hs16[t * fs + r0 + 32 * wn + 16 * h + c] = (_Float16)(silu(acc[i][h][r]) * acc[i][h + 2][r]);
      }
    }
}

// Shared down: row tile nt = output rows nt*256 .. +255; wave wn owns rows
// 64 wn .. +63.
__global__ __launch_bounds__(dense::kW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_shared_down(
    const _Float16* __restrict__ hs16, int64_t T, int fs, int d, const uint16_t* __restrict__ wd, int ntt,
    float* __restrict__ y) {
  using namespace dense;
  __shared__ __align__(16) _Float16 s_ring[ring<false>() * slot_halves<false>()];
  int nt, tt;
  if (!item_of(d / kBN, ntt, nt, tt)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
  const int c = lane & 15, q = lane >> 4;
  const int64_t t0 = (int64_t)tt * kBM;
  const int o0 = nt * kBN;
  auto arow = [&](int r) { return (int64_t)min(t0 + r, T - 1) * fs; };
  auto brow = [&](int r) { return (const _Float16*)wd + (int64_t)(o0 + r) * fs; };
  auto bfrag = [&](int j) { return 64 * wn + 16 * j; };
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  gemm<false>(fs, hs16, nullptr, arow, brow, bfrag, s_ring, acc, wave, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 64 * wm + 16 * i + 4 * q + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y[t * d + o0 + 64 * wn + 16 * j + c] = acc[i][j][r];
      }
    }
}

// Router: block (part p, expert tile nt, token tile tt) over inputs
// [p d/P, (p+1) d/P); expert rows past E repeat the last one and are not
// stored.  One part: logits + bias directly; more: partials part[p][t][e].
template <bool LO>
__global__ __launch_bounds__(dense::kW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_router_gemm(
    const _Float16* __restrict__ xh, const _Float16* __restrict__ xl, int64_t T, int d, int E,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int ntt, int parts, float* __restrict__ part,
    float* __restrict__ logits) {
  using namespace dense;
  __shared__ __align__(16) _Float16 s_ring[ring<LO>() * slot_halves<LO>()];
  const int ntn = (E + kBN - 1) / kBN;
  int item;
  if (!xcd_item(parts * ntn * ntt, item)) return;
  const int p = item / (ntn * ntt), nt = (item / ntt) % ntn, tt = item % ntt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
  const int c = lane & 15, q = lane >> 4;
  const int kc = d / parts, kb = p * kc;
  const int64_t t0 = (int64_t)tt * kBM;
  const int e0 = nt * kBN;
  auto arow = [&](int r) { return (int64_t)min(t0 + r, T - 1) * d; };
  auto brow = [&](int r) { return (const _Float16*)wr + (int64_t)min(e0 + r, E - 1) * d + kb; };
  auto bfrag = [&](int j) { return 64 * wn + 16 * j; };
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  gemm<LO>(kc, xh + kb, LO ? xl + kb : nullptr, arow, brow, bfrag, s_ring, acc, wave, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 64 * wm + 16 * i + 4 * q + r;
      if (t >= T) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 64 * wn + 16 * j + c;
        if (e >= E) continue;
        if (parts == 1) logits[t * E + e] = acc[i][j][r] + (bias ? bias[e] : 0.0f);
        else part[((int64_t)p * T + t) * E + e] = acc[i][j][r];
      }
    }
}

// logits[t][e] = sum_p part[p][t][e] (p ascending) + bias[e]
__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ part, int parts, int64_t T, int E,
                                                       const float* __restrict__ bias, float* __restrict__ logits) {
  const int64_t n = T * E;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float v = part[i];
    for (int p = 1; p < parts; ++p) v += part[(int64_t)p * n + i];
    logits[i] = v + (bias ? bias[i % E] : 0.0f);
  }
}

hipError_t launch_router_logits(const ds4moe_layer& L, int64_t T, bool lo, const _Float16* xh, const _Float16* xl,
                                float* part, float* logits, hipStream_t st) {
  using namespace dense;
  const int d = L.d_model, E = L.n_experts;
  const int ntt = (int)((T + kBM - 1) / kBM), ntn = (E + kBN - 1) / kBN;
  const int parts = router_splits(T, E, d);
  const dim3 grid((unsigned)(parts * ntn * ntt)), blk(kW * 64);
  if (lo)
    DS4_LAUNCH((k_router_gemm<true>), grid, blk, 0, st, xh, xl, T, d, E, (const uint16_t*)L.router_w, L.router_bias,
               ntt, parts, part, logits);
  else
    DS4_LAUNCH((k_router_gemm<false>), grid, blk, 0, st, xh, xl, T, d, E, (const uint16_t*)L.router_w,
               L.router_bias, ntt, parts, part, logits);
  if (parts > 1) {
    const int64_t n = T * E;
    const int nb = (int)std::min<int64_t>((n + 255) / 256, 4096);
    DS4_LAUNCH(k_router_reduce, dim3(nb), dim3(256), 0, st, part, parts, T, E, L.router_bias, logits);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_shared(const ds4moe_layer& L, int64_t T, bool lo, const _Float16* xh, const _Float16* xl,
                                 _Float16* hs16, float* y, hipStream_t st) {
  using namespace dense;
  const int d = L.d_model, fs = L.d_ff_shared;
  const int ntt = (int)((T + kBM - 1) / kBM);
  const dim3 blk(kW * 64), ggu((unsigned)((fs / 128) * ntt)), gdn((unsigned)((d / kBN) * ntt));
  if (lo)
    DS4_LAUNCH((k_pf_shared_gateup<true>), ggu, blk, 0, st, xh, xl, T, d, fs, (const uint16_t*)L.sh_gate,
               (const uint16_t*)L.sh_up, ntt, hs16);
  else
    DS4_LAUNCH((k_pf_shared_gateup<false>), ggu, blk, 0, st, xh, xl, T, d, fs, (const uint16_t*)L.sh_gate,
               (const uint16_t*)L.sh_up, ntt, hs16);
  DS4_LAUNCH(k_pf_shared_down, gdn, blk, 0, st, hs16, T, fs, d, (const uint16_t*)L.sh_down, ntt, y);
  return hipGetLastError();
}

}  // namespace ds4
