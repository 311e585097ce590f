// Prefill (any T): grouped expert products over the (expert, 16-token group)
// work list built by the grouping kernels, plus the dense shared expert.
//
//   k_shared_gateup_prefill   hs16[t]  = silu(Wsg x_t) * (Wsu x_t)        (binary16)
//   k_gateup_prefill          hw16[s]  = w_s * silu(G_e x_t) * (U_e x_t)  (binary16)
//                             hsum[s]  = its per-16-row sums (Q2K min term)
//   k_down_prefill            yp[s]    = D_e hw16[s]                       (fp32)
//   k_shared_down_prefill     y[t]     = Wsd hs16[t]                       (fp32)
//   k_combine                 y[t]    += sum_j yp[t*k + j], j ascending
// Slots s = t*k + j; the combine order is fixed, so results are deterministic.
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

// Column c of work tile (e, g) is slot perm[offsets[e] + 16 g + c], if any.
__device__ inline int tile_slot(const int32_t* tiles, const int32_t* counts, const int32_t* offsets,
                                const int32_t* perm, int tile, int c, int* e_out) {
  const int e = tiles[2 * tile], g = tiles[2 * tile + 1];
  *e_out = e;
  const int r = 16 * g + c;
  return r < counts[e] ? perm[offsets[e] + r] : -1;
}

template <bool LO>
__global__ __launch_bounds__(kPW * 64) void k_gateup_prefill(ds4moe_layer L, const _Float16* __restrict__ xh,
                                                             const _Float16* __restrict__ xl,
                                                             const int32_t* __restrict__ tiles,
                                                             const int32_t* __restrict__ ntiles,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ perm,
                                                             const float* __restrict__ topk_w,
                                                             _Float16* __restrict__ hw16, float* __restrict__ hsum) {
  __shared__ uint32_t s_mag[256 * 4];
  __shared__ uint32_t s_sgn[128 * 4];
  __shared__ float s_red[kPW * 64 * 4];
  const int tile = blockIdx.y;
  if (tile >= *ntiles) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, k = L.top_k;
  stage_grid_tables(s_mag, s_sgn, c_pre_tables);
  __syncthreads();
  int e;
  const int slot = tile_slot(tiles, counts, offsets, perm, tile, c, &e);
  const _Float16* bh = slot >= 0 ? xh + (int64_t)(slot / k) * d : nullptr;
  const _Float16* bl = (LO && slot >= 0) ? xl + (int64_t)(slot / k) * d : nullptr;
  const int nb = d / QK;
  const size_t mb = (size_t)f * nb;
  const uint8_t* gc = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* uc = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const int row0 = blockIdx.x * 16;
  int ks0, ks1;
  split_range(d / 32, kPW, wave, ks0, ks1);
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  cb2_tile<true, LO>(gc, (const uint16_t*)(gc + mb * 64), uc, (const uint16_t*)(uc + mb * 64), nb, row0, bh, bl,
                     ks0, ks1, lane, s_mag, s_sgn, ag, au);
  ag = block_reduce_waves<kPW>(ag, s_red, wave, lane);
  au = block_reduce_waves<kPW>(au, s_red, wave, lane);
  if (wave == 0) {
    float part = 0.0f;
    if (slot >= 0) {
      const float wt = topk_w[slot];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16 hv = (_Float16)(wt * (silu(ag[r]) * au[r]));
        hw16[(int64_t)slot * f + row0 + 4 * q + r] = hv;
        part += (float)hv;
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (slot >= 0 && q == 0) hsum[(int64_t)slot * (f / 16) + blockIdx.x] = part;
  }
}

__global__ __launch_bounds__(kPW * 64) void k_down_prefill(ds4moe_layer L, const int32_t* __restrict__ tiles,
                                                           const int32_t* __restrict__ ntiles,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ perm,
                                                           const _Float16* __restrict__ hw16,
                                                           const float* __restrict__ hsum, float* __restrict__ yp) {
  __shared__ float s_red[kPW * 64 * 4];
  const int tile = blockIdx.y;
  if (tile >= *ntiles) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff;
  int e;
  const int slot = tile_slot(tiles, counts, offsets, perm, tile, c, &e);
  const _Float16* bcol = slot >= 0 ? hw16 + (int64_t)slot * f : nullptr;
  const float* cs = slot >= 0 ? hsum + (int64_t)slot * (f / 16) : nullptr;
  const int nb = f / QK;
  const size_t mb = (size_t)d * nb;
  const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mb * 84;
  const int row0 = blockIdx.x * 16;
  int ks0, ks1;
  split_range(f / 32, kPW, wave, ks0, ks1);
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  q2k_tile(base, base + mb * 64, (const uint16_t*)(base + mb * 80), nb, row0, bcol, cs, ks0, ks1, lane, acc);
  acc = block_reduce_waves<kPW>(acc, s_red, wave, lane);
  if (wave == 0 && slot >= 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) yp[(int64_t)slot * d + row0 + 4 * q + r] = acc[r];
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
  const int maxtiles = (int)((S + 15) / 16 + E);  // >= sum_e ceil(n_e / 16)
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
  auto hsum = (float*)(ws + y.hsum);
  auto yp = (float*)(ws + y.yp);
  const unsigned tg = (unsigned)((T + 15) / 16);
  const dim3 blk(kPW * 64);
  if (f.lo) {
    DS4_LAUNCH(k_shared_gateup_prefill<true>, dim3(L.d_ff_shared / 16, tg), blk, 0, f.st, L, T, xh, xl, hs16);
    DS4_LAUNCH(k_gateup_prefill<true>, dim3(L.d_ff / 16, maxtiles), blk, 0, f.st, L, xh, xl, tiles, ntiles,
                       counts, offsets, perm, w, hw16, hsum);
  } else {
    DS4_LAUNCH(k_shared_gateup_prefill<false>, dim3(L.d_ff_shared / 16, tg), blk, 0, f.st, L, T, xh, xl, hs16);
    DS4_LAUNCH(k_gateup_prefill<false>, dim3(L.d_ff / 16, maxtiles), blk, 0, f.st, L, xh, xl, tiles, ntiles,
                       counts, offsets, perm, w, hw16, hsum);
  }
  DS4_LAUNCH(k_down_prefill, dim3(d / 16, maxtiles), blk, 0, f.st, L, tiles, ntiles, counts, offsets, perm,
                     hw16, hsum, yp);
  DS4_LAUNCH(k_shared_down_prefill, dim3(d / 16, tg), blk, 0, f.st, L, T, hs16, f.y);
  const int64_t n4 = T * d / 4;
  const int cb = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  DS4_LAUNCH(k_combine, dim3(cb), dim3(256), 0, f.st, T, d, k, yp, f.y);
  return hipGetLastError();
}

}  // namespace ds4
