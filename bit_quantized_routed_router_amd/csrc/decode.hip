// Batched decode (T <= 16 tokens per group): expert products as dequant-in-
// register MFMA tiles whose 16 columns are the group's tokens.
//
// Two kernels after routing:
//   k_gateup_decode  shared expert and every distinct selected expert:
//                    h = silu(G x) * (U x); routed h is stored pre-multiplied
//                    by the token's gate weight, as binary16, with fp32
//                    per-16-row sums for the Q2K min term of the down product.
//   k_down_decode    per 16 output rows: sum over distinct experts of
//                    D_e (w h) plus the shared expert's down, in a fixed order
//                    (ascending expert, then shared), written once as fp32.
// The routed experts' order and the combine are therefore deterministic.
// The shared expert's gate/up runs in the same grid as the routed experts'
// (it needs no routing), and each distinct expert is read once per call
// however many of the tokens chose it.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "trace.h"
#include "tiles.h"

namespace ds4 {

__constant__ GridTables c_dec_tables = make_grid_tables();

constexpr int kGuWaves = 4;
constexpr int kDnWaves = 4;

template <bool LO>
__global__ __launch_bounds__(kGuWaves * 64) void k_gateup_decode(
    ds4moe_layer L, int T, const _Float16* __restrict__ xh, const _Float16* __restrict__ xl,
    const int32_t* __restrict__ ndist, const int32_t* __restrict__ distinct, const int32_t* __restrict__ tok_slot,
    const float* __restrict__ topk_w, _Float16* __restrict__ hs16, _Float16* __restrict__ hw16,
    float* __restrict__ hsum) {
  __shared__ uint32_t s_mag[256 * 4];
  __shared__ uint32_t s_sgn[128 * 4];
  __shared__ float s_red[kGuWaves * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, fs = L.d_ff_shared, k = L.top_k;
  const int nsh = fs / 16, nr = f / 16;
  int ks0, ks1;
  split_range(d / 32, kGuWaves, wave, ks0, ks1);
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;

  if ((int)blockIdx.x < nsh) {  // ---------------- shared expert
    const int row0 = blockIdx.x * 16;
    const _Float16* bh = c < T ? xh + (int64_t)c * d : nullptr;
    const _Float16* bl = (LO && c < T) ? xl + (int64_t)c * d : nullptr;
    const int64_t ar = (int64_t)(row0 + c) * d;
    f16_tile<true, LO>(L.sh_gate + ar, L.sh_up + ar, bh, bl, ks0, ks1, lane, ag, au);
    ag = block_reduce_waves<kGuWaves>(ag, s_red, wave, lane);
    au = block_reduce_waves<kGuWaves>(au, s_red, wave, lane);
    if (wave == 0 && c < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) hs16[(int64_t)c * fs + row0 + 4 * q + r] = (_Float16)(silu(ag[r]) * au[r]);
    }
    return;
  }
  // ---------------- routed: distinct expert i, row tile
  const int rel = blockIdx.x - nsh;
  const int i = rel / nr, tile = rel % nr;
  if (i >= *ndist) return;
  stage_grid_tables(s_mag, s_sgn, c_dec_tables);
  __syncthreads();
  const int e = distinct[i];
  const int slot = tok_slot[i * kDecodeGroup + c];
  const _Float16* bh = slot >= 0 ? xh + (int64_t)(slot / k) * d : nullptr;
  const _Float16* bl = (LO && slot >= 0) ? xl + (int64_t)(slot / k) * d : nullptr;
  const int nb = d / QK;
  const size_t mb = (size_t)f * nb;  // blocks per expert matrix
  const uint8_t* gc = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* uc = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const int row0 = tile * 16;
  cb2_tile<true, LO>(gc, (const uint16_t*)(gc + mb * 64), uc, (const uint16_t*)(uc + mb * 64), nb, row0, bh, bl,
                     ks0, ks1, lane, s_mag, s_sgn, ag, au);
  ag = block_reduce_waves<kGuWaves>(ag, s_red, wave, lane);
  au = block_reduce_waves<kGuWaves>(au, s_red, wave, lane);
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
    if (slot >= 0 && q == 0) hsum[(int64_t)slot * (f / 16) + tile] = part;
  }
}

__global__ __launch_bounds__(kDnWaves * 64) void k_down_decode(
    ds4moe_layer L, int T, const int32_t* __restrict__ ndist, const int32_t* __restrict__ distinct,
    const int32_t* __restrict__ tok_slot, const _Float16* __restrict__ hs16, const _Float16* __restrict__ hw16,
    const float* __restrict__ hsum, float* __restrict__ y) {
  __shared__ float s_red[kDnWaves * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, fs = L.d_ff_shared;
  const int row0 = blockIdx.x * 16;
  const int nb = f / QK;
  const size_t mb = (size_t)d * nb;
  int ks0, ks1;
  split_range(f / 32, kDnWaves, wave, ks0, ks1);
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nd = *ndist;
  for (int i = 0; i < nd; ++i) {
    const int e = distinct[i];
    const int slot = tok_slot[i * kDecodeGroup + c];
    const _Float16* bcol = slot >= 0 ? hw16 + (int64_t)slot * f : nullptr;
    const float* cs = slot >= 0 ? hsum + (int64_t)slot * (f / 16) : nullptr;
    const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mb * 84;
    q2k_tile(base, base + mb * 64, (const uint16_t*)(base + mb * 80), nb, row0, bcol, cs, ks0, ks1, lane, acc);
  }
  {
    int s0, s1;
    split_range(fs / 32, kDnWaves, wave, s0, s1);
    const _Float16* bcol = c < T ? hs16 + (int64_t)c * fs : nullptr;
    float4_t unused = acc;
    f16_tile<false, false>(L.sh_down + (int64_t)(row0 + c) * fs, nullptr, bcol, nullptr, s0, s1, lane, acc, unused);
  }
  acc = block_reduce_waves<kDnWaves>(acc, s_red, wave, lane);
  if (wave == 0 && c < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[(int64_t)c * d + row0 + 4 * q + r] = acc[r];
  }
}

hipError_t launch_decode_experts(const Fwd& f) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  const int maxd = std::min(L.n_experts, T * L.top_k);
  const int nsh = L.d_ff_shared / 16, nr = L.d_ff / 16;
  const dim3 gu(nsh + maxd * nr);
  auto xh = (const _Float16*)(ws + y.x_hi);
  auto xl = f.lo ? (const _Float16*)(ws + y.x_lo) : nullptr;
  auto nd = (const int32_t*)(ws + y.ndist);
  auto dist = (const int32_t*)(ws + y.distinct);
  auto tslot = (const int32_t*)(ws + y.tok_slot);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (float*)(ws + y.hsum);
  if (f.lo)
    DS4_LAUNCH(k_gateup_decode<true>, gu, dim3(kGuWaves * 64), 0, f.st, L, T, xh, xl, nd, dist, tslot,
                       (const float*)(ws + y.topk_w), hs16, hw16, hsum);
  else
    DS4_LAUNCH(k_gateup_decode<false>, gu, dim3(kGuWaves * 64), 0, f.st, L, T, xh, xl, nd, dist, tslot,
                       (const float*)(ws + y.topk_w), hs16, hw16, hsum);
  DS4_LAUNCH(k_down_decode, dim3(L.d_model / 16), dim3(kDnWaves * 64), 0, f.st, L, T, nd, dist, tslot, hs16,
                     hw16, hsum, f.y);
  return hipGetLastError();
}

}  // namespace ds4
