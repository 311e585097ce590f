// Router, top-k, gate weights and token -> expert grouping.
//
// The pages give only "an F16 router picks 6 of 256 experts" (DS4 (DwarfStar
// 4) wiki note, "Architecture" / "Key Techniques").  This library's reading:
// logits = x . Wr^T (+ bias), the k largest win with equal logits going to
// the lower index, a token's experts are listed in ascending index, and the
// gate weights are the softmax of the selected logits.  Grouping lists the
// slots s = t*k + j by (expert, token): counts, exclusive offsets, perm and
// its inverse.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "routefin.h"
#include "tiles.h"
#include "trace.h"

namespace ds4 {

// ---------------------------------------------------------------- activations
// x (fp32 or bf16) -> binary16 hi part, and for fp32 input the lo part
// fp16(x - hi), so that hi + lo carries ~22 bits.  8 elements per lane.
__global__ __launch_bounds__(256) void k_convert_x(const void* __restrict__ x, int dtype, int64_t n8,
                                                   _Float16* __restrict__ hi, _Float16* __restrict__ lo) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    if (dtype == DS4MOE_DT_BF16) {
      u32x4_t u = ((const u32x4_t*)x)[i];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[2 * p] = __builtin_bit_cast(float, u[p] << 16);
        v[2 * p + 1] = __builtin_bit_cast(float, u[p] & 0xFFFF0000u);
      }
    } else {
      const float4* src = (const float4*)x + 2 * i;
      float4 a = src[0], b = src[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    half8_t h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (_Float16)v[e];
      l[e] = (_Float16)(v[e] - (float)h[e]);
    }
    ((half8_t*)hi)[i] = h;
    if (lo) ((half8_t*)lo)[i] = l;
  }
}

// Decode router: block = 16 experts x one K chunk of CK = 256 inputs (4 waves,
// two K-steps each); writes partial logits plog[kc][t][e].  Activations are
// read in their input type and converted in registers; the blocks of expert
// tile 0 also store the binary16 copy (hi, and lo for fp32 input) that the
// expert kernels read.  Block (0, 0) clears the down kernel's tile counters.
template <bool LO>
__global__ __launch_bounds__(256) void k_router_partial(const uint16_t* __restrict__ wr, int E, int d,
                                                        const void* __restrict__ x, int T,
                                                        float* __restrict__ plog, _Float16* __restrict__ xh,
                                                        _Float16* __restrict__ xl, int32_t* __restrict__ zero_ctr,
                                                        int nzero) {
  __shared__ float red[4 * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int e0 = blockIdx.x * 16, kc = blockIdx.y;
  if (blockIdx.x == 0 && kc == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero_ctr[i] = 0;
  const int arow = min(e0 + c, E - 1);
  const uint16_t* rp = wr + (int64_t)arow * d;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ks = kc * 8 + wave * 2 + h;
    const int k0 = ks * 32 + 8 * q;
    half8_t a = *(const half8_t*)(rp + k0);
    half8_t bh = zero_half8(), bl = zero_half8();
    if (c < T) {
      float v[8];
      if (!LO) {
        u32x4_t u = *(const u32x4_t*)((const uint16_t*)x + (int64_t)c * d + k0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          v[2 * p] = __builtin_bit_cast(float, u[p] << 16);
          v[2 * p + 1] = __builtin_bit_cast(float, u[p] & 0xFFFF0000u);
        }
      } else {
        const float4* src = (const float4*)((const float*)x + (int64_t)c * d + k0);
        float4 a0 = src[0], a1 = src[1];
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bh[e] = (_Float16)v[e];
        bl[e] = (_Float16)(v[e] - (float)bh[e]);
      }
      if (blockIdx.x == 0) {
        *(half8_t*)(xh + (int64_t)c * d + k0) = bh;
        if (LO) *(half8_t*)(xl + (int64_t)c * d + k0) = bl;
      }
    }
    acc = mfma16x16x32(a, bh, acc);
    if (LO) acc = mfma16x16x32(a, bl, acc);
  }
  acc = block_reduce_waves<4>(acc, red, wave, lane);
  if (wave == 0 && c < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 4 * q + r;
      if (e < E) plog[((int64_t)kc * T + c) * E + e] = acc[r];
    }
  }
}

// ---------------------------------------------------------------- decode finish (routing only)
__global__ __launch_bounds__(256) void k_route_finish_decode(const float* __restrict__ plog, int nparts,
                                                             const float* __restrict__ bias, int E, int k, int T,
                                                             RouteOut o) {
  __shared__ RouteLdsGroup lds;
  route_finish_block(lds, plog, nparts, bias, E, k, T, o);
}

// ---------------------------------------------------------------- prefill: top-k per token
__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ logits, int E, int k, int64_t T,
                                                   int32_t* __restrict__ idx, float* __restrict__ w,
                                                   int32_t* idx_out, float* w_out) {
  __shared__ int s_sel_e[4][kMaxTopK];
  __shared__ float s_sel_v[4][kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 4;
  if (t0 + wave < T) wave_select(logits + (t0 + wave) * E, E, k, lane, s_sel_e[wave], s_sel_v[wave]);
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * k; i += blockDim.x) {
    const int tw = i / k, j = i % k;
    const int64_t t = t0 + tw;
    if (t < T) {
      const int e = s_sel_e[tw][j];
      const float wj = gate_weight(s_sel_v[tw], k, j);
      idx[t * k + j] = e;
      w[t * k + j] = wj;
      if (idx_out) idx_out[t * k + j] = e;
      if (w_out) w_out[t * k + j] = wj;
    }
  }
}

// prefill grouping, pass 1: counts[e] (one block per expert)
__global__ __launch_bounds__(256) void k_count_experts(const int32_t* __restrict__ idx, int64_t S,
                                                       int32_t* __restrict__ counts) {
  __shared__ int s_tmp[8];
  const int e = blockIdx.x;
  int c = 0;
  // 16-byte loads (idx sits in the 256-byte aligned workspace), four in
  // flight per thread, so the loop does not wait on each load in turn
  const int64_t S4 = S / 4;
  const int4* v = (const int4*)idx;
#pragma unroll 4
  for (int64_t i = threadIdx.x; i < S4; i += blockDim.x) {
    const int4 a = v[i];
    c += (a.x == e) + (a.y == e) + (a.z == e) + (a.w == e);
  }
  for (int64_t s = 4 * S4 + threadIdx.x; s < S; s += blockDim.x) c += idx[s] == e;
  int tot;
  block_excl_scan(c, s_tmp, &tot);
  if (threadIdx.x == 0) counts[e] = tot;
}

// prefill grouping, pass 2: offsets, perm, inv, and the GEMM work lists of
// (expert, run of its slots) tiles (one block per expert): runs of
// kPrefillTile slots go to `tiles`, an expert's remainder of at most
// kSmallTile slots to `stiles` (ntiles[0], ntiles[1]: their lengths).  A
// tile (e, g) covers positions offsets[e] + kPrefillTile g onward.
__global__ __launch_bounds__(256) void k_scatter_experts(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                         const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv, int32_t* counts_out,
                                                         int32_t* offsets_out, int32_t* perm_out,
                                                         int32_t* __restrict__ tiles, int32_t* __restrict__ stiles,
                                                         int32_t* __restrict__ ntiles) {
  __shared__ int s_tmp[8];
  const int e = blockIdx.x;
  int a = 0, b = 0, c = 0;
  for (int u = threadIdx.x; u < E; u += blockDim.x) {
    if (u < e) {
      a += counts[u];
      b += big_tiles(counts[u]);
      c += small_tiles(counts[u]);
    }
  }
  int off, tstart, sstart;
  block_excl_scan(a, s_tmp, &off);
  block_excl_scan(b, s_tmp, &tstart);
  block_excl_scan(c, s_tmp, &sstart);
  const int cnt = counts[e];
  if (threadIdx.x == 0) {
    offsets[e] = off;
    if (offsets_out) offsets_out[e] = off;
    if (counts_out) counts_out[e] = cnt;
    if (e == E - 1) {
      offsets[E] = off + cnt;
      if (offsets_out) offsets_out[E] = off + cnt;
      ntiles[0] = tstart + big_tiles(cnt);
      ntiles[1] = sstart + small_tiles(cnt);
    }
    if (small_tiles(cnt)) {
      stiles[2 * sstart] = e;
      stiles[2 * sstart + 1] = cnt / kPrefillTile;
    }
  }
  for (int g = threadIdx.x; g < big_tiles(cnt); g += blockDim.x) {
    tiles[2 * (tstart + g)] = e;
    tiles[2 * (tstart + g) + 1] = g;
  }
  int base = off;
  for (int64_t t0 = 0; t0 < T; t0 += blockDim.x) {
    const int64_t t = t0 + threadIdx.x;
    int jj = -1;
    if (t < T)
      for (int j = 0; j < k; ++j)
        if (idx[t * k + j] == e) jj = j;
    int tot;
    const int r = block_excl_scan(jj >= 0, s_tmp, &tot);
    if (jj >= 0) {
      const int pos = base + r;
      const int s = (int)(t * k + jj);
      perm[pos] = s;
      inv[s] = pos;
      if (perm_out) perm_out[pos] = s;
    }
    base += tot;
  }
}

// ---------------------------------------------------------------- launcher
hipError_t launch_route(const Fwd& f, bool decode) {
  const ds4moe_layer& L = f.L;
  const int d = L.d_model, E = L.n_experts, k = L.top_k;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  _Float16* xh = (_Float16*)(ws + y.x_hi);
  _Float16* xl = f.lo ? (_Float16*)(ws + y.x_lo) : nullptr;
  float* logits = (float*)(ws + y.logits);
  int32_t* idx = (int32_t*)(ws + y.topk_idx);
  float* w = (float*)(ws + y.topk_w);
  int32_t* counts = (int32_t*)(ws + y.counts);
  int32_t* offsets = (int32_t*)(ws + y.offsets);
  int32_t* perm = (int32_t*)(ws + y.perm);
  int32_t* inv = (int32_t*)(ws + y.inv);

  if (decode) {
    const int T = (int)f.T;
    const int kr = d / QK;  // one partial per 256-input chunk
    float* plog = (float*)(ws + y.plog);
    const dim3 pg((E + 15) / 16, kr);
    int32_t* ctrl = (int32_t*)(ws + y.ctrl);
    const int nctrl = ctrl_ints(L);
    if (f.lo)
      DS4_LAUNCH(k_router_partial<true>, pg, dim3(256), 0, f.st, L.router_w, E, d, f.x, T, plog, xh, xl, ctrl, nctrl);
    else
      DS4_LAUNCH(k_router_partial<false>, pg, dim3(256), 0, f.st, L.router_w, E, d, f.x, T, plog, xh, xl, ctrl, nctrl);
    DS4_LAUNCH(k_route_finish_decode, dim3(1), dim3(256), 0, f.st, plog, kr, L.router_bias, E, k, T, route_out(f));
  } else {
    const int64_t n8 = f.T * d / 8;
    const int cblocks = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
    DS4_LAUNCH(k_convert_x, dim3(cblocks), dim3(256), 0, f.st, f.x, f.x_dtype, n8, xh, xl);
    const hipError_t e = launch_router_logits(L, f.T, f.lo, xh, xl, (float*)(ws + y.rpart), logits, f.st);
    if (e != hipSuccess) return e;
    DS4_LAUNCH(k_topk_rows, dim3((unsigned)((f.T + 3) / 4)), dim3(256), 0, f.st, logits, E, k, f.T, idx, w,
                       f.idx_out, f.w_out);
    DS4_LAUNCH(k_count_experts, dim3(E), dim3(256), 0, f.st, idx, f.T * k, counts);
    DS4_LAUNCH(k_scatter_experts, dim3(E), dim3(256), 0, f.st, idx, f.T, k, E, counts, offsets, perm, inv,
                       f.counts_out, f.offsets_out, f.perm_out, (int32_t*)(ws + y.tiles), (int32_t*)(ws + y.stiles),
                       (int32_t*)(ws + y.ntiles));
  }
  return hipGetLastError();
}

}  // namespace ds4
