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
#include "trace.h"
#include "tiles.h"

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

// ---------------------------------------------------------------- logits
// Block: 16 experts x 16 tokens, NW waves splitting K.  logits [T, E] fp32.
template <int NW, bool LO>
__global__ __launch_bounds__(NW * 64) void k_router_logits(const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int E, int d,
                                                           const _Float16* __restrict__ xh,
                                                           const _Float16* __restrict__ xl, int64_t T,
                                                           float* __restrict__ logits) {
  __shared__ float red[NW * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * 16;
  const int64_t t = (int64_t)blockIdx.y * 16 + (lane & 15);
  const _Float16* bh = t < T ? xh + t * d : nullptr;
  const _Float16* bl = (LO && t < T) ? xl + t * d : nullptr;
  const int arow = min(e0 + (lane & 15), E - 1);
  int ks0, ks1;
  split_range(d / 32, NW, wave, ks0, ks1);
  float4_t acc = {0.f, 0.f, 0.f, 0.f}, unused = acc;
  f16_tile<false, LO>(wr + (int64_t)arow * d, nullptr, bh, bl, ks0, ks1, lane, acc, unused);
  acc = block_reduce_waves<NW>(acc, red, wave, lane);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 4 * (lane >> 4) + r;
      if (e < E) logits[t * E + e] = acc[r] + (bias ? bias[e] : 0.0f);
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wave selects the k largest of E logits (lane owns e = lane + 64 i),
// leaving the chosen indices/values in LDS (sel_e, sel_v, round order).
__device__ inline void wave_topk(const float* __restrict__ l, int E, int k, int lane, int* sel_e, float* sel_v) {
  float v[kMaxExperts / 64];
  uint32_t taken = 0;
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxExperts / 64; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per && e < E) ? l[e] : -__builtin_inff();
  }
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      const int e = lane + 64 * i;
      // strict '>' keeps the lower index among equal logits (e grows with i)
      if (i < per && e < E && !((taken >> i) & 1u) && (v[i] > bv || be == 0x7FFFFFFF)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == 0) {
      sel_e[j] = be;
      sel_v[j] = bv;
    }
  }
}

// Lane 0: sort the k selected experts by index and compute their softmax.
__device__ inline void finish_token(int* sel_e, float* sel_v, int k, int64_t t, int32_t* idx, float* w,
                                    int32_t* idx_out, float* w_out) {
  const float lmax = sel_v[0];
  for (int a = 1; a < k; ++a) {  // insertion sort by expert index
    int e = sel_e[a];
    float v = sel_v[a];
    int b = a - 1;
    while (b >= 0 && sel_e[b] > e) {
      sel_e[b + 1] = sel_e[b];
      sel_v[b + 1] = sel_v[b];
      --b;
    }
    sel_e[b + 1] = e;
    sel_v[b + 1] = v;
  }
  float den = 0.0f;
  for (int j = 0; j < k; ++j) den += expf(sel_v[j] - lmax);
  for (int j = 0; j < k; ++j) {
    const float wj = expf(sel_v[j] - lmax) / den;
    idx[t * k + j] = sel_e[j];
    w[t * k + j] = wj;
    if (idx_out) idx_out[t * k + j] = sel_e[j];
    if (w_out) w_out[t * k + j] = wj;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads); returns the
// thread's exclusive prefix and writes the block total to *total.
__device__ inline int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) pre += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return pre + inc - v;
}

// ---------------------------------------------------------------- decode: one block does it all
// T <= 16 tokens.  Produces idx/w, counts, offsets, perm, inv and the
// distinct-expert table: distinct[i] (ascending expert), tok_slot[i*16 + t]
// = slot of token t in expert distinct[i], or -1.
__global__ __launch_bounds__(256) void k_route_finish_decode(
    const float* __restrict__ logits, int E, int k, int T, int32_t* __restrict__ idx, float* __restrict__ w,
    int32_t* idx_out, float* w_out, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* counts_out, int32_t* offsets_out,
    int32_t* perm_out, int32_t* __restrict__ ndist, int32_t* __restrict__ distinct, int32_t* __restrict__ tok_slot) {
  __shared__ int s_sel_e[4][kMaxTopK];
  __shared__ float s_sel_v[4][kMaxTopK];
  __shared__ int s_idx[kDecodeGroup * kMaxTopK];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_dpos[kMaxExperts];
  __shared__ int s_tmp[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  for (int t = wave; t < T; t += 4) {
    wave_topk(logits + (int64_t)t * E, E, k, lane, s_sel_e[wave], s_sel_v[wave]);
    if (lane == 0) {
      finish_token(s_sel_e[wave], s_sel_v[wave], k, t, idx, w, idx_out, w_out);
      for (int j = 0; j < k; ++j) s_idx[t * k + j] = s_sel_e[wave][j];
    }
  }
  __syncthreads();
  const int S = T * k;
  for (int s = threadIdx.x; s < S; s += blockDim.x) atomicAdd(&s_cnt[s_idx[s]], 1);
  __syncthreads();
  // exclusive scans over experts: thread owns EPT consecutive experts
  const int EPT = (E + 255) / 256;
  int csum = 0, dsum = 0;
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x * EPT + i;
    if (e < E) {
      csum += s_cnt[e];
      dsum += s_cnt[e] > 0;
    }
  }
  int ctot, dtot;
  int cpre = block_excl_scan(csum, s_tmp, &ctot);
  int dpre = block_excl_scan(dsum, s_tmp, &dtot);
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x * EPT + i;
    if (e < E) {
      s_off[e] = cpre;
      s_dpos[e] = s_cnt[e] > 0 ? dpre : -1;
      counts[e] = s_cnt[e];
      offsets[e] = cpre;
      if (counts_out) counts_out[e] = s_cnt[e];
      if (offsets_out) offsets_out[e] = cpre;
      if (s_cnt[e] > 0) distinct[dpre] = e;
      cpre += s_cnt[e];
      dpre += s_cnt[e] > 0;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = ctot;
    if (offsets_out) offsets_out[E] = ctot;
    *ndist = dtot;
  }
  for (int i = threadIdx.x; i < dtot * kDecodeGroup; i += blockDim.x) tok_slot[i] = -1;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = s_idx[s], t = s / k;
    int rank = 0;
    for (int u = 0; u < t; ++u)
      for (int j = 0; j < k; ++j) rank += s_idx[u * k + j] == e;
    const int pos = s_off[e] + rank;
    perm[pos] = s;
    inv[s] = pos;
    if (perm_out) perm_out[pos] = s;
    tok_slot[s_dpos[e] * kDecodeGroup + t] = s;
  }
}

// ---------------------------------------------------------------- prefill: top-k per token
__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ logits, int E, int k, int64_t T,
                                                   int32_t* __restrict__ idx, float* __restrict__ w,
                                                   int32_t* idx_out, float* w_out) {
  __shared__ int s_sel_e[4][kMaxTopK];
  __shared__ float s_sel_v[4][kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  wave_topk(logits + t * E, E, k, lane, s_sel_e[wave], s_sel_v[wave]);
  if (lane == 0) finish_token(s_sel_e[wave], s_sel_v[wave], k, t, idx, w, idx_out, w_out);
}

// prefill grouping, pass 1: counts[e] (one block per expert)
__global__ __launch_bounds__(256) void k_count_experts(const int32_t* __restrict__ idx, int64_t S,
                                                       int32_t* __restrict__ counts) {
  __shared__ int s_tmp[8];
  const int e = blockIdx.x;
  int c = 0;
  for (int64_t s = threadIdx.x; s < S; s += blockDim.x) c += idx[s] == e;
  int tot;
  block_excl_scan(c, s_tmp, &tot);
  if (threadIdx.x == 0) counts[e] = tot;
}

// prefill grouping, pass 2: offsets, perm, inv, and the GEMM work list of
// (expert, group of 16 tokens) tiles (one block per expert).
__global__ __launch_bounds__(256) void k_scatter_experts(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                         const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv, int32_t* counts_out,
                                                         int32_t* offsets_out, int32_t* perm_out,
                                                         int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int s_tmp[8];
  const int e = blockIdx.x;
  int a = 0, b = 0;
  for (int u = threadIdx.x; u < E; u += blockDim.x) {
    if (u < e) {
      a += counts[u];
      b += (counts[u] + 15) / 16;
    }
  }
  int off, tstart;
  block_excl_scan(a, s_tmp, &off);
  block_excl_scan(b, s_tmp, &tstart);
  const int cnt = counts[e];
  if (threadIdx.x == 0) {
    offsets[e] = off;
    if (offsets_out) offsets_out[e] = off;
    if (counts_out) counts_out[e] = cnt;
    if (e == E - 1) {
      offsets[E] = off + cnt;
      if (offsets_out) offsets_out[E] = off + cnt;
      *ntiles = tstart + (cnt + 15) / 16;
    }
  }
  for (int g = threadIdx.x; g < (cnt + 15) / 16; g += blockDim.x) {
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

  const int64_t n8 = f.T * d / 8;
  const int cblocks = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
  DS4_LAUNCH(k_convert_x, dim3(cblocks), dim3(256), 0, f.st, f.x, f.x_dtype, n8, xh, xl);
  const dim3 lg((E + 15) / 16, (unsigned)((f.T + 15) / 16));
  if (decode) {
    if (f.lo)
      DS4_LAUNCH((k_router_logits<16, true>), lg, dim3(1024), 0, f.st, L.router_w, L.router_bias, E, d, xh, xl, f.T, logits);
    else
      DS4_LAUNCH((k_router_logits<16, false>), lg, dim3(1024), 0, f.st, L.router_w, L.router_bias, E, d, xh, xl, f.T, logits);
    DS4_LAUNCH(k_route_finish_decode, dim3(1), dim3(256), 0, f.st, logits, E, k, (int)f.T, idx, w,
                       f.idx_out, f.w_out, counts, offsets, perm, inv, f.counts_out, f.offsets_out, f.perm_out,
                       (int32_t*)(ws + y.ndist), (int32_t*)(ws + y.distinct), (int32_t*)(ws + y.tok_slot));
  } else {
    if (f.lo)
      DS4_LAUNCH((k_router_logits<4, true>), lg, dim3(256), 0, f.st, L.router_w, L.router_bias, E, d, xh, xl, f.T, logits);
    else
      DS4_LAUNCH((k_router_logits<4, false>), lg, dim3(256), 0, f.st, L.router_w, L.router_bias, E, d, xh, xl, f.T, logits);
    DS4_LAUNCH(k_topk_rows, dim3((unsigned)((f.T + 3) / 4)), dim3(256), 0, f.st, logits, E, k, f.T, idx, w,
                       f.idx_out, f.w_out);
    DS4_LAUNCH(k_count_experts, dim3(E), dim3(256), 0, f.st, idx, f.T * k, counts);
    DS4_LAUNCH(k_scatter_experts, dim3(E), dim3(256), 0, f.st, idx, f.T, k, E, counts, offsets, perm, inv,
                       f.counts_out, f.offsets_out, f.perm_out, (int32_t*)(ws + y.tiles), (int32_t*)(ws + y.ntiles));
  }
  return hipGetLastError();
}

}  // namespace ds4
