// Hyper-connection mixer on either side of the layer: coefficients, the
// reduce to one row, and the expand back to n streams.  Definitions (and the
// reading taken of the DS4 (DwarfStar 4) wiki note, "Key Techniques",
// hyper-connections with Sinkhorn normalization) are in include/ds4moe.h at
// ds4moe_hc.
//
// Three kernels, all HBM-bound:
//   k_hc_partial  split-K partial projections of the flattened streams onto
//                 the 24 mixer rows (fp32 MFMA 16x16x4) plus partial sums of
//                 squares; block (tile of 16 tokens, K-slice).  For one or
//                 two tokens its last-arriving block also does k_hc_reduce's
//                 work, so the step is one launch
//   k_hc_reduce   one block per token: adds the partials, finishes the
//                 logits, sigmoid weights and the Sinkhorn mixer in one wave,
//                 then writes x_in = sum_i pre_i X_i (fp32 and/or bf16)
//   k_hc_post     X'_i = sum_j M_ij X_j + post_i y, elementwise over d
#include "common.h"
#include "internal.h"
#include "trace.h"

namespace ds4 {

constexpr int kHcN = 4;                          // streams
constexpr int kHcOut = 2 * kHcN + kHcN * kHcN;  // mixer logits per token
constexpr int kHcPart = 32;                      // floats per (K-slice, token) partial: [0, 24) sums, [24] squares

static_assert(kHcOut <= 24, "the second MFMA tile holds rows 16..31 and the squares in row 24");

// Inputs of the flattened streams per K-slice: short slices (more blocks)
// when few tokens share each projection row, long ones otherwise.
int hc_slice(int64_t T) { return T > 64 ? 1024 : 256; }

// Tokens up to which one launch does everything (the partial kernel's last
// block finishes them).
constexpr int kHcFusedT = 2;

static size_t hc_part_bytes(int d, int64_t T) {
  const int64_t nd = (int64_t)kHcN * d;
  return ((size_t)(nd / hc_slice(T)) * (size_t)T * kHcPart * sizeof(float) + 255) & ~(size_t)255;
}

// partials, then the arrival counter (256 bytes)
size_t hc_ws_bytes(int d, int64_t T) { return hc_part_bytes(d, T) + 256; }

struct HcParams {
  float eps, alpha_pre, alpha_post, alpha_res;
  int iters;
  const float* bias;
};

__device__ inline float4_t mfma_f32_4(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline uint16_t bf16_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);  // NaN stays NaN
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Lane swaps within rows of 16 lanes (DPP): quad_perm [1,0,3,2] and
// [2,3,0,1] exchange within quads, row_ror:8 and row_ror:4 rotate the row.
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor8 = 0x128, kDppRor4 = 0x124;

// Finish of token t by one block of 256 threads.  Threads (g, o), g = tid /
// 32, add slices g, g + 8, ... of partial o (eight independent loads at a
// time; coherent loads when COH, for partials other blocks of the running
// kernel wrote); wave 0 then finishes: lanes 0..23 the logits, 0..7 the
// sigmoid weights, and lanes 0..15 (one DPP row) the Sinkhorn mixer, entry
// p = lane = 4 i + j: a row is a quad, a column the lanes p, p +- 4, p +- 8
// of the row.  Each sum pairs the same terms in every lane that uses it, so
// a row's (column's) lanes divide by the same value.  Then every thread
// reduces float4 columns of the token's streams (loaded before the
// partials, which they do not depend on, up to kHcPre columns per thread).
constexpr int kHcPre = 4;  // float4 columns per thread loaded ahead (all of them up to d = 4096)
struct HcLds {
  float sum[8][kHcPart];
  float pre[kHcN];
};

template <bool COH>
__device__ void hc_finish_token(int t, const float* __restrict__ X, const float* part, int nslices, int T, int d,
                                const HcParams& P, float* __restrict__ coef, float* __restrict__ xout,
                                uint16_t* __restrict__ xbf, HcLds& lds) {
  const int tid = threadIdx.x;
  const float4* xs = (const float4*)(X + (int64_t)t * kHcN * d);
  const int d4 = d / 4;
  float4 w[kHcPre][kHcN];  // the thread's first kHcPre float4 columns of every stream
#pragma unroll
  for (int u = 0; u < kHcPre; ++u) {
    const int c4 = min(tid + 256 * u, d4 - 1);
#pragma unroll
    for (int i = 0; i < kHcN; ++i) w[u][i] = xs[i * d4 + c4];
  }
  {
    const int o = tid & 31, g = tid >> 5;
    float acc = 0.f;
    for (int s0 = g; s0 < nslices; s0 += 64) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + 8 * u;
        const float* src = part + ((int64_t)min(s, nslices - 1) * T + t) * kHcPart + o;
        v[u] = s < nslices ? (COH ? ld_coh(src) : *src) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    lds.sum[g][o] = acc;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    float v = 0.f;
    if (lane < kHcPart) {
#pragma unroll
      for (int g = 0; g < 8; ++g) v += lds.sum[g][lane];
    }
    const float r = sqrtf(__shfl(v, 24) / (float)(kHcN * d) + P.eps);
    const float alpha = lane < kHcN ? P.alpha_pre : (lane < 2 * kHcN ? P.alpha_post : P.alpha_res);
    const float z = lane < kHcOut ? alpha * (v / r) + P.bias[min(lane, kHcOut - 1)] : 0.f;
    const float sg = 1.0f / (1.0f + expf(-z));
    const float zz = __shfl(z, 2 * kHcN + (lane & 15));
    float m = fmaxf(zz, dpp_f32<kDppXor1>(zz));
    m = fmaxf(m, dpp_f32<kDppXor2>(m));
    float a = expf(zz - m);
    for (int it = 0; it < P.iters; ++it) {  // a / sum as a * rcp(sum): within 2 ulp of the quotient
      float rs = a + dpp_f32<kDppXor1>(a);
      rs = rs + dpp_f32<kDppXor2>(rs);
      a = a * __builtin_amdgcn_rcpf(rs);
      float cs = a + dpp_f32<kDppRor8>(a);
      cs = cs + dpp_f32<kDppRor4>(cs);
      a = a * __builtin_amdgcn_rcpf(cs);
    }
    float* cf = coef + (int64_t)t * kHcOut;
    if (lane < kHcN) {
      cf[lane] = sg;
      lds.pre[lane] = sg;
    } else if (lane < 2 * kHcN) {
      cf[lane] = 2.0f * sg;
    }
    if (lane < kHcN * kHcN) cf[2 * kHcN + lane] = a;
  }
  __syncthreads();
  const float p0 = lds.pre[0], p1 = lds.pre[1], p2 = lds.pre[2], p3 = lds.pre[3];
  auto out = [&](int c4, const float4& v0, const float4& v1, const float4& v2, const float4& v3) {
    float4 o;
    o.x = fmaf(p3, v3.x, fmaf(p2, v2.x, fmaf(p1, v1.x, p0 * v0.x)));
    o.y = fmaf(p3, v3.y, fmaf(p2, v2.y, fmaf(p1, v1.y, p0 * v0.y)));
    o.z = fmaf(p3, v3.z, fmaf(p2, v2.z, fmaf(p1, v1.z, p0 * v0.z)));
    o.w = fmaf(p3, v3.w, fmaf(p2, v2.w, fmaf(p1, v1.w, p0 * v0.w)));
    if (xout) ((float4*)(xout + (int64_t)t * d))[c4] = o;
    if (xbf) {
      const uint32_t lo = bf16_rne(o.x) | ((uint32_t)bf16_rne(o.y) << 16);
      const uint32_t hi = bf16_rne(o.z) | ((uint32_t)bf16_rne(o.w) << 16);
      ((uint2*)(xbf + (int64_t)t * d))[c4] = make_uint2(lo, hi);
    }
  };
#pragma unroll
  for (int u = 0; u < kHcPre; ++u) {
    const int c4 = tid + 256 * u;
    if (c4 < d4) out(c4, w[u][0], w[u][1], w[u][2], w[u][3]);
  }
  for (int c4 = tid + 256 * kHcPre; c4 < d4; c4 += 256) out(c4, xs[c4], xs[d4 + c4], xs[2 * d4 + c4], xs[3 * d4 + c4]);
}

// Block (tile, slice): tokens [16 tile, +16) (the last clamped to T - 1 and
// not stored), inputs [slice * ks, +ks), a quarter per wave in steps of 16
// (ks is 256 or 1024, so a wave's share is a whole number of 64-input groups).
// MFMA A = projection rows (row lane & 15, and 16 + (lane & 15) for the
// second tile), B = streams transposed (token lane & 15); lane l feeds
// K-slot l >> 4 the inputs k0 + 4 (l >> 4) + j at sub-step j, so D[o][t]
// leaves outputs 4 (l >> 4) .. +3 of token l & 15 in lane l.  Projection
// rows past the last are zero; row 24 of the second tile carries the sum of
// squares.  part: [slices][T][32].
//
// FUSED (T <= kHcFusedT, one tile): the partials are stored write-through
// (agent-scope stores) and each block, once those stores have completed,
// takes a ticket from the tile's arrival counter; the block that takes the
// last ticket reads every partial with agent-scope loads, finishes every
// token of the tile itself and clears the counter for the next call.  No
// cache-wide fence is needed: the stores reach the device coherence point
// before the ticket is taken, and the loads are served from it.
template <bool FUSED>
__global__ __launch_bounds__(256) void k_hc_partial(const float* __restrict__ X, const float* __restrict__ phi,
                                                    int T, int nd, int ks, float* __restrict__ part,
                                                    int32_t* __restrict__ ctr, HcParams P, float* __restrict__ coef,
                                                    float* __restrict__ xout, uint16_t* __restrict__ xbf) {
  __shared__ float4_t red[3][64][2];
  __shared__ HcLds lds;
  __shared__ int last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int tile = blockIdx.x, slice = blockIdx.y;
  const int t = min(tile * 16 + c, T - 1);
  const float* xr = X + (int64_t)t * nd;
  const float* pa = phi + (int64_t)c * nd;
  const bool hb = c < kHcOut - 16;
  const float* pb = phi + (int64_t)(hb ? 16 + c : 0) * nd;
  const int kw = ks / 4;
  const int k0 = slice * ks + wave * kw + 4 * q;
  float4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  float ss = 0.f;
  // kw is 64 or 256: groups of four 16-input steps, the group's loads issued together
  for (int k = k0; k < k0 + kw; k += 64) {
    float4 xv[4], av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xv[u] = *(const float4*)(xr + k + 16 * u);
      av[u] = *(const float4*)(pa + k + 16 * u);
      bv[u] = hb ? *(const float4*)(pb + k + 16 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0 = mfma_f32_4(av[u].x, xv[u].x, a0);
      a0 = mfma_f32_4(av[u].y, xv[u].y, a0);
      a0 = mfma_f32_4(av[u].z, xv[u].z, a0);
      a0 = mfma_f32_4(av[u].w, xv[u].w, a0);
      a1 = mfma_f32_4(bv[u].x, xv[u].x, a1);
      a1 = mfma_f32_4(bv[u].y, xv[u].y, a1);
      a1 = mfma_f32_4(bv[u].z, xv[u].z, a1);
      a1 = mfma_f32_4(bv[u].w, xv[u].w, a1);
      ss = fmaf(xv[u].x, xv[u].x, ss);
      ss = fmaf(xv[u].y, xv[u].y, ss);
      ss = fmaf(xv[u].z, xv[u].z, ss);
      ss = fmaf(xv[u].w, xv[u].w, ss);
    }
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  if (q == 2) a1[0] = ss;  // row 16 + 4*2 + 0 = 24 (no projection row there)
  if (wave > 0) {
    red[wave - 1][lane][0] = a0;
    red[wave - 1][lane][1] = a1;
  }
  __syncthreads();
  if (wave == 0 && tile * 16 + c < T) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      a0 += red[w][lane][0];
      a1 += red[w][lane][1];
    }
    float* dst = part + ((int64_t)slice * T + tile * 16 + c) * kHcPart;
    if (FUSED) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st_coh(dst + 4 * q + r, a0[r]);
        st_coh(dst + 16 + 4 * q + r, a1[r]);
      }
      wait_stores();
    } else {
      *(float4_t*)(dst + 4 * q) = a0;
      *(float4_t*)(dst + 16 + 4 * q) = a1;
    }
  }
  if (!FUSED) return;
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(ctr, 1) == (int)gridDim.y - 1;
  __syncthreads();
  if (!last) return;
  for (int tt = 0; tt < T; ++tt) {
    hc_finish_token<true>(tt, X, part, gridDim.y, T, nd / kHcN, P, coef, xout, xbf, lds);
    __syncthreads();
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One block per token (tokens the partial kernel did not finish itself).
__global__ __launch_bounds__(256) void k_hc_reduce(const float* __restrict__ X, const float* __restrict__ part,
                                                   int nslices, int T, int d, HcParams P, float* __restrict__ coef,
                                                   float* __restrict__ xout, uint16_t* __restrict__ xbf) {
  __shared__ HcLds lds;
  hc_finish_token<false>(blockIdx.x, X, part, nslices, T, d, P, coef, xout, xbf, lds);
}

// Block b: token b / nbt, float4 columns (b % nbt) * 256 + tid.  X and Xo
// may be the same array: each thread reads its four stream values before
// it writes them, and no other thread touches them.
__global__ __launch_bounds__(256) void k_hc_post(const float* X, const float* __restrict__ y,
                                                 const float* __restrict__ coef, int d, int nbt, float* Xo) {
  const int t = blockIdx.x / nbt;
  const int c4 = (blockIdx.x % nbt) * 256 + threadIdx.x;
  const int d4 = d / 4;
  if (c4 >= d4) return;
  const float* cf = coef + (int64_t)t * kHcOut;
  const float4* xs = (const float4*)(X + (int64_t)t * kHcN * d);
  const float4 v0 = xs[c4], v1 = xs[d4 + c4], v2 = xs[2 * d4 + c4], v3 = xs[3 * d4 + c4];
  const float4 yv = ((const float4*)(y + (int64_t)t * d))[c4];
  float4* os = (float4*)(Xo + (int64_t)t * kHcN * d);
#pragma unroll
  for (int i = 0; i < kHcN; ++i) {
    const float* M = cf + 2 * kHcN + kHcN * i;
    const float pi = cf[kHcN + i];
    float4 o;
    o.x = fmaf(pi, yv.x, fmaf(M[3], v3.x, fmaf(M[2], v2.x, fmaf(M[1], v1.x, M[0] * v0.x))));
    o.y = fmaf(pi, yv.y, fmaf(M[3], v3.y, fmaf(M[2], v2.y, fmaf(M[1], v1.y, M[0] * v0.y))));
    o.z = fmaf(pi, yv.z, fmaf(M[3], v3.z, fmaf(M[2], v2.z, fmaf(M[1], v1.z, M[0] * v0.z))));
    o.w = fmaf(pi, yv.w, fmaf(M[3], v3.w, fmaf(M[2], v2.w, fmaf(M[1], v1.w, M[0] * v0.w))));
    os[i * d4 + c4] = o;
  }
}

hipError_t launch_hc_pre(const ds4moe_hc& H, const float* X, int64_t T, float* coef, float* xout, uint16_t* xbf,
                         void* ws, hipStream_t st) {
  const int d = H.d_model, nd = kHcN * d, ks = hc_slice(T);
  const int nslices = nd / ks;
  float* part = (float*)ws;
  int32_t* ctr = (int32_t*)((char*)ws + hc_part_bytes(d, T));
  const HcParams P{H.eps, H.alpha_pre, H.alpha_post, H.alpha_res, H.sinkhorn_iters, H.bias};
  const dim3 grid((unsigned)((T + 15) / 16), (unsigned)nslices);
  if (T <= kHcFusedT) {
    DS4_LAUNCH(k_hc_partial<true>, grid, dim3(256), 0, st, X, H.phi, (int)T, nd, ks, part, ctr, P, coef, xout, xbf);
    return hipGetLastError();
  }
  DS4_LAUNCH(k_hc_partial<false>, grid, dim3(256), 0, st, X, H.phi, (int)T, nd, ks, part, ctr, P, coef, xout, xbf);
  DS4_LAUNCH(k_hc_reduce, dim3((unsigned)T), dim3(256), 0, st, X, (const float*)part, nslices, (int)T, d, P, coef,
             xout, xbf);
  return hipGetLastError();
}

hipError_t launch_hc_post(const ds4moe_hc& H, const float* X, const float* y, const float* coef, int64_t T,
                          float* Xo, hipStream_t st) {
  const int d = H.d_model, nbt = (d / 4 + 255) / 256;
  DS4_LAUNCH(k_hc_post, dim3((unsigned)(T * nbt)), dim3(256), 0, st, X, y, coef, d, nbt, Xo);
  return hipGetLastError();
}

}  // namespace ds4
