// Batched decode (T <= 16 tokens per group): expert products as dequant-in-
// register MFMA tiles whose 16 columns are the group's tokens.  Three
// kernels per group:
//   k_router_partial  (route.hip) partial router logits per 256-input chunk,
//                     binary16 copy of x, clears the control words.
//   k_gateup_decode   block 0 finishes routing (logits, top-k, softmax,
//                     grouping) and raises a ready flag; the shared expert's
//                     16-row tiles run as 4 K-chunks each, the last chunk of a
//                     tile summing the chunk partials in order and applying
//                     SwiGLU; each distinct selected expert's 16-row tiles run
//                     once routing is ready.  Routed h is stored pre-multiplied
//                     by the token's gate weight as binary16, with fp32 sums
//                     over each 16 rows (one Q2K sub-block of the down input).
//   k_down_decode     one block per (16-row tile of y, source), the sources
//                     being 4 K-chunks of the shared expert and each distinct
//                     expert; the last block to finish a tile adds the partials
//                     in a fixed order (shared chunks, then experts by
//                     ascending index) into y.
// Each distinct expert is read once per call however many tokens chose it,
// and results do not depend on block scheduling.  Blocks hand data to each
// other inside a kernel with a device-scope release (L2 write-back) before a
// counter or flag, and coherent (sc1) loads on the reading side.
//
// Lane mapping.  For packed weights every lane owns a contiguous 16-byte
// piece of its row's super-block and feeds those weights to consecutive MFMA
// steps (CB2: lane group q holds sub-blocks 2q, 2q+1; Q2K: sub-blocks
// 4q..4q+3); the activation column is read at the matching K offsets, so no
// two lanes load the same bytes.  F16 weights use the plain mapping (K-step
// ks, lane group q -> K = 32 ks + 8 q).
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "routefin.h"
#include "tiles.h"
#include "trace.h"

namespace ds4 {

__constant__ GridTables c_dec_tables = make_grid_tables();

constexpr int kGW = 8;  // waves per gate/up block
constexpr int kDW = 8;  // waves per down block

__device__ inline int cb2_boff(int q, int s) { return 32 * (2 * q + (s >> 2)) + 8 * (s & 3); }
__device__ inline int q2k_boff(int q, int s) { return 16 * (4 * q + (s >> 1)) + 8 * (s & 1); }

// One CB2 super-block of two matrices (gate, up).  cg/cu: this lane's 16
// code bytes (sub-blocks 2q, 2q+1 of its row); bcol/bl: activation column at
// the super-block start; dg/du: d of the lane's four output rows.
template <bool LO>
__device__ inline void cb2_pair_superblock(u32x4_t cg, u32x4_t cu, const _Float16* bcol, const _Float16* bl,
                                           int q, const float* dg, const float* du, const uint32_t* mag,
                                           const uint32_t* sgn, float4_t& ag, float4_t& au) {
  half8_t bv[8], blv[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    bv[s] = bcol ? *(const half8_t*)(bcol + cb2_boff(q, s)) : zero_half8();
    if (LO) blv[s] = bl ? *(const half8_t*)(bl + cb2_boff(q, s)) : zero_half8();
  }
  float4_t pg = {0.f, 0.f, 0.f, 0.f}, pu = pg;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const half8_t a0 = cb2_frag((s & 4) ? cg.z : cg.x, (s & 4) ? cg.w : cg.y, s & 3, mag, sgn);
    const half8_t a1 = cb2_frag((s & 4) ? cu.z : cu.x, (s & 4) ? cu.w : cu.y, s & 3, mag, sgn);
    pg = mfma16x16x32(a0, bv[s], pg);
    pu = mfma16x16x32(a1, bv[s], pu);
    if (LO) {
      pg = mfma16x16x32(a0, blv[s], pg);
      pu = mfma16x16x32(a1, blv[s], pu);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ag[r] += dg[r] * pg[r];
    au[r] += du[r] * pu[r];
  }
}

// Bounded wait (thread 0) for a flag another block of this kernel raises.
// The writer is always an earlier block of the same grid, so the wait ends;
// the bound only guards against a broken invariant.
__device__ inline void wait_flag(const int32_t* flag) {
  if (threadIdx.x == 0) {
    for (int n = 0; ld_acq_int(flag) == 0 && n < (1 << 22); ++n) __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();
}

template <bool LO>
__global__ __launch_bounds__(kGW * 64) void k_gateup_decode(
    ds4moe_layer L, int T, const float* __restrict__ plog, RouteOut ro, const _Float16* __restrict__ xh,
    const _Float16* __restrict__ xl, int32_t* __restrict__ ctrl, float* __restrict__ sh_part,
    _Float16* __restrict__ hs16, _Float16* __restrict__ hw16, float* __restrict__ hsum) {
  __shared__ uint32_t s_mag[256 * 4];
  __shared__ uint32_t s_sgn[128 * 4];
  __shared__ float4_t s_red[kGW][2][64];
  __shared__ int s_flag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, fs = L.d_ff_shared, k = L.top_k;
  const int nsh = fs / 16, nr = f / 16, nb = d / QK;
  const int Tp = min(T, kDecodeGroup);

  if (blockIdx.x == 0) {  // ---------------- routing: top-k, weights, grouping
    route_finish_block(plog, nb, L.router_bias, L.n_experts, k, T, ro);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(&ctrl[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  const int bid = blockIdx.x - 1;
  if (bid < nsh * kShChunks) {  // ---------------- shared expert: tile x K chunk
    const int tile = bid / kShChunks, kc = bid % kShChunks;
    const int row0 = tile * 16;
    const int nks = d / 32;
    const int c0 = kc * nks / kShChunks, c1 = (kc + 1) * nks / kShChunks;
    int ks0, ks1;
    split_range(c1 - c0, kGW, wave, ks0, ks1);
    const _Float16* bh = c < T ? xh + (int64_t)c * d : nullptr;
    const _Float16* bl = (LO && c < T) ? xl + (int64_t)c * d : nullptr;
    const int64_t ar = (int64_t)(row0 + c) * d;
    f16_tile<true, LO>(L.sh_gate + ar, L.sh_up + ar, bh, bl, c0 + ks0, c0 + ks1, lane, ag, au);
    s_red[wave][0][lane] = ag;
    s_red[wave][1][lane] = au;
    __syncthreads();
    float* part = sh_part + (size_t)tile * kShChunks * 2 * 16 * Tp;
    if (wave == 0) {
      ag = s_red[0][0][lane];
      au = s_red[0][1][lane];
#pragma unroll
      for (int w = 1; w < kGW; ++w) {
        ag += s_red[w][0][lane];
        au += s_red[w][1][lane];
      }
      if (c < T) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st_coh(&part[((size_t)(kc * 2 + 0) * 16 + 4 * q + r) * Tp + c], ag[r]);
          st_coh(&part[((size_t)(kc * 2 + 1) * 16 + 4 * q + r) * Tp + c], au[r]);
        }
      }
      wait_stores();
    }
    __syncthreads();
    if (threadIdx.x == 0) s_flag = atomicAdd(&ctrl[1 + tile], 1) == kShChunks - 1;
    __syncthreads();
    if (!s_flag || wave != 0 || c >= T) return;
    float4_t g = {0.f, 0.f, 0.f, 0.f}, u = g;
    for (int j = 0; j < kShChunks; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        g[r] += ld_coh(&part[((size_t)(j * 2 + 0) * 16 + 4 * q + r) * Tp + c]);
        u[r] += ld_coh(&part[((size_t)(j * 2 + 1) * 16 + 4 * q + r) * Tp + c]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) hs16[(int64_t)c * fs + row0 + 4 * q + r] = (_Float16)(silu(g[r]) * u[r]);
    return;
  }
  // ---------------- routed: distinct expert i, 16-row tile
  const int rel = bid - nsh * kShChunks;
  const int i = rel / nr, tile = rel % nr;
  const int row0 = tile * 16;
  stage_grid_tables(s_mag, s_sgn, c_dec_tables);
  wait_flag(&ctrl[0]);  // includes a barrier for the staged tables
  if (i >= ld_acq_int(ro.ndist)) return;
  const int e = ld_acq_int(&ro.distinct[i]);
  const int slot = ld_acq_int(&ro.tok_slot[i * kDecodeGroup + c]);
  const _Float16* bh = slot >= 0 ? xh + (int64_t)(slot / k) * d : nullptr;
  const _Float16* bl = (LO && slot >= 0) ? xl + (int64_t)(slot / k) * d : nullptr;
  const size_t mb = (size_t)f * nb;  // blocks per matrix
  const uint8_t* gc = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* uc = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const uint16_t* gd = (const uint16_t*)(gc + mb * 64);
  const uint16_t* ud = (const uint16_t*)(uc + mb * 64);
  const uint8_t* grow = gc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  const uint8_t* urow = uc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  const int orow = row0 + 4 * q;
  int sb0, sb1;
  split_range(nb, kGW, wave, sb0, sb1);
  for (int b = sb0; b < sb1; ++b) {
    const u32x4_t cg = __builtin_nontemporal_load((const u32x4_t*)(grow + b * 64));
    const u32x4_t cu = __builtin_nontemporal_load((const u32x4_t*)(urow + b * 64));
    float dg[4], du[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dg[r] = h2f(gd[(size_t)(orow + r) * nb + b]);
      du[r] = h2f(ud[(size_t)(orow + r) * nb + b]);
    }
    cb2_pair_superblock<LO>(cg, cu, bh ? bh + b * QK : nullptr, bl ? bl + b * QK : nullptr, q, dg, du, s_mag, s_sgn,
                            ag, au);
  }
  s_red[wave][0][lane] = ag;
  s_red[wave][1][lane] = au;
  __syncthreads();
  if (wave != 0) return;
  ag = s_red[0][0][lane];
  au = s_red[0][1][lane];
#pragma unroll
  for (int w = 1; w < kGW; ++w) {
    ag += s_red[w][0][lane];
    au += s_red[w][1][lane];
  }
  float psum = 0.0f;
  if (slot >= 0) {
    const float wt = ld_coh(&ro.w[slot]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 hv = (_Float16)(wt * (silu(ag[r]) * au[r]));
      hw16[(int64_t)slot * f + row0 + 4 * q + r] = hv;
      psum += (float)hv;
    }
  }
  psum += __shfl_xor(psum, 16);
  psum += __shfl_xor(psum, 32);
  if (slot >= 0 && q == 0) hsum[(int64_t)slot * (f / 16) + tile] = psum;
  (void)Tp;
}

// One Q2K super-block, lane (i, q) owning sub-blocks 4q..4q+3 of its row.
// rc: row's code block, rs: row's 16 subscale bytes, dd/dm: d and dmin of the
// lane's four output rows, bcol: activation column at the super-block start,
// cs: its 16 sub-block sums (nullptr with bcol).
__device__ inline void q2k_superblock(const uint8_t* rc, const uint8_t* rs, const float* dd, const float* dm,
                                      const _Float16* bcol, const float* cs, int q, float4_t& acc) {
  const u32x4_t codes = __builtin_nontemporal_load((const u32x4_t*)(rc + 16 * q));
  const uint32_t sc4 = *(const uint32_t*)(rs + 4 * q);
  half8_t bv[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) bv[s] = bcol ? *(const half8_t*)(bcol + q2k_boff(q, s)) : zero_half8();
  half8_t am = zero_half8(), bh = zero_half8(), bl = zero_half8();
  if (q < 2) {
    const u32x2_t mb = *(const u32x2_t*)(rs + 8 * q);
    u32x4_t t;
    t.x = nib_hi_pair_f16(mb.x, 0);
    t.y = nib_hi_pair_f16(mb.x, 2);
    t.z = nib_hi_pair_f16(mb.y, 0);
    t.w = nib_hi_pair_f16(mb.y, 2);
    am = as_half8(t);
    if (cs) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = cs[8 * q + e];
        const _Float16 h = (_Float16)v;
        bh[e] = h;
        bl[e] = (_Float16)(v - (float)h);
      }
    }
  }
  float4_t p = {0.f, 0.f, 0.f, 0.f}, pm = p;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const half8_t a = q2k_frag(codes[s >> 1], s & 1, (sc4 >> (8 * (s >> 1))) & 15u);
    p = mfma16x16x32(a, bv[s], p);
  }
  pm = mfma16x16x32(am, bh, pm);
  pm = mfma16x16x32(am, bl, pm);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] += dd[r] * p[r] - dm[r] * pm[r];
}

__global__ __launch_bounds__(kDW * 64) void k_down_decode(
    ds4moe_layer L, int T, const int32_t* __restrict__ ndist, const int32_t* __restrict__ distinct,
    const int32_t* __restrict__ tok_slot, const _Float16* __restrict__ hs16, const _Float16* __restrict__ hw16,
    const float* __restrict__ hsum, int dmax, float* __restrict__ part, int32_t* __restrict__ ctr,
    float* __restrict__ y) {
  __shared__ float4_t s_red[kDW][64];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, fs = L.d_ff_shared;
  const int tile = blockIdx.x, row0 = tile * 16;
  const int src = blockIdx.y;  // < kDnShChunks: shared-expert K chunk; else distinct expert src - kDnShChunks
  const int nd = *ndist;
  const int nsrc = kDnShChunks + nd;
  if (src >= nsrc) return;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (src < kDnShChunks) {
    const int nks = fs / 32;
    const int c0 = src * nks / kDnShChunks, c1 = (src + 1) * nks / kDnShChunks;
    int ks0, ks1;
    split_range(c1 - c0, kDW, wave, ks0, ks1);
    const _Float16* bcol = c < T ? hs16 + (int64_t)c * fs : nullptr;
    float4_t unused = acc;
    f16_tile<false, false>(L.sh_down + (int64_t)(row0 + c) * fs, nullptr, bcol, nullptr, c0 + ks0, c0 + ks1, lane,
                           acc, unused);
  } else {
    const int i = src - kDnShChunks;
    const int e = distinct[i];
    const int slot = tok_slot[i * kDecodeGroup + c];
    const _Float16* bcol = slot >= 0 ? hw16 + (int64_t)slot * f : nullptr;
    const float* cs = slot >= 0 ? hsum + (int64_t)slot * (f / 16) : nullptr;
    const int nb = f / QK;
    const size_t mb = (size_t)d * nb;
    const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mb * 84;
    const uint8_t* rcodes = base + (size_t)(row0 + c) * nb * 64;
    const uint8_t* rsub = base + mb * 64 + (size_t)(row0 + c) * nb * 16;
    const uint16_t* sup = (const uint16_t*)(base + mb * 80);
    int sb0, sb1;
    split_range(nb, kDW, wave, sb0, sb1);
    for (int b = sb0; b < sb1; ++b) {
      float dd[4], dm[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t pr = *(const uint32_t*)(sup + ((size_t)(row0 + 4 * q + r) * nb + b) * 2);
        dd[r] = h2f((uint16_t)(pr & 0xFFFFu));
        dm[r] = h2f((uint16_t)(pr >> 16));
      }
      q2k_superblock(rcodes + b * 64, rsub + b * 16, dd, dm, bcol ? bcol + b * QK : nullptr, cs ? cs + b * 16 : nullptr,
                     q, acc);
    }
  }
  s_red[wave][lane] = acc;
  __syncthreads();
  const int Tp = min(T, kDecodeGroup);
  float* tile_part = part + ((size_t)tile * (kDnShChunks + dmax)) * 16 * Tp;
  if (wave == 0) {
    acc = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < kDW; ++w) acc += s_red[w][lane];
    if (c < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st_coh(&tile_part[((size_t)src * 16 + 4 * q + r) * Tp + c], acc[r]);
    }
    wait_stores();
  }
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(&ctr[tile], 1) == nsrc - 1;
  __syncthreads();
  if (!s_last || wave != 0 || c >= T) return;
  float4_t sum = {0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < nsrc; ++s2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += ld_coh(&tile_part[((size_t)s2 * 16 + 4 * q + r) * Tp + c]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) y[(int64_t)c * d + row0 + 4 * q + r] = sum[r];
}

hipError_t launch_decode_experts(const Fwd& f) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  const int maxd = std::min(L.n_experts, T * L.top_k);
  const int nsh = L.d_ff_shared / 16, nr = L.d_ff / 16;
  const dim3 gu(1 + nsh * kShChunks + maxd * nr);
  auto xh = (const _Float16*)(ws + y.x_hi);
  auto xl = f.lo ? (const _Float16*)(ws + y.x_lo) : nullptr;
  auto plog = (const float*)(ws + y.plog);
  auto ctrl = (int32_t*)(ws + y.ctrl);
  auto sh_part = (float*)(ws + y.sh_part);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (float*)(ws + y.hsum);
  const RouteOut ro = route_out(f);
  if (f.lo)
    DS4_LAUNCH(k_gateup_decode<true>, gu, dim3(kGW * 64), 0, f.st, L, T, plog, ro, xh, xl, ctrl, sh_part, hs16, hw16,
               hsum);
  else
    DS4_LAUNCH(k_gateup_decode<false>, gu, dim3(kGW * 64), 0, f.st, L, T, plog, ro, xh, xl, ctrl, sh_part, hs16, hw16,
               hsum);
  const int dmax = std::min(L.n_experts, std::min(T, kDecodeGroup) * L.top_k);
  DS4_LAUNCH(k_down_decode, dim3(L.d_model / 16, kDnShChunks + maxd), dim3(kDW * 64), 0, f.st, L, T, ro.ndist,
             ro.distinct, ro.tok_slot, hs16, hw16, hsum, dmax, (float*)(ws + y.dn_part),
             ctrl + 1 + L.d_ff_shared / 16, f.y);
  return hipGetLastError();
}

}  // namespace ds4
