// Top-k selection, gate weights and token grouping, shared by the routing
// kernels.  Reading of the pages (DS4 (DwarfStar 4) wiki note, "Architecture":
// an F16 router picks 6 of 256 experts): the k largest logits win, equal
// logits go to the lower expert index, a token's experts are listed in
// ascending index, and their weights are the softmax of their logits.
#pragma once

#include "common.h"
#include "internal.h"

namespace ds4 {

// One wave selects the k largest of E logits l[0..E) (lane owns
// e = lane + 64 i) and leaves the chosen indices/values in sel_e/sel_v in
// selection order.
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
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
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
    const int e = sel_e[a];
    const float v = sel_v[a];
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

// Block-wide exclusive scan of one int per thread (blockDim a multiple of
// 64, at most 1024); returns the thread's exclusive prefix and the total.
__device__ inline int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
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

// Everything routing writes for one decode group (T <= 16 tokens).
struct RouteOut {
  float* logits;  // [T, E] (scratch)
  int32_t *idx, *idx_out;
  float *w, *w_out;
  int32_t *counts, *offsets, *perm, *inv;
  int32_t *counts_out, *offsets_out, *perm_out;
  int32_t *ndist, *distinct, *tok_slot;  // distinct experts, slot of token t in distinct[i] at [i*16 + t]
};

// Run by a whole block (any multiple of 64 threads up to 1024): logits =
// sum of nparts partial rows plog[p][t][e] (+ bias), top-k and softmax per
// token, then counts, offsets, perm (slots t*k + j by expert, then token),
// inv, and the distinct-expert table.
__device__ inline void route_finish_block(const float* __restrict__ plog, int nparts, const float* __restrict__ bias,
                                          int E, int k, int T, const RouteOut& o) {
  __shared__ int s_sel_e[16][kMaxTopK];
  __shared__ float s_sel_v[16][kMaxTopK];
  __shared__ int s_idx[kDecodeGroup * kMaxTopK];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_dpos[kMaxExperts];
  __shared__ int s_tmp[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6, nthr = blockDim.x;
  for (int e = threadIdx.x; e < E; e += nthr) s_cnt[e] = 0;
  for (int i = threadIdx.x; i < T * E; i += nthr) {
    const int e = i % E;
    float a = 0.0f;
#pragma unroll 8
    for (int p = 0; p < nparts; ++p) a += plog[(int64_t)p * T * E + i];
    o.logits[i] = bias ? a + bias[e] : a;
  }
  __syncthreads();
  for (int t = wave; t < T; t += nwaves) {
    wave_topk(o.logits + (int64_t)t * E, E, k, lane, s_sel_e[wave], s_sel_v[wave]);
    if (lane == 0) {
      finish_token(s_sel_e[wave], s_sel_v[wave], k, t, o.idx, o.w, o.idx_out, o.w_out);
      for (int j = 0; j < k; ++j) s_idx[t * k + j] = s_sel_e[wave][j];
    }
  }
  __syncthreads();
  const int S = T * k;
  for (int s = threadIdx.x; s < S; s += nthr) atomicAdd(&s_cnt[s_idx[s]], 1);
  __syncthreads();
  const int EPT = (E + nthr - 1) / nthr;  // consecutive experts per thread
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
      o.counts[e] = s_cnt[e];
      o.offsets[e] = cpre;
      if (o.counts_out) o.counts_out[e] = s_cnt[e];
      if (o.offsets_out) o.offsets_out[e] = cpre;
      if (s_cnt[e] > 0) o.distinct[dpre] = e;
      cpre += s_cnt[e];
      dpre += s_cnt[e] > 0;
    }
  }
  if (threadIdx.x == 0) {
    o.offsets[E] = ctot;
    if (o.offsets_out) o.offsets_out[E] = ctot;
    *o.ndist = dtot;
  }
  for (int i = threadIdx.x; i < dtot * kDecodeGroup; i += nthr) o.tok_slot[i] = -1;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += nthr) {
    const int e = s_idx[s], t = s / k;
    int rank = 0;
    for (int u = 0; u < t; ++u)
      for (int j = 0; j < k; ++j) rank += s_idx[u * k + j] == e;
    const int pos = s_off[e] + rank;
    o.perm[pos] = s;
    o.inv[s] = pos;
    if (o.perm_out) o.perm_out[pos] = s;
    o.tok_slot[s_dpos[e] * kDecodeGroup + t] = s;
  }
}

inline RouteOut route_out(const Fwd& f) {
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  RouteOut o;
  o.logits = (float*)(ws + y.logits);
  o.idx = (int32_t*)(ws + y.topk_idx);
  o.idx_out = f.idx_out;
  o.w = (float*)(ws + y.topk_w);
  o.w_out = f.w_out;
  o.counts = (int32_t*)(ws + y.counts);
  o.offsets = (int32_t*)(ws + y.offsets);
  o.perm = (int32_t*)(ws + y.perm);
  o.inv = (int32_t*)(ws + y.inv);
  o.counts_out = f.counts_out;
  o.offsets_out = f.offsets_out;
  o.perm_out = f.perm_out;
  o.ndist = (int32_t*)(ws + y.ndist);
  o.distinct = (int32_t*)(ws + y.distinct);
  o.tok_slot = (int32_t*)(ws + y.tok_slot);
  return o;
}

// Coherent (device-scope) loads of data another block wrote in the same
// kernel, after observing its release.
__device__ inline int ld_acq_int(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
// Write-through (device-coherent) store for data handed to another block of
// the same kernel; a writer waits for its coherent stores to complete
// (wait_stores) before the counter that publishes them is incremented, so no
// L2 write-back is needed.
__device__ inline void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace ds4
