// Top-k selection, gate weights and token grouping, shared by the routing
// kernels.  Reading of the pages (DS4 (DwarfStar 4) wiki note, "Architecture":
// an F16 router picks 6 of 256 experts): the k largest logits win, equal
// logits go to the lower expert index, a token's experts are listed in
// ascending index, and their weights are the softmax of their logits.
#pragma once

#include "common.h"
#include "internal.h"

namespace ds4 {

// Order-preserving map of a float to a u32 key: a > b  <=>  key(a) > key(b)
// for non-NaN values, and a == b  <=>  key(a) == key(b) (-0 is keyed as +0).
__device__ inline uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects the k largest of E logits l[0..E) (lane owns
// e = lane + 64 i, i < PER, PER * 64 >= E), equal logits going to the lower
// expert index, and writes the chosen experts and logits to sel_e/sel_v in
// ascending expert order.  The k-th largest key is found bit by bit from the
// top: a candidate threshold is kept when at least k keys reach it.  Counting
// uses only ballots and popcounts, so no data crosses lanes, and every step
// is straight-line code.  Slots past E get key 0, which no candidate (>= 1)
// admits; k <= E guarantees k real keys.
// NT tokens at once (logits lp(t); outputs ep(t), vp(t)): the tokens'
// selections are independent, so their ballot and popcount chains overlap.
template <int PER, int NT, typename LP, typename EP, typename VP>
__device__ inline void wave_select_n(LP lp, EP ep, VP vp, int E, int k, int lane) {
  float v[NT][PER];
  uint32_t key[NT][PER];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      v[t][i] = lp(t)[e < E ? e : E - 1];
    }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < PER; ++i) key[t][i] = lane + 64 * i < E ? order_key(v[t][i]) : 0u;
  uint32_t thr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) thr[t] = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t cand = thr[t] | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(key[t][i] >= cand));
      thr[t] = cnt >= k ? cand : thr[t];
    }
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes under this one
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int gt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) gt += __popcll(__ballot(key[t][i] > thr[t]));
    const int need_eq = k - gt;  // keys equal to the threshold still to take, lowest index first
    int eq_before = 0, pos0 = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool eq = key[t][i] == thr[t];
      const uint64_t eqm = __ballot(eq);
      const bool sel = key[t][i] > thr[t] || (eq && eq_before + __popcll(eqm & below) < need_eq);
      eq_before += __popcll(eqm);
      const uint64_t sm = __ballot(sel);
      if (sel) {
        const int pos = pos0 + __popcll(sm & below);
        ep(t)[pos] = lane + 64 * i;
        vp(t)[pos] = v[t][i];
      }
      pos0 += __popcll(sm);
    }
  }
}

template <int NT, typename LP, typename EP, typename VP>
__device__ inline void wave_select_t(LP lp, EP ep, VP vp, int E, int k, int lane) {
  if (E <= 256)
    wave_select_n<4, NT>(lp, ep, vp, E, k, lane);
  else if (E <= 512)
    wave_select_n<8, NT>(lp, ep, vp, E, k, lane);
  else
    wave_select_n<16, NT>(lp, ep, vp, E, k, lane);
}

__device__ inline void wave_select(const float* l, int E, int k, int lane, int* sel_e, float* sel_v) {
  wave_select_t<1>([&](int) { return l; }, [&](int) { return sel_e; }, [&](int) { return sel_v; }, E, k, lane);
}

// Gate weight of selected slot j: softmax over the k selected logits,
// shifted by their maximum, with the denominator summed in slot order.
__device__ inline float gate_weight(const float* sel_v, int k, int j) {
  float vmax = sel_v[0];
  for (int a = 1; a < k; ++a) vmax = fmaxf(vmax, sel_v[a]);
  float den = 0.0f;
  for (int a = 0; a < k; ++a) den += __expf(sel_v[a] - vmax);
  return __expf(sel_v[j] - vmax) / den;
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

// LDS of route_finish_block (a struct so kernels can place it beside the
// LDS of their other block roles).
// LDS of the routing finish, NL logits kept in LDS: 1024 for one token (a
// small footprint for the launch the single-token step waits on), 4096 for a
// group (16 tokens of 256 experts).
template <int NL>
struct RouteLdsN {
  float logit[NL];                      // logits when T * E <= NL (else the workspace copy)
  int sel_e[kDecodeGroup][kMaxTopK];    // per token: chosen experts, ascending
  float sel_v[kDecodeGroup][kMaxTopK];  // their logits
  int fe[kDecodeGroup * kMaxTopK];      // expert of slot s = t * k + j
  uint32_t tokm[kMaxExperts];           // bit t: token t chose expert e
  uint32_t selm[kMaxExperts / 32];      // bit e: some token chose expert e
  int selpre[kMaxExperts / 32 + 1];     // chosen experts below word w of selm
  int dist[kDecodeGroup * kMaxTopK];    // distinct experts, ascending
  int wsel[16];                         // one token: chosen experts per wave
  int off[kMaxExperts];                 // per expert: slots of lower experts
  int scan[16];                         // block scan: one total per wave
};
using RouteLdsOne = RouteLdsN<1024>;
using RouteLdsGroup = RouteLdsN<4096>;

// Number of experts below e that some token chose (e's distinct position).
template <typename RL>
__device__ inline int distinct_below(const RL& R, int e) {
  return R.selpre[e >> 5] + __popc(R.selm[e >> 5] & ((1u << (e & 31)) - 1u));
}

// One key per lane: flags the k largest valid keys, equal keys going to the
// lower lane; every valid lane is flagged when fewer than k are valid.  The
// k-th largest key is found bit by bit with ballots (valid order keys are
// never 0).
__device__ inline bool wave_top_flags(uint32_t key, bool valid, int k, int lane) {
  key = valid ? key : 0u;
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    thr = __popcll(__ballot(key >= cand)) >= k ? cand : thr;
  }
  const int need_eq = k - __popcll(__ballot(key > thr));
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const bool eq = valid && key == thr;
  return key > thr || (eq && __popcll(__ballot(eq) & below) < need_eq);
}

// One token (T = 1, E <= 64 * waves, waves * k <= 64): each wave flags the k
// largest logits of its 64 experts, wave 0 then flags the k largest of those
// candidates.  Lane order is expert order at both levels, so ties go to the
// lower expert index and the winners, compacted by ballot, come out in
// ascending expert order.  With one token, slot j holds the j-th chosen
// expert, so perm and inv are the identity.  logits are filled and the block
// has passed a barrier.
template <typename RL>
__device__ inline void route_finish_one(RL& R, const float* logits, int E, int k, const RouteOut& o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int e = threadIdx.x;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int* cand_e = R.fe;              // [nwaves][k] candidates, ascending within a wave
  int* cand_n = R.wsel;            // candidates per wave
  {
    const bool f = wave_top_flags(e < E ? order_key(logits[e]) : 0u, e < E, k, lane);
    const uint64_t fm = __ballot(f);
    if (f) cand_e[wave * k + __popcll(fm & below)] = e;
    if (lane == 0) cand_n[wave] = __popcll(fm);
  }
  __syncthreads();
  if (wave == 0) {
    const int w = lane / k, j = lane - w * k;
    const bool valid = w < nwaves && j < cand_n[w];
    const int ce = valid ? cand_e[lane] : 0;
    const float cv = valid ? logits[ce] : 0.0f;
    const bool f = wave_top_flags(order_key(cv), valid, k, lane);
    const uint64_t fm = __ballot(f);
    if (f) {
      const int pos = __popcll(fm & below);
      R.sel_e[0][pos] = ce;
      R.sel_v[0][pos] = cv;
      atomicOr(&R.selm[ce >> 5], 1u << (ce & 31));
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
      const int ej = R.sel_e[0][lane];
      float vmax = R.sel_v[0][0];
      for (int a = 1; a < k; ++a) vmax = fmaxf(vmax, R.sel_v[0][a]);
      float den = 0.0f;  // summed in slot order, as in gate_weight
      for (int a = 0; a < k; ++a) den += __expf(R.sel_v[0][a] - vmax);
      const float wj = __expf(R.sel_v[0][lane] - vmax) / den;
      o.idx[lane] = ej;
      o.w[lane] = wj;
      if (o.idx_out) o.idx_out[lane] = ej;
      if (o.w_out) o.w_out[lane] = wj;
      o.perm[lane] = lane;
      o.inv[lane] = lane;
      if (o.perm_out) o.perm_out[lane] = lane;
      o.distinct[lane] = ej;
    }
    if (lane == 0) {
      o.offsets[E] = k;
      if (o.offsets_out) o.offsets_out[E] = k;
      *o.ndist = k;
    }
  }
  __syncthreads();
  if (e < E) {  // counts and offsets from the chosen-expert bitmask
    const uint32_t wd = R.selm[e >> 5];
    const int c = (wd >> (e & 31)) & 1u;
    int off = __popc(wd & ((1u << (e & 31)) - 1u));
    for (int w = 0; w < (e >> 5); ++w) off += __popc(R.selm[w]);
    o.counts[e] = c;
    o.offsets[e] = off;
    if (o.counts_out) o.counts_out[e] = c;
    if (o.offsets_out) o.offsets_out[e] = off;
  }
  for (int i = threadIdx.x; i < k * kDecodeGroup; i += blockDim.x)
    o.tok_slot[i] = (i % kDecodeGroup) == 0 ? i / kDecodeGroup : -1;
}

// Run by a whole block (any multiple of 64 threads up to 1024), T <= 16
// (so S = T * k <= 256): logits = sum of nparts partial rows plog[p][t][e]
// (+ bias), top-k and gate weights per token, then counts, offsets, perm
// (slots t*k + j by expert, then token), inv, and the distinct-expert table.
// COH: the partials were written by other blocks of the running kernel (read
// them with coherent loads).
// KLF: logits a thread sums at a time; above 1 the selection also runs two
// tokens per wave at once (1 keeps the one-token finish's register
// footprint).
template <bool COH = false, int KLF = 4, typename RL>
__device__ inline void route_finish_block(RL& R, const float* __restrict__ plog, int nparts,
                                          const float* __restrict__ bias, int E, int k, int T, const RouteOut& o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6, nthr = blockDim.x;
  const int S = T * k;
  for (int e = threadIdx.x; e < E; e += nthr) R.tokm[e] = 0u;
  for (int w = threadIdx.x; w < (E + 31) / 32; w += nthr) R.selm[w] = 0u;
  // logits in LDS when they fit, else in memory.  The stores and the
  // one-token finish name the array itself: through a pointer that may be
  // either, the compiler emits flat accesses, slower than LDS ones on this
  // latency-bound chain.
  const bool in_lds = T * E <= (int)(sizeof(R.logit) / sizeof(float));
  float* logits = in_lds ? R.logit : o.logits;
  // kLf logits per thread at a time, kPb partials each, all loads in flight
  // before the first add (a loop that waits for each load, or for each
  // logit's loads, would pay one memory round trip per partial or per
  // logit); each logit summed in ascending p
  constexpr int kLf = KLF, kPb = KLF > 1 ? 8 : 16;
  const int n = T * E;
  for (int i0 = threadIdx.x; i0 < n; i0 += kLf * nthr) {
    float a[kLf];
#pragma unroll
    for (int u = 0; u < kLf; ++u) a[u] = 0.0f;
    for (int p0 = 0; p0 < nparts; p0 += kPb) {
      float v[kLf][kPb];
#pragma unroll
      for (int u = 0; u < kLf; ++u) {
        const int i = i0 + u * nthr;
#pragma unroll
        for (int j = 0; j < kPb; ++j) {
          if (i < n && p0 + j < nparts) {
            const float* src = plog + (int64_t)(p0 + j) * n + i;
            v[u][j] = COH ? __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *src;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kLf; ++u)
#pragma unroll
        for (int j = 0; j < kPb; ++j)
          if (i0 + u * nthr < n && p0 + j < nparts) a[u] += v[u][j];
    }
#pragma unroll
    for (int u = 0; u < kLf; ++u) {
      const int i = i0 + u * nthr;
      if (i < n) {
        const float lg = bias ? a[u] + bias[i % E] : a[u];
        if (in_lds) R.logit[i] = lg;
        else o.logits[i] = lg;
      }
    }
  }
  __syncthreads();
  if (T == 1 && in_lds && E <= 64 * nwaves && nwaves * k <= 64) {
    route_finish_one(R, R.logit, E, k, o);
    return;
  }
  if constexpr (KLF > 1) {
    // tokens two at a time per wave (t and t + nwaves), one when it is the last
    for (int t = wave; t < T; t += 2 * nwaves) {
      if (t + nwaves < T && E <= 512) {  // (past 512 experts two tokens' keys outgrow the registers)
        const int tt[2] = {t, t + nwaves};
        const auto lp = [&](int u) { return logits + (int64_t)tt[u] * E; };
        const auto ep = [&](int u) { return R.sel_e[tt[u]]; };
        const auto vp = [&](int u) { return R.sel_v[tt[u]]; };
        if (E <= 256) wave_select_n<4, 2>(lp, ep, vp, E, k, lane);
        else wave_select_n<8, 2>(lp, ep, vp, E, k, lane);
      } else if (t + nwaves < T) {
        wave_select(logits + (int64_t)t * E, E, k, lane, R.sel_e[t], R.sel_v[t]);
        wave_select(logits + (int64_t)(t + nwaves) * E, E, k, lane, R.sel_e[t + nwaves], R.sel_v[t + nwaves]);
      } else {
        wave_select(logits + (int64_t)t * E, E, k, lane, R.sel_e[t], R.sel_v[t]);
      }
    }
  } else {
    for (int t = wave; t < T; t += nwaves) wave_select(logits + (int64_t)t * E, E, k, lane, R.sel_e[t], R.sel_v[t]);
  }
  __syncthreads();
  // per slot: gate weight, and the expert/token bitmaps
  for (int s = threadIdx.x; s < S; s += nthr) {
    const int t = s / k, j = s - t * k;
    const int e = R.sel_e[t][j];
    const float wj = gate_weight(R.sel_v[t], k, j);
    o.idx[s] = e;
    o.w[s] = wj;
    if (o.idx_out) o.idx_out[s] = e;
    if (o.w_out) o.w_out[s] = wj;
    R.fe[s] = e;
    atomicOr(&R.tokm[e], 1u << t);
    atomicOr(&R.selm[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // prefix counts of chosen experts per 32-expert word
    int n = 0;
    for (int w = 0; w <= (E + 31) / 32; ++w) {
      R.selpre[w] = n;
      if (w < (E + 31) / 32) n += __popc(R.selm[w]);
    }
  }
  __syncthreads();
  // per expert: count, offset (the selected slots of lower experts: an
  // exclusive scan of the counts, in chunks of the block's threads), and the
  // distinct table
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += nthr) {  // uniform trip count: every thread scans
    const int e = e0 + (int)threadIdx.x;
    const int c = e < E ? __popc(R.tokm[e]) : 0;
    int tot;
    const int off = base + block_excl_scan(c, R.scan, &tot);
    base += tot;
    if (e < E) {
      R.off[e] = off;
      o.counts[e] = c;
      o.offsets[e] = off;
      if (o.counts_out) o.counts_out[e] = c;
      if (o.offsets_out) o.offsets_out[e] = off;
      if (c > 0) {
        const int dp = distinct_below(R, e);
        o.distinct[dp] = e;
        R.dist[dp] = e;
      }
    }
  }
  if (threadIdx.x == 0) {
    o.offsets[E] = S;
    if (o.offsets_out) o.offsets_out[E] = S;
    *o.ndist = R.selpre[(E + 31) / 32];
  }
  __syncthreads();
  // per slot: position in the expert-major order
  for (int s = threadIdx.x; s < S; s += nthr) {
    const int t = s / k;
    const int e = R.fe[s];
    const int pos = R.off[e] + __popc(R.tokm[e] & ((1u << t) - 1u));  // earlier tokens of expert e
    o.perm[pos] = s;
    o.inv[s] = pos;
    if (o.perm_out) o.perm_out[pos] = s;
  }
  // per (distinct expert, token): its slot, or -1
  const int nd = R.selpre[(E + 31) / 32];
  for (int i = threadIdx.x; i < nd * kDecodeGroup; i += nthr) {
    const int di = i / kDecodeGroup, t = i % kDecodeGroup;
    const int e = R.dist[di];
    int slot = -1;
    if (t < T && ((R.tokm[e] >> t) & 1u)) {
      int j = 0;
      while (R.sel_e[t][j] != e) ++j;  // e is among token t's k experts
      slot = t * k + j;
    }
    o.tok_slot[i] = slot;
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


}  // namespace ds4
