// Batched decode (T <= 16 tokens per group): the whole layer in three
// streaming kernels whose 16 MFMA columns are the group's tokens.  Routing
// gates the routed experts; the F16 shared expert (independent of it)
// streams beside the routed work of stages 2 and 3:
//
//   k_dec_stage1  router partial logits per input chunk; the last router
//                 block to arrive finishes routing (top-k, gate weights,
//                 grouping).  x is read in its input type; the router chunk
//                 owners keep the binary16 copy for stage 2.
//   k_dec_stage2  for every distinct selected expert its gate/up tiles:
//                 w * silu(G x) * (U x) as binary16 plus the sums over each
//                 16 rows (one Q2K sub-block of the down input) as binary16
//                 hi/lo; behind them the shared expert's gate and up, two
//                 blocks per 16 rows, the second of which forms
//                 h = silu(g) * u as binary16.
//   k_dec_stage3  one block per 16 output rows: the shared expert's down
//                 product for those rows (an F16 stream that overlaps the
//                 routed decode arithmetic) and every distinct expert's down
//                 super-blocks; it writes y = ys + the routed terms and clears
//                 the earlier stages' arrival counters.  One token takes the
//                 dot-product form k_dec_stage3_one.
// Each distinct expert is read once per call however many tokens chose it,
// and results do not depend on block scheduling.  Blocks hand partials to
// the last arriver (router logits, shared gate/up tiles) with
// device-coherent (sc1) stores and loads around an atomic counter, which
// needs no L2 write-back.
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
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "ring.h"
#include "routefin.h"
#include "tiles.h"
#include "trace.h"

namespace ds4 {

__constant__ GridTables c_dec_tables = make_grid_tables();

constexpr int kW = 4;           // waves per block
constexpr int kStageHalves = 4096;        // binary16 activations a stage-1/2 block may stage (per hi/lo part)
constexpr int kStageHalvesGroup = 16384;  // the same for a group of tokens (T d <= 16384: 4 tokens of 4096)
// Stage 3 LDS for staged activations and sums (dynamic, beside 32 KB of
// static reduction buffers within the CU's 160 KB; one 16-wave block per
// CU): T = 1 (MXFP4, Q4K) and groups up to T = 4 at the decode1 layer shape.
constexpr size_t kStage3Bytes = 128 * 1024;
constexpr size_t kStage3OneBytes = 40 * 1024;  // the same for the one-token form

__device__ inline int cb2_boff(int q, int s) { return 32 * (2 * q + (s >> 2)) + 8 * (s & 3); }
__device__ inline int q2k_boff(int q, int s) { return 16 * (4 * q + (s >> 1)) + 8 * (s & 1); }

// Decode's h keeps each 16-row sub-block pair-interleaved for the Q2K down
// product: row r of the sub-block is stored at q2k_pair_pos(r), i.e. in the
// order 0, 8, 1, 9, ..., 7, 15, so binary16 pair i of the activations holds
// rows i and i + 8, the two codes of weight pair i.
__host__ __device__ constexpr int q2k_pair_pos(int r) { return 2 * (r & 7) + (r >> 3); }

__device__ inline int clamp_index(int v, int n) { return (unsigned)v < (unsigned)n ? v : 0; }

// 8 activations x[t][k0 .. k0+7] (bf16 bits or fp32), loaded (load_x8_raw)
// and turned into binary16 hi and lo parts (cvt_x8) as separate steps.
struct X8Raw {
  u32x4_t u;    // bf16
  float4 a, b;  // fp32
};
template <bool LO>
__device__ inline X8Raw load_x8_raw(const void* x, int d, int t, int k0) {
  X8Raw r;
  if (!LO) {
    r.u = *(const u32x4_t*)((const uint16_t*)x + (int64_t)t * d + k0);
  } else {
    const float4* src = (const float4*)((const float*)x + (int64_t)t * d + k0);
    r.a = src[0];
    r.b = src[1];
  }
  return r;
}
template <bool LO>
__device__ inline void cvt_x8(const X8Raw& r, half8_t& h, half8_t& l) {
  float v[8];
  if (!LO) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      v[2 * p] = __builtin_bit_cast(float, r.u[p] << 16);
      v[2 * p + 1] = __builtin_bit_cast(float, r.u[p] & 0xFFFF0000u);
    }
  } else {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (_Float16)v[e];
    l[e] = LO ? (_Float16)(v[e] - (float)h[e]) : (_Float16)0.0f;
  }
}
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

// Rows of the tokens in tmask (bit t: token t; wave-uniform), ascending,
// into consecutive LDS rows of stride st: 256 halves each from src + t ld,
// one wave instruction a row (lanes 0..31).
__device__ inline void dma_token_rows(const _Float16* src, int ld, uint32_t tmask, _Float16* dst, int st, int lane) {
  int r = 0;
  for (uint32_t m = tmask; m != 0u; m &= m - 1u, ++r) {
    const int t = __builtin_ctz(m);
    if (lane < QK / 8)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + (int64_t)t * ld + lane * 8),
                                       (__attribute__((address_space(3))) void*)(dst + r * st), 16, 0, 0);
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

// ============================================================== stage 1
template <bool GRP>
struct Stage1Lds {
  std::conditional_t<GRP, RouteLdsGroup, RouteLdsOne> route;
  float4_t red[kW][64];
  int last;
};


// inputs per router block: 512, or 256 when d is an odd multiple of 256
__host__ __device__ inline int router_chunk(int d) { return d % 512 == 0 ? 512 : 256; }

// F16 rows (the lane's A row) x K-steps [ks0, ks1) of one staged or global
// activation set, accumulated into acc.  a[]: the first kBatch steps,
// loaded by the caller; later batches load here.
// TRANS: the weights are the MFMA's B operand, so a lane's four outputs are
// tokens 4q..4q+3 of its own row (otherwise rows 4q..4q+3 of its column).
template <bool LO, bool BL, int kBatch, typename GetB, bool TRANS = false>
__device__ inline void f16_steps(const uint16_t* __restrict__ rowp, int ks0, int ks1, int q, half8_t (&a)[kBatch],
                                 GetB getb, float4_t& acc) {
  for (int ks = ks0; ks < ks1; ks += kBatch) {
    if (ks != ks0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) a[j] = *(const half8_t*)(rowp + max(min(ks + j, ks1 - 1), 0) * 32 + 8 * q);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // steps past the range multiply a zero A fragment
      const int ksj = max(min(ks + j, ks1 - 1), 0);
      const half8_t aj = ks + j < ks1 ? a[j] : zero_half8();
      half8_t bh, bl;
      getb(ksj * 32 + 8 * q, bh, bl);
      acc = TRANS ? mfma16x16x32(bh, aj, acc) : mfma16x16x32(aj, bh, acc);
      if (LO) acc = TRANS ? mfma16x16x32(bl, aj, acc) : mfma16x16x32(aj, bl, acc);
    }
  }
}

// Shared expert gate and up, block sb = (tile, part, half): part 0 is the
// gate, part 1 the up product of 16 rows, over input part `half` of KS;
// the last of a tile's 2 KS blocks to arrive forms h = silu(g) * u as
// binary16.  It does not depend on routing: for a group of tokens these
// blocks run beside the router's (XR: x read as the input itself and
// turned into binary16 hi/lo parts as the router's blocks do); for one
// token behind the routed gate/up blocks, whose stream they overlap best (x
// as the binary16 copy xh, xl the router wrote, staged in LDS (bhs, bls)
// when BL).  KS = kShSplit: a wave's K-steps are one batch of loads at
// d_model 4096.  red: the wave reduction, last: one LDS int.
template <bool LO, bool BL, bool XR, int KS>
__device__ inline void shared_gateup_block(const ds4moe_layer& L, int T, const void* __restrict__ x,
                                           const _Float16* __restrict__ xh, const _Float16* __restrict__ xl, int sb,
                                           float* __restrict__ gu_part, _Float16* __restrict__ hs16,
                                           int32_t* __restrict__ ctrl, _Float16* bhs, _Float16* bls,
                                           float4_t (*red)[64], int& last) {
  static_assert(KS <= kShSplit && !(XR && BL), "shared gate/up block form");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);  // token feeding MFMA column c
  const int d = L.d_model, fs = L.d_ff_shared;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int tile = sb / (2 * KS), part = (sb / KS) & 1, half = sb % KS;
  const uint16_t* rp = (part == 0 ? L.sh_gate : L.sh_up) + (int64_t)(tile * 16 + c) * d;
  const int nks = d / 32 / KS;  // K-steps of one part
  int ks0, ks1;
  split_range(nks, kW, wave, ks0, ks1);
  ks0 += half * nks;
  ks1 += half * nks;
  if constexpr (!XR) {
    const int st = stage_stride(d);
    if (BL) dma_rows(xh, d, T, d, bhs, st, wave, kW, lane);
    if (BL && LO) dma_rows(xl, d, T, d, bls, st, wave, kW, lane);
    constexpr int kBatch = 16;
    half8_t a[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) a[j] = *(const half8_t*)(rp + max(min(ks0 + j, ks1 - 1), 0) * 32 + 8 * q);
    if (BL) {
      wait_all();
      __syncthreads();
    }
    f16_steps<LO, BL, kBatch>(rp, ks0, ks1, q, a,
                              [&](int kk, half8_t& bh, half8_t& bl) {
                                if (BL) {
                                  bh = *(const half8_t*)(bhs + tc * st + kk);
                                  if (LO) bl = *(const half8_t*)(bls + tc * st + kk);
                                } else {
                                  bh = *(const half8_t*)(xh + (int64_t)tc * d + kk);
                                  if (LO) bl = *(const half8_t*)(xl + (int64_t)tc * d + kk);
                                }
                              },
                              acc);
  }
  // XR: batches of kBatch K-steps, the weights and the raw x of a batch
  // requested together and waited for once (an x read at its step would
  // wait behind every weight load requested before it)
  constexpr int kBatch = 8;
  for (int ks = ks0; XR && ks < ks1; ks += kBatch) {
    half8_t a[kBatch];
    X8Raw xr[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int kk = max(min(ks + j, ks1 - 1), 0) * 32 + 8 * q;
      a[j] = *(const half8_t*)(rp + kk);
      xr[j] = load_x8_raw<LO>(x, d, tc, kk);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // steps past the range multiply a zero A fragment
      half8_t bh, bl;
      cvt_x8<LO>(xr[j], bh, bl);
      const half8_t aj = ks + j < ks1 ? a[j] : zero_half8();
      acc = mfma16x16x32(aj, bh, acc);
      if (LO) acc = mfma16x16x32(aj, bl, acc);
    }
  }
  acc = reduce_waves<kW>(acc, red, wave, lane);
  float* tp = gu_part + (size_t)tile * 2 * KS * 16 * T;  // [part][half][row][t]
  if (wave == 0) {
    if (c < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st_coh(&tp[((size_t)(part * KS + half) * 16 + 4 * q + r) * T + c], acc[r]);
    }
    wait_stores();
  }
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(&ctrl[1 + tile], 1) == 2 * KS - 1;
  __syncthreads();
  if (!last || wave != 0) return;
  if (c < T) {
    float pv[2][KS][4];  // [part][half][r]: every coherent load in flight before the first use
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int hf = 0; hf < KS; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[pt][hf][r] = ld_coh(&tp[((size_t)(pt * KS + hf) * 16 + 4 * q + r) * T + c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float g = pv[0][0][r], u = pv[1][0][r];
#pragma unroll
      for (int hf = 1; hf < KS; ++hf) {
        g += pv[0][hf][r];
        u += pv[1][hf][r];
      }
      hs16[(int64_t)c * fs + tile * 16 + 4 * q + r] = (_Float16)(silu(g) * u);
    }
  }
  if (lane == 0) ctrl[1 + tile] = 0;
}

// One block per (expert tile, input chunk) of the router, chunk-major; the
// last block to arrive finishes routing.  GRP: a group of tokens (T >= 2),
// whose finish keeps 4096 logits in LDS and sums eight logits' partials at
// a time (KLF; 16 for large groups, whose partials then all go out in one
// pass at the cost of the kernel's register budget); one token keeps the
// smaller footprint.  With GRP, blocks from rblocks on are the shared
// expert's gate/up blocks.
template <bool LO, bool GRP, int KLF = GRP ? 8 : 1>
__global__ __launch_bounds__(kW * 64) void k_dec_stage1(ds4moe_layer L, int T, const void* __restrict__ x,
                                                        int rblocks, float* __restrict__ plog, RouteOut ro,
                                                        _Float16* __restrict__ xh, _Float16* __restrict__ xl,
                                                        float* __restrict__ gu_part, _Float16* __restrict__ hs16,
                                                        int32_t* __restrict__ ctrl) {
  __shared__ Stage1Lds<GRP> lds;
  if (GRP && (int)blockIdx.x >= rblocks) {
    shared_gateup_block<LO, false, true, kShSplit>(L, T, x, nullptr, nullptr, blockIdx.x - rblocks, gu_part, hs16,
                                                   ctrl, nullptr, nullptr, lds.red, lds.last);
    return;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);  // token feeding MFMA column c
  const int d = L.d_model, E = L.n_experts;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  {  // ---------------- router partial logits
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
        if (et == 0 && c < T) {  // binary16 copy of x for stage 2
          const int k0 = (kc * (ck / 32) + wave * spw + h) * 32 + 8 * q;
          *(half8_t*)(xh + (int64_t)c * d + k0) = bh[h];
          if (LO) *(half8_t*)(xl + (int64_t)c * d + k0) = bl[h];
        }
        acc = mfma16x16x32(a[h], bh[h], acc);
        if (LO) acc = mfma16x16x32(a[h], bl[h], acc);
      }
    }
    acc = reduce_waves<kW>(acc, lds.red, wave, lane);
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
    if (threadIdx.x == 0) lds.last = atomicAdd(&ctrl[0], 1) == rblocks - 1;  // cleared by stage 3
    __syncthreads();
    if (lds.last) route_finish_block<true, KLF>(lds.route, plog, d / ck, L.router_bias, E, L.top_k, T, ro);
  }
}

// ============================================================== stage 2
// Activation rows of one super-block per wave when the group's x is not
// staged whole: 16 token rows of 256 inputs, 8 halves of padding per row.
constexpr int kSbRow = QK + 8;
constexpr int kSbRows = kDecodeGroup * kSbRow;

// BL: the group's whole x staged once per block (bh, bl); otherwise each
// wave stages the super-block it is about to decode (xw, xwl).
// NS: binary16 activations the block stages when BL (T rows of d_model,
// each padded by 8 halves, T <= 16).
// Codebook form of a routed CB2 gate/up kernel: byte tables (half the LDS
// bytes, two byte permutes more per weight pair) for groups of tokens, whose
// gate/up is bound by LDS reads; binary16 pairs for the one-token form,
// whose decode hides behind its weight stream.
template <bool BL, int NS>
constexpr bool cb2_bytes() { return !BL || NS != kStageHalves; }

template <bool LO, bool BL, int NS = kStageHalves>
struct Stage2Lds {
  static constexpr int kEnt = cb2_bytes<BL, NS>() ? 2 : 4;  // words per table entry
  uint32_t mag[256 * kEnt];  // sgn right after mag
  uint32_t sgn[128 * kEnt];
  _Float16 bh[BL ? NS + 16 * 8 : 8];
  _Float16 bl[BL && LO ? NS + 16 * 8 : 8];
  _Float16 xw[BL ? 8 : kW * kSbRows];
  _Float16 xwl[BL || !LO ? 8 : kW * kSbRows];
  float4_t red[kW][64];
  float4_t red2[kW][64];
  int last;
};

constexpr int kSb2 = 4;  // CB2 super-blocks a wave loads at once

// One CB2 group's codebook entries, read ahead of their use: magnitudes and
// signs of the 8 weights.  B8 (byte form): byte k is the high byte of
// binary16 m_k (its low byte is zero for m in {1, 3, 5}), and 0x80 in the
// sign entry's byte k if weight k is negative.  Else binary16 pairs and
// their sign masks (bits 15 and 31).
template <bool B8>
struct Cb2Raw {
  using V = std::conditional_t<B8, u32x2_t, u32x4_t>;
  V m, s;
};
template <bool B8>
struct Cb2Step {  // one sub-block step of a routed gate/up wave
  Cb2Raw<B8> g, u;
  half8_t bh, bl;
};
template <bool B8>
__device__ inline void cb2_lookup(Cb2Raw<B8>& R, uint32_t idxw, uint32_t aux, int q, const uint32_t* mag,
                                  const uint32_t* sgn) {
  using V = typename Cb2Raw<B8>::V;
  constexpr int kEnt = B8 ? 2 : 4;
  R.m = *(const V*)(mag + kEnt * ((idxw >> (8 * q)) & 0xFFu));
  R.s = *(const V*)(sgn + kEnt * ((aux >> (7 * q)) & 0x7Fu));
}
// sign * (2s+1) * m as binary16 (exact integers <= 155), s from aux bits 28..31
template <bool B8>
__device__ inline half8_t cb2_apply(const Cb2Raw<B8>& R, uint32_t aux) {
  const _Float16 S = (_Float16)(float)(2 * (aux >> 28) + 1);
  const half2_t S2 = {S, S};
  u32x4_t r;
  if constexpr (B8) {
    const uint32_t b0 = R.m.x ^ R.s.x, b1 = R.m.y ^ R.s.y;
    // bytes 2p, 2p + 1 -> high bytes of a binary16 pair (selector 0x0C: zero)
    r.x = as_u32(as_half2(__builtin_amdgcn_perm(0u, b0, 0x010C000Cu)) * S2);
    r.y = as_u32(as_half2(__builtin_amdgcn_perm(0u, b0, 0x030C020Cu)) * S2);
    r.z = as_u32(as_half2(__builtin_amdgcn_perm(0u, b1, 0x010C000Cu)) * S2);
    r.w = as_u32(as_half2(__builtin_amdgcn_perm(0u, b1, 0x030C020Cu)) * S2);
  } else {
    r.x = as_u32(as_half2(R.m.x ^ R.s.x) * S2);
    r.y = as_u32(as_half2(R.m.y ^ R.s.y) * S2);
    r.z = as_u32(as_half2(R.m.z ^ R.s.z) * S2);
    r.w = as_u32(as_half2(R.m.w ^ R.s.w) * S2);
  }
  return as_half8(r);
}

// Per lane and super-block b of an MXFP4 [rows, K] matrix: the lane's two
// blocks 8b + 2q and 8b + 2q + 1 of its row (64 elements, the same K range
// as a CB2 lane's two sub-blocks) and their two scale bytes.
struct Mx4Sb {
  u32x4_t c0, c1;
  uint32_t sc;  // scale of block 2q in bits 0..7, of block 2q + 1 in bits 8..15
};
// step s2 (0..7) of super-block: block 2q + (s2 >> 2), code word s2 & 3
__device__ inline half8_t mx4_step(const Mx4Sb& W, int s2) {
  const u32x4_t& c = (s2 & 4) ? W.c1 : W.c0;
  const uint32_t w = (s2 & 3) == 0 ? c.x : ((s2 & 3) == 1 ? c.y : ((s2 & 3) == 2 ? c.z : c.w));
  return mx4_frag(w, e8m0_f32((W.sc >> ((s2 & 4) ? 8 : 0)) & 0xFFu));
}
// Per lane and super-block b of a Q4K [rows, K] matrix: the lane's two
// sub-blocks 2q and 2q + 1 of its row (64 elements), the block's three
// scale words and its (d, dmin) word.
struct Q4kSb {
  u32x4_t c0, c1;
  uint32_t w0, w1, w2, sup;
};
// binary16 scales of the lane's two sub-blocks: [0] = 2q, [1] = 2q + 1
struct Q4kS {
  half2_t ds[2], nm[2];
};
__device__ inline Q4kS q4k_lane_scales(const Q4kSb& W, int q) {
  Q4kS S;
  q4k_scales(W.w0, W.w1, W.w2, W.sup, 2 * q, S.ds[0], S.nm[0]);
  q4k_scales(W.w0, W.w1, W.w2, W.sup, 2 * q + 1, S.ds[1], S.nm[1]);
  return S;
}
__device__ inline half8_t q4k_step(const Q4kSb& W, const Q4kS& S, int s2) {
  const u32x4_t& c = (s2 & 4) ? W.c1 : W.c0;
  const uint32_t w = (s2 & 3) == 0 ? c.x : ((s2 & 3) == 1 ? c.y : ((s2 & 3) == 2 ? c.z : c.w));
  return q4k_frag(w, S.ds[s2 >> 2], S.nm[s2 >> 2]);
}

// Blocks [0, maxd * f/16): one per (distinct expert, 16-row tile) of the
// routed gate/up products, whose codebook decoding is the arithmetic; then
// two per 16-row tile of the shared expert (gate, up), an F16 stream
// dispatched behind the routed blocks.
// Waves per SIMD that stage 2's LDS allows: 4 blocks per CU with x staged
// whole, 3 with the per-wave super-block buffers, fewer with fp32 input.
constexpr int stage2_waves(bool lo, bool bl, int ns = kStageHalves) {
  return bl ? (lo ? 2 : (ns > kStageHalves ? 3 : 4)) : (lo ? 1 : 3);
}

template <bool LO, bool BL, bool Q4, int NS>
__device__ void routed_gateup_mx(const ds4moe_layer& L, int T, const RouteOut& ro, const _Float16* __restrict__ xh,
                                 const _Float16* __restrict__ xl, _Float16* __restrict__ hw16,
                                 Stage2Lds<LO, BL, NS>& lds);

// Blocks from rtiles on (launched for one token) are the shared expert's
// gate/up blocks.
template <bool LO, bool BL, bool MX, bool Q4 = false, int NS = kStageHalves>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(stage2_waves(LO, BL, NS)))) void k_dec_stage2(
    ds4moe_layer L, int T, RouteOut ro, const _Float16* __restrict__ xh,
    const _Float16* __restrict__ xl, _Float16* __restrict__ hw16, _Float16* __restrict__ hsum, int rtiles,
    float* __restrict__ gu_part, _Float16* __restrict__ hs16, int32_t* __restrict__ ctrl) {
  __shared__ Stage2Lds<LO, BL, NS> lds;
  if ((int)blockIdx.x >= rtiles) {
    shared_gateup_block<LO, BL, false, kShSplit>(L, T, nullptr, xh, xl, blockIdx.x - rtiles, gu_part, hs16, ctrl,
                                                 lds.bh, lds.bl, lds.red, lds.last);
    return;
  }
  if constexpr (MX || Q4) {
    routed_gateup_mx<LO, BL, Q4, NS>(L, T, ro, xh, xl, hw16, lds);
    return;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);
  const int d = L.d_model, f = L.d_ff, k = L.top_k;
  const int nr = f / 16, nb = d / QK;
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  // ---------------- routed gate/up: distinct expert i, 16-row tile
  const int rel = blockIdx.x;
  const int i = rel / nr, tile = rel % nr;
  const int row0 = tile * 16;
  // phase 1: copies into LDS (activations, grid tables), independent of routing
  const int st = stage_stride(d);
  if (BL) dma_rows(xh, d, T, d, lds.bh, st, wave, kW, lane);
  if (BL && LO) dma_rows(xl, d, T, d, lds.bl, st, wave, kW, lane);
  constexpr bool B8 = cb2_bytes<BL, NS>();
  static_assert(offsetof(GridTables, sgn) == sizeof(GridTables::mag) &&
                offsetof(GridTables, sgn8) == offsetof(GridTables, mag8) + sizeof(GridTables::mag8));
  // mag, then sgn (in 16-byte pieces: 256 + 128, or 128 + 64 in byte form)
  dma_pieces(B8 ? &c_dec_tables.mag8[0][0] : &c_dec_tables.mag[0][0], B8 ? 192 : 384, lds.mag, wave, kW, lane);
  // phase 2: routing tables by scalar loads, which do not wait for the
  // copies: the first weight batch goes out while they are in flight
  const int nd = ld_uniform(ro.ndist);
  if (i >= nd) {  // whole block
    wait_all();   // no copy into LDS left in flight
    return;
  }
  const int e = clamp_index(ld_uniform(ro.distinct + i), L.n_experts);
  // Transposed products: x (token c') is the MFMA's A operand, the weights
  // its B operand, so lane (c, q) ends with tokens 4q..4q+3 of row row0 + c.
  const size_t mb = (size_t)f * nb;  // blocks per matrix
  const uint8_t* gc = (const uint8_t*)L.gate + (size_t)e * mb * 66;
  const uint8_t* uc = (const uint8_t*)L.up + (size_t)e * mb * 66;
  const uint16_t* gd = (const uint16_t*)(gc + mb * 64) + (size_t)(row0 + c) * nb;
  const uint16_t* ud = (const uint16_t*)(uc + mb * 64) + (size_t)(row0 + c) * nb;
  const uint8_t* grow = gc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  const uint8_t* urow = uc + (size_t)(row0 + c) * nb * 64 + 16 * q;
  int sb0, sb1;
  split_range(nb, kW, wave, sb0, sb1);
  // d of kSb2 consecutive super-blocks in one load per matrix when aligned
  const bool dvec = nb % kSb2 == 0;
  u32x4_t cg[kSb2], cu[kSb2];
  float dg[kSb2], du[kSb2];
  // phase 3: weight loads of kSb2 super-blocks from b0, consumed as they
  // arrive (indices clamped into [0, nb): a wave with an empty range loads
  // a valid block it never uses)
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int j = 0; j < kSb2; ++j) {
      const int b = max(min(b0 + j, sb1 - 1), 0);
      cg[j] = __builtin_nontemporal_load((const u32x4_t*)(grow + b * 64));
      cu[j] = __builtin_nontemporal_load((const u32x4_t*)(urow + b * 64));
    }
    if (dvec && b0 + kSb2 <= sb1) {
      const u32x2_t g4 = *(const u32x2_t*)(gd + b0), u4 = *(const u32x2_t*)(ud + b0);
#pragma unroll
      for (int j = 0; j < kSb2; ++j) {
        dg[j] = h2f((uint16_t)((j < 2 ? g4.x : g4.y) >> (16 * (j & 1))));
        du[j] = h2f((uint16_t)((j < 2 ? u4.x : u4.y) >> (16 * (j & 1))));
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSb2; ++j) {
        const int b = max(min(b0 + j, sb1 - 1), 0);
        dg[j] = h2f(gd[b]);
        du[j] = h2f(ud[b]);
      }
    }
  };
  load_batch(sb0);
  // !BL: the tokens that chose expert i (bit t; a distinct expert has at
  // least one), compacted: MFMA row j is the j-th of them, so only their
  // activation rows are staged
  uint32_t tmask = 0u;
  int ntok = T;
  if constexpr (!BL) {
    const int slc = c < T ? ro.tok_slot[i * kDecodeGroup + c] : -1;
    tmask = (uint32_t)__ballot(slc >= 0) & 0xFFFFu;  // lanes 0..15 (c = lane)
    ntok = max(1, __popc(tmask));
  }
  wait_all();  // the copies (and the first batch)
  __syncthreads();
  if constexpr (!BL) {
    // Each wave stages the activations of the super-block it decodes next
    // (the expert's token rows x 256 inputs) and waits for its own copies;
    // the buffer is its own, so no block barrier is needed.  Rows at or
    // beyond ntok are never read (those MFMA rows repeat row ntok - 1).
    _Float16* xw = lds.xw + wave * kSbRows;
    _Float16* xwl = LO ? lds.xwl + wave * kSbRows : nullptr;
    const int tcx = min(c, ntok - 1);
    // with at most kDecodeGroup / kSb2 tokens, the whole batch's rows fit
    // the buffer (super-block j at rows j ntok ..): one copy pass and one
    // wait per batch instead of one per super-block
    const bool whole = ntok * kSb2 <= kDecodeGroup;  // wave-uniform
    for (int b0 = sb0; b0 < sb1; b0 += kSb2) {
      if (b0 != sb0) load_batch(b0);
      if (whole) {
        pin();
#pragma unroll
        for (int j = 0; j < kSb2; ++j) {
          if (b0 + j < sb1) {
            dma_token_rows(xh + (int64_t)(b0 + j) * QK, d, tmask, xw + j * ntok * kSbRow, kSbRow, lane);
            if (LO) dma_token_rows(xl + (int64_t)(b0 + j) * QK, d, tmask, xwl + j * ntok * kSbRow, kSbRow, lane);
          }
        }
        wait_all();
      }
#pragma unroll
      for (int j = 0; j < kSb2; ++j) {
        if (b0 + j >= sb1) break;  // wave-uniform
        pin();
        if (!whole) {
          dma_token_rows(xh + (int64_t)(b0 + j) * QK, d, tmask, xw, kSbRow, lane);
          if (LO) dma_token_rows(xl + (int64_t)(b0 + j) * QK, d, tmask, xwl, kSbRow, lane);
          wait_all();
        }
        pin();
        const _Float16* xj = xw + (whole ? j * ntok * kSbRow : 0);
        const _Float16* xjl = LO ? xwl + (whole ? j * ntok * kSbRow : 0) : nullptr;
        Cb2Step<B8> F[2];
        auto fetch = [&](Cb2Step<B8>& G, int s2) {
          const int kk = cb2_boff(q, s2);
          G.bh = *(const half8_t*)(xj + tcx * kSbRow + kk);
          if (LO) G.bl = *(const half8_t*)(xjl + tcx * kSbRow + kk);
          cb2_lookup(G.g, (s2 & 4) ? cg[j].z : cg[j].x, (s2 & 4) ? cg[j].w : cg[j].y, s2 & 3, lds.mag, lds.sgn);
          cb2_lookup(G.u, (s2 & 4) ? cu[j].z : cu[j].x, (s2 & 4) ? cu[j].w : cu[j].y, s2 & 3, lds.mag, lds.sgn);
        };
        float4_t pg = {0.f, 0.f, 0.f, 0.f}, pu = pg;
        fetch(F[0], 0);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          if (s2 + 1 < 8) fetch(F[(s2 + 1) & 1], s2 + 1);
          pin();
          const Cb2Step<B8>& G = F[s2 & 1];
          const half8_t a0 = cb2_apply(G.g, (s2 & 4) ? cg[j].w : cg[j].y);
          const half8_t a1 = cb2_apply(G.u, (s2 & 4) ? cu[j].w : cu[j].y);
          pg = mfma16x16x32(G.bh, a0, pg);
          pu = mfma16x16x32(G.bh, a1, pu);
          if (LO) {
            pg = mfma16x16x32(G.bl, a0, pg);
            pu = mfma16x16x32(G.bl, a1, pu);
          }
          pin();
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // the lane's own row: its own d
          ag[r] += dg[j] * pg[r];
          au[r] += du[j] * pu[r];
        }
      }
    }
  }
  for (int b0 = sb0; BL && b0 < sb1; b0 += kSb2) {
    if (b0 != sb0) load_batch(b0);
    pin();
    // 8 steps per super-block (one per sub-block); each step's LDS reads
    // (activations, codebook magnitudes and signs) are issued one step ahead
    Cb2Step<B8> F[2];
    auto fetch = [&](Cb2Step<B8>& G, int t) {
      const int j = t >> 3, s2 = t & 7;
      const int kk = min(b0 + j, sb1 - 1) * QK + cb2_boff(q, s2);
      if (BL) {
        G.bh = *(const half8_t*)(lds.bh + tc * st + kk);
        if (LO) G.bl = *(const half8_t*)(lds.bl + tc * st + kk);
      } else {
        G.bh = *(const half8_t*)(xh + (int64_t)tc * d + kk);
        if (LO) G.bl = *(const half8_t*)(xl + (int64_t)tc * d + kk);
      }
      cb2_lookup(G.g, (s2 & 4) ? cg[j].z : cg[j].x, (s2 & 4) ? cg[j].w : cg[j].y, s2 & 3, lds.mag, lds.sgn);
      cb2_lookup(G.u, (s2 & 4) ? cu[j].z : cu[j].x, (s2 & 4) ? cu[j].w : cu[j].y, s2 & 3, lds.mag, lds.sgn);
    };
    float4_t pg = {0.f, 0.f, 0.f, 0.f}, pu = pg;
    fetch(F[0], 0);
#pragma unroll
    for (int t = 0; t < 8 * kSb2; ++t) {
      if (t + 1 < 8 * kSb2) fetch(F[(t + 1) & 1], t + 1);
      pin();
      const Cb2Step<B8>& G = F[t & 1];
      const int j = t >> 3, s2 = t & 7;
      const half8_t a0 = cb2_apply(G.g, (s2 & 4) ? cg[j].w : cg[j].y);
      const half8_t a1 = cb2_apply(G.u, (s2 & 4) ? cu[j].w : cu[j].y);
      pg = mfma16x16x32(G.bh, a0, pg);
      pu = mfma16x16x32(G.bh, a1, pu);
      if (LO) {
        pg = mfma16x16x32(G.bl, a0, pg);
        pu = mfma16x16x32(G.bl, a1, pu);
      }
      pin();
      if (s2 == 7) {  // super-blocks past the range get a zero scale
        const float sg = b0 + j < sb1 ? dg[j] : 0.0f, su = b0 + j < sb1 ? du[j] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // the lane's own row: its own d
          ag[r] += sg * pg[r];
          au[r] += su * pu[r];
        }
        pg = float4_t{0.f, 0.f, 0.f, 0.f};
        pu = pg;
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
  // MFMA rows 4q..4q+3: their tokens' slots for this expert (BL: row j is
  // token j; else the j-th token of tmask); h = w * silu(g) * u as binary16
  // into hw16[slot][row] (pair-interleaved within the 16-row tile), and the
  // 16-row sums into hsum
  int slots[4];
  if constexpr (BL) {
    const int4 sl4 = *(const int4*)(ro.tok_slot + i * kDecodeGroup + 4 * q);
    slots[0] = sl4.x;
    slots[1] = sl4.y;
    slots[2] = sl4.z;
    slots[3] = sl4.w;
  } else {
    uint32_t m = tmask;
    for (int x = 0; x < 4 * q; ++x) m &= m - 1u;  // drop the first 4q tokens
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      slots[r] = m != 0u ? ro.tok_slot[i * kDecodeGroup + __builtin_ctz(m)] : -1;
      m &= m - 1u;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = slots[r];
    const bool has = (BL ? 4 * q + r < T : 4 * q + r < ntok) && slot >= 0 && slot < T * k;
    float hv = 0.0f;
    if (has) {
      const _Float16 h16 = (_Float16)(ro.w[slot] * (silu(ag[r]) * au[r]));
      hw16[(int64_t)slot * f + row0 + q2k_pair_pos(c)] = h16;  // pair-interleaved for the Q2K down product
      hv = (float)h16;
    }
    // sum over the 16 rows (lanes 16q..16q+15): quad, half-row and row mirrors
    hv += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hv), 0xB1, 0xF, 0xF, true));
    hv += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hv), 0x4E, 0xF, 0xF, true));
    hv += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hv), 0x141, 0xF, 0xF, true));
    hv += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hv), 0x140, 0xF, 0xF, true));
    if (has && c == 0) {  // binary16 hi and lo planes of the sum (the Q2K min term's A operand)
      const _Float16 hi = (_Float16)hv;
      hsum[(int64_t)slot * (f / 16) + tile] = hi;
      hsum[(int64_t)(T * k + slot) * (f / 16) + tile] = (_Float16)(hv - (float)hi);
    }
  }
}

// Routed gate/up tile of an MXFP4 (Q4 false) or Q4K (Q4) layer: as the CB2
// tile, with the lane's two 32-element blocks of each super-block turned
// into binary16 fragments with their scales folded in (MXFP4 by the FP4
// conversion, exact for the documented scale range; Q4K as q * binary16(d s)
// - binary16(dmin m), rounded once), so no per-super-block scale after the
// products.  Activations come from LDS when staged (BL), else from the
// binary16 copy in memory.
// super-blocks a wave loads at once (32 code bytes per matrix and lane each):
// four for MXFP4; two for Q4K, whose three scale words and (d, dmin) per
// super-block would not fit four blocks' worth in the 128 registers of a
// 4-wave-per-SIMD kernel
template <bool Q4>
constexpr int sb_batch() { return Q4 ? 2 : 4; }

template <bool LO, bool BL, bool Q4, int NS>
__device__ void routed_gateup_mx(const ds4moe_layer& L, int T, const RouteOut& ro, const _Float16* __restrict__ xh,
                                 const _Float16* __restrict__ xl, _Float16* __restrict__ hw16,
                                 Stage2Lds<LO, BL, NS>& lds) {
  constexpr int kSbMx = sb_batch<Q4>();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int tc = min(c, T - 1);
  const int d = L.d_model, f = L.d_ff, k = L.top_k;
  const int nr = f / 16, nb = d / QK;
  const int i = blockIdx.x / nr, tile = blockIdx.x % nr;
  const int row0 = tile * 16;
  const int st = stage_stride(d);
  if (BL) dma_rows(xh, d, T, d, lds.bh, st, wave, kW, lane);
  if (BL && LO) dma_rows(xl, d, T, d, lds.bl, st, wave, kW, lane);
  const int nd = ld_uniform(ro.ndist);
  if (i >= nd) {
    wait_all();
    return;
  }
  const int e = clamp_index(ld_uniform(ro.distinct + i), L.n_experts);
  // one packed [f, d] matrix; a row's code bytes per super-block are 128 in both formats
  const size_t mbytes = Q4 ? (size_t)f * nb * 144 : (size_t)f * d * 17 / 32;
  const uint8_t* gm = (const uint8_t*)L.gate + (size_t)e * mbytes;
  const uint8_t* um = (const uint8_t*)L.up + (size_t)e * mbytes;
  const uint8_t* grow = gm + (size_t)(row0 + c) * (d / 2) + 32 * q;
  const uint8_t* urow = um + (size_t)(row0 + c) * (d / 2) + 32 * q;
  // MXFP4: the lane's two scale bytes; Q4K: the block's scale words, then (d, dmin)
  const uint8_t* gsc = Q4 ? gm + (size_t)f * nb * 128 + (size_t)(row0 + c) * nb * 12
                          : gm + (size_t)f * d / 2 + (size_t)(row0 + c) * (d / 32) + 2 * q;
  const uint8_t* usc = Q4 ? um + (size_t)f * nb * 128 + (size_t)(row0 + c) * nb * 12
                          : um + (size_t)f * d / 2 + (size_t)(row0 + c) * (d / 32) + 2 * q;
  const uint8_t* gsp = gm + (size_t)f * nb * 140 + (size_t)(row0 + c) * nb * 4;  // Q4K only
  const uint8_t* usp = um + (size_t)f * nb * 140 + (size_t)(row0 + c) * nb * 4;
  int sb0, sb1;
  split_range(nb, kW, wave, sb0, sb1);
  Mx4Sb wg[kSbMx], wu[kSbMx];
  Q4kSb qg[kSbMx], qu[kSbMx];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int j = 0; j < kSbMx; ++j) {
      const int b = max(min(b0 + j, sb1 - 1), 0);
      if constexpr (Q4) {
        qg[j].c0 = __builtin_nontemporal_load((const u32x4_t*)(grow + 128 * b));
        qg[j].c1 = __builtin_nontemporal_load((const u32x4_t*)(grow + 128 * b + 16));
        qu[j].c0 = __builtin_nontemporal_load((const u32x4_t*)(urow + 128 * b));
        qu[j].c1 = __builtin_nontemporal_load((const u32x4_t*)(urow + 128 * b + 16));
        const u32x3_t gw = *(const u32x3_a4_t*)(gsc + 12 * b);  // one 12-byte load each
        const u32x3_t uw = *(const u32x3_a4_t*)(usc + 12 * b);
        qg[j].w0 = gw.x; qg[j].w1 = gw.y; qg[j].w2 = gw.z;
        qu[j].w0 = uw.x; qu[j].w1 = uw.y; qu[j].w2 = uw.z;
        qg[j].sup = *(const uint32_t*)(gsp + 4 * b);
        qu[j].sup = *(const uint32_t*)(usp + 4 * b);
      } else {
        wg[j].c0 = __builtin_nontemporal_load((const u32x4_t*)(grow + 128 * b));
        wg[j].c1 = __builtin_nontemporal_load((const u32x4_t*)(grow + 128 * b + 16));
        wu[j].c0 = __builtin_nontemporal_load((const u32x4_t*)(urow + 128 * b));
        wu[j].c1 = __builtin_nontemporal_load((const u32x4_t*)(urow + 128 * b + 16));
        wg[j].sc = *(const uint16_t*)(gsc + 8 * b);
        wu[j].sc = *(const uint16_t*)(usc + 8 * b);
      }
    }
  };
  load_batch(sb0);
  wait_all();  // the copies (and the first batch)
  __syncthreads();
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  for (int b0 = sb0; b0 < sb1; b0 += kSbMx) {
    if (b0 != sb0) load_batch(b0);
    pin();
    // nested constant-trip loops (fully unrolled, so the per-super-block
    // registers are indexed statically); super-blocks past the range are
    // skipped by a wave-uniform test
#pragma unroll
    for (int j = 0; j < kSbMx; ++j) {
      if (b0 + j < sb1) {
        Q4kS sg, su;  // Q4K: this super-block's binary16 scales, formed just before use
        if constexpr (Q4) {
          sg = q4k_lane_scales(qg[j], q);
          su = q4k_lane_scales(qu[j], q);
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int kk = (b0 + j) * QK + cb2_boff(q, s2);
          half8_t bh, bl;
          if (BL) {
            bh = *(const half8_t*)(lds.bh + tc * st + kk);
            if (LO) bl = *(const half8_t*)(lds.bl + tc * st + kk);
          } else {
            bh = *(const half8_t*)(xh + (int64_t)tc * d + kk);
            if (LO) bl = *(const half8_t*)(xl + (int64_t)tc * d + kk);
          }
          const half8_t a0 = Q4 ? q4k_step(qg[j], sg, s2) : mx4_step(wg[j], s2);
          const half8_t a1 = Q4 ? q4k_step(qu[j], su, s2) : mx4_step(wu[j], s2);
          ag = mfma16x16x32(bh, a0, ag);
          au = mfma16x16x32(bh, a1, au);
          if (LO) {
            ag = mfma16x16x32(bl, a0, ag);
            au = mfma16x16x32(bl, a1, au);
          }
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
  const int4 sl4 = *(const int4*)(ro.tok_slot + i * kDecodeGroup + 4 * q);
  const int slots[4] = {sl4.x, sl4.y, sl4.z, sl4.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = slots[r];
    if (4 * q + r < T && slot >= 0 && slot < T * k)
      hw16[(int64_t)slot * f + row0 + c] = (_Float16)(ro.w[slot] * (silu(ag[r]) * au[r]));
  }
}

// ============================================================== stage 3
// Weight operands of one (expert, super-block) Q2K unit for lane (c, q):
// its row is row0 + c.
struct Q2kW {
  u32x4_t codes;  // sub-blocks 4q..4q+3 of the lane's row
  uint32_t sc4;   // their scale/min bytes
  u32x2_t mins;   // scale/min bytes 8(q&1)..+7 (min MFMA operand; used by lanes q < 2)
  uint32_t sup;   // (d, dmin) of the lane's row
};

// Per-lane byte offsets of a Q2K unit's operands within one expert's packed
// matrix, for super-block 0 (add b * 64, b * 16, b * 4 for super-block b).
struct Q2kOff {
  uint32_t codes, sc, mins, sup;
};

__device__ inline Q2kOff q2k_offsets(size_t mb, int nb, int row0, int c, int q) {
  Q2kOff o;
  o.codes = (uint32_t)((size_t)(row0 + c) * nb * 64 + 16 * q);
  o.sc = (uint32_t)(mb * 64 + (size_t)(row0 + c) * nb * 16 + 4 * q);
  o.mins = (uint32_t)(mb * 64 + (size_t)(row0 + c) * nb * 16 + 8 * (q & 1));
  o.sup = (uint32_t)(mb * 80 + (size_t)(row0 + c) * nb * 4);
  return o;
}

// Activation operands of one unit for lane (c, q): its token's binary16 h at
// the lane's K offsets and the hi/lo sums of the 16 sub-blocks.
struct Q2kA {
  half8_t b[8], bh, bl;
};

// bcol: the activation row of the lane's token at the unit's super-block
// (LDS); csh/csl: binary16 hi/lo of its 16 sub-block sums.
__device__ inline void q2k_act(Q2kA& A, const _Float16* bcol, const _Float16* csh, const _Float16* csl, int q) {
#pragma unroll
  for (int s = 0; s < 8; ++s) A.b[s] = *(const half8_t*)(bcol + q2k_boff(q, s));
  A.bh = *(const half8_t*)(csh + 8 * (q & 1));
  A.bl = *(const half8_t*)(csl + 8 * (q & 1));
}

// Q2K codes at unit weight.  The two codes of pair i of a sub-block (codes i
// and i + 8: bits 2i and 2i + 16 of its u32 u, the same bits of the word's
// two 16-bit halves) are taken by one three-input bit operation from u << 4,
// u >> 2 or u >> 8, which puts them at mantissa bit 4, 6 or 8 under an
// exponent that gives that bit weight one: each binary16 half reads
// base + q exactly, base 64, 16 or 4.
//   pairs 0, 3, 6 -> bit 4 (base 64), 1, 4, 7 -> bit 6 (base 16), 2, 5 -> bit 8 (base 4).
__host__ __device__ constexpr int q2k_pair_base(int i) { return i % 3 == 0 ? 64 : (i % 3 == 1 ? 16 : 4); }

__device__ inline void q2k_pairs_unit_weight(uint32_t u, uint32_t (&w)[8]) {
  const uint32_t a = u << 4, b = u >> 2, c = u >> 8;
  // (x & mask) | magic: 0x5400 = 64, 0x4C00 = 16, 0x4400 = 4 (binary16)
  w[0] = __builtin_amdgcn_bitop3_b32(a, 0x00300030u, 0x54005400u, 0xEA);
  w[1] = __builtin_amdgcn_bitop3_b32(a, 0x00C000C0u, 0x4C004C00u, 0xEA);
  w[2] = __builtin_amdgcn_bitop3_b32(a, 0x03000300u, 0x44004400u, 0xEA);
  w[3] = __builtin_amdgcn_bitop3_b32(b, 0x00300030u, 0x54005400u, 0xEA);
  w[4] = __builtin_amdgcn_bitop3_b32(b, 0x00C000C0u, 0x4C004C00u, 0xEA);
  w[5] = __builtin_amdgcn_bitop3_b32(b, 0x03000300u, 0x44004400u, 0xEA);
  w[6] = __builtin_amdgcn_bitop3_b32(c, 0x00300030u, 0x54005400u, 0xEA);
  w[7] = __builtin_amdgcn_bitop3_b32(c, 0x00C000C0u, 0x4C004C00u, 0xEA);
}

// Both B fragments of one Q2K sub-block in pair order (dwords 0..3: pairs
// 0..3, then 4..7), as binary16 s q, exact: one fma per pair scales the
// unit-weight pair and removes its base, (base + q) s - base s.
__device__ inline void q2k_subblock_paired(uint32_t u, uint32_t s, half8_t& lo, half8_t& hi) {
  uint32_t w[8];
  q2k_pairs_unit_weight(u, w);
  const _Float16 S = (_Float16)(uint16_t)s;
  const half2_t S2 = {S, S};
  const half2_t C[3] = {S2 * (half2_t){(_Float16)-64.0f, (_Float16)-64.0f},
                        S2 * (half2_t){(_Float16)-16.0f, (_Float16)-16.0f},
                        S2 * (half2_t){(_Float16)-4.0f, (_Float16)-4.0f}};  // -base s, by pair i % 3
  u32x4_t a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = as_u32(__builtin_elementwise_fma(as_half2(w[i]), S2, C[i % 3]));
    b[i] = as_u32(__builtin_elementwise_fma(as_half2(w[4 + i]), S2, C[(4 + i) % 3]));
  }
  lo = as_half8(a);
  hi = as_half8(b);
}

// The high nibbles (the 4-bit mins) of bytes j and j + 1 of w as a binary16
// pair: one byte permute puts byte j in the low half and byte j + 1 in the
// high half, the bit operation sets the exponent that gives bit 4 weight one
// (64 + m), and one subtraction removes the 64.
template <int J>
__device__ inline uint32_t min_pair_f16(uint32_t w) {
  constexpr uint32_t sel = J == 0 ? 0x01010000u : 0x03030202u;
  const uint32_t x = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(0u, w, sel), 0x00F000F0u, 0x54005400u, 0xEA);
  return as_u32(as_half2(x) - (half2_t){(_Float16)64.0f, (_Float16)64.0f});
}

// One unit, transposed: the activations are the MFMA's A operand (row c' =
// token c'), the weights its B operand, so lane (c, q) ends with tokens
// 4q..4q+3 of row row0 + c.  The activations are pair-interleaved
// (q2k_pair_pos).  MASKED: bit r of vmask set when token 4q + r has a slot
// for this expert, the other tokens' products are dropped; else those
// tokens' activations (and the sums of lanes q >= 2) are zeros already, so
// their products are exactly zero.
template <bool MASKED>
__device__ inline void q2k_unit(const Q2kW& U, const Q2kA& A, uint32_t vmask, int q, float4_t& acc) {
  float4_t p = {0.f, 0.f, 0.f, 0.f}, pm = p;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // sub-block 4q + j: two MFMA steps share its scale
    half8_t alo, ahi;
    q2k_subblock_paired(U.codes[j], (U.sc4 >> (8 * j)) & 15u, alo, ahi);
    p = mfma16x16x32(A.b[2 * j], alo, p);
    p = mfma16x16x32(A.b[2 * j + 1], ahi, p);
  }
  // min term: K-slots 0..15 are the 16 sub-blocks (lane groups q >= 2 add zeros)
  u32x4_t t;
  t.x = min_pair_f16<0>(U.mins.x);
  t.y = min_pair_f16<1>(U.mins.x);
  t.z = min_pair_f16<0>(U.mins.y);
  t.w = min_pair_f16<1>(U.mins.y);
  const half8_t am = !MASKED || q < 2 ? as_half8(t) : zero_half8();
  pm = mfma16x16x32(A.bh, am, pm);
  pm = mfma16x16x32(A.bl, am, pm);
  const float dd = h2f((uint16_t)(U.sup & 0xFFFFu)), dm = h2f((uint16_t)(U.sup >> 16));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (MASKED) {
      acc[r] += ((vmask >> r) & 1u) ? dd * p[r] - dm * pm[r] : 0.0f;
    } else {
      acc[r] = __builtin_fmaf(dd, p[r], acc[r]);
      acc[r] = __builtin_fmaf(-dm, pm[r], acc[r]);
    }
  }
}

constexpr int kW3 = 16;     // waves per stage-3 block: 4 per SIMD, few units each
constexpr int kUnits3 = 3;  // units whose weight loads a wave keeps in flight
constexpr int kRing3 = 3;   // stage-3 ring slots per wave: one unit computing, the next two requested

// Block `tile`: output rows tile*16 .. tile*16+15 of the shared expert's
// down product and of every (distinct expert, super-block) unit, so the
// whole sum stays in the block and it writes y = ys + the routed terms
// itself.  The routed weights are requested first: their decode is the
// arithmetic, and the shared expert's F16 rows stream in behind them.
// One MXFP4 or Q4K down unit, transposed like q2k_unit: 8 steps over the
// lane's two 32-element blocks (scales folded into the binary16 weights).
__device__ inline void mx4_unit(const Mx4Sb& U, const Q2kA& A, uint32_t vmask, float4_t& acc) {
  float4_t p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) p = mfma16x16x32(A.b[s2], mx4_step(U, s2), p);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] += ((vmask >> r) & 1u) ? p[r] : 0.0f;
}
__device__ inline void q4k_unit(const Q4kSb& U, const Q2kA& A, uint32_t vmask, int q, float4_t& acc) {
  const Q4kS S = q4k_lane_scales(U, q);
  float4_t p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) p = mfma16x16x32(A.b[s2], q4k_step(U, S, s2), p);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] += ((vmask >> r) & 1u) ? p[r] : 0.0f;
}

template <bool BL, bool MX, bool Q4 = false, bool PH = false>
__global__ __launch_bounds__(kW3 * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_stage3(
    ds4moe_layer L, int T, const int32_t* __restrict__ ndist, const int32_t* __restrict__ distinct,
    const int32_t* __restrict__ tok_slot, const _Float16* __restrict__ hw16, const _Float16* __restrict__ hsum,
    const _Float16* __restrict__ hs16, int32_t* __restrict__ ctrl, int nctrl1, int maxd, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char s_dyn[];  // staged activations when BL
  __shared__ float4_t s_red[kW3][64];
  __shared__ float4_t s_red2[kW3][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, k = L.top_k, fs = L.d_ff_shared;
  const int tile = blockIdx.x, row0 = tile * 16;
  const int nb = f / QK, fs16 = f / 16;
  const size_t mb = (size_t)d * nb;
  const int S = T * k;
  const int tc = min(c, T - 1);  // token feeding MFMA row c of the shared product
  const uint8_t* down = (const uint8_t*)L.down;
  // staged: routed activations [S][f], their sums [2][S][f / 16], the
  // shared expert's activations [T][fs]
  _Float16* s_h = (_Float16*)s_dyn;
  _Float16* s_cs = s_h + (size_t)S * f;
  _Float16* s_hs = s_cs + (size_t)2 * S * fs16;
  // phased (PH): super-block p's activation columns [S][QK] and (Q2K) their
  // sums [2S][16] in LDS buffer p % 2, the next super-block's copy in flight
  // into the other buffer while this one computes.  A phase is copied in
  // 1 KB chunks, buffer loads straight into LDS: h chunk ch = rows 2ch,
  // 2ch + 1 (32 lanes a row), sums chunk cs = rows 32cs .. 32cs + 31 (2
  // lanes a row); rows past the last read zeros (the buffer's range check).
  // Padding: h to S + 1 rows rounded up to even, the sums to 2S + 1 rounded
  // up to 32, so h row S and sums row 2S are zero rows.  Chunks ch and cs are
  // wave ch % kW3's and cs % kW3's.
  const int ph_hrows = (S + 2) & ~1, ph_srows = MX || Q4 ? 0 : (2 * S + 32) & ~31;
  const int ph_hch = ph_hrows / 2, ph_sch = ph_srows / 32;
  const uint32_t ph_bytes = (uint32_t)(ph_hrows * QK * 2 + ph_srows * 32);
  auto ph_h = [&](int p) { return (_Float16*)(s_dyn + (p & 1) * ph_bytes); };
  auto ph_cs = [&](int p) { return ph_h(p) + (size_t)ph_hrows * QK; };
  unsigned char* ph_sink = s_dyn + 2 * ph_bytes;  // 1 KB that chunks past the last land in (reading nothing)
  const uint32_t ph_vh = (uint32_t)(lane >> 5) * (uint32_t)(2 * f) + (uint32_t)(lane & 31) * 16u;
  const uint32_t ph_vs = (uint32_t)(lane >> 1) * (uint32_t)(2 * fs16) + (uint32_t)(lane & 1) * 16u;
  const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hw16, (uint32_t)(S * f * 2));
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(hsum, (uint32_t)(2 * S * fs16 * 2));
  auto dma_h = [&](int p, int ch) {  // h chunk ch of phase p; none past the last
    const bool in = ch < ph_hch;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rh, (__attribute__((address_space(3))) void*)(in ? (unsigned char*)(ph_h(p) + ch * 512) : ph_sink), 16,
        in ? ph_vh + (uint32_t)ch * (uint32_t)(4 * f) : kOob, (uint32_t)p * (2 * QK), 0, 0);
  };
  auto dma_s = [&](int p, int cs) {  // sums chunk cs of phase p; none past the last
    const bool in = cs < ph_sch;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(in ? (unsigned char*)(ph_cs(p) + cs * 512) : ph_sink), 16,
        in ? ph_vs + (uint32_t)cs * (uint32_t)(64 * fs16) : kOob, (uint32_t)p * 32u, 0, 0);
  };
  // this wave's chunks of phase p: a fixed number of instructions (at most
  // 4 h chunks and 1 sums chunk are its own)
  auto send_phase = [&](int p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_h(p, wave + kW3 * j);
    if constexpr (!MX && !Q4) dma_s(p, wave);
  };
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctrl1; i += blockDim.x) ctrl[i] = 0;
  // copies of the activations into LDS; one barrier publishes them
  if (BL) {
    dma_rows(hw16, f, S, f, s_h, f, wave, kW3, lane);
    if (!MX && !Q4) dma_rows(hsum, fs16, 2 * S, fs16, s_cs, fs16, wave, kW3, lane);
    dma_rows(hs16, fs, T, fs, s_hs, fs, wave, kW3, lane);
  }
  if (PH) send_phase(0);
  // routing tables: expert ids by scalar loads, which do not wait for the
  // copies, so the first weight batch goes out while they are in flight
  const int nd = max(1, min(ld_uniform(ndist), maxd));  // a call selects at least one expert
  // PH pads the experts to at least 32 (see below): units of padding slots
  // read the last expert's weights again and take no token
  const int nde = PH ? max(nd, 32) : nd;
  const int nunits = nde * nb;  // only the selected experts' units: their weights alone are read
  // units u = (expert slot u / nb, super-block u % nb), or with PH
  // super-block major, (u % nd, u / nd); wave w takes
  // u = w, w + kW3, ...  Its m-th unit sits in ring slot m % kRing3 and its
  // weights are requested kRing3 - 1 units before that unit computes, so a
  // wave always has the next units' loads in flight behind the current one.
  int sj[kRing3], bsb[kRing3];  // per slot: slot of token c, super-block
  bool rl[kRing3];              // per slot: a selected expert's unit (not padding)
  Q2kW W[kRing3];
  Mx4Sb WM[kRing3];  // MXFP4: the lane's two blocks of the unit's super-block
  Q4kSb WQ[kRing3];  // Q4K: the same, with the block's scale words
  const Q2kOff off = q2k_offsets(mb, nb, row0, c, q);
  const size_t mx_bytes = Q4 ? mb * 144 : (size_t)d * f * 17 / 32;  // one packed MXFP4 / Q4K [d, f] matrix
  const uint32_t mx_codes = (uint32_t)((size_t)(row0 + c) * (f / 2) + 32 * q);
  const uint32_t mx_sc = (uint32_t)((size_t)d * f / 2 + (size_t)(row0 + c) * (f / 32) + 2 * q);
  const uint32_t q4_sc = (uint32_t)(mb * 128 + (size_t)(row0 + c) * nb * 12);
  const uint32_t q4_sp = (uint32_t)(mb * 140 + (size_t)(row0 + c) * nb * 4);
  const uint32_t ebytes = (uint32_t)(MX || Q4 ? mx_bytes : mb * 84);  // one expert's packed down matrix
  // unstaged activations come from the buffers rh and rs: a lane whose
  // token has no slot for the unit's expert reads zeros (offset kOob), so
  // its products are zero and need no mask
  // the unit to request next as (major, minor) index, stepped by kW3
  // without a division per unit
  const int nmin = PH ? nde : nb;
  const int dmaj = kW3 / nmin, dmin = kW3 % nmin;
  int pmaj = wave / nmin, pmin = wave - (wave / nmin) * nmin;
  auto load_unit = [&](int r) {  // r: ring slot, fixed once unrolled
    int i = PH ? pmin : pmaj, b = PH ? pmaj : pmin;
    if (!PH && i >= nd) {  // past the end and never computed: no loads
      pmaj += dmaj;
      pmin += dmin;
      if (pmin >= nmin) {
        pmin -= nmin;
        ++pmaj;
      }
      return;
    }
    if (PH && b >= nb) {  // past the end: the last unit again (the phased walk sends a fixed count)
      i = nd - 1;
      b = nb - 1;
    }
    rl[r] = i < nd;
    i = min(i, nd - 1);
    const int e = clamp_index(ld_uniform(distinct + i), L.n_experts);
    // the expert's matrix as a buffer: the lane's offsets stay in VGPRs, the
    // super-block's goes in an SGPR, so no per-unit address arithmetic
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(down + (size_t)e * ebytes, ebytes);
    if constexpr (Q4) {
      WQ[r].c0 = buf_ld128<kBufNt>(rw, mx_codes, 128 * b);
      WQ[r].c1 = buf_ld128<kBufNt>(rw, mx_codes + 16, 128 * b);
      const u32x3_t sw = buf_ld96(rw, q4_sc, 12 * b);  // one 12-byte load
      WQ[r].w0 = sw.x;
      WQ[r].w1 = sw.y;
      WQ[r].w2 = sw.z;
      WQ[r].sup = buf_ld32(rw, q4_sp, 4 * b);
    } else if constexpr (MX) {
      WM[r].c0 = buf_ld128<kBufNt>(rw, mx_codes, 128 * b);
      WM[r].c1 = buf_ld128<kBufNt>(rw, mx_codes + 16, 128 * b);
      WM[r].sc = buf_ld16(rw, mx_sc, 8 * b);
    } else {
      W[r].codes = buf_ld128<kBufNt>(rw, off.codes, 64 * b);
      W[r].sc4 = buf_ld32(rw, off.sc, 16 * b);
      W[r].mins = buf_ld64(rw, off.mins, 16 * b);
      W[r].sup = buf_ld32(rw, off.sup, 4 * b);
    }
    sj[r] = tok_slot[i * kDecodeGroup + c];
    bsb[r] = b;
    pmaj += dmaj;
    pmin += dmin;
    if (pmin >= nmin) {
      pmin -= nmin;
      ++pmaj;
    }
  };
#pragma unroll
  for (int r = 0; r < kRing3 - 1; ++r) load_unit(r);
#pragma unroll
  for (int r = 0; r < kRing3 - 1; ++r) asm volatile("" ::"v"(sj[r]));  // keeps these loads ahead of the barrier
  asm volatile("" ::"s"(nd));
  wait_all();  // the copies (and the first units)
  __syncthreads();
  // PH, with the experts padded to at least 32: every wave has at least two
  // units a phase and meets at most one phase change a unit.  Entering
  // phase p, a wave sends its chunks of phase p + 1; at least two units'
  // kLdU weight loads follow them before it enters p + 1, so its copies are
  // done once all but the last 2 kLdU loads are (the weights of the next
  // two units stay in flight).  The barrier then publishes everyone's copies
  // and shows every wave done with the buffer the next phase's copy
  // overwrites.
  const bool phased = PH;
  constexpr int kLdU = MX ? 4 : 5;  // vector-memory instructions of load_unit
  int cur = 0;  // phased: the phase (super-block) in LDS buffer cur % 2
  if (PH) send_phase(min(1, nb - 1));  // one phase only: its own chunks again, unchanged data
  // the shared expert's down rows (this wave's K-steps)
  const uint16_t* srow = L.sh_down + (int64_t)(row0 + c) * fs;
  int sk0, sk1;
  split_range(fs / 32, kW3, wave, sk0, sk1);
  constexpr int kBatchS = 4;
  half8_t sa[kBatchS];
  auto load_sa = [&]() {
#pragma unroll
    for (int j = 0; j < kBatchS; ++j) sa[j] = *(const half8_t*)(srow + max(min(sk0 + j, sk1 - 1), 0) * 32 + 8 * q);
    pin();
  };
  // they stream in while the routed units compute, except in the phased
  // form, where their registers are worth more to the routed loop
  if constexpr (!PH) load_sa();
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  // one step: activations of the slot's unit, the request of the unit
  // kRing3 - 1 ahead into the slot freed last step, then the products.
  // Global activations go out before that request (a wait for them then
  // leaves it in flight); LDS ones after it (the expert id's scalar load
  // is waited for with a count that would include them).
  auto routed = [&](auto phased_tag) {
    constexpr bool P = decltype(phased_tag)::value;  // activations from the phase buffers
    for (int m0 = 0;; m0 += kRing3) {
#pragma unroll
      for (int r = 0; r < kRing3; ++r) {
        if (wave + (m0 + r) * kW3 >= nunits) return;
        if constexpr (P) {
          if (bsb[r] != cur) {  // the next phase (wave-uniform)
            vm_wait<2 * kLdU>();
            ring_barrier();
            cur = bsb[r];
            send_phase(min(cur + 1, nb - 1));  // in the last phase: its own chunks again, unchanged data
          }
          pin();
        }
        const int slot = sj[r];  // slot of token c for this unit's expert
        const bool has = rl[r] && slot >= 0 && slot < S;  // tokens without a slot add nothing
        // staged: every lane reads a valid row and the products of tokens
        // without a slot are masked (tokens 4q..4q+3); unstaged: those
        // tokens read zeros, which leaves Q2K products exactly zero (its
        // weights are small integers), while MXFP4 and Q4K weights, scaled
        // in binary16, keep the mask in case a scale overflowed to inf
        // Q2K, phased: tokens without a slot (and the min sums of lane
        // groups q >= 2) read the buffer's zero rows, whose products are
        // exactly zero, so no mask
        constexpr bool kZeroRows = P && !MX && !Q4;
        const uint32_t vmask = (BL || P || MX || Q4) && !kZeroRows ? (uint32_t)(__ballot(has) >> (4 * q)) & 15u : 15u;
        const int row = has ? slot : (kZeroRows ? S : 0);
        const int b = bsb[r];  // super-block
        Q2kA A;
        auto act = [&]() {
          if constexpr (BL || P) {
            const _Float16* bcol = BL ? s_h + (size_t)row * f + b * QK : ph_h(b) + (size_t)row * QK;
            if constexpr (MX || Q4) {
#pragma unroll
              for (int s2 = 0; s2 < 8; ++s2) A.b[s2] = *(const half8_t*)(bcol + q2k_boff(q, s2));
            } else if constexpr (BL) {
              q2k_act(A, bcol, s_cs + (size_t)row * fs16 + b * 16, s_cs + (size_t)(S + row) * fs16 + b * 16, q);
            } else {
              const bool sm = has && q < 2;  // hi and lo sum rows, else the zero row
              q2k_act(A, bcol, ph_cs(b) + (size_t)(sm ? row : 2 * S) * 16, ph_cs(b) + (size_t)(sm ? S + row : 2 * S) * 16,
                      q);
            }
          } else {
            // byte offsets: row * 2f + 2 q2k_boff(q, s2) in the activations,
            // row * 2 fs16 + 16 (q & 1) in the hi sums, S * 2 fs16 further on
            // in the lo sums; the super-block's part is wave-uniform
            const uint32_t vo = has ? (uint32_t)row * (uint32_t)(2 * f) + 128u * q : kOob;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) A.b[s2] = as_half8(buf_ld128(rh, vo + 16u * s2, (uint32_t)b * (2 * QK)));
            if constexpr (!MX && !Q4) {  // lane groups q >= 2 take zero sums (their min operand is unused)
              const uint32_t vs = has && q < 2 ? (uint32_t)row * (uint32_t)(2 * fs16) + 16u * q : kOob;
              A.bh = as_half8(buf_ld128(rs, vs, (uint32_t)b * 32u));
              A.bl = as_half8(buf_ld128(rs, vs, (uint32_t)b * 32u + (uint32_t)(S * fs16 * 2)));
            }
          }
        };
        if (!BL && !P) act();
        pin();
        load_unit((r + kRing3 - 1) % kRing3);
        pin();
        if (BL || P) act();
        if constexpr (Q4) q4k_unit(WQ[r], A, vmask, q, acc);
        else if constexpr (MX) mx4_unit(WM[r], A, vmask, acc);
        else q2k_unit<BL>(W[r], A, vmask, q, acc);
      }
    }
  };
  if (phased) {
    routed(std::true_type{});
    // every wave meets every phase's barrier and sends its chunks of each
    while (cur < nb - 1) {
      vm_wait<0>();
      ring_barrier();
      ++cur;
      send_phase(min(cur + 1, nb - 1));
    }
  } else {
    if constexpr (!PH) routed(std::false_type{});
  }
  // shared expert, transposed like the routed units: lane (c, q) ends with
  // tokens 4q..4q+3 of row row0 + c
  if constexpr (PH) load_sa();
  float4_t accs = {0.f, 0.f, 0.f, 0.f};
  {
    auto getb = [&](int kk, half8_t& bh, half8_t&) {
      bh = BL ? *(const half8_t*)(s_hs + tc * fs + kk) : *(const half8_t*)(hs16 + (int64_t)tc * fs + kk);
    };
    f16_steps<false, BL, kBatchS, decltype(getb), true>(srow, sk0, sk1, q, sa, getb, accs);
  }
  s_red[wave][lane] = acc;  // lane (c, q): tokens 4q + r of row row0 + c
  s_red2[wave][lane] = accs;
  __syncthreads();
  if (wave == 0) {
    float4_t ar = s_red[0][lane], as = s_red2[0][lane];
#pragma unroll
    for (int w = 1; w < kW3; ++w) {
      ar += s_red[w][lane];
      as += s_red2[w][lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q + r < T) y[(int64_t)(4 * q + r) * d + row0 + c] = as[r] + ar[r];
  }
}

// ============================================================== stage 3, one token
// With one token the MFMA's 16 token columns would carry one useful column,
// so the routed down product runs on v_dot2_f32_f16 instead, each lane
// over its own row.  Codes become binary16 without a per-weight rescale: a
// three-input bit operation puts the two codes of a pair (codes i and i + 8
// of a sub-block, the same bits of its two 16-bit halves) into the low
// mantissa bits under an exponent that gives them unit weight, so each half
// reads base + q exactly, base being 64, 16 or 4 for mantissa bit 4, 6 or 8.
// The dot product of a sub-block's 8 pairs with (h_i, h_{i+8}) is then
// sum_k q_k h_k + OFF, OFF = sum_k base_k h_k, and the sub-block adds
// d s (dot - OFF) - dmin m HS with HS = sum_k h_k.  OFF and HS come from the
// same binary16 h, once per block.
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_half2(a), as_half2(b), c, false);
}

// Block `tile` (16 waves): output rows tile*16 .. +15 of token 0.  Lane
// (c, q) works on row row0 + c, sub-blocks 4q .. 4q + 3 of each unit's
// super-block.  LDS: h as pairs [S][f/16][8] (u32), OFF and HS [S][f/16]
// (fp32), the shared expert's h [fs] (binary16).
__global__ __launch_bounds__(kW3 * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_stage3_one(
    ds4moe_layer L, const int32_t* __restrict__ ndist, const int32_t* __restrict__ distinct,
    const int32_t* __restrict__ tok_slot, const _Float16* __restrict__ hw16, const _Float16* __restrict__ hs16,
    int32_t* __restrict__ ctrl, int nctrl1, int maxd, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ float s_row[kW3][16];
  __shared__ float4_t s_red2[kW3][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int d = L.d_model, f = L.d_ff, k = L.top_k, fs = L.d_ff_shared;
  const int tile = blockIdx.x, row0 = tile * 16;
  const int nb = f / QK, nsb = f / 16;
  const size_t mb = (size_t)d * nb;
  const int S = k;  // one token: k slots
  uint32_t* s_pair = (uint32_t*)s_dyn;                   // [S][nsb][8]
  float* s_off = (float*)(s_pair + (size_t)S * nsb * 8);  // [S][nsb]
  float* s_hs = s_off + (size_t)S * nsb;                  // [S][nsb]
  _Float16* s_sh = (_Float16*)(s_hs + (size_t)S * nsb);   // [fs]
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctrl1; i += blockDim.x) ctrl[i] = 0;
  const uint8_t* down = (const uint8_t*)L.down;
  const int nd = min(ld_uniform(ndist), maxd);
  const int maxunits = maxd * nb, nunits = nd * nb;
  // units u = (expert slot u / nb, super-block u % nb); wave w takes
  // u = w, w + kW3, ... in batches of kUnits3
  struct W1 {
    u32x4_t codes;  // sub-blocks 4q .. 4q + 3 of the lane's row
    uint32_t sc4;   // their scale/min bytes
    uint32_t sup;   // (d, dmin) of the lane's row
  };
  W1 W[kUnits3];
  int ib[kUnits3][2];  // per unit: slot of the token for its expert, super-block
  const uint32_t o_codes = (uint32_t)((size_t)(row0 + c) * nb * 64 + 16 * q);
  const uint32_t o_sc = (uint32_t)(mb * 64 + (size_t)(row0 + c) * nb * 16 + 4 * q);
  const uint32_t o_sup = (uint32_t)(mb * 80 + (size_t)(row0 + c) * nb * 4);
  auto load_batch = [&](int u0) {
    int ej[kUnits3];
#pragma unroll
    for (int j = 0; j < kUnits3; ++j) {  // units past the end repeat the last one
      const int u = min(u0 + j * kW3, maxunits - 1);
      const int i = u / nb;  // distinct expert
      ib[j][1] = u - i * nb;
      ej[j] = ld_uniform(distinct + i);  // all ids and slots in flight before the first address needs one
      ib[j][0] = clamp_index(ld_uniform(tok_slot + i * kDecodeGroup), S);
    }
    pin();
#pragma unroll
    for (int j = 0; j < kUnits3; ++j) {
      const uint8_t* base = down + (size_t)clamp_index(ej[j], L.n_experts) * mb * 84;
      const int b = ib[j][1];
      W[j].codes = __builtin_nontemporal_load((const u32x4_t*)(base + o_codes + b * 64));
      W[j].sc4 = *(const uint32_t*)(base + o_sc + b * 16);
      W[j].sup = *(const uint32_t*)(base + o_sup + b * 4);
    }
  };
  load_batch(wave);
  // staging: the routed h as pairs with their OFF and HS sums, one
  // (slot, sub-block) per thread; the shared expert's h by copy
  dma_rows(hs16, fs, 1, fs, s_sh, fs, wave, kW3, lane);
  for (int t = threadIdx.x; t < S * nsb; t += blockDim.x) {
    // h is pair-interleaved already: binary16 pair i holds rows i and i + 8
    const u32x4_t p0 = *(const u32x4_t*)(hw16 + (size_t)t * 16), p1 = *(const u32x4_t*)(hw16 + (size_t)t * 16 + 8);
    const half8_t h0 = as_half8(p0), h1 = as_half8(p1);
    auto row_i = [&](int i) { return (float)(i < 4 ? h0[2 * i] : h1[2 * (i - 4)]); };             // row i
    auto row_i8 = [&](int i) { return (float)(i < 4 ? h0[2 * i + 1] : h1[2 * (i - 4) + 1]); };  // row i + 8
    float off = 0.0f, hs = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) off += (float)q2k_pair_base(i) * (row_i(i) + row_i8(i));
#pragma unroll
    for (int i = 0; i < 8; ++i) hs += row_i(i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hs += row_i8(i);
    *(u32x4_t*)(s_pair + (size_t)t * 8) = p0;
    *(u32x4_t*)(s_pair + (size_t)t * 8 + 4) = p1;
    s_off[t] = off;
    s_hs[t] = hs;
  }
#pragma unroll
  for (int j = 0; j < kUnits3; ++j) asm volatile("" ::"v"(W[j].sup));  // keeps these loads ahead of the barrier
  wait_all();
  __syncthreads();
  // the shared expert's down rows stream in while the routed units compute
  const uint16_t* srow = L.sh_down + (int64_t)(row0 + c) * fs;
  int sk0, sk1;
  split_range(fs / 32, kW3, wave, sk0, sk1);
  constexpr int kBatchS = 4;
  half8_t sa[kBatchS];
#pragma unroll
  for (int j = 0; j < kBatchS; ++j) sa[j] = *(const half8_t*)(srow + max(min(sk0 + j, sk1 - 1), 0) * 32 + 8 * q);
  pin();
  float yr = 0.0f;  // row row0 + c, this lane's sub-blocks
  for (int u0 = wave; u0 < maxunits; u0 += kW3 * kUnits3) {
    if (u0 != wave) load_batch(u0);
    pin();
#pragma unroll
    for (int j = 0; j < kUnits3; ++j) {
      if (u0 + j * kW3 >= nunits) continue;  // wave-uniform
      const int sbase = ib[j][0] * nsb + ib[j][1] * 16 + 4 * q;  // (slot, first sub-block) of the lane
      const float4_t off4 = *(const float4_t*)(s_off + sbase), hs4 = *(const float4_t*)(s_hs + sbase);
      float as = 0.0f, am = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x4_t h0 = *(const u32x4_t*)(s_pair + (size_t)(sbase + jj) * 8);
        const u32x4_t h1 = *(const u32x4_t*)(s_pair + (size_t)(sbase + jj) * 8 + 4);
        uint32_t w[8];
        q2k_pairs_unit_weight(W[j].codes[jj], w);
        float acc = dot2(w[0], h0.x, 0.0f);
        acc = dot2(w[1], h0.y, acc);
        acc = dot2(w[2], h0.z, acc);
        acc = dot2(w[3], h0.w, acc);
        acc = dot2(w[4], h1.x, acc);
        acc = dot2(w[5], h1.y, acc);
        acc = dot2(w[6], h1.z, acc);
        acc = dot2(w[7], h1.w, acc);
        const uint32_t sm = (W[j].sc4 >> (8 * jj)) & 0xFFu;
        as += (float)(sm & 15u) * (acc - off4[jj]);
        am += (float)(sm >> 4) * hs4[jj];
      }
      const float dd = h2f((uint16_t)(W[j].sup & 0xFFFFu)), dm = h2f((uint16_t)(W[j].sup >> 16));
      yr += dd * as - dm * am;
    }
  }
  // shared expert, transposed MFMA: lane (c, 0) ends with token 0 of row c
  float4_t accs = {0.f, 0.f, 0.f, 0.f};
  {
    auto getb = [&](int kk, half8_t& bh, half8_t&) { bh = *(const half8_t*)(s_sh + kk); };
    f16_steps<false, true, kBatchS, decltype(getb), true>(srow, sk0, sk1, q, sa, getb, accs);
  }
  // row sums over the four lane groups, then over the waves
  yr += __shfl_xor(yr, 16);
  yr += __shfl_xor(yr, 32);
  if (q == 0) s_row[wave][c] = yr;
  s_red2[wave][lane] = accs;
  __syncthreads();
  if (wave == 0 && q == 0) {
    float ar = s_row[0][c], as = s_red2[0][lane][0];
#pragma unroll
    for (int w = 1; w < kW3; ++w) {
      ar += s_row[w][c];
      as += s_red2[w][lane][0];
    }
    y[row0 + c] = as + ar;
  }
}

// ============================================================== launcher
template <bool LO, bool BL, bool MX, bool Q4, int NS = kStageHalves>
static void launch_stages12(const Fwd& f, int rblocks, int nsh, int maxd, int nr, const RouteOut& ro) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  auto xh = (_Float16*)(ws + y.x_hi);
  auto xl = LO ? (_Float16*)(ws + y.x_lo) : nullptr;
  auto plog = (float*)(ws + y.plog);
  auto ctrl = (int32_t*)(ws + y.ctrl);
  auto gu = (float*)(ws + y.gu_part);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (_Float16*)(ws + y.hsum);
  const dim3 blk(kW * 64);
  // the shared expert's gate/up blocks: for a group of tokens behind the
  // router's in stage 1 (its 2 MB leave the chip idle), for one token behind
  // the routed gate/up blocks of stage 2 (whose stream they overlap best)
  if (T >= 12) {  // the finish sums 16 logits' partials at a time
    DS4_LAUNCH((k_dec_stage1<LO, true, 16>), dim3(rblocks + 2 * kShSplit * nsh), blk, 0, f.st, L, T, f.x, rblocks,
               plog, ro, xh, xl, gu, hs16, ctrl);
    DS4_LAUNCH((k_dec_stage2<LO, BL, MX, Q4, NS>), dim3(maxd * nr), blk, 0, f.st, L, T, ro, xh, xl, hw16, hsum,
               maxd * nr, gu, hs16, ctrl);
  } else if (T > 1) {
    DS4_LAUNCH((k_dec_stage1<LO, true>), dim3(rblocks + 2 * kShSplit * nsh), blk, 0, f.st, L, T, f.x, rblocks, plog,
               ro, xh, xl, gu, hs16, ctrl);
    DS4_LAUNCH((k_dec_stage2<LO, BL, MX, Q4, NS>), dim3(maxd * nr), blk, 0, f.st, L, T, ro, xh, xl, hw16, hsum,
               maxd * nr, gu, hs16, ctrl);
  } else {
    DS4_LAUNCH((k_dec_stage1<LO, false>), dim3(rblocks), blk, 0, f.st, L, T, f.x, rblocks, plog, ro, xh, xl, gu, hs16,
               ctrl);
    DS4_LAUNCH((k_dec_stage2<LO, BL, MX, Q4, NS>), dim3(maxd * nr + 2 * kShSplit * nsh), blk, 0, f.st, L, T, ro, xh,
               xl, hw16, hsum, maxd * nr, gu, hs16, ctrl);
  }
}

hipError_t launch_decode(const Fwd& f) {
  const ds4moe_layer& L = f.L;
  const WsLayout& y = f.lay;
  char* ws = f.ws;
  const int T = (int)f.T;
  const int d = L.d_model, E = L.n_experts, fs = L.d_ff_shared;
  const int rblocks = ((E + 15) / 16) * (d / router_chunk(d));
  const int nsh = fs / 16, nr = L.d_ff / 16, ndt = d / 16;
  const int maxd = std::min(E, T * L.top_k);
  const RouteOut ro = route_out(f);
  // stage 2 stages the group's x in LDS once per block when it fits: one
  // token (kStageHalves) or, with a larger block footprint of its own, a few
  // (kStageHalvesGroup, binary16 x only); else each wave stages the
  // super-block it decodes next
  const bool bl = (int64_t)T * d <= kStageHalves;
  const bool blg = !bl && !f.lo && (int64_t)T * d <= kStageHalvesGroup;
  const bool mx = L.expert_fmt == DS4MOE_EXPERTS_MXFP4, q4 = L.expert_fmt == DS4MOE_EXPERTS_Q4K;
#define DS4_S12(LO_, BL_, ...)                                                                   \
  (mx   ? launch_stages12<LO_, BL_, true, false, ##__VA_ARGS__>(f, rblocks, nsh, maxd, nr, ro)   \
   : q4 ? launch_stages12<LO_, BL_, false, true, ##__VA_ARGS__>(f, rblocks, nsh, maxd, nr, ro)   \
        : launch_stages12<LO_, BL_, false, false, ##__VA_ARGS__>(f, rblocks, nsh, maxd, nr, ro))
  if (f.lo) {
    if (bl) DS4_S12(true, true);
    else DS4_S12(true, false);
  } else {
    if (bl) DS4_S12(false, true);
    else if (blg) DS4_S12(false, true, kStageHalvesGroup);
    else DS4_S12(false, false);
  }
#undef DS4_S12
  auto ctrl = (int32_t*)(ws + y.ctrl);
  auto hs16 = (const _Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto hsum = (_Float16*)(ws + y.hsum);  // hi plane [S][f/16], then lo plane
  const int S = T * L.top_k;
  // stage 3 stages the routed activations, their sums and the shared
  // expert's activations
  const size_t stage_bytes =
      (size_t)S * L.d_ff * 2 + (size_t)2 * S * (L.d_ff / 16) * 2 + (size_t)T * L.d_ff_shared * 2;
  const dim3 blk3(kW3 * 64);
  // one token: the dot-product form (pairs, OFF and HS sums, shared h)
  const size_t one_bytes = (size_t)L.top_k * L.d_ff * 2 + (size_t)2 * L.top_k * (L.d_ff / 16) * 4 +
                           (size_t)L.d_ff_shared * 2;
  if (T == 1 && one_bytes <= kStage3OneBytes && !mx && !q4) {
    DS4_LAUNCH(k_dec_stage3_one, dim3(ndt), blk3, one_bytes, f.st, L, ro.ndist, ro.distinct, ro.tok_slot, hw16,
               hs16, ctrl, ctrl_ints(L), maxd, f.y);
    return hipGetLastError();
  }
#define DS4_S3(BL_, MX_, Q4_, BYTES, ...)                                                                        \
  DS4_LAUNCH((k_dec_stage3<BL_, MX_, Q4_, ##__VA_ARGS__>), dim3(ndt), blk3, BYTES, f.st, L, T, ro.ndist, ro.distinct, \
             ro.tok_slot, hw16, hsum, hs16, ctrl, ctrl_ints(L), maxd, f.y)
  // else one super-block's columns at a time, double-buffered (rows padded
  // as the kernel pads them, its 1 KB sink; at most 4 h and 1 sums copy
  // chunks a wave and phase)
  const int ph_hrows = (S + 2) & ~1, ph_srows = mx || q4 ? 0 : (2 * S + 32) & ~31;
  const size_t phase_bytes = (size_t)2 * (ph_hrows * QK * 2 + ph_srows * 32) + 1024;
  const bool ph_fits = phase_bytes <= kStage3Bytes && ph_hrows / 2 <= 4 * kW3 && ph_srows / 32 <= kW3;
  if (stage_bytes <= kStage3Bytes) {
    if (mx) DS4_S3(true, true, false, stage_bytes);
    else if (q4) DS4_S3(true, false, true, stage_bytes);
    else DS4_S3(true, false, false, stage_bytes);
  } else if (ph_fits) {
    if (mx) DS4_S3(false, true, false, phase_bytes, true);
    else if (q4) DS4_S3(false, false, true, phase_bytes, true);
    else DS4_S3(false, false, false, phase_bytes, true);
  } else {
    if (mx) DS4_S3(false, true, false, 0);
    else if (q4) DS4_S3(false, false, true, 0);
    else DS4_S3(false, false, false, 0);
  }
#undef DS4_S3
  return hipGetLastError();
}

}  // namespace ds4
