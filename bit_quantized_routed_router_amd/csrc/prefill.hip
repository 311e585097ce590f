// Prefill (any T): grouped expert products over the work list of (expert,
// run of up to 128 of its slots) tiles built by the grouping kernels; the
// dense shared expert runs first (dense.hip: hs16 and y = Wsd hs16).
//
//   k_pf_gateup          hw16[p] = w_s * silu(G_e x_t) * (U_e x_t)    (binary16)
//   k_pf_down            yp[s]   = D_e hw16[p]                         (fp32)
//   k_combine            y[t]   += sum_j yp[t*k + j], j ascending
// Slots s = t*k + j sit at position p of the expert-sorted list (perm[p] = s).
// The combine order is fixed, so results are deterministic.
//
// Grouped GEMM.  A block takes one work tile (a routed expert's run of up to
// 128 slots) and a slice of output rows.  Each of its four waves owns four 16-row weight fragments
// and all of the tile's slots (up to eight 16-slot fragments), so a weight is
// decoded once per tile and a staged activation fragment feeds four MFMAs
// (v_mfma_f32_16x16x32_f16 with the slots as A rows and the weights as B
// columns: lane (c, q) holds slots 4q..4q+3 of weight row c).  Activation
// chunks of 128 inputs are copied straight into LDS (global_load_lds), double
// buffered, in a layout whose 16-byte pieces are XOR-swizzled by row so that
// the fragment reads of 16 rows hit distinct banks.  Inside a chunk the
// K-steps are permuted so that a lane's weight codes for the whole chunk are
// one 8-byte piece of its row (CB2: one sub-block; Q2K: two sub-blocks): at
// step j lane group q covers inputs 32q + 8j .. +7 of the chunk, and the
// activation fragments are read at the same offsets.  Routed weights are
// decoded to binary16 with the block scales folded in (CB2: d*(2s+1) rounded
// to binary16, then its product with sign*m; Q2K: d*s and dmin*m rounded to
// binary16, then q*(d*s) - dmin*m rounded once); F16 weights are used as
// stored.  The MFMA accumulates in fp32.  Work items are laid out so that each XCD takes a contiguous
// range (blocks are dealt to the 8 XCDs round-robin): the row slices of one
// tile and the tiles of one expert share that XCD's L2.
#include <algorithm>

#include "common.h"
#include "ring.h"
#include "internal.h"
#include "trace.h"

namespace ds4 {

__constant__ GridTables c_pre_tables = make_grid_tables();



constexpr int kTT = kPrefillTile;  // slots per work tile (128)
constexpr int kKC = 128;           // inputs per staged activation chunk
constexpr int kGW = 4;             // waves per block
constexpr int kChunk = kTT * kKC;  // halves per staged chunk of 128 rows (32 KB)
// Halves of a block's activation ring: 64 KB for tiles of up to 128 slots,
// 32 KB for small tiles (<= 32 slots).
constexpr int ring_halves(bool small) { return small ? kChunk : 2 * kChunk; }

// Ring slots of a tile: as many as the activation ring holds (R * 16 NF
// rows of KC inputs) and the 6-bit load counter can track (R - 1 batches of
// `loads` vector-memory instructions in flight, <= 63), at most 6.
// Small tiles have little work per chunk, so they need the deepest prefetch.
constexpr int ring_depth(int nf, int loads, bool lo, int ring, int rmax = 6, int kc = kKC) {
  int r = lo ? 2 : rmax;
  while (r > 2 && (r * nf * 16 * kc > ring || (r - 1) * loads > 63)) --r;
  return r;
}

// Copy instructions per wave and chunk for 16 NF rows of KC inputs (one
// instruction moves 1 KB: 512 / KC rows) over NW waves; every wave issues the
// same number.
constexpr int dma_groups(int nf, int kc = kKC) { return nf * 16 * kc / 512; }
constexpr int dma_per_wave(int nf, int nw, int kc = kKC) { return (dma_groups(nf, kc) + nw - 1) / nw; }

// One KC-input chunk of the tile's first 16 NF activation rows into a
// swizzled LDS buffer: wave instruction m moves the P = 512 / KC rows of
// group g = wave + NW m, lane l writing physical piece l % (KC / 8) of row
// P g + l / (KC / 8), which holds logical piece (l % (KC / 8)) ^ (row & 15).
// row_of(r): element offset of tile row r from src (src is the same for the
// whole block, offsets fit 32 bits).
template <bool LO, int NF, int NW, int KC = kKC, typename RowOf>
__device__ inline void stage_rows(const _Float16* __restrict__ src, const _Float16* __restrict__ src_lo, RowOf row_of,
                                  int ch, _Float16* dh, _Float16* dl, int wave, int lane) {
  constexpr int kPieces = KC / 8, kRowsPer = 64 / kPieces;
#pragma unroll
  for (int m = 0; m < dma_per_wave(NF, NW, KC); ++m) {  // groups dealt to NW waves
    const int g = min(wave + NW * m, dma_groups(NF, KC) - 1);  // a spare slot repeats the last group (same bytes)
    const int r = kRowsPer * g + lane / kPieces;
    const int u = (lane % kPieces) ^ (r & 15);
    const uint32_t off = 2u * ((uint32_t)row_of(r) + (uint32_t)(ch * KC + 8 * u));
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)src + off),
                                     (__attribute__((address_space(3))) void*)(dh + g * kRowsPer * KC), 16, 0, 0);
    if (LO)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)src_lo + off),
                                       (__attribute__((address_space(3))) void*)(dl + g * kRowsPer * KC), 16, 0, 0);
  }
}

template <typename T>
__device__ inline T ld_at(const void* base, uint32_t byte_off) {
  return *(const T*)((const char*)base + byte_off);
}

// A fragment of slot fragment i at step j: row 16i + c, inputs (KC / 4) q + 8j .. +7.
template <int KC = kKC>
__device__ inline half8_t slot_frag(const _Float16* buf, int i, int c, int q, int j) {
  return *(const half8_t*)(buf + (16 * i + c) * KC + 8 * (((KC / 32) * q + j) ^ c));
}

// CB2 group j of a sub-block (index word idxw, aux word aux) as binary16
// sign * m * D, with D = binary16(d * (2s+1)) in both halves of D2.  The
// tables hold one byte per element (the high byte of binary16 sign * m, whose
// low byte is zero), 8 bytes an entry: the sign bytes are XORed in, then a
// byte permute widens two elements to a binary16 pair (low bytes zero) for
// the scale multiply.  mag/sgn point at this lane's copy of the tables, whose
// entries are TC copies apart.
template <int TC>
__device__ inline half8_t cb2_frag_scaled(uint32_t idxw, uint32_t aux, int j, const uint32_t* mag,
                                          const uint32_t* sgn, half2_t D2) {
  const uint32_t idx = (idxw >> (8 * j)) & 0xFFu;
  const uint32_t code = (aux >> (7 * j)) & 0x7Fu;
  const u32x2_t m = *(const u32x2_t*)(mag + 2 * TC * idx);
  const u32x2_t s = *(const u32x2_t*)(sgn + 2 * TC * code);
  const uint32_t b0 = m.x ^ s.x, b1 = m.y ^ s.y;
  // byte k of b -> high byte of a half: selector 0x0C yields a zero byte
  u32x4_t r;
  r.x = as_u32(as_half2(__builtin_amdgcn_perm(0u, b0, 0x010C000Cu)) * D2);
  r.y = as_u32(as_half2(__builtin_amdgcn_perm(0u, b0, 0x030C020Cu)) * D2);
  r.z = as_u32(as_half2(__builtin_amdgcn_perm(0u, b1, 0x010C000Cu)) * D2);
  r.w = as_u32(as_half2(__builtin_amdgcn_perm(0u, b1, 0x030C020Cu)) * D2);
  return as_half8(r);
}

__device__ inline float f16f(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }
__device__ inline half2_t h2splat(float v) {
  const _Float16 h = (_Float16)v;
  return (half2_t){h, h};
}

// Codebook tables in LDS (byte forms, 8 bytes an entry): TC interleaved
// copies of each entry, lane l reading copy l % TC.
template <int TC>
struct CbTables {
  uint32_t mag[256 * TC * 2];
  uint32_t sgn[128 * TC * 2];
  __device__ inline void stage(const GridTables& t) {
    for (int i = threadIdx.x; i < 256 * TC * 2; i += blockDim.x) mag[i] = t.mag8[i / (TC * 2)][i % 2];
    for (int i = threadIdx.x; i < 128 * TC * 2; i += blockDim.x) sgn[i] = t.sgn8[i / (TC * 2)][i % 2];
  }
};

// CB2 block scales staged per block: the first NBS blocks of each of the
// block's 128 gate and 128 up rows.  The scale plane of a row spans its whole
// K range, so read per chunk its cache lines stay live for the block's whole
// life and are evicted and fetched again; staged once, each is read once.
template <bool LO, int TC, int RING, int NBS>
struct GuLds {
  _Float16 xh[RING];
  _Float16 xl[LO ? RING : 8];
  CbTables<TC> tab;
  int tok[kTT];
  float w[kTT];
  uint16_t dsc[NBS ? 2 * 128 * NBS : 2];
};
template <bool MX = false, bool Q4 = false>
constexpr int gu_nbs() { return MX || Q4 ? 0 : 16; }

// Weights of one 128-input chunk for a lane's four fragments.  CB2: the lane's sub-block (8 bytes) and its block's d;
// with WIDE, chunks of 256 inputs (one block per row): the lane's two sub-blocks (16 bytes, in mw).
// kLoads counts the vector-memory loads of a chunk when every scale comes from LDS; kMaxLoads when they are all read
// from memory (blocks past the staged ones).
// MXFP4: the lane's 32 inputs of the chunk are one MX block, 16 code bytes and
// one scale byte per fragment.
// Q4K (Q4): the lane's 32 inputs are one sub-block, 16 code bytes, plus its
// super-block's three scale words and (d, dmin) word per fragment.
template <bool MX = false, bool Q4 = false, bool WIDE = false>
struct GuW {
  u32x2_t cw[MX || Q4 || WIDE ? 1 : 4];
  uint32_t dv[4];
  u32x4_t mw[MX || Q4 || WIDE ? 4 : 1];
  u32x3_t qs[Q4 ? 4 : 1];  // Q4K: the super-block's three scale words (one 12-byte load)
  int jq;  // Q4K: the lane's sub-block within its super-block (set at issue)
  static constexpr int kLoads = Q4 ? 12 : (MX ? 8 : 4);
  static constexpr int kMaxLoads = Q4 ? 12 : 8;
  // loads per chunk that size the ring: Q4K keeps the depth of 20 loads, which
  // its registers allow (a deeper ring spills)
  static constexpr int kRingLoads = Q4 ? 20 : kMaxLoads;
};

// Gate/up of one work tile (up to 128 slots) for a 128-row slice of h, NF
// slot fragments, routed expert e (CB2 weights, or MXFP4 with MX, Q4K with
// Q4; routing weights s.w), in chunks of KC inputs (CB2: 128 or 256).  FS:
// every block's scale is staged (d_model <= 256 NBS), so the scale reads are
// LDS reads only; otherwise blocks past the staged ones read theirs from
// memory (the compiler then forms one flat load over both address spaces,
// which the LDS waits of the compute also wait for).
template <bool LO, int NW, int TC, int RING, int NF, int NBS, bool MX = false, bool Q4 = false, int KC = kKC,
          bool FS = false>
__device__ __attribute__((always_inline)) inline void gateup_tile(const ds4moe_layer& L, GuLds<LO, TC, RING, NBS>& s,
                                                                  const _Float16* __restrict__ xh,
                                                                  const _Float16* __restrict__ xl, int e, int rt,
                                                                  int pos0, int n, _Float16* __restrict__ hout) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, q = lane >> 4;
  constexpr bool WIDE = KC == 2 * kKC;  // CB2, one block per row and chunk
  static_assert(KC == kKC || (WIDE && !MX && !Q4), "256-input chunks: CB2 only");
  using WT = GuW<MX, Q4, WIDE>;
  const int d = L.d_model, fd = L.d_ff, nb = d / QK, nch = d / KC;
  const size_t mb = (size_t)fd * nb;
  const size_t mat_bytes = Q4 ? mb * 144 : (MX ? (size_t)fd * d * 17 / 32 : mb * 66);
  const uint8_t* gb = (const uint8_t*)L.gate + (size_t)e * mat_bytes;
  const uint8_t* ub = (const uint8_t*)L.up + (size_t)e * mat_bytes;
  // CB2 d plane / MXFP4 scale plane / Q4K scale words
  const uint8_t* gd = gb + (Q4 ? mb * 128 : (MX ? (size_t)fd * d / 2 : mb * 64));
  const uint8_t* ud = ub + (Q4 ? mb * 128 : (MX ? (size_t)fd * d / 2 : mb * 64));
  const uint8_t* gsp = gb + mb * 140;  // Q4K (d, dmin) words
  const uint8_t* usp = ub + mb * 140;
  const int hr0 = rt * 32 * NW + 32 * wave;
  // fragment f: rows hr0 + 16 (f & 1) + c of gate (f < 2) or up (f >= 2)
  uint32_t rowu[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) rowu[h] = (uint32_t)((hr0 + 16 * h + c) * nb);
  auto load_w = [&](int ch, WT& W) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if constexpr (WIDE) {  // block ch of the row: sub-blocks 2q, 2q + 1
        const uint32_t blk = rowu[f & 1] + (uint32_t)ch;
        W.mw[f] = ld_at<u32x4_t>(f < 2 ? gb : ub, blk * 64u + 16u * (uint32_t)q);
        if (NBS > 0 && (FS || ch < NBS))
          W.dv[f] = s.dsc[((f >> 1) * 128 + 32 * wave + 16 * (f & 1) + c) * NBS + ch];
        else
          W.dv[f] = ld_at<uint16_t>(f < 2 ? gd : ud, blk * 2u);
      } else if constexpr (Q4) {  // row hr0 + 16 (f & 1) + c, sub-block 4 (ch & 1) + q of super-block ch / 2
        const uint32_t r = (uint32_t)(hr0 + 16 * (f & 1) + c), blk = r * (uint32_t)nb + (uint32_t)(ch >> 1);
        W.mw[f] = ld_at<u32x4_t>(f < 2 ? gb : ub, blk * 128u + 16u * (uint32_t)(4 * (ch & 1) + q));
        W.qs[f] = ld_at<u32x3_a4_t>(f < 2 ? gd : ud, blk * 12u);
        W.dv[f] = ld_at<uint32_t>(f < 2 ? gsp : usp, blk * 4u);
        W.jq = 4 * (ch & 1) + q;
      } else if constexpr (MX) {  // row hr0 + 16 (f & 1) + c, block 4 ch + q
        const uint32_t r = (uint32_t)(hr0 + 16 * (f & 1) + c), blk = (uint32_t)(4 * ch + q);
        W.mw[f] = ld_at<u32x4_t>(f < 2 ? gb : ub, r * (uint32_t)(d / 2) + 16u * blk);
        W.dv[f] = ld_at<uint8_t>(f < 2 ? gd : ud, r * (uint32_t)(d / 32) + blk);
      } else {
        const uint32_t blk = rowu[f & 1] + (uint32_t)(ch >> 1);
        W.cw[f] = ld_at<u32x2_t>(f < 2 ? gb : ub, blk * 64u + (uint32_t)(32 * (ch & 1) + 8 * q));
        if (NBS > 0 && (FS || (ch >> 1) < NBS))
          W.dv[f] = s.dsc[((f >> 1) * 128 + 32 * wave + 16 * (f & 1) + c) * NBS + (ch >> 1)];
        else
          W.dv[f] = ld_at<uint16_t>(f < 2 ? gd : ud, blk * 2u);
      }
    }
  };
  auto rows = [&](int r) { return s.tok[r] * d; };
  float4_t acc[4][NF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // Loads per chunk and lane.  The ring depth keeps the largest count within the load counter; the waits use the
  // smallest, which is exact when every scale is staged and waits longer than needed otherwise.
  constexpr int kDma = dma_per_wave(NF, NW, KC) * (LO ? 2 : 1);
  constexpr int kBatch = kDma + WT::kLoads;
  constexpr int R = ring_depth(NF, kDma + WT::kRingLoads, LO, RING, 6, KC);
  constexpr int kSlot = NF * 16 * KC;  // halves per ring slot
  static_assert(R * kSlot <= RING, "ring slots exceed the staging buffer");
  WT W[R];
  auto issue = [&](int ch, int u) {
    stage_rows<LO, NF, NW, KC>(xh, xl, rows, ch, s.xh + u * kSlot, s.xl + (LO ? u * kSlot : 0), wave, lane);
    load_w(ch, W[u]);
  };
  const uint32_t* tmag = s.tab.mag + 2 * (lane % TC);
  const uint32_t* tsgn = s.tab.sgn + 2 * (lane % TC);
  auto compute = [&](int u) {
    half2_t D2[4];
    float XS[4];  // MXFP4 block scales
    half2_t QD[4], QN[4];  // Q4K binary16 d*s and -dmin*m of the lane's sub-block
    if constexpr (Q4) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        q4k_scales(W[u].qs[f][0], W[u].qs[f][1], W[u].qs[f][2], W[u].dv[f], W[u].jq, QD[f], QN[f]);
    } else if constexpr (MX) {
#pragma unroll
      for (int f = 0; f < 4; ++f) XS[f] = e8m0_f32(W[u].dv[f] & 0xFFu);
    } else if constexpr (!WIDE) {
#pragma unroll
      for (int f = 0; f < 4; ++f) D2[f] = h2splat(f16f(W[u].dv[f]) * (float)(2 * (W[u].cw[f].y >> 28) + 1));
    }
    const _Float16* bh = s.xh + u * kSlot;
    const _Float16* bl = s.xl + (LO ? u * kSlot : 0);
    // step j: lane group q covers inputs (KC / 4) q + 8j .. +7 of the chunk
    auto step = [&](int j) {
      half8_t wf[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if constexpr (WIDE)  // sub-block 2q + j / 4: words (x, y) or (z, w)
          wf[f] = cb2_frag_scaled<TC>(j < 4 ? W[u].mw[f].x : W[u].mw[f].z, j < 4 ? W[u].mw[f].y : W[u].mw[f].w,
                                      j & 3, tmag, tsgn, D2[f]);
        else if constexpr (Q4)
          wf[f] = q4k_frag(W[u].mw[f][j], QD[f], QN[f]);
        else if constexpr (MX)
          wf[f] = mx4_frag(W[u].mw[f][j], XS[f]);
        else
          wf[f] = cb2_frag_scaled<TC>(W[u].cw[f].x, W[u].cw[f].y, j, tmag, tsgn, D2[f]);
      }
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const half8_t a = slot_frag<KC>(bh, i, c, q, j);
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(a, wf[f], acc[f][i]);
        if (LO) {
          const half8_t al = slot_frag<KC>(bl, i, c, q, j);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(al, wf[f], acc[f][i]);
        }
      }
    };
    if constexpr (WIDE) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // sub-block 2q + h: its scale, then its four steps
#pragma unroll
        for (int f = 0; f < 4; ++f)
          D2[f] = h2splat(f16f(W[u].dv[f]) * (float)(2 * ((h ? W[u].mw[f].w : W[u].mw[f].y) >> 28) + 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) step(4 * h + j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) step(j);
    }
  };
  ring_loop<R, kBatch>(nch, issue, compute);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * i + 4 * q + r;
      if (t < n) {
        const float wt = s.w[t];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          hout[(int64_t)(pos0 + t) * fd + hr0 + 16 * h + c] =
              (_Float16)(wt * (silu(acc[h][i][r]) * acc[h + 2][i][r]));
      }
    }
  }
}

// Item -> (work tile, row slice); false for blocks without work.
template <bool SMALL>
__device__ inline bool tile_of(int rowtiles, const int32_t* big, const int32_t* small, const int32_t* ntiles,
                               const int32_t* counts, const int32_t* offsets, int& e, int& rt, int& pos0, int& n) {
  const int32_t* tiles = SMALL ? small : big;
  const int ntile = ntiles[SMALL ? 1 : 0];
  int item;
  if (!xcd_item(ntile * rowtiles, item)) return false;
  const int tile = item / rowtiles;
  rt = item - tile * rowtiles;
  e = tiles[2 * tile];
  const int g = tiles[2 * tile + 1];
  pos0 = offsets[e] + kTT * g;
  n = min(kTT, counts[e] - kTT * g);
  return true;
}

// Slot fragments of a tile with n slots: small-tile kernels see 1-2, large
// ones 3-8.
#define DS4_NF_SWITCH(n, SMALL, CALL)                  \
  switch (((n) + 15) >> 4) {                           \
    case 1: if constexpr (SMALL) CALL(1); break;       \
    case 2: if constexpr (SMALL) CALL(2); break;       \
    case 3: if constexpr (!SMALL) CALL(3); break;      \
    case 4: if constexpr (!SMALL) CALL(4); break;      \
    case 5: if constexpr (!SMALL) CALL(5); break;      \
    case 6: if constexpr (!SMALL) CALL(6); break;      \
    case 7: if constexpr (!SMALL) CALL(7); break;      \
    default: if constexpr (!SMALL) CALL(8); break;     \
  }

// Routed gate/up over the work list into hw16.
// Waves per gate/up block (each owns 32 rows of h) and codebook table copies.
constexpr int kGuWaves = 4;
constexpr int kGuCopies = 1;

// SMALL: the small-tile list (at most 32 slots per tile, a smaller ring).
// MX / Q4: the routed experts are MXFP4 / Q4K.
template <bool LO, bool SMALL, bool MX = false, bool Q4 = false, bool FS = false>
__global__ __launch_bounds__((kGuWaves * 64))
__attribute__((amdgpu_waves_per_eu(LO ? 1 : 2))) void k_pf_gateup(
    ds4moe_layer L, const _Float16* __restrict__ xh, const _Float16* __restrict__ xl,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ stiles, const int32_t* __restrict__ ntiles,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float* __restrict__ topk_w, _Float16* __restrict__ hout) {
  constexpr int NW = kGuWaves, TC = kGuCopies, RING = ring_halves(SMALL);
  // small CB2 tiles: 256-input chunks, so that a lane's codes of a row are one
  // 16-byte load (a wave instruction reads 16 rows x 64 bytes)
  constexpr int kGuKC = SMALL && !MX && !Q4 ? 2 * kKC : kKC;
  constexpr int NBS = gu_nbs<MX, Q4>();
  static_assert(NW == 4, "the staged scales cover 4 waves x 32 rows");
  __shared__ GuLds<LO, TC, RING, NBS> s;
  int e, rt, pos0, n;
  if (!tile_of<SMALL>(L.d_ff / (32 * NW), tiles, stiles, ntiles, counts, offsets, e, rt, pos0, n)) return;
  if constexpr (!MX && !Q4) {
    s.tab.stage(c_pre_tables);
    // scales of rows rt*128 .. +127 of gate (g = 0) and up (g = 1), blocks 0 .. ns-1
    const int nb = L.d_model / QK, ns = min(nb, NBS);
    const size_t mb = (size_t)L.d_ff * nb;
    const uint16_t* gd = (const uint16_t*)((const uint8_t*)L.gate + (size_t)e * mb * 66 + mb * 64);
    const uint16_t* ud = (const uint16_t*)((const uint8_t*)L.up + (size_t)e * mb * 66 + mb * 64);
    for (int i = threadIdx.x; i < 2 * 128 * ns; i += blockDim.x) {
      const int g = i / (128 * ns), r = (i / ns) % 128, b = i % ns;
      s.dsc[(g * 128 + r) * NBS + b] = (g ? ud : gd)[(size_t)(rt * 128 + r) * nb + b];
    }
  }
  if ((int)threadIdx.x < kTT) {
    const int r = min((int)threadIdx.x, n - 1);
    const int slot = perm[pos0 + r];
    s.tok[threadIdx.x] = slot / L.top_k;
    s.w[threadIdx.x] = topk_w[slot];
  }
  __syncthreads();
#define DS4_GU(NF) gateup_tile<LO, NW, TC, RING, NF, NBS, MX, Q4, kGuKC, FS>(L, s, xh, xl, e, rt, pos0, n, hout)
  DS4_NF_SWITCH(n, SMALL, DS4_GU)
#undef DS4_GU
}

// Q2K scales staged per block: d/dmin (4 bytes per block) of the first NBS
// blocks and, with SC, the sub-block bytes (16 per block) too, for the
// block's 256 rows; rows padded by one word so that 16 rows read at once hit
// distinct banks.
template <int RING, int NBS, bool SC>
struct DnLds {
  _Float16 xh[RING];
  int slot[kTT];
  uint32_t sc[SC ? 256 * (4 * NBS + 1) : 1];
  uint32_t dd[NBS ? 256 * (NBS + 1) : 1];
};
// Staged Q2K blocks.  Small tiles: d/dmin and the sub-block bytes of the
// first 8 blocks, later blocks read from memory in the loop (DDS: every
// block staged, d_ff <= 2048, so the scale reads are LDS reads only).  Large tiles
// (the ring leaves room for d/dmin only): d/dmin when the whole row fits
// (d_ff <= 2048, DDS), with no in-loop fallback, which would not fit the
// register budget.
template <bool SMALL, bool DDS>
constexpr int dn_nbs() { return !SMALL && !DDS ? 0 : 8; }
constexpr int kDnStagedMax = 8;

// Down weights of one chunk.  Q2K: the lane's two sub-blocks of codes, the
// aligned word holding their two scale bytes, the block's d/dmin.  kLoads /
// kMaxLoads: vector-memory loads of a chunk with the scales staged in LDS /
// read from memory.  WIDE (Q2K, 256-input chunks, one block per row): the
// lane's four sub-blocks of codes (16 bytes, in mw) and the word of their
// four scale bytes.
template <bool SC, bool DD, bool MX = false, bool Q4 = false, bool WIDE = false>
struct DnW {
  u32x2_t cw[MX || Q4 || WIDE ? 1 : 4];
  uint32_t sc[4], dd[MX ? 1 : 4];
  u32x4_t mw[MX || Q4 || WIDE ? 4 : 1];  // MXFP4 / Q4K: the lane's 32 elements (16 code bytes); MXFP4's scale byte in sc
  u32x3_t qs[Q4 ? 4 : 1];  // Q4K: scale words (one 12-byte load); (d, dmin) in dd
  int jq;                   // Q4K: the lane's sub-block within its super-block
  static constexpr int kMaxLoads = Q4 ? 12 : (MX ? 8 : 12);
  static constexpr int kLoads = Q4 ? 12 : (MX ? 8 : 4 + (SC ? 0 : 4) + (DD ? 0 : 4));
  static constexpr int kRingLoads = Q4 ? 20 : kMaxLoads;  // as in GuW
};

// Down product of one work tile for a 256-row slice of the output (Q2K, or
// MXFP4 with MX, Q4K with Q4): yp[slot] = D_e h, in chunks of KC inputs
// (Q2K: 128 or 256).
template <int RING, int NF, int NBS, bool SC, bool FULL, bool MX = false, bool Q4 = false, int KC = kKC>
__device__ __attribute__((always_inline)) inline void down_tile(const ds4moe_layer& L, DnLds<RING, NBS, SC>& s,
                                                                const _Float16* __restrict__ hin, int e, int rt,
                                                                int pos0, int n, float* __restrict__ yp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, q = lane >> 4;
  constexpr bool WIDE = KC == 2 * kKC;
  static_assert(KC == kKC || (WIDE && !MX && !Q4), "256-input chunks: Q2K only");
  const int d = L.d_model, fd = L.d_ff, nb = fd / QK, nch = fd / KC;
  const size_t mb = (size_t)d * nb;
  const size_t mat_bytes = Q4 ? mb * 144 : (MX ? (size_t)d * fd * 17 / 32 : mb * 84);
  const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mat_bytes;
  // Q2K sub-scales / MXFP4 scale plane / Q4K scale words
  const uint8_t* sub = base + (Q4 ? mb * 128 : (MX ? (size_t)d * fd / 2 : mb * 64));
  const uint8_t* sup = base + (Q4 ? mb * 140 : mb * 80);
  const int r0 = rt * 256 + 64 * wave;
  const uint32_t row0 = (uint32_t)((r0 + c) * nb);  // fragment f: + 16 f nb
  using WT = DnW<SC, (NBS > 0), MX, Q4, WIDE>;
  auto load_w = [&](int ch, WT& W) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if constexpr (WIDE) {  // block ch of row r0 + 16 f + c: sub-blocks 4q .. 4q + 3
        const uint32_t blk = row0 + (uint32_t)(16 * f * nb + ch);
        W.mw[f] = ld_at<u32x4_t>(base, blk * 64u + 16u * (uint32_t)q);
        const int lr = 64 * wave + 16 * f + c;
        if (SC && (FULL || ch < NBS))
          W.sc[f] = s.sc[lr * (4 * NBS + 1) + 4 * ch + q];
        else
          W.sc[f] = ld_at<uint32_t>(sub, blk * 16u + 4u * (uint32_t)q);
        if (NBS > 0 && (FULL || ch < NBS))
          W.dd[f] = s.dd[lr * (NBS + 1) + ch];
        else
          W.dd[f] = ld_at<uint32_t>(sup, blk * 4u);
      } else if constexpr (Q4) {  // row r0 + 16 f + c, sub-block 4 (ch & 1) + q of super-block ch / 2
        const uint32_t r = (uint32_t)(r0 + 16 * f + c), blk = r * (uint32_t)nb + (uint32_t)(ch >> 1);
        W.mw[f] = ld_at<u32x4_t>(base, blk * 128u + 16u * (uint32_t)(4 * (ch & 1) + q));
        W.qs[f] = ld_at<u32x3_a4_t>(sub, blk * 12u);
        W.dd[f] = ld_at<uint32_t>(sup, blk * 4u);
        W.jq = 4 * (ch & 1) + q;
      } else if constexpr (MX) {  // row r0 + 16 f + c, block 4 ch + q
        const uint32_t r = (uint32_t)(r0 + 16 * f + c), blk = (uint32_t)(4 * ch + q);
        W.mw[f] = ld_at<u32x4_t>(base, r * (uint32_t)(fd / 2) + 16u * blk);
        W.sc[f] = ld_at<uint8_t>(sub, r * (uint32_t)(fd / 32) + blk);
      } else {
        const uint32_t blk = row0 + (uint32_t)(16 * f * nb + (ch >> 1));
        W.cw[f] = ld_at<u32x2_t>(base, blk * 64u + (uint32_t)(32 * (ch & 1) + 8 * q));
        const int lr = 64 * wave + 16 * f + c;
        if (SC && (FULL || (ch >> 1) < NBS))
          W.sc[f] = s.sc[lr * (4 * NBS + 1) + 4 * (ch >> 1) + 2 * (ch & 1) + (q >> 1)];
        else
          W.sc[f] = ld_at<uint32_t>(sub, blk * 16u + (uint32_t)(8 * (ch & 1) + 4 * (q >> 1)));
        if (NBS > 0 && (FULL || (ch >> 1) < NBS))
          W.dd[f] = s.dd[lr * (NBS + 1) + (ch >> 1)];
        else
          W.dd[f] = ld_at<uint32_t>(sup, blk * 4u);
      }
    }
  };
  const _Float16* hbase = hin + (int64_t)pos0 * fd;
  auto rows = [&](int r) { return min(r, n - 1) * fd; };
  float4_t acc[4][NF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // As in gate/up: the depth bounds the largest load count, the waits use the smallest.
  constexpr int kDma = dma_per_wave(NF, kGW, KC);
  constexpr int kBatch = kDma + WT::kLoads;
  constexpr int R = ring_depth(NF, kDma + WT::kRingLoads, false, RING,
                               RING < 2 * kChunk ? 3 : 6, KC);  // small: register budget
  constexpr int kSlot = NF * 16 * KC;
  static_assert(R * kSlot <= RING, "ring slots exceed the staging buffer");
  WT W[R];
  auto issue = [&](int ch, int u) {
    stage_rows<false, NF, kGW, KC>(hbase, nullptr, rows, ch, s.xh + u * kSlot, nullptr, wave, lane);
    load_w(ch, W[u]);
  };
  const half2_t k1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  auto compute = [&](int u) {
    const _Float16* bh = s.xh + u * kSlot;
    if constexpr (MX || Q4) {
      float XS[4];
      half2_t QD[4], QN[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if constexpr (Q4) q4k_scales(W[u].qs[f][0], W[u].qs[f][1], W[u].qs[f][2], W[u].dd[f], W[u].jq, QD[f], QN[f]);
        else XS[f] = e8m0_f32(W[u].sc[f] & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // code word j: inputs 32q + 8j .. +7 of the chunk
        half8_t wf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) wf[f] = Q4 ? q4k_frag(W[u].mw[f][j], QD[f], QN[f]) : mx4_frag(W[u].mw[f][j], XS[f]);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          const half8_t a = slot_frag(bh, i, c, q, j);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(a, wf[f], acc[f][i]);
        }
      }
      return;
    }
    // Q2K: sub-block h of the lane's chunk piece (2q + h, or 4q + h with WIDE)
    // feeds steps 2h, 2h+1
    auto half_chunk = [&](int h) {
      half2_t A2[4], nB2[4];         // binary16 d * s and -(dmin * m) of the sub-block
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t sm = (W[u].sc[f] >> (WIDE ? 8 * h : 16 * (q & 1) + 8 * h)) & 0xFFu;
        A2[f] = h2splat(f16f(W[u].dd[f]) * (float)(sm & 15u));
        nB2[f] = h2splat(-f16f(W[u].dd[f] >> 16) * (float)(sm >> 4));
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {  // Q2K: codes 8jj .. 8jj+7 of the sub-block
        const int j = 2 * h + jj;
        half8_t wf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          uint32_t word;
          if constexpr (WIDE) word = W[u].mw[f][h];
          else word = h ? W[u].cw[f].y : W[u].cw[f].x;
          const uint32_t fld = (word >> (16 * jj)) & 0xFFFFu;
          uint32_t pr[4];
          q2k_pairs(fld | (fld << 14), pr);
          u32x4_t a;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            a[p] = as_u32(__builtin_elementwise_fma(as_half2(pr[p]) + k1024, A2[f], nB2[f]));
          wf[f] = as_half8(a);
        }
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          const half8_t a = slot_frag<KC>(bh, i, c, q, j);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(a, wf[f], acc[f][i]);
        }
      }
    };
#pragma unroll
    for (int h = 0; h < (WIDE ? 4 : 2); ++h) half_chunk(h);
  };
  ring_loop<R, kBatch>(nch, issue, compute);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * i + 4 * q + r;
      if (t < n) {
        const int64_t row = (int64_t)s.slot[t] * d;
#pragma unroll
        for (int f = 0; f < 4; ++f) yp[row + r0 + 16 * f + c] = acc[f][i][r];
      }
    }
  }
}

// Routed down (Q2K, or MXFP4 with MX, Q4K with Q4) over the work list into yp.
template <bool SMALL, bool DDS, bool MX = false, bool Q4 = false>
__global__ __launch_bounds__(kGW * 64)
__attribute__((amdgpu_waves_per_eu(2))) void k_pf_down(
    ds4moe_layer L, const int32_t* __restrict__ tiles, const int32_t* __restrict__ stiles,
    const int32_t* __restrict__ ntiles, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const _Float16* __restrict__ hin, float* __restrict__ yp) {
  constexpr int RING = ring_halves(SMALL);
  constexpr int NBS = MX || Q4 ? 0 : dn_nbs<SMALL, DDS>();
  constexpr bool SC = SMALL && !MX && !Q4;
  // small Q2K tiles: 256-input chunks (a lane's codes of a row in one 16-byte load)
  constexpr int kDnKC = SMALL && !MX && !Q4 ? 2 * kKC : kKC;
  __shared__ DnLds<RING, NBS, SC> s;
  int e, rt, pos0, n;
  if (!tile_of<SMALL>(L.d_model / 256, tiles, stiles, ntiles, counts, offsets, e, rt, pos0, n)) return;
  if ((int)threadIdx.x < kTT) s.slot[threadIdx.x] = perm[pos0 + min((int)threadIdx.x, n - 1)];
  if constexpr (NBS > 0) {
    // scales of rows rt*256 .. +255, blocks 0 .. ns-1
    const int nb = L.d_ff / QK, ns = min(nb, NBS);
    const size_t mb = (size_t)L.d_model * nb;
    const uint8_t* base = (const uint8_t*)L.down + (size_t)e * mb * 84;
    const uint32_t* sub = (const uint32_t*)(base + mb * 64);
    const uint32_t* sup = (const uint32_t*)(base + mb * 80);
    if constexpr (SC) {
      for (int i = threadIdx.x; i < 256 * 4 * ns; i += blockDim.x) {
        const int r = i / (4 * ns), wd = i % (4 * ns);  // word wd of the row's first ns blocks
        s.sc[r * (4 * NBS + 1) + wd] = sub[(size_t)(rt * 256 + r) * nb * 4 + wd];
      }
    }
    for (int i = threadIdx.x; i < 256 * ns; i += blockDim.x) {
      const int r = i / ns, b = i % ns;
      s.dd[r * (NBS + 1) + b] = sup[(size_t)(rt * 256 + r) * nb + b];
    }
  }
  __syncthreads();
#define DS4_DN(NF) down_tile<RING, NF, NBS, SC, DDS, MX, Q4, kDnKC>(L, s, hin, e, rt, pos0, n, yp)
  DS4_NF_SWITCH(n, SMALL, DS4_DN)
#undef DS4_DN
}

// y[t][i] += sum_j yp[t*k + j][i] in ascending j, four columns per lane.
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
  const int64_t maxtiles = (S + kTT - 1) / kTT + E;  // >= the large-tile count; the small list holds <= E
  auto xh = (const _Float16*)(ws + y.x_hi);
  auto xl = f.lo ? (const _Float16*)(ws + y.x_lo) : nullptr;
  auto tiles = (const int32_t*)(ws + y.tiles);
  auto stiles = (const int32_t*)(ws + y.stiles);
  auto ntiles = (const int32_t*)(ws + y.ntiles);
  auto counts = (const int32_t*)(ws + y.counts);
  auto offsets = (const int32_t*)(ws + y.offsets);
  auto perm = (const int32_t*)(ws + y.perm);
  auto w = (const float*)(ws + y.topk_w);
  auto hs16 = (_Float16*)(ws + y.hs16);
  auto hw16 = (_Float16*)(ws + y.hw16);
  auto yp = (float*)(ws + y.yp);
  const dim3 blk(kGW * 64);
  const int gr = L.d_ff / (32 * kGuWaves);  // gate/up row slices
  const dim3 ggu((unsigned)(maxtiles * gr)), ggs((unsigned)(E * gr));
  const dim3 gdn((unsigned)(maxtiles * (d / 256))), gds((unsigned)(E * (d / 256)));
  const bool mx = L.expert_fmt == DS4MOE_EXPERTS_MXFP4, q4 = L.expert_fmt == DS4MOE_EXPERTS_Q4K;
  // every scale block staged in LDS (CB2 gate/up: d_model; Q2K down: d_ff)
  const bool fsg = L.d_model / QK <= gu_nbs(), fsd = L.d_ff / QK <= kDnStagedMax;
#define DS4_GU_LAUNCH(LO, SMALL, MX, Q4, grid, ...)                                                              \
  DS4_LAUNCH((k_pf_gateup<LO, SMALL, MX, Q4, ##__VA_ARGS__>), grid, blk, 0, f.st, L, xh, xl, tiles, stiles, ntiles, \
             counts, offsets, perm, w, hw16)
#define DS4_GU_ROUTED(LO)                                \
  do {                                                   \
    if (mx) {                                            \
      DS4_GU_LAUNCH(LO, false, true, false, ggu);        \
      DS4_GU_LAUNCH(LO, true, true, false, ggs);         \
    } else if (q4) {                                     \
      DS4_GU_LAUNCH(LO, false, false, true, ggu);        \
      DS4_GU_LAUNCH(LO, true, false, true, ggs);         \
    } else if (fsg) {                                    \
      DS4_GU_LAUNCH(LO, false, false, false, ggu, true); \
      DS4_GU_LAUNCH(LO, true, false, false, ggs, true);  \
    } else {                                             \
      DS4_GU_LAUNCH(LO, false, false, false, ggu);       \
      DS4_GU_LAUNCH(LO, true, false, false, ggs);        \
    }                                                    \
  } while (0)
  // the shared expert first (dense GEMMs; its down product writes y, which
  // the combine completes)
  hipError_t e = launch_prefill_shared(L, T, f.lo, xh, xl, hs16, f.y, f.st);
  if (e != hipSuccess) return e;
  if (f.lo) DS4_GU_ROUTED(true);
  else DS4_GU_ROUTED(false);
#undef DS4_GU_ROUTED
#undef DS4_GU_LAUNCH
#define DS4_DN_LAUNCH(SMALL, DDS, MX, Q4, grid)                                                                    \
  DS4_LAUNCH((k_pf_down<SMALL, DDS, MX, Q4>), grid, blk, 0, f.st, L, tiles, stiles, ntiles, counts, offsets, perm, \
             hw16, yp)
  if (mx) {
    DS4_DN_LAUNCH(false, false, true, false, gdn);
    DS4_DN_LAUNCH(true, false, true, false, gds);
  } else if (q4) {
    DS4_DN_LAUNCH(false, false, false, true, gdn);
    DS4_DN_LAUNCH(true, false, false, true, gds);
  } else {
    if (fsd) {
      DS4_DN_LAUNCH(false, true, false, false, gdn);
      DS4_DN_LAUNCH(true, true, false, false, gds);
    } else {
      DS4_DN_LAUNCH(false, false, false, false, gdn);
      DS4_DN_LAUNCH(true, false, false, false, gds);
    }
  }
#undef DS4_DN_LAUNCH
  const int64_t n4 = T * d / 4;
  const int cb = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  DS4_LAUNCH(k_combine, dim3(cb), dim3(256), 0, f.st, T, d, k, yp, f.y);
  return hipGetLastError();
}

}  // namespace ds4
