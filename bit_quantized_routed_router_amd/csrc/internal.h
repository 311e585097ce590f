// Internal host-side declarations of the ds4moe library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ds4moe.h"

namespace ds4 {

constexpr int kDecodeGroup = 16;  // tokens per decode group (one MFMA column tile)
constexpr int kMaxDim = 16384;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kPrefillTile = 128;  // slots per prefill work tile (one expert)
constexpr int kSmallTile = 32;     // tiles of at most this many slots go to the small-tile list
// Prefill work tiles of an expert with n slots: runs of kPrefillTile; the
// remainder is a small tile when it holds at most kSmallTile slots.
__host__ __device__ inline int big_tiles(int n) { return n / kPrefillTile + (n % kPrefillTile > kSmallTile ? 1 : 0); }
__host__ __device__ inline int small_tiles(int n) {
  const int r = n % kPrefillTile;
  return r > 0 && r <= kSmallTile ? 1 : 0;
}

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
  size_t x_hi, x_lo, logits, topk_idx, topk_w, counts, offsets, perm, inv;
  size_t ndist, distinct, tok_slot;  // decode: distinct experts and their token slots
  size_t hs16, hw16, hsum, yp;        // activations between the kernels
  size_t tiles, stiles, ntiles;       // prefill: (expert, run) work lists of large and small tiles, their counts
  size_t plog;                        // decode: partial router logits [d/128][Tg][E]
  size_t rpart;                       // prefill/route: router GEMM partials [parts][T][E] (parts > 1 only)
  size_t ctrl;                        // decode: arrival counters (see ctrl_ints)
  size_t gu_part;                     // decode: shared-expert gate and up tiles handed to the tile's last block
  size_t total;
};

WsLayout ws_layout(const ds4moe_layer& L, int64_t T, int mode);

// Decode arrival counters at workspace offset 0: [0] router blocks (stage 1),
// then one per 16-row tile of the shared expert's gate/up (stage 2).  Each counter is
// reset by the block that sees the last arrival, and stage 3 clears them all
// again, so they are zero whenever no call is running; a new workspace must
// start zeroed.
constexpr int kCtrlInts = 1 + kMaxDim / 16;
inline int ctrl_ints(const ds4moe_layer& L) { return 1 + L.d_ff_shared / 16; }  // router + shared tiles
// decode: blocks a shared-expert gate or up row tile is split into along its
// input (contiguous parts), so that a wave has few K-steps to load at once
constexpr int kShSplit = 2;

// Everything a forward launch needs, resolved on the host.
struct Fwd {
  ds4moe_layer L;
  int64_t T;
  bool lo;  // activations arrived as fp32: use a hi/lo binary16 split
  const void* x;
  int x_dtype;
  float* y;
  int32_t* idx_out;
  float* w_out;
  int32_t* counts_out;
  int32_t* offsets_out;
  int32_t* perm_out;
  char* ws;
  WsLayout lay;
  hipStream_t st;
};

hipError_t launch_quant_cb2(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st);
hipError_t launch_quant_q2k(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st);
hipError_t launch_dequant_cb2(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st);
hipError_t launch_dequant_q2k(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st);
hipError_t launch_quant_mx4(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st);
hipError_t launch_dequant_mx4(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st);
hipError_t launch_quant_q4k(const float* w, int64_t rows, int64_t cols, void* packed, hipStream_t st);
hipError_t launch_dequant_q4k(const void* packed, int64_t rows, int64_t cols, float* out, hipStream_t st);

// routing: x conversion + logits + top-k + grouping.  decode == true builds
// the distinct-expert tables of a <= 16-token group.
hipError_t launch_route(const Fwd& f, bool decode);
hipError_t launch_decode(const Fwd& f);  // full layer for one group of <= 16 tokens
hipError_t launch_prefill_experts(const Fwd& f);
// router logits [T][E] (+ bias) of binary16 activations; part: fp32
// partials of router_splits(T, E, d) > 1 K parts ([parts][T][E])
int router_splits(int64_t T, int E, int d);
hipError_t launch_router_logits(const ds4moe_layer& L, int64_t T, bool lo, const _Float16* xh, const _Float16* xl,
                                float* part, float* logits, hipStream_t st);
// prefill shared expert: gate/up into hs16 (binary16), down into y (fp32)
hipError_t launch_prefill_shared(const ds4moe_layer& L, int64_t T, bool lo, const _Float16* xh, const _Float16* xl,
                                 _Float16* hs16, float* y, hipStream_t st);

// hyper-connection mixer (ds4moe_hc); hc_ws_bytes: workspace of hc_pre
constexpr int64_t kHcMaxT = 1 << 20;
size_t hc_ws_bytes(int d, int64_t T);
hipError_t launch_hc_pre(const ds4moe_hc& H, const float* X, int64_t T, float* coef, float* xout, uint16_t* xbf,
                         void* ws, hipStream_t st);
hipError_t launch_hc_post(const ds4moe_hc& H, const float* X, const float* y, const float* coef, int64_t T,
                          float* Xo, hipStream_t st);

}  // namespace ds4
