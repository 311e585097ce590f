// Internal host-side declarations of the ds4moe library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ds4moe.h"

namespace ds4 {

constexpr int kDecodeGroup = 16;  // tokens per decode group (one MFMA column tile)
constexpr int kMaxDim = 16384;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
  size_t x_hi, x_lo, logits, topk_idx, topk_w, counts, offsets, perm, inv;
  size_t ndist, distinct, tok_slot;  // decode: distinct experts and their token slots
  size_t hs16, hw16, hsum, yp;        // activations between the kernels
  size_t tiles, ntiles;               // prefill: (expert, token group) work list
  size_t total;
};

WsLayout ws_layout(const ds4moe_layer& L, int64_t T, int mode);

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

// routing: x conversion + logits + top-k + grouping.  decode == true builds
// the distinct-expert tables of a <= 16-token group.
hipError_t launch_route(const Fwd& f, bool decode);
hipError_t launch_decode_experts(const Fwd& f);
hipError_t launch_prefill_experts(const Fwd& f);

}  // namespace ds4
