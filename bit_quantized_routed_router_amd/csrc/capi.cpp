// C ABI of the ds4moe library: argument validation, workspace layout and
// dispatch.  Nothing is enqueued unless every check passes.
#include <cmath>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "common.h"
#include "internal.h"
#include "trace.h"

namespace ds4 {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const ds4moe_layer& L, int64_t T, int mode) {
  WsLayout y{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += align256(bytes);
    return r;
  };
  const int64_t d = L.d_model, E = L.n_experts, k = L.top_k, f = L.d_ff, fs = L.d_ff_shared;
  const int64_t Tg = mode == DS4MOE_MODE_DECODE ? std::min<int64_t>(T, kDecodeGroup) : T;
  const int64_t S = Tg * k;
  // first and of fixed size, so every mode and layer shape finds its counters
  // at the same place in a shared workspace
  y.ctrl = take((size_t)kCtrlInts * 4);
  y.x_hi = take(Tg * d * 2);
  y.x_lo = take(Tg * d * 2);
  y.logits = take(Tg * E * 4);
  y.topk_idx = take(S * 4);
  y.topk_w = take(S * 4);
  y.counts = take(E * 4);
  y.offsets = take((E + 1) * 4);
  y.perm = take(S * 4);
  y.inv = take(S * 4);
  const int64_t dmax = std::min<int64_t>(E, std::min<int64_t>(Tg, kDecodeGroup) * k);
  y.ndist = take(4);
  y.distinct = take(E * 4);
  y.tok_slot = take(dmax * kDecodeGroup * 4);
  y.tiles = take(((S + kPrefillTile - 1) / kPrefillTile + E) * 2 * 4);
  y.stiles = take(E * 2 * 4);
  y.ntiles = take(2 * 4);
  const int64_t Tdec = std::min<int64_t>(Tg, kDecodeGroup);
  y.plog = take((d / 128) * Tdec * E * 4);  // one partial per 256 (routing only) or 128 inputs (forward)
  if (mode != DS4MOE_MODE_DECODE) {
    const int parts = router_splits(Tg, (int)E, (int)d);
    y.rpart = take(parts > 1 ? (size_t)parts * Tg * E * 4 : 0);
  }
  if (mode != DS4MOE_MODE_ROUTE) {  // expert buffers (not needed for routing alone)
    y.hs16 = take(Tg * fs * 2);
    y.hw16 = take(S * f * 2);
    y.hsum = take(S * (f / 16) * 4);
    if (mode == DS4MOE_MODE_PREFILL) y.yp = take(S * d * 4);
    if (mode == DS4MOE_MODE_DECODE) {
      y.gu_part = take((fs / 16) * 2 * kShSplit * 16 * Tdec * 4);
    }
  }
  y.total = o;
  return y;
}

static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
static bool dim_ok(int64_t v) { return v >= 256 && v <= kMaxDim && v % 256 == 0; }

static int check_layer(const ds4moe_layer* L) {
  if (!L) return DS4MOE_EINVAL;
  if (!L->router_w || !L->sh_gate || !L->sh_up || !L->sh_down || !L->gate || !L->up || !L->down) return DS4MOE_EINVAL;
  if (!dim_ok(L->d_model) || !dim_ok(L->d_ff) || !dim_ok(L->d_ff_shared)) return DS4MOE_ESHAPE;
  if (L->n_experts < 1 || L->n_experts > kMaxExperts) return DS4MOE_ESHAPE;
  if (L->top_k < 1 || L->top_k > L->n_experts || L->top_k > kMaxTopK) return DS4MOE_ESHAPE;
  if (!al16(L->router_w) || !al16(L->sh_gate) || !al16(L->sh_up) || !al16(L->sh_down) || !al16(L->gate) ||
      !al16(L->up) || !al16(L->down))
    return DS4MOE_EALIGN;
  if (L->router_bias && ((uintptr_t)L->router_bias & 3)) return DS4MOE_EALIGN;
  if (L->expert_fmt != DS4MOE_EXPERTS_CB2_Q2K && L->expert_fmt != DS4MOE_EXPERTS_MXFP4 &&
      L->expert_fmt != DS4MOE_EXPERTS_Q4K)
    return DS4MOE_EINVAL;
  return DS4MOE_OK;
}

static int check_io(const void* x, int x_dtype, int64_t T, const void* ws, size_t ws_bytes, size_t need) {
  if (!x || !ws) return DS4MOE_EINVAL;
  if (x_dtype != DS4MOE_DT_F32 && x_dtype != DS4MOE_DT_BF16) return DS4MOE_EINVAL;
  if (T < 1) return DS4MOE_ESHAPE;
  if (!al16(x) || ((uintptr_t)ws & 255)) return DS4MOE_EALIGN;
  if (ws_bytes < need) return DS4MOE_EWORKSPACE;
  return DS4MOE_OK;
}

static bool opt_al4(const void* p) { return !p || ((uintptr_t)p & 3) == 0; }

static Fwd make_fwd(const ds4moe_layer* L, const void* x, int x_dtype, int64_t T, float* y, int32_t* idx_out,
                    float* w_out, void* ws, int mode, void* stream) {
  Fwd f{};
  f.L = *L;
  f.T = T;
  f.lo = x_dtype == DS4MOE_DT_F32;
  f.x = x;
  f.x_dtype = x_dtype;
  f.y = y;
  f.idx_out = idx_out;
  f.w_out = w_out;
  f.ws = (char*)ws;
  f.lay = ws_layout(*L, T, mode);
  f.st = (hipStream_t)stream;
  return f;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? DS4MOE_OK : DS4MOE_EHIP; }

__global__ __launch_bounds__(256) void k_zero_bytes(uint8_t* __restrict__ p, size_t n) {
  const size_t n16 = n / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    ((u32x4_t*)p)[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x < n % 16) p[n16 * 16 + threadIdx.x] = 0;
}

// ---------------------------------------------------------------- static scratch
// Device memory of ds4moe_forward_decode_static: a fixed array in place of
// the caller's workspace.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); it takes each
// device's copy from hipGetSymbolAddress once, with that device current.
static __device__ __align__(256) unsigned char scratch[DS4MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
static StaticScratch g_static;

// This device's scratch address; on the first call for a device, looks it up
// and clears the whole array with a kernel on `st` (the arrival counters the
// decode kernels keep at its start must be zero before the first call; each
// call returns them to zero).
static int static_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DS4MOE_EHIP;
  std::lock_guard<std::mutex> lk(g_static.mu);
  if (!g_static.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DS4MOE_EHIP;
    const size_t n = DS4MOE_STATIC_SCRATCH_BYTES;
    DS4_LAUNCH(k_zero_bytes, dim3(1024), dim3(256), 0, st, (uint8_t*)p, n);
    if (hipGetLastError() != hipSuccess) return DS4MOE_EHIP;
    g_static.ptr[dev] = p;
  }
  *out = g_static.ptr[dev];
  return DS4MOE_OK;
}

}  // namespace ds4

using namespace ds4;

extern "C" {

size_t ds4moe_packed_bytes(int fmt, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  if (fmt == DS4MOE_FMT_F16) return (size_t)rows * (size_t)cols * 2;
  if (cols % QK != 0) return 0;
  const size_t nblk = (size_t)rows * (size_t)(cols / QK);
  if (fmt == DS4MOE_FMT_CB2) return nblk * 66;
  if (fmt == DS4MOE_FMT_Q2K) return nblk * 84;
  if (fmt == DS4MOE_FMT_MXFP4) return nblk * 136;
  if (fmt == DS4MOE_FMT_Q4K) return nblk * 144;
  return 0;
}

static bool codec_fmt(int fmt) {
  return fmt == DS4MOE_FMT_CB2 || fmt == DS4MOE_FMT_Q2K || fmt == DS4MOE_FMT_MXFP4 || fmt == DS4MOE_FMT_Q4K;
}

int ds4moe_quantize(int fmt, const float* w, int64_t rows, int64_t cols, void* packed, void* stream) {
  if (!codec_fmt(fmt)) return DS4MOE_EINVAL;
  if (rows < 0 || cols < 0) return DS4MOE_EINVAL;
  if (cols % QK != 0) return DS4MOE_ESHAPE;
  if (rows == 0 || cols == 0) return DS4MOE_OK;
  if (!w || !packed) return DS4MOE_EINVAL;
  if (!al16(w) || !al16(packed)) return DS4MOE_EALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = fmt == DS4MOE_FMT_CB2   ? launch_quant_cb2(w, rows, cols, packed, st)
                 : fmt == DS4MOE_FMT_Q2K ? launch_quant_q2k(w, rows, cols, packed, st)
                 : fmt == DS4MOE_FMT_Q4K ? launch_quant_q4k(w, rows, cols, packed, st)
                                         : launch_quant_mx4(w, rows, cols, packed, st);
  return hip_status(e);
}

int ds4moe_dequantize(int fmt, const void* packed, int64_t rows, int64_t cols, float* w, void* stream) {
  if (!codec_fmt(fmt)) return DS4MOE_EINVAL;
  if (rows < 0 || cols < 0) return DS4MOE_EINVAL;
  if (cols % QK != 0) return DS4MOE_ESHAPE;
  if (rows == 0 || cols == 0) return DS4MOE_OK;
  if (!w || !packed) return DS4MOE_EINVAL;
  if (!al16(w) || !al16(packed)) return DS4MOE_EALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = fmt == DS4MOE_FMT_CB2   ? launch_dequant_cb2(packed, rows, cols, w, st)
                 : fmt == DS4MOE_FMT_Q2K ? launch_dequant_q2k(packed, rows, cols, w, st)
                 : fmt == DS4MOE_FMT_Q4K ? launch_dequant_q4k(packed, rows, cols, w, st)
                                         : launch_dequant_mx4(packed, rows, cols, w, st);
  return hip_status(e);
}

size_t ds4moe_workspace_bytes(const ds4moe_layer* L, int64_t T, int mode) {
  if (!L || T < 1 || (mode != DS4MOE_MODE_DECODE && mode != DS4MOE_MODE_PREFILL && mode != DS4MOE_MODE_ROUTE)) return 0;
  if (!dim_ok(L->d_model) || !dim_ok(L->d_ff) || !dim_ok(L->d_ff_shared)) return 0;
  if (L->n_experts < 1 || L->n_experts > kMaxExperts || L->top_k < 1 || L->top_k > L->n_experts) return 0;
  return ws_layout(*L, T, mode).total;
}

int ds4moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return DS4MOE_EINVAL;
  if ((uintptr_t)ws & 255) return DS4MOE_EALIGN;
  if (ws_bytes == 0) return DS4MOE_OK;
  const size_t blocks = std::min<size_t>((ws_bytes / 16 + 255) / 256 + 1, 4096);
  hipStream_t st = (hipStream_t)stream;
  DS4_LAUNCH(k_zero_bytes, dim3((unsigned)blocks), dim3(256), 0, st, (uint8_t*)ws, ws_bytes);
  return hip_status(hipGetLastError());
}

int ds4moe_route(const ds4moe_layer* L, const void* x, int x_dtype, int64_t T, int32_t* topk_idx, float* topk_w,
                 int32_t* counts, int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T > 1 << 20) return DS4MOE_ESHAPE;
  if ((rc = check_io(x, x_dtype, T, ws, ws_bytes, ws_layout(*L, T, DS4MOE_MODE_ROUTE).total))) return rc;
  if (!topk_idx || !topk_w) return DS4MOE_EINVAL;
  if (!opt_al4(topk_idx) || !opt_al4(topk_w) || !opt_al4(counts) || !opt_al4(offsets) || !opt_al4(perm))
    return DS4MOE_EALIGN;
  Fwd f = make_fwd(L, x, x_dtype, T, nullptr, topk_idx, topk_w, ws, DS4MOE_MODE_ROUTE, stream);
  f.counts_out = counts;
  f.offsets_out = offsets;
  f.perm_out = perm;
  return hip_status(launch_route(f, T <= kDecodeGroup));
}

int ds4moe_forward_decode(const ds4moe_layer* L, const void* x, int x_dtype, int64_t T, float* y,
                          int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T > DS4MOE_DECODE_MAX_T) return DS4MOE_ESHAPE;
  if ((rc = check_io(x, x_dtype, T, ws, ws_bytes, ws_layout(*L, T, DS4MOE_MODE_DECODE).total))) return rc;
  if (!y) return DS4MOE_EINVAL;
  if (!al16(y)) return DS4MOE_EALIGN;
  if (!opt_al4(topk_idx_out) || !opt_al4(topk_w_out)) return DS4MOE_EALIGN;
  const size_t xes = x_dtype == DS4MOE_DT_F32 ? 4 : 2;
  const int64_t d = L->d_model, k = L->top_k;
  for (int64_t t0 = 0; t0 < T; t0 += kDecodeGroup) {  // groups of up to 16 tokens, in order on the stream
    const int64_t tg = std::min<int64_t>(kDecodeGroup, T - t0);
    Fwd f = make_fwd(L, (const char*)x + t0 * d * xes, x_dtype, tg, y + t0 * d,
                     topk_idx_out ? topk_idx_out + t0 * k : nullptr, topk_w_out ? topk_w_out + t0 * k : nullptr, ws,
                     DS4MOE_MODE_DECODE, stream);
    if (launch_decode(f) != hipSuccess) return DS4MOE_EHIP;
  }
  return DS4MOE_OK;
}

int ds4moe_forward_decode_static(const ds4moe_layer* L, const void* x, int x_dtype, int64_t T, float* y,
                                 int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !y) return DS4MOE_EINVAL;
  if (x_dtype != DS4MOE_DT_F32 && x_dtype != DS4MOE_DT_BF16) return DS4MOE_EINVAL;
  if (T < 1 || T > DS4MOE_DECODE_MAX_T) return DS4MOE_ESHAPE;
  const size_t need = ws_layout(*L, T, DS4MOE_MODE_DECODE).total;
  if (need > DS4MOE_STATIC_SCRATCH_BYTES) return DS4MOE_EWORKSPACE;
  if (!al16(x) || !al16(y) || !opt_al4(topk_idx_out) || !opt_al4(topk_w_out)) return DS4MOE_EALIGN;
  void* ws = nullptr;
  if ((rc = static_scratch((hipStream_t)stream, &ws))) return rc;
  return ds4moe_forward_decode(L, x, x_dtype, T, y, topk_idx_out, topk_w_out, ws, need, stream);
}

int ds4moe_forward_prefill(const ds4moe_layer* L, const void* x, int x_dtype, int64_t T, float* y,
                           int32_t* topk_idx_out, float* topk_w_out, int32_t* perm_out, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T > 65535 * 16 / 2) return DS4MOE_ESHAPE;  // 16-token groups along a grid's y dimension
  // the grouped products address activations and h with 32-bit byte offsets
  if (T * L->d_model >= (int64_t)1 << 31 || T * L->top_k * L->d_ff >= (int64_t)1 << 31) return DS4MOE_ESHAPE;
  if ((rc = check_io(x, x_dtype, T, ws, ws_bytes, ws_layout(*L, T, DS4MOE_MODE_PREFILL).total))) return rc;
  if (!y) return DS4MOE_EINVAL;
  if (!al16(y)) return DS4MOE_EALIGN;
  if (!opt_al4(topk_idx_out) || !opt_al4(topk_w_out) || !opt_al4(perm_out)) return DS4MOE_EALIGN;
  Fwd f = make_fwd(L, x, x_dtype, T, y, topk_idx_out, topk_w_out, ws, DS4MOE_MODE_PREFILL, stream);
  f.perm_out = perm_out;
  hipError_t e = launch_route(f, false);
  if (e == hipSuccess) e = launch_prefill_experts(f);
  return hip_status(e);
}

// ---------------------------------------------------------------- hyper-connection mixer
static int check_hc(const ds4moe_hc* H) {
  if (!H || !H->phi || !H->bias) return DS4MOE_EINVAL;
  if (H->n_streams < 1) return DS4MOE_EINVAL;
  if (H->n_streams != 4) return DS4MOE_EUNSUPPORTED;
  if (!dim_ok(H->d_model)) return DS4MOE_ESHAPE;
  if (H->sinkhorn_iters < 1 || H->sinkhorn_iters > 64) return DS4MOE_EINVAL;
  if (!(H->eps >= 0.0f) || !std::isfinite(H->eps) || !std::isfinite(H->alpha_pre) || !std::isfinite(H->alpha_post) ||
      !std::isfinite(H->alpha_res))
    return DS4MOE_EINVAL;
  if (!al16(H->phi) || ((uintptr_t)H->bias & 3)) return DS4MOE_EALIGN;
  return DS4MOE_OK;
}

size_t ds4moe_hc_workspace_bytes(const ds4moe_hc* H, int64_t T) {
  if (check_hc(H) != DS4MOE_OK || T < 1 || T > kHcMaxT) return 0;
  return hc_ws_bytes(H->d_model, T);
}

int ds4moe_hc_pre(const ds4moe_hc* H, const float* X, int64_t T, float* coef, float* x_out, uint16_t* x_bf16,
                  void* ws, size_t ws_bytes, void* stream) {
  const int st = check_hc(H);
  if (st != DS4MOE_OK) return st;
  if (!X || !coef || !ws) return DS4MOE_EINVAL;
  if (T < 1 || T > kHcMaxT) return DS4MOE_ESHAPE;
  if (!al16(X) || !al16(coef) || (x_out && !al16(x_out)) || ((uintptr_t)x_bf16 & 7) || ((uintptr_t)ws & 255))
    return DS4MOE_EALIGN;
  if (ws_bytes < hc_ws_bytes(H->d_model, T)) return DS4MOE_EWORKSPACE;
  return hip_status(launch_hc_pre(*H, X, T, coef, x_out, x_bf16, ws, (hipStream_t)stream));
}

int ds4moe_hc_post(const ds4moe_hc* H, const float* X, const float* y, const float* coef, int64_t T, float* X_out,
                   void* stream) {
  const int st = check_hc(H);
  if (st != DS4MOE_OK) return st;
  if (!X || !y || !coef || !X_out) return DS4MOE_EINVAL;
  if (T < 1 || T > kHcMaxT) return DS4MOE_ESHAPE;
  if (!al16(X) || !al16(y) || !al16(coef) || !al16(X_out)) return DS4MOE_EALIGN;
  return hip_status(launch_hc_post(*H, X, y, coef, T, X_out, (hipStream_t)stream));
}

const char* ds4moe_strerror(int status) {
  switch (status) {
    case DS4MOE_OK: return "ok";
    case DS4MOE_EINVAL: return "invalid argument (NULL pointer, unknown enum or negative size)";
    case DS4MOE_ESHAPE: return "unsupported shape (dimensions must be multiples of 256, 1 <= k <= E, T in range)";
    case DS4MOE_EALIGN: return "misaligned pointer (16 bytes for tensors, 256 for the workspace)";
    case DS4MOE_EWORKSPACE: return "workspace smaller than ds4moe_workspace_bytes()";
    case DS4MOE_EHIP: return "HIP runtime error at launch";
    case DS4MOE_EUNSUPPORTED: return "not supported by this library";
    default: return "unknown status";
  }
}

void ds4moe_grid_levels(uint8_t* levels) {
  if (!levels) return;
  for (int i = 0; i < 256; ++i)
    for (int k = 0; k < 8; ++k) levels[8 * i + k] = kGridLevels.lv[i][k];
}

}  // extern "C"
