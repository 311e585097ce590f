/*
 * ds4moe -- routed mixture-of-experts layer with 2-bit quantized experts on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The layer (DS4 (DwarfStar 4) wiki note, "Architecture" and "Key
 * Techniques"; TopDigg "DwarfStar (ds4) Deep Dive", section 3.4 "Asymmetric
 * Quantization"): an F16 router scores E experts and picks the top k; one
 * F16 shared expert always runs; each expert is a SwiGLU block
 * down(silu(gate x) * up x) whose routed gate/up weights are stored in the
 * CB2 codebook format (IQ2_XXS class) and whose routed down weights are in
 * the Q2K super-block format (Q2_K class), dequantized inside the products.
 * DeepSeek V4 Flash's shape is d_model 4096, E 256, k 6.
 *
 * Readings where the pages are silent: the routing weights are the softmax
 * of the selected logits (sum 1, no extra scale); the k selected experts of a
 * token are listed in ascending expert index; equal logits go to the lower
 * index; the shared expert has weight 1; silu(z) = z / (1 + e^-z).
 *
 * ---------------------------------------------------------------- conventions
 * Every pointer is a device pointer owned by the caller unless marked host.
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream).  Arguments are validated on the host before anything
 * is enqueued: a nonzero return means nothing was launched, except
 * DS4MOE_EHIP, which reports a launch failure.  Buffers must stay alive until
 * the stream has passed the call.  The library allocates no device memory:
 * the caller provides a workspace of ds4moe_workspace_bytes() bytes (256-byte
 * aligned) for each call; calls that share a workspace must be ordered on one
 * stream.  A workspace must be all zero before its first forward call
 * (ds4moe_workspace_init); every call leaves it ready for the next one.
 * The codebook grid is a compile-time table; the only mutable global state
 * is the opt-in kernel timer (ds4moe_trace_enable).
 *
 * Numeric range.  The forward calls carry activations in binary16: x (bf16
 * as one binary16 value, fp32 as a binary16 hi + lo pair) and the SwiGLU
 * rows h = silu(gate x) * up x of the routed and the shared experts.  So
 * |x| and every |h| must stay below 65504: larger values become infinities
 * and the outputs non-finite (nothing checks this).  Below 2^-14 they keep
 * less precision (binary16 subnormals) and below 2^-25 they become zero.
 * Inputs that have been RMS-normalised, as the layer's
 * input is in the model, keep x and h of order one.  Products accumulate
 * in fp32 and y is fp32.
 *
 * ---------------------------------------------------------------- formats
 * A matrix W [rows, cols] is quantized along cols (the input dimension) in
 * super-blocks of 256; cols % 256 == 0, nb = cols / 256.  A packed matrix is
 * one buffer holding its planes back to back; E experts are E packed
 * matrices back to back (expert e at e * ds4moe_packed_bytes(...)).
 *
 * CB2 (2.0625 bits per weight; 66 bytes per 256 weights):
 *   code plane  rows*nb*64 bytes: block (r, b) at (r*nb + b)*64.  Sub-block
 *               j (32 weights) occupies bytes 8j..8j+7: bytes 8j+g (g = 0..3)
 *               are the grid indices of its groups of 8; bytes 8j+4..8j+7 are
 *               a little-endian u32 aux: bits 7g..7g+6 = sign code of group
 *               g, bits 28..31 = sub-block scale s (0..15).
 *   scale plane rows*nb binary16 d, at byte offset rows*nb*64.
 *   Weight K = 256b + 32j + 8g + k = sign_k * (d * (2s + 1)) * m_k with
 *   m_k = 2*level + 1 of grid entry idx, coordinate k.  sign_k (1 = negative)
 *   is bit k of the code for k < 7 and the parity of the code for k = 7.
 *   Grid: 256 entries x 8 levels in {0,1,2}; entry i is drawn with
 *   splitmix64 seeded with 0x44533447524944, level = (draw >> 32) % 3, in
 *   coordinate order; an entry equal to an earlier one is drawn again.
 *   Every product is exact in binary32, so decoding is bit-exact.
 *
 * Q2K (2.625 bits per weight; 84 bytes per 256 weights):
 *   code plane      rows*nb*64 bytes: sub-block j (16 weights) is the LE u32
 *                   at bytes 4j..4j+3 of its block, element i at bits 2i..2i+1.
 *   subscale plane  rows*nb*16 bytes at offset rows*nb*64: byte j =
 *                   s_j | m_j << 4.
 *   superscale      rows*nb pairs (binary16 d, binary16 dmin) at offset
 *                   rows*nb*80.
 *   Weight K = 256b + 16j + i = (d * s_j) * q - dmin * m_j; both products
 *   are exact in binary32 and the difference is rounded once.
 *
 * MXFP4 (4.25 bits per weight; 136 bytes per 256 weights): the OCP
 * Microscaling format with FP4 E2M1 elements and one E8M0 scale per 32.
 *   code plane   rows*cols/2 bytes: element K of row r at byte
 *                (r*cols + K)/2, even K in the low nibble; nibble = sign bit
 *                (bit 3), 2 exponent bits (bias 1), 1 mantissa bit, so
 *                magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   scale plane  rows*cols/32 bytes at offset rows*cols/2: E8M0, value
 *                2^(E - 127) (0xFF is NaN).
 *   Weight = e2m1 * 2^(E - 127), exact in binary32.  The quantizer follows
 *   the OCP MX conversion: shared exponent floor(log2 max|w|) - 2, elements
 *   to the nearest E2M1 value (ties to the even code, saturating at 6); a
 *   negative weight that rounds to zero is stored as +0.
 *   The forward calls form each weight in binary16 with its block scale
 *   folded in, which is exact for scale codes 104..140 (2^-23 .. 2^13);
 *   other scales round (binary16) or overflow.  The quantizer gives codes in
 *   that range for blocks whose largest |w| lies in [2^-21, 2^16).
 *
 * Q4K (4.5 bits per weight; 144 bytes per 256 weights), Q4_K class: 8
 * sub-blocks of 32 per super-block, 4-bit codes, 6-bit scale and min per
 * sub-block, binary16 d and dmin.
 *   code plane      rows*nb*128 bytes: sub-block j at bytes 16j..16j+15 of
 *                   its block; LE u32 word k of a sub-block holds elements
 *                   8k..8k+7, element 8k+2p at bits 4p..4p+3 and element
 *                   8k+2p+1 at bits 16+4p..19+4p (p = 0..3).
 *   scale plane     rows*nb*12 bytes at offset rows*nb*128: LE u32 w0, w1,
 *                   w2; nibble j of w0 = s_j & 15, nibble j of w1 = m_j & 15,
 *                   bits 2j..2j+1 of w2 = s_j >> 4, bits 16+2j..17+2j of w2 =
 *                   m_j >> 4.
 *   superscale      rows*nb pairs (binary16 d, binary16 dmin) at offset
 *                   rows*nb*140.
 *   Weight K = 256b + 32j + i = (d * s_j) * q - dmin * m_j, exact products,
 *   one rounding.  The forward calls round each weight to binary16 with
 *   the scales folded in: q * binary16(d * s_j) - binary16(dmin * m_j),
 *   rounded once, so weights must stay within binary16 range.
 *
 * F16 weights are plain row-major binary16 [rows, cols].
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DS4MOE_OK = 0,
  DS4MOE_EINVAL = -1,       /* NULL pointer, bad enum, negative size */
  DS4MOE_ESHAPE = -2,       /* dimension not a multiple of 256, k > E, T out of range */
  DS4MOE_EALIGN = -3,       /* pointer not aligned as required */
  DS4MOE_EWORKSPACE = -4,   /* workspace smaller than ds4moe_workspace_bytes() */
  DS4MOE_EHIP = -5,         /* the HIP runtime reported an error at launch */
  DS4MOE_EUNSUPPORTED = -6  /* valid but not supported by this library */
};

enum { DS4MOE_FMT_F16 = 0, DS4MOE_FMT_CB2 = 1, DS4MOE_FMT_Q2K = 2, DS4MOE_FMT_MXFP4 = 3, DS4MOE_FMT_Q4K = 4 };
/* Formats of a layer's routed experts (ds4moe_layer.expert_fmt):
 * CB2_Q2K: gate/up CB2, down Q2K (the pages' 2-bit recipe);
 * MXFP4: gate, up and down all MXFP4 (the model's native expert format,
 * TopDigg "DwarfStar (ds4) Deep Dive" 5.2, download options);
 * Q4K: gate, up and down all Q4K (the Q4 layers of the q2-q4 mix, same
 * section: the last six routed-expert layers at Q4). */
enum { DS4MOE_EXPERTS_CB2_Q2K = 0, DS4MOE_EXPERTS_MXFP4 = 1, DS4MOE_EXPERTS_Q4K = 2 };
enum { DS4MOE_DT_F32 = 0, DS4MOE_DT_BF16 = 1 };
enum { DS4MOE_MODE_DECODE = 0, DS4MOE_MODE_PREFILL = 1, DS4MOE_MODE_ROUTE = 2 };

/* Largest T accepted by ds4moe_forward_decode (tokens beyond 16 are run as
 * consecutive groups of 16). */
#define DS4MOE_DECODE_MAX_T 64
/* Limits of this library: d_model, d_ff, d_ff_shared <= 16384; E <= 1024;
 * k <= 16. */

/* Layer descriptor.  Plain data: read during the call, not retained.
 * Alignment: every pointer 16-byte aligned. */
typedef struct {
  int32_t d_model;      /* d, multiple of 256 */
  int32_t n_experts;    /* E */
  int32_t top_k;        /* k, 1 <= k <= E */
  int32_t d_ff;         /* routed expert intermediate f, multiple of 256 */
  int32_t d_ff_shared;  /* shared expert intermediate fs, multiple of 256 */
  const uint16_t *router_w;    /* F16 [E, d] */
  const float *router_bias;    /* fp32 [E] added to the logits, or NULL */
  const uint16_t *sh_gate;     /* F16 [fs, d] */
  const uint16_t *sh_up;       /* F16 [fs, d] */
  const uint16_t *sh_down;     /* F16 [d, fs] */
  const void *gate;            /* E packed [f, d] matrices (CB2, MXFP4 or Q4K) */
  const void *up;              /* E packed [f, d] matrices (CB2, MXFP4 or Q4K) */
  const void *down;            /* E packed [d, f] matrices (Q2K, MXFP4 or Q4K) */
  int32_t expert_fmt;          /* DS4MOE_EXPERTS_*; 0 (CB2/Q2K) when the struct is zero-initialised */
} ds4moe_layer;

/* Bytes of one packed [rows, cols] matrix (host function; 0 if cols % 256 != 0
 * or fmt is unknown).  F16: rows*cols*2; CB2 66, Q2K 84, MXFP4 136, Q4K 144
 * bytes per 256 weights. */
size_t ds4moe_packed_bytes(int fmt, int64_t rows, int64_t cols);

/* Quantize fp32 [rows, cols] (row-major, finite values) into the packed
 * matrix `packed` (ds4moe_packed_bytes bytes).  fmt: DS4MOE_FMT_CB2,
 * DS4MOE_FMT_Q2K, DS4MOE_FMT_MXFP4 or DS4MOE_FMT_Q4K.  Deterministic: the bytes equal those
 * of the format's reference quantizer (steps in the library's
 * documentation).
 * Passage: DS4 (DwarfStar 4) wiki note, "Key Techniques" (only the routed
 * experts are quantized: gate/up IQ2_XXS, down Q2_K); TopDigg "DwarfStar
 * (ds4) Deep Dive" 3.4 "Asymmetric Quantization"; 5.2 for the MXFP4 and
 * Q4 expert downloads. */
int ds4moe_quantize(int fmt, const float *w, int64_t rows, int64_t cols, void *packed, void *stream);

/* Decode a packed matrix to fp32 [rows, cols] (bit-exact). */
int ds4moe_dequantize(int fmt, const void *packed, int64_t rows, int64_t cols, float *w, void *stream);

/* Workspace bytes for a call with T tokens (host function).  mode:
 * DS4MOE_MODE_DECODE for ds4moe_forward_decode, DS4MOE_MODE_PREFILL for
 * ds4moe_forward_prefill, DS4MOE_MODE_ROUTE for ds4moe_route.  0 on invalid
 * input. */
size_t ds4moe_workspace_bytes(const ds4moe_layer *L, int64_t T, int mode);

/* Zero ws_bytes bytes of a new workspace with a kernel on `stream` (no memset
 * node, so the call may be captured in a HIP graph).  The decode kernels hand
 * partial results between blocks through arrival counters kept in the
 * workspace; each call returns them to zero, so this is needed once per
 * allocation.  A forward call on a workspace that was never zeroed may return
 * wrong outputs; it still reads and writes only inside its buffers.
 * ws: 256-byte aligned device pointer. */
int ds4moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Router + top-k + gate weights + token grouping for T tokens.
 * Passage: DS4 (DwarfStar 4) wiki note, "Architecture" (256 routed experts,
 * 6 active per token) and "Key Techniques" (the router stays F16).
 * x: [T, d] fp32 or bf16 (x_dtype).  Outputs: topk_idx [T, k] int32 (ascending
 * expert index per token), topk_w [T, k] fp32 (softmax of the selected
 * logits), counts [E], offsets [E+1] (exclusive scan of counts), perm [T*k]
 * (slot ids t*k + j sorted by expert, then token).  counts/offsets/perm may
 * be NULL (not written).  1 <= T. */
int ds4moe_route(const ds4moe_layer *L, const void *x, int x_dtype, int64_t T, int32_t *topk_idx,
                 float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm, void *ws,
                 size_t ws_bytes, void *stream);

/* Full layer for 1 <= T <= DS4MOE_DECODE_MAX_T tokens (batched decode).
 * y: [T, d] fp32.  topk_idx_out / topk_w_out: optional [T, k] copies of the
 * routing (NULL = not written).
 * Passage: DS4 (DwarfStar 4) wiki note, "Architecture" (6 routed + 1 shared
 * expert per token); the batch bound covers TopDigg "DwarfStar (ds4) Deep
 * Dive" 5.4's 16 batched sessions and its speculative-verify batches. */
int ds4moe_forward_decode(const ds4moe_layer *L, const void *x, int x_dtype, int64_t T, float *y,
                          int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                          void *stream);

/* Bytes of the device array that ds4moe_forward_decode_static uses as its
 * workspace (one copy per GPU, held until the process ends). */
#define DS4MOE_STATIC_SCRATCH_BYTES ((size_t)4 << 20)

/* ds4moe_forward_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * ds4moe_forward_decode (bit for bit: the same kernels run), with the
 * library's own device array of DS4MOE_STATIC_SCRATCH_BYTES as workspace.
 * Allocates nothing: on its first call on a device it looks up that device's
 * copy of the array and clears it with a kernel on `stream`.  Returns
 * DS4MOE_EWORKSPACE, with nothing launched, when the call's workspace
 * (ds4moe_workspace_bytes(L, T, DS4MOE_MODE_DECODE)) exceeds the array
 * (DeepSeek V4 Flash's shape needs 1.6 MB at any T).  All calls on one GPU
 * share its array: calls that may overlap (on different streams or host
 * threads without ordering between them) race and give wrong outputs; calls
 * ordered on one stream are safe. */
int ds4moe_forward_decode_static(const ds4moe_layer *L, const void *x, int x_dtype, int64_t T, float *y,
                                 int32_t *topk_idx_out, float *topk_w_out, void *stream);

/* Passage: DS4 (DwarfStar 4) wiki note, "Architecture" (prefill runs in
 * chunks, 2048 tokens by default).
 * Full layer for 1 <= T <= 524280 tokens (prefill chunk; grouped GEMMs),
 * with T * d_model < 2^31 and T * k * d_ff < 2^31 (DS4MOE_ESHAPE otherwise).
 * Same outputs as ds4moe_forward_decode plus the optional permutation
 * perm_out [T*k].  The routed products round each dequantized weight to
 * binary16 (block scales folded in), so weights must stay within binary16
 * range; the decode entry point applies the block scales in fp32. */
int ds4moe_forward_prefill(const ds4moe_layer *L, const void *x, int x_dtype, int64_t T, float *y,
                           int32_t *topk_idx_out, float *topk_w_out, int32_t *perm_out, void *ws,
                           size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------------
 * Hyper-connection mixer on either side of the layer (DS4 (DwarfStar 4)
 * wiki note, "Key Techniques", hyper-connections with Sinkhorn
 * normalization: the activations travel as n = 4 streams of d values; a
 * learned mixer normalised by Sinkhorn iterations reduces them to the one
 * row the sublayer consumes and expands its output back into n streams).
 * The note gives no formulas; this library takes the manifold-constrained
 * hyper-connection reading (per token t, streams X[n][d] flattened as
 * k = i*d + c):
 *   r      = sqrt(sum_k X_k^2 / (n d) + eps)
 *   z_o    = alpha_g * (sum_k phi[o][k] X_k) / r + bias[o], o < 2n + n*n;
 *            g = pre (o < n), post (o < 2n), res (otherwise)
 *   pre_i  = 1 / (1 + e^-z_i),  post_i = 2 / (1 + e^-z_{n+i})
 *   M      = sinkhorn_iters Sinkhorn iterations on exp(Z), Z[i][j] =
 *            z_{2n+n*i+j}; one iteration divides every row by its sum, then
 *            every column by its sum (the GPU subtracts each row's maximum
 *            before exp, which the first row step cancels)
 *   x_in   = sum_i pre_i X[i]                      (ds4moe_hc_pre)
 *   X'[i]  = sum_j M[i][j] X[j] + post_i y          (ds4moe_hc_post)
 * Everything is fp32 (binary32 inputs, fp32 accumulation).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_streams;      /* n; this library runs n = 4 (else DS4MOE_EUNSUPPORTED) */
  int32_t d_model;        /* d: multiple of 256, <= 16384 */
  int32_t sinkhorn_iters; /* 1..64 (the note: 20) */
  float eps;              /* RMS epsilon, finite, >= 0 */
  float alpha_pre, alpha_post, alpha_res;
  const float *phi;       /* fp32 [2n + n*n][n*d] row-major, 16-byte aligned */
  const float *bias;      /* fp32 [2n + n*n], 4-byte aligned */
} ds4moe_hc;

/* Workspace bytes ds4moe_hc_pre needs for T tokens (0 on invalid input). */
size_t ds4moe_hc_workspace_bytes(const ds4moe_hc *H, int64_t T);

/* Coefficients and reduced rows of T tokens (1 <= T <= 1048576).
 *   X      fp32 [T][n][d], 16-byte aligned (read only)
 *   coef   fp32 [T][2n + n*n] out: pre (n), post (n), M row-major (n*n);
 *          16-byte aligned
 *   x_out  fp32 [T][d] out, or NULL; 16-byte aligned
 *   x_bf16 bfloat16 bits [T][d] out (x_out rounded to nearest-even, the
 *          layer's bf16 input), or NULL; 8-byte aligned
 *   ws     device workspace of at least ds4moe_hc_workspace_bytes,
 *          256-byte aligned, zeroed once before its first use
 *          (ds4moe_workspace_init); every call leaves its arrival counter
 *          at zero again.  Calls that share a workspace must not overlap.
 * For T <= 2 the whole step is one kernel launch (the last block to finish
 * its partial projection completes the tokens), otherwise two.
 * Asynchronous on `stream`; nothing is enqueued on a non-zero return. */
int ds4moe_hc_pre(const ds4moe_hc *H, const float *X, int64_t T, float *coef, float *x_out, uint16_t *x_bf16,
                  void *ws, size_t ws_bytes, void *stream);

/* Expanded streams X_out [T][n][d] = M X + post y per token, with coef as
 * ds4moe_hc_pre wrote it and y fp32 [T][d] the sublayer's output (the
 * layer's y).  X_out may equal X (in place); no other overlap.  All
 * pointers 16-byte aligned.  Asynchronous on `stream`. */
int ds4moe_hc_post(const ds4moe_hc *H, const float *X, const float *y, const float *coef, int64_t T,
                   float *X_out, void *stream);

/* Opt-in per-kernel timing (profiling aid).  While enabled, every kernel
 * the library launches is bracketed by two HIP events on its stream, which
 * adds a little launch overhead.  Thread-safe. */
int ds4moe_trace_enable(int on);

/* Wait for the recorded events and accumulate them; then write, for up to
 * `cap` kernels, the accumulated milliseconds (ms[i]) and launch counts
 * (counts[i]), and their names as one '\n'-separated string into `names`
 * (host buffers; any may be NULL).  reset != 0 clears the totals afterwards.
 * Returns the number of kernels seen, or DS4MOE_EHIP. */
int ds4moe_trace_read(char *names, size_t names_cap, double *ms, long long *counts, int cap, int reset);

/* Static string for a status code. */
const char *ds4moe_strerror(int status);

/* Host copy of the codebook grid levels, levels[256*8] (entry-major). */
void ds4moe_grid_levels(uint8_t *levels);

#ifdef __cplusplus
}
#endif

#endif /* DS4MOE_H */
