/*
 * Driver that runs every function of the CPU oracle (oracle/ds4moe_oracle.c)
 * at the shapes and edge cases of its pins, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and
 * runs it).  It checks only cheap consistency properties itself -- the values
 * are pinned by the Python tests -- its job is that no out-of-bounds access,
 * overflow or other undefined behaviour happens on those inputs.  Test
 * infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_f16_to_f64(uint16_t h);
uint16_t orc_f64_to_f16(double v);
double orc_bf16_to_f64(uint16_t b);
uint64_t orc_splitmix64(uint64_t *state);
void orc_grid_levels(uint8_t *levels);
void orc_cb2_dequantize(const uint8_t *codes, const uint16_t *dplane, int64_t rows, int64_t cols, float *out);
void orc_cb2_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint16_t *dplane);
void orc_q2k_dequantize(const uint8_t *codes, const uint8_t *sub, const uint16_t *sup, int64_t rows, int64_t cols,
                        float *out);
void orc_q2k_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *sub, uint16_t *sup);
void orc_q4k_dequantize(const uint8_t *codes, const uint8_t *scales, const uint16_t *sup, int64_t rows, int64_t cols,
                        float *out);
void orc_q4k_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales, uint16_t *sup);
void orc_q4k_matmul(const uint8_t *codes, const uint8_t *scales, const uint16_t *sup, int64_t rows, int64_t cols,
                    const double *X, int64_t n, double *Y);
double orc_e2m1_value(int code);
double orc_e8m0_value(int code);
void orc_mx4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, float *out);
void orc_mx4_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales);
void orc_cb2_matmul(const uint8_t *codes, const uint16_t *dplane, int64_t rows, int64_t cols, const double *X,
                    int64_t n, double *Y);
void orc_q2k_matmul(const uint8_t *codes, const uint8_t *sub, const uint16_t *sup, int64_t rows, int64_t cols,
                    const double *X, int64_t n, double *Y);
void orc_mx4_matmul(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, const double *X,
                    int64_t n, double *Y);
void orc_f16_matmul(const uint16_t *w, int64_t rows, int64_t cols, const double *X, int64_t n, double *Y);
void orc_router_logits(const double *X, int64_t T, int64_t d, const uint16_t *wr, int64_t E, const float *bias,
                       double *logits);
void orc_topk(const double *logits, int64_t T, int64_t E, int k, int32_t *idx, double *w);
void orc_permute(const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts, int32_t *offsets, int32_t *perm,
                 int32_t *inv);
void orc_swiglu(const double *g, const double *u, int64_t n, double *h);
void orc_sinkhorn(const double *Z, int n, int iters, double *A);
void orc_hc_pre(const double *X, int64_t T, int n, int64_t d, const double *phi, const double *bias,
                const double *alpha, double eps, int iters, double *coef, double *xin);
void orc_hc_post(const double *X, const double *y, const double *coef, int64_t T, int n, int64_t d, double *Xout);
void orc_set_threads(int n);

static int g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      g_fail = 1;                                                  \
    }                                                              \
  } while (0)

static uint64_t g_state = 12345;
static double unif(void) { return (double)(orc_splitmix64(&g_state) >> 11) * (1.0 / 9007199254740992.0); }
static double gauss(void) {
  double u = unif(), v = unif();
  if (u < 1e-300) u = 1e-300;
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

/* rows x cols fp32 weights with edge rows: zeros, one spike, tiny values,
 * huge values of both signs, all-negative, exact ties. */
static float *weights(int64_t rows, int64_t cols, double scale) {
  float *w = malloc(sizeof(float) * (size_t)(rows * cols));
  for (int64_t i = 0; i < rows * cols; i++) w[i] = (float)(gauss() * scale);
  if (rows >= 6) {
    for (int64_t c = 0; c < cols; c++) {
      w[0 * cols + c] = 0.0f;
      w[1 * cols + c] = c == 17 ? 0.5f : 0.0f;
      w[2 * cols + c] = 1e-9f;
      w[3 * cols + c] = (c % 2) ? 3e38f : -3e38f;
      w[4 * cols + c] = -0.01f;
      w[5 * cols + c] = (c % 2) ? 0.03f : -0.03f;
    }
  }
  return w;
}

static void codecs(void) {
  const int64_t rows = 12, cols = 512, nb = cols / 256;
  float *w = weights(rows, cols, 0.02);
  float *out = malloc(sizeof(float) * (size_t)(rows * cols));
  double *X = malloc(sizeof(double) * 3 * (size_t)cols), *Y = malloc(sizeof(double) * 3 * (size_t)rows);
  for (int64_t i = 0; i < 3 * cols; i++) X[i] = gauss();
  /* CB2 */
  uint8_t *cc = calloc((size_t)(rows * nb * 64), 1);
  uint16_t *cd = calloc((size_t)(rows * nb), 2);
  orc_cb2_quantize(w, rows, cols, cc, cd);
  orc_cb2_dequantize(cc, cd, rows, cols, out);
  orc_cb2_matmul(cc, cd, rows, cols, X, 3, Y);
  for (int64_t c = 0; c < cols; c++) CHECK(out[c] == 0.0f); /* zero row */
  /* Q2K */
  uint8_t *qc = calloc((size_t)(rows * nb * 64), 1), *qs = calloc((size_t)(rows * nb * 16), 1);
  uint16_t *qp = calloc((size_t)(rows * nb * 2), 2);
  orc_q2k_quantize(w, rows, cols, qc, qs, qp);
  orc_q2k_dequantize(qc, qs, qp, rows, cols, out);
  orc_q2k_matmul(qc, qs, qp, rows, cols, X, 3, Y);
  /* Q4K */
  uint8_t *kc = calloc((size_t)(rows * nb * 128), 1), *ks = calloc((size_t)(rows * nb * 12), 1);
  uint16_t *kp = calloc((size_t)(rows * nb * 2), 2);
  orc_q4k_quantize(w, rows, cols, kc, ks, kp);
  orc_q4k_dequantize(kc, ks, kp, rows, cols, out);
  orc_q4k_matmul(kc, ks, kp, rows, cols, X, 3, Y);
  for (int64_t c = 0; c < cols; c++) CHECK(out[c] == 0.0f);
  /* MXFP4, including random code and scale bytes (NaN scale 0xFF included) */
  uint8_t *mc = calloc((size_t)(rows * cols / 2), 1), *ms = calloc((size_t)(rows * cols / 32), 1);
  orc_mx4_quantize(w, rows, cols, mc, ms);
  orc_mx4_dequantize(mc, ms, rows, cols, out);
  orc_mx4_matmul(mc, ms, rows, cols, X, 3, Y);
  for (int64_t i = 0; i < rows * cols / 2; i++) mc[i] = (uint8_t)orc_splitmix64(&g_state);
  for (int64_t i = 0; i < rows * cols / 32; i++) ms[i] = (uint8_t)orc_splitmix64(&g_state);
  orc_mx4_dequantize(mc, ms, rows, cols, out);
  for (int c = 0; c < 16; c++) CHECK(fabs(orc_e2m1_value(c)) <= 6.0);
  CHECK(isnan(orc_e8m0_value(255)) && orc_e8m0_value(127) == 1.0);
  /* random bytes through the other decoders */
  for (int64_t i = 0; i < rows * nb * 64; i++) cc[i] = qc[i] = (uint8_t)orc_splitmix64(&g_state);
  for (int64_t i = 0; i < rows * nb * 16; i++) qs[i] = (uint8_t)orc_splitmix64(&g_state);
  for (int64_t i = 0; i < rows * nb * 128; i++) kc[i] = (uint8_t)orc_splitmix64(&g_state);
  for (int64_t i = 0; i < rows * nb * 12; i++) ks[i] = (uint8_t)orc_splitmix64(&g_state);
  for (int64_t i = 0; i < rows * nb; i++) cd[i] = (uint16_t)(orc_splitmix64(&g_state) & 0x3BFF);
  for (int64_t i = 0; i < rows * nb * 2; i++) qp[i] = kp[i] = (uint16_t)(orc_splitmix64(&g_state) & 0x3BFF);
  orc_cb2_dequantize(cc, cd, rows, cols, out);
  orc_q2k_dequantize(qc, qs, qp, rows, cols, out);
  orc_q4k_dequantize(kc, ks, kp, rows, cols, out);
  free(w); free(out); free(X); free(Y);
  free(cc); free(cd); free(qc); free(qs); free(qp); free(kc); free(ks); free(kp); free(mc); free(ms);
}

static void conversions(void) {
  for (uint32_t h = 0; h < 65536; h++) {
    const double v = orc_f16_to_f64((uint16_t)h);
    if (!isnan(v)) CHECK(orc_f64_to_f16(v) == (uint16_t)h || v == 0.0);
    (void)orc_bf16_to_f64((uint16_t)h);
  }
  CHECK(orc_f64_to_f16(1e9) == 0x7C00 && orc_f64_to_f16(-1e9) == 0xFC00);
  uint8_t *lv = malloc(256 * 8);
  orc_grid_levels(lv);
  for (int i = 0; i < 256 * 8; i++) CHECK(lv[i] <= 2);
  free(lv);
}

static void layer_steps(void) {
  const int64_t T = 9, d = 256, E = 40, f = 256;
  const int k = 6;
  double *X = malloc(sizeof(double) * (size_t)(T * d));
  for (int64_t i = 0; i < T * d; i++) X[i] = gauss();
  uint16_t *wr = malloc(2 * (size_t)(E * d));
  for (int64_t i = 0; i < E * d; i++) wr[i] = orc_f64_to_f16(gauss() * 0.02);
  for (int64_t c = 0; c < d; c++) wr[1 * d + c] = wr[0 * d + c]; /* an exact tie */
  float *bias = malloc(sizeof(float) * (size_t)E);
  for (int64_t e = 0; e < E; e++) bias[e] = (float)(0.1 * gauss());
  /* idx and w sized for the k = E call */
  double *lg = malloc(sizeof(double) * (size_t)(T * E)), *w = malloc(sizeof(double) * (size_t)(T * E));
  int32_t *idx = malloc(4 * (size_t)(T * E)), *cnt = malloc(4 * (size_t)E), *off = malloc(4 * (size_t)(E + 1));
  int32_t *perm = malloc(4 * (size_t)(T * k)), *inv = malloc(4 * (size_t)(T * k));
  orc_router_logits(X, T, d, wr, E, bias, lg);
  orc_router_logits(X, T, d, wr, E, NULL, lg);
  orc_topk(lg, T, E, k, idx, w);
  orc_topk(lg, T, E, 1, idx, w);
  orc_topk(lg, T, E, (int)E, idx, w); /* k = E */
  orc_topk(lg, T, E, k, idx, w);
  orc_permute(idx, T, k, E, cnt, off, perm, inv);
  CHECK(off[E] == T * k);
  for (int64_t s = 0; s < T * k; s++) CHECK(perm[inv[s]] == s);
  double *g = malloc(sizeof(double) * (size_t)(T * f)), *u = malloc(sizeof(double) * (size_t)(T * f));
  double *h = malloc(sizeof(double) * (size_t)(T * f));
  uint16_t *wg = malloc(2 * (size_t)(f * d));
  for (int64_t i = 0; i < f * d; i++) wg[i] = orc_f64_to_f16(gauss() * 0.02);
  orc_f16_matmul(wg, f, d, X, T, g);
  orc_f16_matmul(wg, f, d, X, T, u);
  orc_swiglu(g, u, T * f, h);
  free(X); free(wr); free(bias); free(lg); free(w); free(idx); free(cnt); free(off); free(perm); free(inv);
  free(g); free(u); free(h); free(wg);
}

static void mixer(void) {
  const int n = 4;
  const int64_t T = 5, d = 256, no = 2 * n + n * n, nd = n * d;
  double Z[16], A[16];
  for (int q = 0; q < 16; q++) Z[q] = 8.0 * (2.0 * unif() - 1.0);
  Z[3] = -800.0; /* exp underflows to zero */
  for (int it = 0; it <= 20; it += 20) orc_sinkhorn(Z, n, it, A);
  for (int j = 0; j < n; j++) {
    double s = 0.0;
    for (int i = 0; i < n; i++) s += A[i * n + j];
    CHECK(fabs(s - 1.0) < 1e-12);
  }
  orc_sinkhorn(Z, 2, 3, A);
  double *X = malloc(sizeof(double) * (size_t)(T * nd)), *phi = malloc(sizeof(double) * (size_t)(no * nd));
  double *bias = malloc(sizeof(double) * (size_t)no), alpha[3] = {1.0, 0.5, 2.0};
  double *coef = malloc(sizeof(double) * (size_t)(T * no)), *xin = malloc(sizeof(double) * (size_t)(T * d));
  double *y = malloc(sizeof(double) * (size_t)(T * d)), *Xo = malloc(sizeof(double) * (size_t)(T * nd));
  for (int64_t i = 0; i < T * nd; i++) X[i] = gauss();
  for (int64_t i = 0; i < nd; i++) X[i] = 0.0; /* an all-zero token: r = sqrt(eps) */
  for (int64_t i = 0; i < no * nd; i++) phi[i] = gauss() / 32.0;
  for (int64_t i = 0; i < no; i++) bias[i] = gauss();
  for (int64_t i = 0; i < T * d; i++) y[i] = gauss();
  orc_hc_pre(X, T, n, d, phi, bias, alpha, 1e-6, 20, coef, xin);
  orc_hc_post(X, y, coef, T, n, d, Xo);
  for (int64_t i = 0; i < T * no; i++) CHECK(isfinite(coef[i]));
  free(X); free(phi); free(bias); free(coef); free(xin); free(y); free(Xo);
}

int main(void) {
  orc_set_threads(2);
  conversions();
  codecs();
  layer_steps();
  mixer();
  if (g_fail) return 1;
  printf("oracle sanitize driver: ok\n");
  return 0;
}
