/*
 * ds4moe CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar implementation of the routed mixture-of-experts layer
 * that DS4 (DwarfStar 4) runs for DeepSeek V4 Flash, written so that a reader
 * can check each step against its definition by eye.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load this
 * file's library; the product path never does.  It shares no code, header,
 * table or constant generator with the GPU library.
 *
 * What the pages fix (DS4 (DwarfStar 4) wiki note, "Architecture" and "Key
 * Techniques"; TopDigg "DwarfStar (ds4) Deep Dive", section 3.4 "Asymmetric
 * Quantization"):
 *   - 256 routed experts, 6 active per token plus 1 shared expert, d = 4096;
 *   - only the routed experts are quantized: gate/up in IQ2_XXS, down in Q2_K;
 *     router and shared expert stay F16.
 * Everything else (grid contents, bit layout, scale rules, score function,
 * slot order) is left open by the pages; the readings taken here are listed
 * next to each function.  Arithmetic is fp64 for the layer math; the codecs
 * follow their written fp32 definitions exactly (every step is one IEEE
 * operation, round-to-nearest-even, no contraction: build with
 * -ffp-contract=off).
 *
 * Parallelism: OpenMP only over independent output rows, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256 /* super-block length along the input (K) dimension */

/* ------------------------------------------------------------------------- */
/* IEEE half precision, written from the binary16 definition                  */
/* ------------------------------------------------------------------------- */

/* binary16 bits -> value (exact in double). */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

float orc_f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

/* value -> nearest binary16, ties to even; overflow -> inf (IEEE rule). */
uint16_t orc_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (a >= 65520.0) /* 65504 + half an ulp (16) rounds to infinity */
        return sign | 0x7C00;
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) -> unbiased exponent e2-1 */
    int unb = (a == 0.0) ? -25 : e2 - 1;
    /* quantum: 2^-24 in the subnormal range, else 2^(unb-10) */
    int qexp = unb < -14 ? -24 : unb - 10;
    double n = nearbyint(ldexp(a, -qexp)); /* integer count of quanta, RNE */
    double r = ldexp(n, qexp);              /* rounded magnitude */
    if (r == 0.0)
        return sign;
    int re2;
    frexp(r, &re2);
    int runb = re2 - 1;
    if (runb < -14) /* subnormal result */
        return sign | (uint16_t)n;
    uint16_t bits = (uint16_t)(((runb + 15) << 10) | ((uint32_t)ldexp(r, -runb + 10) & 0x3FF));
    return sign | bits;
}

/* bf16 bits -> value (the upper half of a binary32). */
double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------- */
/* Codebook grid (the pages call the gate/up format IQ2_XXS and say its       */
/* layout comes from GGML; the GGML tables are not used).  The grid is 256    */
/* entries of 8 magnitude levels in {0,1,2} -> magnitudes {1,3,5}, drawn with */
/* splitmix64 (Steele, Lea & Flood, OOPSLA 2014) from a fixed seed; an entry  */
/* equal to an earlier one is drawn again.                                    */
/* ------------------------------------------------------------------------- */

#define ORC_GRID_SEED 0x44533447524944ULL /* ASCII "DS4GRID" */

uint64_t orc_splitmix64(uint64_t *state)
{
    *state += 0x9E3779B97F4A7C15ULL;
    uint64_t z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* levels[256*8]: level (0,1,2) of coordinate k of entry i at [8*i + k]. */
void orc_grid_levels(uint8_t *levels)
{
    uint64_t st = ORC_GRID_SEED;
    for (int i = 0; i < 256; i++) {
        for (;;) {
            for (int k = 0; k < 8; k++)
                levels[8 * i + k] = (uint8_t)((orc_splitmix64(&st) >> 32) % 3);
            int dup = 0;
            for (int j = 0; j < i && !dup; j++)
                dup = memcmp(levels + 8 * j, levels + 8 * i, 8) == 0;
            if (!dup)
                break;
        }
    }
}

/* Magnitudes m = 2*level + 1 of the grid, filled once before any parallel
 * region by ensure_grid(). */
static int32_t g_mag[256 * 8];
static int32_t g_magT[8][256]; /* g_magT[k][e] = m_ek */
static int g_grid_ready = 0;

static void ensure_grid(void)
{
    if (!g_grid_ready) {
        uint8_t lv[256 * 8];
        orc_grid_levels(lv);
        for (int i = 0; i < 256 * 8; i++)
            g_mag[i] = 2 * lv[i] + 1;
        for (int e = 0; e < 256; e++)
            for (int k = 0; k < 8; k++)
                g_magT[k][e] = g_mag[8 * e + k];
        g_grid_ready = 1;
    }
}

static int grid_mag(int entry, int k) { return g_mag[8 * entry + k]; }

/* Sign of element k (0..7) of a group with 7-bit sign code c: bits 0..6 are
 * explicit, bit 7 is the parity of c, so every group has an even number of
 * negative elements.  Returns 1 for negative. */
static int sign_bit(uint32_t c, int k)
{
    if (k < 7)
        return (c >> k) & 1;
    return __builtin_popcount(c & 0x7F) & 1;
}

/* ------------------------------------------------------------------------- */
/* CB2: the 2-bit codebook format for gate/up (IQ2_XXS class).                */
/*                                                                            */
/* A [rows, cols] matrix, cols % 256 == 0, nb = cols/256 blocks per row, is   */
/* stored as two planes:                                                      */
/*   code plane  [rows][nb][64] bytes: for sub-block j (32 weights) bytes     */
/*               8j..8j+3 are the grid indices of its 4 groups of 8, bytes    */
/*               8j+4..8j+7 a little-endian u32 "aux": bits 7g..7g+6 the sign */
/*               code of group g, bits 28..31 the sub-block scale s (0..15).  */
/*   scale plane [rows][nb] binary16 d.                                       */
/* Weight K = 256 b + 32 j + 8 g + k has value                                */
/*     sign * (d * (2 s + 1)) * m,   m = 2 * level + 1 of grid[idx][k]        */
/* Each product is exact in binary32 (at most 11+5+3 significant bits).       */
/* ------------------------------------------------------------------------- */

void orc_cb2_dequantize(const uint8_t *codes, const uint16_t *dplane, int64_t rows, int64_t cols,
                        float *out)
{
    ensure_grid();
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = codes + (r * nb + b) * 64;
            float d = orc_f16_to_f32(dplane[r * nb + b]);
            for (int j = 0; j < 8; j++) {
                uint32_t aux = (uint32_t)blk[8 * j + 4] | (uint32_t)blk[8 * j + 5] << 8 |
                               (uint32_t)blk[8 * j + 6] << 16 | (uint32_t)blk[8 * j + 7] << 24;
                int s = (int)(aux >> 28);
                float ds = d * (float)(2 * s + 1);
                for (int g = 0; g < 4; g++) {
                    int idx = blk[8 * j + g];
                    uint32_t c = (aux >> (7 * g)) & 0x7F;
                    for (int k = 0; k < 8; k++) {
                        float w = ds * (float)grid_mag(idx, k);
                        out[r * cols + b * QK + 32 * j + 8 * g + k] = sign_bit(c, k) ? -w : w;
                    }
                }
            }
        }
    }
}

/* binary32 -> binary16 with the quantizer's clamp: values above the largest
 * finite half are stored as 65504 (never as infinity). */
static uint16_t f16_clamped(float v)
{
    if (v > 65504.0f)
        v = 65504.0f;
    return orc_f64_to_f16((double)v);
}

/* Integer score of all 256 grid entries for one group:
 *   sum_k (4096 m_ek^2 - 2 R_k m_ek)  [+ 4 min_k R_k m_ek if odd]
 * Values stay below 2^25, so int32 is exact. */

__attribute__((target_clones("avx2", "default"))) static void search_scores(const int32_t R[8], int odd,
                                                                           int32_t score[256])
{
    int32_t mn[256];
    for (int e = 0; e < 256; e++) {
        score[e] = 0;
        mn[e] = INT32_MAX;
    }
    for (int k = 0; k < 8; k++) {
        for (int e = 0; e < 256; e++) {
            int32_t m = g_magT[k][e];
            int32_t f = R[k] * m;
            score[e] += 4096 * m * m - 2 * f;
            mn[e] = f < mn[e] ? f : mn[e];
        }
    }
    if (odd)
        for (int e = 0; e < 256; e++)
            score[e] += 4 * mn[e];
}

/*
 * CB2 quantizer (deterministic; its steps are this library's own, since the
 * pages give none):
 *  1. per sub-block j:  A_j = max|x| / 5            (binary32 division)
 *  2. d = half(max_j A_j / 31), clamped to 65504; if d == 0 every code is 0
 *  3. s_j = clamp(rne((A_j / d - 1) * 0.5), 0, 15); a_j = d * (2 s_j + 1)
 *  4. per group of 8: r_k = min(|x_k| / a_j, 64), R_k = rne(r_k * 4096)
 *     (integers); score of entry e is
 *         sum_k (4096 m_ek^2 - 2 R_k m_ek)        (= 4096 * SSE/a^2 - const)
 *     plus, when the number of negative x_k is odd, 4 * min_k R_k m_ek (the
 *     cheapest single sign flip that restores even parity).  The entry with
 *     the lowest score wins, ties to the lower index; the flipped element is
 *     the k of lowest R_k m_ek, ties to the lower k.  Sign code = bits 0..6.
 * x_k < 0 is the sign test (so -0.0 counts as positive).  Inputs must be
 * finite.
 */
static void cb2_quantize_block(const float *x, uint8_t *blk, uint16_t *dout)
{
    float A[8];
    float amax = 0.0f;
    for (int j = 0; j < 8; j++) {
        float mx = 0.0f;
        for (int i = 0; i < 32; i++) {
            float v = fabsf(x[32 * j + i]);
            if (v > mx)
                mx = v;
        }
        A[j] = mx / 5.0f;
        if (A[j] > amax)
            amax = A[j];
    }
    uint16_t dbits = f16_clamped(amax / 31.0f);
    float d = orc_f16_to_f32(dbits);
    memset(blk, 0, 64);
    *dout = dbits;
    if (d == 0.0f)
        return;
    for (int j = 0; j < 8; j++) {
        float t = A[j] / d;
        float u = (t - 1.0f) * 0.5f;
        float sr = rintf(u);
        int s = sr < 0.0f ? 0 : (sr > 15.0f ? 15 : (int)sr);
        float a = d * (float)(2 * s + 1);
        uint32_t aux = (uint32_t)s << 28;
        for (int g = 0; g < 4; g++) {
            const float *xg = x + 32 * j + 8 * g;
            int32_t R[8];
            int neg = 0, nneg = 0;
            for (int k = 0; k < 8; k++) {
                float r = fabsf(xg[k]) / a;
                if (r > 64.0f)
                    r = 64.0f;
                R[k] = (int32_t)rintf(r * 4096.0f);
                if (xg[k] < 0.0f) {
                    neg |= 1 << k;
                    nneg++;
                }
            }
            int odd = nneg & 1;
            /* score of every entry, then the lowest (lower index on ties) */
            int32_t score[256];
            search_scores(R, odd, score);
            int best = 0;
            for (int e = 1; e < 256; e++)
                if (score[e] < score[best])
                    best = e;
            if (odd) {
                int kf = 0;
                int64_t fmin = -1;
                for (int k = 0; k < 8; k++) {
                    int64_t f = (int64_t)R[k] * grid_mag(best, k);
                    if (fmin < 0 || f < fmin) {
                        fmin = f;
                        kf = k;
                    }
                }
                neg ^= 1 << kf;
            }
            blk[8 * j + g] = (uint8_t)best;
            aux |= (uint32_t)(neg & 0x7F) << (7 * g);
        }
        blk[8 * j + 4] = (uint8_t)(aux & 0xFF);
        blk[8 * j + 5] = (uint8_t)((aux >> 8) & 0xFF);
        blk[8 * j + 6] = (uint8_t)((aux >> 16) & 0xFF);
        blk[8 * j + 7] = (uint8_t)(aux >> 24);
    }
}

void orc_cb2_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint16_t *dplane)
{
    ensure_grid();
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            cb2_quantize_block(w + r * cols + b * QK, codes + (r * nb + b) * 64, dplane + r * nb + b);
}

/* ------------------------------------------------------------------------- */
/* Q2K: the 2-bit super-block format for down (Q2_K class).                   */
/*                                                                            */
/* [rows, cols], nb = cols/256, three planes:                                 */
/*   code plane     [rows][nb][64]: sub-block j (16 weights) is the LE u32    */
/*                  at bytes 4j..4j+3, element i at bits 2i..2i+1 (q 0..3)    */
/*   subscale plane [rows][nb][16]: byte j = s_j | m_j << 4                   */
/*   superscale     [rows][nb][2] binary16: d, then dmin                      */
/* Weight K = 256 b + 16 j + i has value (d * s_j) * q - dmin * m_j: both     */
/* products are exact in binary32, the difference is rounded once.           */
/* ------------------------------------------------------------------------- */

static float q2k_value(float d, float dmin, int s, int m, int q)
{
    float t1 = d * (float)s;
    t1 = t1 * (float)q;
    float t2 = dmin * (float)m;
    return t1 - t2;
}

void orc_q2k_dequantize(const uint8_t *codes, const uint8_t *sub, const uint16_t *sup, int64_t rows,
                        int64_t cols, float *out)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = codes + (r * nb + b) * 64;
            const uint8_t *sc = sub + (r * nb + b) * 16;
            float d = orc_f16_to_f32(sup[(r * nb + b) * 2 + 0]);
            float dmin = orc_f16_to_f32(sup[(r * nb + b) * 2 + 1]);
            for (int j = 0; j < 16; j++) {
                uint32_t u = (uint32_t)blk[4 * j] | (uint32_t)blk[4 * j + 1] << 8 |
                             (uint32_t)blk[4 * j + 2] << 16 | (uint32_t)blk[4 * j + 3] << 24;
                int s = sc[j] & 0xF, m = sc[j] >> 4;
                for (int i = 0; i < 16; i++) {
                    int q = (int)((u >> (2 * i)) & 3);
                    out[r * cols + b * QK + 16 * j + i] = q2k_value(d, dmin, s, m, q);
                }
            }
        }
    }
}

/*
 * Q2K quantizer (this library's own deterministic steps):
 *  1. per sub-block j of 16: b_j = max(0, -min x), a_j = (max x + b_j) / 3
 *  2. d = half(max_j a_j / 15), dmin = half(max_j b_j / 15), clamped to 65504
 *  3. s_j = d > 0 ? clamp(rne(a_j / d), 0, 15) : 0; m_j likewise with dmin
 *  4. q = argmin over 0..3 of |value(q) - x| using the decoder's own binary32
 *     formula, ties to the lower q.
 */
static void q2k_quantize_block(const float *x, uint8_t *blk, uint8_t *sc, uint16_t *sup)
{
    float a[16], bb[16];
    float amax = 0.0f, bmax = 0.0f;
    for (int j = 0; j < 16; j++) {
        float mx = x[16 * j], mn = x[16 * j];
        for (int i = 1; i < 16; i++) {
            float v = x[16 * j + i];
            if (v > mx)
                mx = v;
            if (v < mn)
                mn = v;
        }
        bb[j] = mn < 0.0f ? -mn : 0.0f;
        a[j] = (mx + bb[j]) / 3.0f;
        if (a[j] > amax)
            amax = a[j];
        if (bb[j] > bmax)
            bmax = bb[j];
    }
    uint16_t dbits = f16_clamped(amax / 15.0f);
    uint16_t mbits = f16_clamped(bmax / 15.0f);
    float d = orc_f16_to_f32(dbits), dmin = orc_f16_to_f32(mbits);
    sup[0] = dbits;
    sup[1] = mbits;
    for (int j = 0; j < 16; j++) {
        int s = 0, m = 0;
        if (d > 0.0f) {
            float v = rintf(a[j] / d);
            s = v < 0.0f ? 0 : (v > 15.0f ? 15 : (int)v);
        }
        if (dmin > 0.0f) {
            float v = rintf(bb[j] / dmin);
            m = v < 0.0f ? 0 : (v > 15.0f ? 15 : (int)v);
        }
        sc[j] = (uint8_t)(s | (m << 4));
        uint32_t u = 0;
        for (int i = 0; i < 16; i++) {
            float xv = x[16 * j + i];
            int bq = 0;
            float berr = 0.0f;
            for (int q = 0; q < 4; q++) {
                float err = fabsf(q2k_value(d, dmin, s, m, q) - xv);
                if (q == 0 || err < berr) {
                    bq = q;
                    berr = err;
                }
            }
            u |= (uint32_t)bq << (2 * i);
        }
        blk[4 * j + 0] = (uint8_t)(u & 0xFF);
        blk[4 * j + 1] = (uint8_t)((u >> 8) & 0xFF);
        blk[4 * j + 2] = (uint8_t)((u >> 16) & 0xFF);
        blk[4 * j + 3] = (uint8_t)(u >> 24);
    }
}

void orc_q2k_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *sub,
                      uint16_t *sup)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            q2k_quantize_block(w + r * cols + b * QK, codes + (r * nb + b) * 64, sub + (r * nb + b) * 16,
                               sup + (r * nb + b) * 2);
}

/* ------------------------------------------------------------------------- */
/* Q4K: the 4-bit super-block format (Q4_K class, 4.5 bits per weight) of the */
/* Q4 layers of the q2-q4 mix (TopDigg "DwarfStar (ds4) Deep Dive", 5.2:      */
/* the last six routed-expert layers at Q4; the wiki note's Comparison Notes  */
/* name the Q4_K layouts).  Layout (this library's own):                      */
/*   code plane     [rows][nb][128]: sub-block j (32 weights) at bytes        */
/*                  16j..16j+15 of its block; LE u32 word k of a sub-block    */
/*                  holds elements 8k..8k+7: element 8k+2p at bits 4p..4p+3,  */
/*                  element 8k+2p+1 at bits 16+4p..19+4p (p = 0..3)           */
/*   scale plane    [rows][nb][12]: LE u32 w0, w1, w2; nibble j of w0 is      */
/*                  s_j & 15, nibble j of w1 is m_j & 15, bits 2j..2j+1 of w2 */
/*                  are s_j >> 4 and bits 16+2j..17+2j are m_j >> 4 (6 bits) */
/*   superscale     [rows][nb][2] binary16: d, then dmin                      */
/* Weight K = 256 b + 32 j + i has value (d * s_j) * q - dmin * m_j: both     */
/* products are exact in binary32, the difference is rounded once.           */
/* ------------------------------------------------------------------------- */

static int q4k_code(const uint8_t *blk, int i) /* element i (0..255) of a block's code plane */
{
    int j = i / 32, r = i % 32, k = r / 8, e = r % 8, p = e / 2;
    const uint8_t *w = blk + 16 * j + 4 * k;
    uint32_t u = (uint32_t)w[0] | (uint32_t)w[1] << 8 | (uint32_t)w[2] << 16 | (uint32_t)w[3] << 24;
    int sh = (e & 1) ? 16 + 4 * p : 4 * p;
    return (int)((u >> sh) & 15u);
}

static void q4k_scale_min(const uint8_t *sc, int j, int *s, int *m)
{
    uint32_t w[3];
    for (int t = 0; t < 3; t++)
        w[t] = (uint32_t)sc[4 * t] | (uint32_t)sc[4 * t + 1] << 8 | (uint32_t)sc[4 * t + 2] << 16 |
               (uint32_t)sc[4 * t + 3] << 24;
    *s = (int)(((w[0] >> (4 * j)) & 15u) | (((w[2] >> (2 * j)) & 3u) << 4));
    *m = (int)(((w[1] >> (4 * j)) & 15u) | (((w[2] >> (16 + 2 * j)) & 3u) << 4));
}

void orc_q4k_dequantize(const uint8_t *codes, const uint8_t *scales, const uint16_t *sup, int64_t rows, int64_t cols,
                        float *out)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = codes + (r * nb + b) * 128;
            const uint8_t *sc = scales + (r * nb + b) * 12;
            float d = orc_f16_to_f32(sup[(r * nb + b) * 2]), dmin = orc_f16_to_f32(sup[(r * nb + b) * 2 + 1]);
            for (int i = 0; i < QK; i++) {
                int s, m;
                q4k_scale_min(sc, i / 32, &s, &m);
                float t1 = d * (float)s;
                t1 = t1 * (float)q4k_code(blk, i);
                float t2 = dmin * (float)m;
                out[r * cols + b * QK + i] = t1 - t2;
            }
        }
}

/*
 * Q4K quantizer (this library's own deterministic steps, those of Q2K at
 * 4-bit codes and 6-bit scales):
 *  1. per sub-block j of 32: b_j = max(0, -min x), a_j = (max x + b_j) / 15
 *  2. d = half(max_j a_j / 63), dmin = half(max_j b_j / 63), clamped to 65504
 *  3. s_j = d > 0 ? clamp(rne(a_j / d), 0, 63) : 0; m_j likewise with dmin
 *  4. q = argmin over 0..15 of |value(q) - x| using the decoder's own binary32
 *     formula, ties to the lower q.
 */
static void q4k_quantize_block(const float *x, uint8_t *blk, uint8_t *sc, uint16_t *sup)
{
    float a[8], bb[8], amax = 0.0f, bmax = 0.0f;
    for (int j = 0; j < 8; j++) {
        float mx = x[32 * j], mn = x[32 * j];
        for (int i = 1; i < 32; i++) {
            float v = x[32 * j + i];
            if (v > mx)
                mx = v;
            if (v < mn)
                mn = v;
        }
        bb[j] = mn < 0.0f ? -mn : 0.0f;
        a[j] = (mx + bb[j]) / 15.0f;
        if (a[j] > amax)
            amax = a[j];
        if (bb[j] > bmax)
            bmax = bb[j];
    }
    uint16_t dbits = f16_clamped(amax / 63.0f), mbits = f16_clamped(bmax / 63.0f);
    float d = orc_f16_to_f32(dbits), dmin = orc_f16_to_f32(mbits);
    sup[0] = dbits;
    sup[1] = mbits;
    uint32_t w[3] = {0u, 0u, 0u};
    memset(blk, 0, 128);
    for (int j = 0; j < 8; j++) {
        int s = 0, m = 0;
        if (d > 0.0f) {
            float v = rintf(a[j] / d);
            s = v < 0.0f ? 0 : (v > 63.0f ? 63 : (int)v);
        }
        if (dmin > 0.0f) {
            float v = rintf(bb[j] / dmin);
            m = v < 0.0f ? 0 : (v > 63.0f ? 63 : (int)v);
        }
        w[0] |= (uint32_t)(s & 15) << (4 * j);
        w[1] |= (uint32_t)(m & 15) << (4 * j);
        w[2] |= (uint32_t)(s >> 4) << (2 * j) | (uint32_t)(m >> 4) << (16 + 2 * j);
        for (int i = 0; i < 32; i++) {
            float xv = x[32 * j + i];
            int bq = 0;
            float berr = 0.0f;
            for (int q = 0; q < 16; q++) {
                float t1 = d * (float)s;
                t1 = t1 * (float)q;
                float err = fabsf((t1 - dmin * (float)m) - xv);
                if (q == 0 || err < berr) {
                    bq = q;
                    berr = err;
                }
            }
            int k = i / 8, e = i % 8, p = e / 2;
            int sh = (e & 1) ? 16 + 4 * p : 4 * p;
            uint8_t *wb = blk + 16 * j + 4 * k;
            uint32_t u = (uint32_t)wb[0] | (uint32_t)wb[1] << 8 | (uint32_t)wb[2] << 16 | (uint32_t)wb[3] << 24;
            u |= (uint32_t)bq << sh;
            wb[0] = (uint8_t)u;
            wb[1] = (uint8_t)(u >> 8);
            wb[2] = (uint8_t)(u >> 16);
            wb[3] = (uint8_t)(u >> 24);
        }
    }
    for (int t = 0; t < 3; t++) {
        sc[4 * t] = (uint8_t)w[t];
        sc[4 * t + 1] = (uint8_t)(w[t] >> 8);
        sc[4 * t + 2] = (uint8_t)(w[t] >> 16);
        sc[4 * t + 3] = (uint8_t)(w[t] >> 24);
    }
}

void orc_q4k_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales, uint16_t *sup)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            q4k_quantize_block(w + r * cols + b * QK, codes + (r * nb + b) * 128, scales + (r * nb + b) * 12,
                               sup + (r * nb + b) * 2);
}

void orc_q4k_matmul(const uint8_t *codes, const uint8_t *scales, const uint16_t *sup, int64_t rows, int64_t cols,
                    const double *X, int64_t n, double *Y)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)cols);
        orc_q4k_dequantize(codes + r * nb * 128, scales + r * nb * 12, sup + r * nb * 2, 1, cols, wrow);
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += (double)wrow[i] * X[t * cols + i];
            Y[t * rows + r] = acc;
        }
        free(wrow);
    }
}

/* ------------------------------------------------------------------------- */
/* MXFP4: the public OCP Microscaling (MX) format with FP4 E2M1 elements, one  */
/* E8M0 scale per block of 32 elements.  It is DeepSeek's native format for    */
/* the routed experts (TopDigg "DwarfStar (ds4) Deep Dive", 5.2, download     */
/* options; diego-rodriguez.work guide, 4, model files).                      */
/*   E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is  */
/*         subnormal (0 and 0.5).  Values 0, 0.5, 1, 1.5, 2, 3, 4, 6.         */
/*   E8M0: 8 exponent bits, bias 127, value 2^(E - 127); 0xFF is NaN.         */
/* [rows, cols], two planes: codes rows*cols/2 bytes (element k of a row at   */
/* byte k/2, even k in the low nibble), then scales rows*cols/32 bytes.       */
/* Weight = e2m1(code) * 2^(scale - 127), exact in binary32 (rounded only     */
/* where it leaves binary32's range, scale codes >= 253).                     */
/* ------------------------------------------------------------------------- */

double orc_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

double orc_e8m0_value(int code)
{
    return code == 255 ? NAN : ldexp(1.0, code - 127);
}

void orc_mx4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols; k++) {
            int byte = codes[(r * cols + k) / 2];
            int c = (k & 1) ? byte >> 4 : byte & 15;
            double v = orc_e2m1_value(c) * orc_e8m0_value(scales[(r * cols + k) / 32]);
            out[r * cols + k] = (float)v;
        }
}

/*
 * MXFP4 quantizer, the OCP MX conversion of a block of 32:
 *  1. amax = max |x|; a block of zeros gets scale code 0 and zero elements;
 *  2. shared exponent = floor(log2(amax)) - 2 (2 = the largest E2M1
 *     exponent), stored biased by 127 and clamped to 0..254;
 *  3. each x / 2^shared is rounded to the nearest E2M1 value, ties to the
 *     even code, values beyond 6 to 6 (saturation: 6 is the nearest);
 *     the sign bit is set for negative x with a non-zero magnitude.
 * Inputs must be finite.
 */
static void mx4_quantize_block(const float *x, uint8_t *codes, uint8_t *scale)
{
    double amax = 0.0;
    for (int i = 0; i < 32; i++) {
        double a = fabs((double)x[i]);
        if (a > amax)
            amax = a;
    }
    memset(codes, 0, 16);
    *scale = 0;
    if (amax == 0.0)
        return;
    int ex;
    frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1 */
    int sc = (ex - 1) - 2 + 127;
    sc = sc < 0 ? 0 : (sc > 254 ? 254 : sc);
    *scale = (uint8_t)sc;
    for (int i = 0; i < 32; i++) {
        double r = ldexp(fabs((double)x[i]), 127 - sc); /* exact */
        int best = 0;
        double bd = r;
        for (int c = 1; c < 8; c++) {
            double dd = fabs(r - orc_e2m1_value(c));
            if (dd < bd || (dd == bd && (c & 1) == 0)) {
                bd = dd;
                best = c;
            }
        }
        int code = best | ((x[i] < 0.0f && best != 0) ? 8 : 0);
        codes[i / 2] |= (uint8_t)((i & 1) ? code << 4 : code);
    }
}

void orc_mx4_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < cols / 32; b++)
            mx4_quantize_block(w + r * cols + b * 32, codes + (r * cols + b * 32) / 2, scales + (r * cols) / 32 + b);
}

/* ------------------------------------------------------------------------- */
/* Products with fp64 accumulation (sequential over K).                       */
/* Y[n][rows] = W[rows][cols] . X[n][cols], W given packed or as F16.         */
/* ------------------------------------------------------------------------- */

void orc_cb2_matmul(const uint8_t *codes, const uint16_t *dplane, int64_t rows, int64_t cols,
                    const double *X, int64_t n, double *Y)
{
    ensure_grid();
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)cols);
        orc_cb2_dequantize(codes + r * nb * 64, dplane + r * nb, 1, cols, wrow);
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += (double)wrow[i] * X[t * cols + i];
            Y[t * rows + r] = acc;
        }
        free(wrow);
    }
}

void orc_q2k_matmul(const uint8_t *codes, const uint8_t *sub, const uint16_t *sup, int64_t rows,
                    int64_t cols, const double *X, int64_t n, double *Y)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)cols);
        orc_q2k_dequantize(codes + r * nb * 64, sub + r * nb * 16, sup + r * nb * 2, 1, cols, wrow);
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += (double)wrow[i] * X[t * cols + i];
            Y[t * rows + r] = acc;
        }
        free(wrow);
    }
}

void orc_mx4_matmul(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, const double *X,
                    int64_t n, double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)cols);
        orc_mx4_dequantize(codes + r * cols / 2, scales + r * cols / 32, 1, cols, wrow);
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += (double)wrow[i] * X[t * cols + i];
            Y[t * rows + r] = acc;
        }
        free(wrow);
    }
}

void orc_f16_matmul(const uint16_t *w, int64_t rows, int64_t cols, const double *X, int64_t n, double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)cols);
        for (int64_t i = 0; i < cols; i++)
            wrow[i] = orc_f16_to_f64(w[r * cols + i]);
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += wrow[i] * X[t * cols + i];
            Y[t * rows + r] = acc;
        }
        free(wrow);
    }
}

/* ------------------------------------------------------------------------- */
/* Router, top-k, gate weights (the pages: an F16 router picks 6 of 256).     */
/* Readings where the pages are silent: logits plus an optional bias; the k   */
/* largest logits win, equal logits to the lower expert index; the selected   */
/* experts are listed in ascending index order; their weights are the        */
/* softmax of their logits (sum 1, no extra scaling factor).                  */
/* ------------------------------------------------------------------------- */

void orc_router_logits(const double *X, int64_t T, int64_t d, const uint16_t *wr, int64_t E,
                       const float *bias, double *logits)
{
    orc_f16_matmul(wr, E, d, X, T, logits); /* logits[t][e] */
    if (bias)
        for (int64_t t = 0; t < T; t++)
            for (int64_t e = 0; e < E; e++)
                logits[t * E + e] += (double)bias[e];
}

void orc_topk(const double *logits, int64_t T, int64_t E, int k, int32_t *idx, double *w)
{
    for (int64_t t = 0; t < T; t++) {
        const double *l = logits + t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        /* k rounds of "largest remaining logit, lower index on ties" */
        for (int j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
        }
        int j = 0;
        for (int64_t e = 0; e < E; e++)
            if (taken[e])
                idx[t * k + j++] = (int32_t)e;
        free(taken);
        double lmax = -INFINITY;
        for (j = 0; j < k; j++)
            if (l[idx[t * k + j]] > lmax)
                lmax = l[idx[t * k + j]];
        double den = 0.0;
        for (j = 0; j < k; j++)
            den += exp(l[idx[t * k + j]] - lmax);
        for (j = 0; j < k; j++)
            w[t * k + j] = exp(l[idx[t * k + j]] - lmax) / den;
    }
}

/* ------------------------------------------------------------------------- */
/* Token -> expert grouping: counts, exclusive offsets, and perm = the slot   */
/* ids s = t*k + j sorted by (expert, token); inv is perm's inverse.          */
/* ------------------------------------------------------------------------- */

void orc_permute(const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts, int32_t *offsets,
                 int32_t *perm, int32_t *inv)
{
    for (int64_t e = 0; e < E; e++)
        counts[e] = 0;
    for (int64_t s = 0; s < T * k; s++)
        counts[idx[s]]++;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int64_t p = 0;
    for (int64_t e = 0; e < E; e++)
        for (int64_t t = 0; t < T; t++)
            for (int j = 0; j < k; j++)
                if (idx[t * k + j] == e) {
                    perm[p] = (int32_t)(t * k + j);
                    inv[t * k + j] = (int32_t)p;
                    p++;
                }
}

/* ------------------------------------------------------------------------- */
/* SwiGLU (reading of "gate/up/down": h = silu(gate) * up, silu(z) =          */
/* z / (1 + e^-z), no clamp).                                                 */
/* ------------------------------------------------------------------------- */

void orc_swiglu(const double *g, const double *u, int64_t n, double *h)
{
    for (int64_t i = 0; i < n; i++)
        h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* ------------------------------------------------------------------------- */
/* Hyper-connection mixer around the layer (DS4 (DwarfStar 4) wiki note, "Key */
/* Techniques": activations travel as n = 4 streams of d = 4096, a learned    */
/* mixer normalised by 20 Sinkhorn iterations reduces them to one row for the */
/* sublayer and expands the sublayer's output back into n streams).          */
/* Readings where the note is silent, after the manifold-constrained          */
/* hyper-connection formulation that pairs a Sinkhorn-normalised residual     */
/* mixer with per-stream reduce and expand weights:                           */
/*   X [n][d] per token, flattened as k = i*d + c;                            */
/*   x' = X / sqrt(mean_k X_k^2 + eps)      (RMS over all n*d values)          */
/*   z_o = alpha_g * sum_k phi[o][k] x'_k + bias[o],  o < 2n + n*n, with      */
/*         g = pre for o < n, post for n <= o < 2n, res otherwise             */
/*   pre_i  = sigmoid(z_i)                  (reduce weights)                  */
/*   post_i = 2 sigmoid(z_{n+i})            (expand weights)                  */
/*   M = Sinkhorn(exp(Z)), Z[i][j] = z_{2n + n*i + j}; one iteration divides   */
/*       every row by its sum, then every column by its sum                   */
/*   reduce:  x_in[c]   = sum_i pre_i X[i][c]                                 */
/*   expand:  X'[i][c]  = sum_j M[i][j] X[j][c] + post_i y[c]                 */
/* ------------------------------------------------------------------------- */

/* A[n][n] <- `iters` Sinkhorn iterations applied to exp(Z). */
void orc_sinkhorn(const double *Z, int n, int iters, double *A)
{
    for (int q = 0; q < n * n; q++)
        A[q] = exp(Z[q]);
    for (int it = 0; it < iters; it++) {
        for (int i = 0; i < n; i++) {
            double s = 0.0;
            for (int j = 0; j < n; j++)
                s += A[i * n + j];
            for (int j = 0; j < n; j++)
                A[i * n + j] /= s;
        }
        for (int j = 0; j < n; j++) {
            double s = 0.0;
            for (int i = 0; i < n; i++)
                s += A[i * n + j];
            for (int i = 0; i < n; i++)
                A[i * n + j] /= s;
        }
    }
}

/* X [T][n][d]; phi [2n+n*n][n*d]; bias [2n+n*n]; alpha {pre, post, res}.
 * coef [T][2n+n*n] = pre (n), post (n), M (n*n, row-major); xin [T][d]. */
void orc_hc_pre(const double *X, int64_t T, int n, int64_t d, const double *phi, const double *bias,
                const double *alpha, double eps, int iters, double *coef, double *xin)
{
    const int no = 2 * n + n * n;
    const int64_t nd = (int64_t)n * d;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const double *x = X + t * nd;
        double ss = 0.0;
        for (int64_t k = 0; k < nd; k++)
            ss += x[k] * x[k];
        const double r = sqrt(ss / (double)nd + eps);
        double *xn = (double *)malloc(sizeof(double) * (size_t)nd);
        for (int64_t k = 0; k < nd; k++)
            xn[k] = x[k] / r;
        double *z = (double *)malloc(sizeof(double) * (size_t)no);
        for (int o = 0; o < no; o++) {
            double acc = 0.0;
            for (int64_t k = 0; k < nd; k++)
                acc += phi[(int64_t)o * nd + k] * xn[k];
            const double a = o < n ? alpha[0] : (o < 2 * n ? alpha[1] : alpha[2]);
            z[o] = a * acc + bias[o];
        }
        double *cf = coef + t * no;
        for (int i = 0; i < n; i++) {
            cf[i] = 1.0 / (1.0 + exp(-z[i]));
            cf[n + i] = 2.0 / (1.0 + exp(-z[n + i]));
        }
        orc_sinkhorn(z + 2 * n, n, iters, cf + 2 * n);
        for (int64_t c = 0; c < d; c++) {
            double acc = 0.0;
            for (int i = 0; i < n; i++)
                acc += cf[i] * x[(int64_t)i * d + c];
            xin[t * d + c] = acc;
        }
        free(z);
        free(xn);
    }
}

/* Xout [T][n][d] = M X + post y, with coef as orc_hc_pre writes it. */
void orc_hc_post(const double *X, const double *y, const double *coef, int64_t T, int n, int64_t d, double *Xout)
{
    const int no = 2 * n + n * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const double *cf = coef + t * no;
        const double *M = cf + 2 * n;
        for (int i = 0; i < n; i++)
            for (int64_t c = 0; c < d; c++) {
                double acc = 0.0;
                for (int j = 0; j < n; j++)
                    acc += M[i * n + j] * X[(t * n + j) * d + c];
                Xout[(t * n + i) * d + c] = acc + cf[n + i] * y[t * d + c];
            }
    }
}

/* ------------------------------------------------------------------------- */
/* Threads of the parallel loops (independent output rows only, so results   */
/* do not depend on the count).                                              */
/* ------------------------------------------------------------------------- */

void orc_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}

int orc_max_threads(void)
{
    return omp_get_max_threads();
}
