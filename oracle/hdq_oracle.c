/*
 * hdq_oracle.c -- plain, slow CPU oracle for the block-Hadamard quantize and
 * quantized linear path of 6Bit-Diffusion's dynamic mixed-precision
 * quantization (DMPQ).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library
 * never calls it.  Every loop is written out in the order the method states;
 * nothing is blocked, fused or vectorised by hand.  Build:
 *     gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (no FMA contraction, so every float32 expression rounds where written).
 *
 * Sources, cited in the comments below as:
 *   [S1] "6Bit-Diffusion" summary of arXiv:2603.18742 (vetunion.cn), section
 *        one, dynamic mixed-precision quantization: two activation formats,
 *        NVFP4 and INT8; INT8 when the previous step's module input/output
 *        difference is large, NVFP4 when it is small; block Hadamard
 *        transform to spread outliers before quantizing.
 *   [S3] same page, section three, purified delta refresh: outlier ratio =
 *        max over mean of the input, full precision when it is too large;
 *        INT8 for every layer when no previous-step difference exists.
 *   [S4] same page, section four: a custom kernel fuses quantization with the
 *        block Hadamard transform.
 *   [S6] same page, section six: the tolerance is predictable by a simple
 *        linear model of the difference.
 *   [G2] "6Bit-Diffusion: Inference-Time Mixed-Precision Quantization for
 *        Video Diffusion Models" (gist.science explainer), section 2 (DMPQ:
 *        stable steps NVFP4, unstable steps INT8); [G4] its section 4 (PDR).
 *   [D1] "DeltaQuant: 4-bit Video Diffusion Models with Spatiotemporal
 *        Delta Smoothing" (paper-radar CVPR 2026 listing), abstract:
 *        activations are grouped in local 3D spatiotemporal cubes; each
 *        cube's mean token is the core token, kept in FP8; only the small
 *        differences from it (delta tokens) are quantized to 4 bits.
 *   [OCP] The pages name NVFP4 but never define it.  Its element and scale
 *        encodings are the public OCP Microscaling Formats v1.0 ones: FP4
 *        E2M1 elements, FP8 E4M3 ("FN": no infinities, one NaN code)
 *        scales; NVFP4 is one E4M3 scale per 16 elements plus one fp32
 *        tensor scale.
 *
 * Readings the pages leave open are listed in the design notes; the ones
 * that fix arithmetic are repeated at the function that applies them.
 * Parity status: every function below is pinned by a CPU test against a
 * closed form, a format definition, an independent library routine or brute
 * force (tests/test_oracle_pins.py); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

/* bf16 -> float is exact: the bf16 bits are the top half of a float. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;
    return (uint16_t)keep;
}

void orc_f32_to_bf16_array(const float *x, int64_t n, uint16_t *y)
{
    for (int64_t i = 0; i < n; i++)
        y[i] = orc_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------- Hadamard */

/* Sylvester Hadamard matrix entry: H[i][j] = (-1)^popcount(i & j).  [S1]
 * names only "block Hadamard transform"; Sylvester (natural) order is the
 * one the fast transform below produces. */
int orc_hadamard_sign(int i, int j)
{
    unsigned v = (unsigned)(i & j);
    int parity = 0;
    while (v) {
        parity ^= (int)(v & 1u);
        v >>= 1;
    }
    return parity ? -1 : 1;
}

/* The float32 normalisation constant c_b = fl32(1/sqrt(b)). */
float orc_hadamard_scale(int b)
{
    return (float)(1.0 / sqrt((double)b));
}

/* Definition of the block rotation, in double: every aligned block of b
 * consecutive elements of a row is multiplied by H_b / sqrt(b).  [S1] */
void orc_rotate_dense_f64(const double *x, int64_t rows, int64_t cols, int b,
                          double *y)
{
    double norm = 1.0 / sqrt((double)b);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j0 = 0; j0 < cols; j0 += b)
            for (int i = 0; i < b; i++) {
                double s = 0.0;
                for (int k = 0; k < b; k++)
                    s += (double)orc_hadamard_sign(i, k) * x[r * cols + j0 + k];
                y[r * cols + j0 + i] = s * norm;
            }
}

/* The rotation as the quantizers evaluate it, in float32.  Quantized codes
 * are integers decided by float arithmetic, so both the oracle and the GPU
 * take them from this one evaluation: the fast Walsh-Hadamard butterfly with
 * strides h = 1, 2, 4, ..., b/2 in that order, each stage replacing the pair
 * (u, v) at positions (i, i + h), i & h == 0, by (u + v, u - v); then one
 * multiply by c_b.  Input is bf16 (exact in float32). */
static void rotate_row_f32(const uint16_t *x, int64_t cols, int b, float *y)
{
    float c = orc_hadamard_scale(b);
    for (int64_t j0 = 0; j0 < cols; j0 += b) {
        float *blk = y + j0;
        for (int i = 0; i < b; i++)
            blk[i] = orc_bf16_to_f32(x[j0 + i]);
        for (int h = 1; h < b; h *= 2)
            for (int i = 0; i < b; i++)
                if ((i & h) == 0) {
                    float u = blk[i];
                    float v = blk[i + h];
                    blk[i] = u + v;
                    blk[i + h] = u - v;
                }
        for (int i = 0; i < b; i++)
            blk[i] = blk[i] * c;
    }
}

void orc_rotate_f32(const uint16_t *x, int64_t rows, int64_t cols, int b,
                    float *y)
{
    for (int64_t r = 0; r < rows; r++)
        rotate_row_f32(x + r * cols, cols, b, y + r * cols);
}

/* Largest |y| over the whole rotated tensor (NVFP4's tensor amax). */
float orc_rotated_amax(const uint16_t *x, int64_t rows, int64_t cols, int b)
{
    float *y = (float *)malloc((size_t)cols * sizeof(float));
    float a = 0.0f;
    for (int64_t r = 0; r < rows; r++) {
        rotate_row_f32(x + r * cols, cols, b, y);
        for (int64_t k = 0; k < cols; k++)
            if (fabsf(y[k]) > a)
                a = fabsf(y[k]);
    }
    free(y);
    return a;
}

/* --------------------------------------------------------------- codecs */

/* FP4 E2M1 [OCP]: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.
 * Magnitudes in code order. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float orc_e2m1_decode(uint8_t code)
{
    double m = E2M1_GRID[code & 7u];
    return (float)((code & 8u) ? -m : m);
}

/* Round to the nearest E2M1 value, ties to the even code, saturating at 6.
 * The sign bit copies the sign of v (so -0.1 gives the code of -0). */
uint8_t orc_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 8u : 0u;
    double a = fabs((double)v);
    if (a >= 6.0)
        return (uint8_t)(sign | 7u);
    int best = 0;
    double bestd = a;
    for (int c = 1; c < 8; c++) {
        double d = fabs(a - E2M1_GRID[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | (uint8_t)best);
}

/* FP8 E4M3 ("FN") [OCP]: sign bit 7, exponent bits 6:3 (bias 7), mantissa
 * bits 2:0; exponent field 0 is subnormal (m * 2^-9); 0x7f/0xff are NaN. */
float orc_e4m3_decode(uint8_t code)
{
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)((code & 0x80u) ? -v : v);
}

/* Unsigned E4M3 block-scale encoder: nearest representable value, ties to
 * the even code, values above 448 saturate to 448 (0x7e).  t >= 0. */
uint8_t orc_e4m3_encode(float t)
{
    if (t >= 448.0f)
        return 0x7e;
    int best = 0;
    double bestd = fabs((double)t);
    for (int c = 1; c < 0x7f; c++) {
        double d = fabs((double)t - (double)orc_e4m3_decode((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------- integer quantizers */

/* Rows whose largest |y| is below this are stored as all-zero codes with a
 * zero scale: below it the reciprocal scales would overflow float32. */
#define ORC_TINY 0x1p-100f

/* Symmetric per-row quantizer of already-rotated float32 rows.
 * qmax = 127: INT8 per token, the "big fire" activation format of [S1];
 * qmax = 7: INT4 per output channel, the 4-bit weights of the W4A6/W4A8
 * configurations [S4 quality paragraph].  Per row: a = max |y|;
 * s = a / qmax; inv = qmax / a; q = clamp(round_half_even(y * inv),
 * -qmax, qmax). */
void orc_quant_int_rotated(const float *y, int64_t rows, int64_t cols,
                           int qmax, int8_t *q, float *s)
{
    for (int64_t r = 0; r < rows; r++) {
        const float *yr = y + r * cols;
        float a = 0.0f;
        for (int64_t k = 0; k < cols; k++)
            if (fabsf(yr[k]) > a)
                a = fabsf(yr[k]);
        if (a < ORC_TINY) {
            s[r] = 0.0f;
            for (int64_t k = 0; k < cols; k++)
                q[r * cols + k] = 0;
            continue;
        }
        s[r] = a / (float)qmax;
        float inv = (float)qmax / a;
        for (int64_t k = 0; k < cols; k++) {
            float t = yr[k] * inv;
            float n = nearbyintf(t); /* default rounding: half to even */
            if (n > (float)qmax)
                n = (float)qmax;
            if (n < -(float)qmax)
                n = -(float)qmax;
            q[r * cols + k] = (int8_t)n;
        }
    }
}

/* Rotate [S1] then quantize (the fused step of [S4], done here in two
 * plain passes). */
void orc_quant_int(const uint16_t *x, int64_t rows, int64_t cols, int b,
                   int qmax, int8_t *q, float *s)
{
    float *y = (float *)malloc((size_t)cols * sizeof(float));
    for (int64_t r = 0; r < rows; r++) {
        rotate_row_f32(x + r * cols, cols, b, y);
        orc_quant_int_rotated(y, 1, cols, qmax, q + r * cols, s + r);
    }
    free(y);
}

/* INT4 storage: two codes per byte, even k in the low nibble, two's
 * complement nibbles. */
void orc_pack_int4(const int8_t *q, int64_t rows, int64_t cols, uint8_t *p)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols; k += 2) {
            uint8_t lo = (uint8_t)(q[r * cols + k] & 0x0f);
            uint8_t hi = (uint8_t)(q[r * cols + k + 1] & 0x0f);
            p[r * (cols / 2) + k / 2] = (uint8_t)(lo | (hi << 4));
        }
}

void orc_unpack_int4(const uint8_t *p, int64_t rows, int64_t cols, int8_t *q)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols; k++) {
            uint8_t byte = p[r * (cols / 2) + k / 2];
            int nib = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            q[r * cols + k] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
}

/* ------------------------------------------------------ NVFP4 quantizer */

/* NVFP4 [S1, OCP], on rotated float32 rows, with the tensor amax A given.
 * mx == 0, plain NVFP4:
 *   s_t = A / 2688 (6 * 448, so the largest block maps to E4M3's top);
 *   per aligned 16-block: a = max |y|; t = a / (6 * s_t);
 *   E = E4M3(t) (nearest, ties even, saturating); d = E * s_t;
 *   codes = E2M1(y * (1 / d)), all zero when d == 0.
 * mx == 1, the MX-compatible variant (power-of-two scales shared by each
 * aligned pair of 16-blocks, so the bytes are also valid MXFP4 blocks):
 *   s_t = A / 1536 (6 * 256); per aligned 32-element group:
 *   a = max |y|; t = a / (6 * s_t); E = the smallest power of two >= t,
 *   clamped to [2^-9, 2^8] (all E4M3-representable); both 16-blocks of the
 *   group store E; then d and codes as above.
 * mx == 2, power-of-two scales per 16-block: as mx == 1 with each aligned
 *   16-block taking its own E (a = max over the 16).  Still valid NVFP4; a
 *   scaled-FP4 matrix instruction with one scale per 32 elements computes it
 *   exactly in two passes, one per 16-block half.
 * A below ORC_TINY: s_t = 0 and every code and scale byte is 0.
 * Layout: codes [rows, cols/2] (even k in the low nibble); scales
 * [rows, cols/16]. */
void orc_quant_nvfp4_rotated(const float *y, int64_t rows, int64_t cols,
                             float amax, int mx, uint8_t *codes,
                             uint8_t *scales, float *s_t_out)
{
    int64_t nblk = cols / 16;
    if (amax < ORC_TINY) {
        *s_t_out = 0.0f;
        memset(codes, 0, (size_t)(rows * cols / 2));
        memset(scales, 0, (size_t)(rows * nblk));
        return;
    }
    float s_t = mx ? amax / 1536.0f : amax / 2688.0f;
    *s_t_out = s_t;
    float six_st = 6.0f * s_t;
    int group = mx == 1 ? 32 : 16;
    for (int64_t r = 0; r < rows; r++) {
        const float *yr = y + r * cols;
        for (int64_t g0 = 0; g0 < cols; g0 += group) {
            float a = 0.0f;
            for (int i = 0; i < group; i++)
                if (fabsf(yr[g0 + i]) > a)
                    a = fabsf(yr[g0 + i]);
            float t = a / six_st;
            uint8_t e;
            if (mx) {
                float p = 0x1p-9f;
                while (p < t && p < 256.0f)
                    p = p * 2.0f;
                e = orc_e4m3_encode(p); /* exact: p is representable */
            } else {
                e = orc_e4m3_encode(t);
            }
            for (int i = 0; i < group; i += 16)
                scales[r * nblk + (g0 + i) / 16] = e;
            float d = orc_e4m3_decode(e) * s_t;
            float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
            for (int i = 0; i < group; i++) {
                int64_t k = g0 + i;
                uint8_t c = (d == 0.0f) ? 0u : orc_e2m1_encode(yr[k] * inv);
                uint8_t *byte = &codes[r * (cols / 2) + k / 2];
                if (k % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xf0u) | c);
                else
                    *byte = (uint8_t)((*byte & 0x0fu) | (uint8_t)(c << 4));
            }
        }
    }
}

/* Rotate [S1] then quantize to NVFP4.  amax < 0 means: take it from the
 * rotated rows given (the whole tensor). */
void orc_quant_nvfp4(const uint16_t *x, int64_t rows, int64_t cols, int b,
                     float amax, int mx, uint8_t *codes, uint8_t *scales,
                     float *s_t_out)
{
    if (amax < 0.0f)
        amax = orc_rotated_amax(x, rows, cols, b);
    float *y = (float *)malloc((size_t)cols * sizeof(float));
    float s_t = 0.0f;
    for (int64_t r = 0; r < rows; r++) {
        rotate_row_f32(x + r * cols, cols, b, y);
        orc_quant_nvfp4_rotated(y, 1, cols, amax, mx, codes + r * (cols / 2),
                                scales + r * (cols / 16), &s_t);
    }
    if (rows == 0)
        s_t = (amax < ORC_TINY) ? 0.0f : (mx ? amax / 1536.0f : amax / 2688.0f);
    *s_t_out = s_t;
    free(y);
}

/* Dequantize NVFP4: value = e2m1(code) * E4M3(scale) * s_t, in float32. */
void orc_dequant_nvfp4(const uint8_t *codes, const uint8_t *scales, float s_t,
                       int64_t rows, int64_t cols, float *out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols; k++) {
            uint8_t byte = codes[r * (cols / 2) + k / 2];
            uint8_t c = (k % 2 == 0) ? (byte & 0x0fu) : (uint8_t)(byte >> 4);
            float d = orc_e4m3_decode(scales[r * (cols / 16) + k / 16]) * s_t;
            out[r * cols + k] = orc_e2m1_decode(c) * d;
        }
}

/* ---------------------------------------------------------------- GEMMs */

/* Integer linear (INT8 activations x INT4 weights, both rotated, so
 * (XQ)(WQ)^T = XW^T [S1]).  acc[m][n] = sum_k qa[m][k] * qw[n][k] exactly
 * in int64; y = fl32(fl32(float(acc) * sa[m]) * sw[n]).  qw holds unpacked
 * codes. */
void orc_gemm_int(const int8_t *qa, const float *sa, const int8_t *qw,
                  const float *sw, int64_t M, int64_t N, int64_t K,
                  int64_t *acc, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t c = 0;
            for (int64_t k = 0; k < K; k++)
                c += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
            if (acc)
                acc[m * N + n] = c;
            float t = (float)c * sa[m];
            y[m * N + n] = t * sw[n];
        }
}

/* NVFP4 linear: y = s_tA * s_tW * sum over 16-blocks of
 * E_A * E_W * sum_k e2m1(a_k) * e2m1(w_k), in double. */
void orc_gemm_nvfp4(const uint8_t *ac, const uint8_t *ae, float ast,
                    const uint8_t *wc, const uint8_t *we, float wst,
                    int64_t M, int64_t N, int64_t K, double *y)
{
    int64_t nblk = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double total = 0.0;
            for (int64_t j = 0; j < nblk; j++) {
                double inner = 0.0;
                for (int64_t k = j * 16; k < j * 16 + 16; k++) {
                    uint8_t ab = ac[m * (K / 2) + k / 2];
                    uint8_t wb = wc[n * (K / 2) + k / 2];
                    uint8_t ca = (k % 2 == 0) ? (ab & 0x0fu) : (uint8_t)(ab >> 4);
                    uint8_t cw = (k % 2 == 0) ? (wb & 0x0fu) : (uint8_t)(wb >> 4);
                    inner += (double)orc_e2m1_decode(ca) * (double)orc_e2m1_decode(cw);
                }
                total += (double)orc_e4m3_decode(ae[m * nblk + j]) *
                         (double)orc_e4m3_decode(we[n * nblk + j]) * inner;
            }
            y[m * N + n] = (double)ast * (double)wst * total;
        }
}

/* Full-precision linear, the fallback of [S3]: y = x w^T on the original
 * (unrotated) bf16 operands, in double. */
void orc_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N,
                   int64_t K, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double s = 0.0;
            for (int64_t k = 0; k < K; k++)
                s += (double)orc_bf16_to_f32(x[m * K + k]) *
                     (double)orc_bf16_to_f32(w[n * K + k]);
            y[m * N + n] = s;
        }
}

/* ----------------------------------------------- selection statistics */

/* Statistics the per-layer, per-timestep choice reads, all in double:
 *   out[0] delta = sum|prev_out - prev_in| / sum|prev_in|  (relative L1
 *          difference of the module's previous-step input and output [S1]);
 *          0 when both sums are 0, +inf when only the denominator is; NaN
 *          when there is no history (prev_in or prev_out NULL);
 *   out[1] ratio = max|x| / mean|x| of the raw current input, the outlier
 *          ratio of [S3]; 0 for an all-zero input; NaN when x holds a NaN
 *          or an infinity;
 *   out[2] max|x|; out[3] mean|x|;
 *   out[4] largest |rotated x| (b > 0), the NVFP4 tensor amax; else 0. */
void orc_stats(const uint16_t *prev_in, const uint16_t *prev_out,
               int64_t prev_numel, const uint16_t *cur, int64_t rows,
               int64_t cols, int b, double *out)
{
    if (prev_in && prev_out) {
        double diff = 0.0, base = 0.0;
        for (int64_t i = 0; i < prev_numel; i++) {
            double a = orc_bf16_to_f32(prev_in[i]);
            double o = orc_bf16_to_f32(prev_out[i]);
            diff += fabs(o - a);
            base += fabs(a);
        }
        if (base == 0.0)
            out[0] = (diff == 0.0) ? 0.0 : INFINITY;
        else
            out[0] = diff / base;
    } else {
        out[0] = NAN;
    }
    int64_t n = rows * cols;
    double mx = 0.0, sum = 0.0;
    int bad = 0;
    for (int64_t i = 0; i < n; i++) {
        double v = fabs((double)orc_bf16_to_f32(cur[i]));
        if (!isfinite(v))
            bad = 1;
        if (v > mx)
            mx = v;
        sum += v;
    }
    double mean = (n > 0) ? sum / (double)n : 0.0;
    out[2] = mx;
    out[3] = mean;
    if (bad)
        out[1] = NAN;
    else
        out[1] = (sum == 0.0) ? 0.0 : mx / mean;
    out[4] = (b > 0 && !bad) ? (double)orc_rotated_amax(cur, rows, cols, b) : 0.0;
}

/* Decision codes: 0 NVFP4, 1 INT8, 2 BF16 (full precision). */
int orc_decide(int has_history, double delta, double ratio, double delta_thresh,
               double ratio_thresh)
{
    /* [S3, G4]: an outlier ratio above the threshold (or not a number)
     * forces full precision, ahead of any other rule. */
    if (!(ratio <= ratio_thresh))
        return 2;
    /* [S3]: with no previous-step difference, fall back to INT8. */
    if (!has_history)
        return 1;
    /* [S1, G2, S6]: a large previous-step difference needs the precise
     * format (INT8), a small one tolerates NVFP4.  The pages' linear
     * predictor compared with a fixed budget is a threshold on delta; a
     * delta at the threshold (or NaN) takes the conservative INT8. */
    if (!(delta < delta_thresh))
        return 1;
    return 0;
}

/* ----------------------------------------- temporal delta cache (TDC) */

/* Skip decision of the temporal delta cache [S2, G3], per module, once per
 * diffusion step.  A module whose output changed little between its last
 * two computed steps is predicted to change little again: the next step
 * reuses the cached output instead of computing.  An accumulator adds the
 * predicted change of every skipped step and forces a computation once the
 * sum would pass its budget; a computation resets it.
 *   state[i]: 0 the module was skipped at this step; 1 computed, with no
 *             earlier output to compare with; 2 computed, sums[2i] =
 *             sum |new - previous output|, sums[2i + 1] = sum |previous|.
 *   c[i]    : float32, relative change between the last two computed
 *             outputs (NaN: none yet); updated when state is 1 or 2.
 *   acc[i]  : float32 accumulator, reset to 0 on a computation.
 *   skip[i] : 1 when the next step reuses the cache:
 *             c < tau_skip and fl32(acc + c) <= tau_acc (NaN compares
 *             false); then acc = fl32(acc + c).
 * c = diff / base in double, rounded to float32; base == 0 gives 0 when
 * diff == 0, else +inf (the same conventions as the difference statistic). */
void orc_tdc_decide(const double *sums, const int32_t *state, float *c, float *acc,
                    int32_t *skip, int64_t n, float tau_skip, float tau_acc)
{
    for (int64_t i = 0; i < n; i++) {
        if (state[i] != 0) {
            acc[i] = 0.0f;
            if (state[i] == 1) {
                c[i] = NAN;
            } else {
                double diff = sums[2 * i], base = sums[2 * i + 1];
                double r = (base == 0.0) ? ((diff == 0.0) ? 0.0 : INFINITY) : diff / base;
                c[i] = (float)r;
            }
        }
        float next = acc[i] + c[i];
        int s = (c[i] < tau_skip) && (next <= tau_acc);
        if (s)
            acc[i] = next;
        skip[i] = s;
    }
}

/* ------------------------------------------------------------ DeltaQuant
 * [D1].  Video tokens form a frames x height x width grid, row-major with the
 * frame outermost (token (f, h, w) is row (f * H + h) * W + w).  Cubes are
 * cf x ch x cw blocks of it, ragged at the far edges, numbered the same way
 * over the cube grid.  Readings the abstract leaves open:
 *   - the core token is the float32 mean: the tokens' values summed in token
 *     order, then divided by their count;
 *   - FP8 is E4M3 [OCP] with one fp32 scale per core token, s = max|c| / 448
 *     (0 and all-zero codes when max|c| < ORC_TINY); a value's code is the
 *     nearest E4M3 of |c| / s with the sign in bit 7 (a zero magnitude is
 *     stored as +0);
 *   - a token's difference is taken from the stored core: fl32(x - fl32(E * s));
 *   - the differences are quantized to NVFP4 (4 bits [D1]; the format of this
 *     path), without rotation.
 */
static int64_t orc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Cube of every token. */
void orc_dq_cube_of(int64_t F, int64_t H, int64_t W, int cf, int ch, int cw, int32_t *cube)
{
    int64_t nH = orc_ceil_div(H, ch), nW = orc_ceil_div(W, cw);
    for (int64_t f = 0; f < F; f++)
        for (int64_t h = 0; h < H; h++)
            for (int64_t w = 0; w < W; w++)
                cube[(f * H + h) * W + w] = (int32_t)(((f / cf) * nH + h / ch) * nW + w / cw);
}

/* Signed E4M3 byte. */
float orc_e4m3s_decode(uint8_t c)
{
    float v = orc_e4m3_decode((uint8_t)(c & 0x7f));
    return (c & 0x80) ? -v : v;
}

/* Core tokens: codes [ncubes, K] (signed E4M3), scale [ncubes]. */
void orc_dq_core(const uint16_t *x, int64_t F, int64_t H, int64_t W, int64_t K, int cf, int ch, int cw,
                 uint8_t *codes, float *scale)
{
    int64_t nF = orc_ceil_div(F, cf), nH = orc_ceil_div(H, ch), nW = orc_ceil_div(W, cw);
    float *core = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t a = 0; a < nF; a++)
        for (int64_t b = 0; b < nH; b++)
            for (int64_t c = 0; c < nW; c++) {
                int64_t cube = (a * nH + b) * nW + c;
                for (int64_t k = 0; k < K; k++) {
                    float sum = 0.0f;
                    int n = 0;
                    for (int64_t f = a * cf; f < F && f < (a + 1) * cf; f++)
                        for (int64_t h = b * ch; h < H && h < (b + 1) * ch; h++)
                            for (int64_t w = c * cw; w < W && w < (c + 1) * cw; w++) {
                                sum = sum + orc_bf16_to_f32(x[((f * H + h) * W + w) * K + k]);
                                n++;
                            }
                    core[k] = sum / (float)n;
                }
                float amax = 0.0f;
                for (int64_t k = 0; k < K; k++)
                    if (fabsf(core[k]) > amax)
                        amax = fabsf(core[k]);
                float s = (amax < ORC_TINY) ? 0.0f : amax / 448.0f;
                scale[cube] = s;
                for (int64_t k = 0; k < K; k++) {
                    uint8_t m = (s == 0.0f) ? 0u : orc_e4m3_encode(fabsf(core[k]) / s);
                    codes[cube * K + k] = (m != 0 && core[k] < 0.0f) ? (uint8_t)(m | 0x80) : m;
                }
            }
    free(core);
}

/* Differences from the stored core, float32 [F * H * W, K]. */
void orc_dq_delta(const uint16_t *x, int64_t F, int64_t H, int64_t W, int64_t K, int cf, int ch, int cw,
                  const uint8_t *codes, const float *scale, float *d)
{
    int64_t M = F * H * W;
    int32_t *cube = (int32_t *)malloc((size_t)M * sizeof(int32_t));
    orc_dq_cube_of(F, H, W, cf, ch, cw, cube);
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++) {
            float core = orc_e4m3s_decode(codes[(int64_t)cube[m] * K + k]) * scale[cube[m]];
            d[m * K + k] = orc_bf16_to_f32(x[m * K + k]) - core;
        }
    free(cube);
}

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the GEMM loops may use (1 when built without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the GEMM loops (timing of the CPU baseline with one
 * thread and with every core); no effect without OpenMP.  Changes no
 * result: every GEMM output element is one thread's sequential sum. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
