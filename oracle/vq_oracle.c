/*
 * vq_oracle.c -- plain, slow, CPU reference for the block-quantized verify GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source, header, table or helper with the HIP
 * library: every decoder below is written out from its closed form.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Qwen3.8-27B on the AMD R9700: up to 227 tok/s" -- sections
 *       "A block-diffusion drafter, verified exactly" (verification checks a
 *       whole draft block in one batched target forward that reads the weights
 *       once) and "What 'lossless' means here, precisely" (batched and 1-row
 *       paths sum in different orders).
 *  [P3] "r9k: a from-scratch inference engine for Qwen3.8-27B on two Radeon AI
 *       PRO R9700" -- opening paragraph (FP8 E4M3 weights in 128 x 128 scale
 *       blocks).
 *  [P4] "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit
 *       activations with a Hadamard rotation" -- section "Prompt processing:
 *       4-bit activations, rotated first" (Q4_0 is a 4-bit value with offset 8;
 *       flipping its top bit gives two's complement; blocks of 32; 32-point
 *       Walsh-Hadamard rotation of activations inside the int8/int4 quantizer,
 *       weights rotated the same way offline so the product is unchanged).
 *
 * Readings where the pages are silent (each one is a choice, not a quote):
 *  - Q4_0 layout: codes u8 [M][K/2]; within each 32-weight block (16 bytes),
 *    byte j holds the code of k = 32b + j in its low nibble and of
 *    k = 32b + 16 + j in its high nibble (the in-block order of GGUF Q4_0, the
 *    container the pages' Q4_0 files use).  Scales: fp16 [M][K/32].
 *  - E4M3: the OCP 8-bit floating point "E4M3FN" variant: bias 7, no
 *    infinities, S.1111.111 is NaN, max +-448.
 *  - FP8 scales: fp32 multiplier per 128 x 128 tile, array [ceil(M/128)][K/128],
 *    tile (i, j) covers output features [128 i, 128 i + 128) and inputs
 *    [128 j, 128 j + 128).
 *  - H32: Sylvester-ordered Walsh-Hadamard matrix with +-1 entries
 *    (H[i][j] = (-1)^popcount(i & j)), applied as the radix-2 butterfly with
 *    h = 1, 2, 4, 8, 16 in that order; unnormalised, so a rotated product is
 *    restored by alpha = 1/32.
 *  - int8 activation quantizer: d = fp16_rne(amax / 127) computed in fp32,
 *    q = clamp(rint_half_even(u / d), -127, 127), amax == 0 gives d = 0, q = 0.
 *    The 4-bit quantizer of the same section is the same rule with 7 in place
 *    of 127 (symmetric 4-bit codes, stored one per byte).
 *  - H32 rotation of Q4_0 weights ([P4]: the weights take the same rotation
 *    once, ahead of time; the pages' tool makes a rotated Q4_0 file from a
 *    plain one): per 32-block, dequantize exactly in fp32, H32 by the butterflies
 *    above, requantize to Q4_0 by the rule of the GGUF Q4_0 format the pages'
 *    files use: m = the block's value of largest magnitude (the first one on
 *    ties), d = m / -8, id = d != 0 ? 1 / d : 0, q = min(15, trunc(x * id +
 *    8.5)), each a single fp32 operation, d stored as fp16_rne(d).
 *  - greedy verification: logits row i is the target's prediction for block
 *    position i (row 0 follows the last committed token, row i the drafted
 *    token i - 1); the target's choice in a row is its argmax, the first NaN
 *    if the row holds one, else the first of its largest values (-0 and +0
 *    equal); the committed tokens are the leading drafted tokens that equal
 *    the target's choices, then the target's own choice at the next position.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * fp-contract is off so that the fp32 quantizer emulation performs exactly one
 * IEEE rounding per written operation.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define VQO_F16 1
#define VQO_BF16 2
#define VQO_F32 3

/* ------------------------------------------------------------------ */
/* Closed-form decoders                                                */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double vqo_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* 2^-14 * f / 2^10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + f, e - 25);           /* 2^(e-15) * (1 + f/2^10) */
    return s ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double vqo_bf16_to_f64(uint16_t b)
{
    int s = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* 2^-126 * f / 2^7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(128.0 + f, e - 134);           /* 2^(e-127) * (1 + f/2^7) */
    return s ? -v : v;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities. */
double vqo_e4m3_to_f64(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                /* 2^-6 * m / 8 */
    else
        v = ldexp(8.0 + m, e - 10);              /* 2^(e-7) * (1 + m/8) */
    return s ? -v : v;
}

static double act_to_f64(const uint16_t *a, int dtype, int64_t i)
{
    return dtype == VQO_BF16 ? vqo_bf16_to_f64(a[i]) : vqo_f16_to_f64(a[i]);
}

/* ------------------------------------------------------------------ */
/* Q4_0 weights                                                        */
/* ------------------------------------------------------------------ */

/* The 4-bit code (0..15) of weight (m, k) in the layout described above. */
int vqo_q4_0_code(const uint8_t *codes, int64_t K, int64_t m, int64_t k)
{
    int64_t b = k / 32, j = k % 32;
    uint8_t byte = codes[m * (K / 2) + b * 16 + (j % 16)];
    return j < 16 ? (byte & 0x0f) : (byte >> 4);
}

/* w[m][k] = d[m][k/32] * (q - 8): offset-8 code times the block's fp16 scale. */
double vqo_q4_0_weight(const uint8_t *codes, const uint16_t *scales,
                       int64_t K, int64_t m, int64_t k)
{
    int q = vqo_q4_0_code(codes, K, m, k);
    return vqo_f16_to_f64(scales[m * (K / 32) + k / 32]) * (double)(q - 8);
}

/* Dequantise the listed rows (output features) into out[nrows][K]. */
void vqo_q4_0_dequant(const uint8_t *codes, const uint16_t *scales,
                      int64_t M, int64_t K,
                      const int64_t *rows, int64_t nrows, double *out)
{
    (void)M;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = vqo_q4_0_weight(codes, scales, K, rows[r], k);
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 weights with 128 x 128 fp32 tile scales                    */
/* ------------------------------------------------------------------ */

double vqo_fp8_weight(const uint8_t *w, const float *tscales,
                      int64_t K, int64_t m, int64_t k)
{
    int64_t kt = K / 128;
    double s = (double)tscales[(m / 128) * kt + (k / 128)];
    return vqo_e4m3_to_f64(w[m * K + k]) * s;
}

void vqo_fp8_dequant(const uint8_t *w, const float *tscales,
                     int64_t M, int64_t K,
                     const int64_t *rows, int64_t nrows, double *out)
{
    (void)M;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = vqo_fp8_weight(w, tscales, K, rows[r], k);
}

/* ------------------------------------------------------------------ */
/* Verify GEMMs: Y[n][m] = alpha * sum_k x[n][k] * w[m][k]            */
/* fp64 accumulation, k ascending, not rounded to any output type.    */
/* Only the output features listed in cols[] are computed; out is     */
/* [N][ncols] row-major.                                              */
/* ------------------------------------------------------------------ */

void vqo_gemm_q4_0(const uint8_t *codes, const uint16_t *scales,
                   const uint16_t *act, int act_dtype,
                   int64_t N, int64_t M, int64_t K,
                   const int64_t *cols, int64_t ncols,
                   double alpha, double *out)
{
    (void)M;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t m = cols[c];
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += act_to_f64(act, act_dtype, n * K + k) *
                       vqo_q4_0_weight(codes, scales, K, m, k);
            out[n * ncols + c] = alpha * acc;
        }
    }
}

void vqo_gemm_fp8_blk128(const uint8_t *w, const float *tscales,
                         const uint16_t *act, int act_dtype,
                         int64_t N, int64_t M, int64_t K,
                         const int64_t *cols, int64_t ncols, double *out)
{
    (void)M;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t m = cols[c];
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += act_to_f64(act, act_dtype, n * K + k) *
                       vqo_fp8_weight(w, tscales, K, m, k);
            out[n * ncols + c] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* W4A8: int8 activations with fp16 per-32-block scales               */
/* Y[n][m] = alpha * sum_b dw[m][b] * dx[n][b] * D_b[n][m],           */
/* D_b = sum_{j<32} (q[m][32b+j] - 8) * qx[n][32b+j]   (exact int64)  */
/* ------------------------------------------------------------------ */

int64_t vqo_w4a8_block_dot(const uint8_t *codes, const int8_t *qx,
                           int64_t K, int64_t n, int64_t m, int64_t b)
{
    int64_t d = 0;
    for (int64_t j = 0; j < 32; ++j) {
        int64_t k = 32 * b + j;
        d += (int64_t)(vqo_q4_0_code(codes, K, m, k) - 8) * (int64_t)qx[n * K + k];
    }
    return d;
}

void vqo_gemm_w4a8(const uint8_t *codes, const uint16_t *wscales,
                   const int8_t *qx, const uint16_t *xscales,
                   int64_t N, int64_t M, int64_t K,
                   const int64_t *cols, int64_t ncols,
                   double alpha, double *out)
{
    (void)M;
    int64_t nb = K / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t m = cols[c];
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                double dw = vqo_f16_to_f64(wscales[m * nb + b]);
                double dx = vqo_f16_to_f64(xscales[n * nb + b]);
                acc += dw * dx * (double)vqo_w4a8_block_dot(codes, qx, K, n, m, b);
            }
            out[n * ncols + c] = alpha * acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* H32 rotation + int8 quantizer, emulated step by step in fp32       */
/* ------------------------------------------------------------------ */

/* fp32 -> fp16 bits, round to nearest, ties to even (IEEE default).
 * Overflow gives +-inf; NaN gives a quiet NaN. */
uint16_t vqo_f32_to_f16_rne(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u)                        /* inf or nan */
        return sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u);
    int e = (int)(ax >> 23);                      /* biased fp32 exponent */
    uint32_t mant = (ax & 0x7fffffu) | (e ? 0x800000u : 0u);
    if (e == 0)
        e = 1;
    /* value = mant * 2^(e - 150).  fp16 keeps an integer significand
     * sig * 2^(he - 25) with he >= 1 (subnormals share he = 1). */
    int he = e - 127 + 15;                        /* tentative fp16 biased exponent */
    int shift;                                    /* how far mant moves right */
    if (he >= 1)
        shift = 13;                               /* 24-bit -> 11-bit significand */
    else {
        shift = 13 + (1 - he);                    /* subnormal: fewer bits kept */
        he = 1;
    }
    if (shift > 30)                               /* far below half the smallest subnormal */
        return sign;
    uint32_t kept = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u)))
        kept += 1;
    /* kept is an 11-bit (or smaller) significand; renormalise on carry */
    if (kept >= 0x800u) {
        kept >>= 1;
        he += 1;
    }
    if (kept < 0x400u)                            /* subnormal (or zero) result */
        return sign | (uint16_t)kept;
    if (he >= 31)
        return sign | 0x7c00u;
    return sign | (uint16_t)((he << 10) | (kept & 0x3ffu));
}

/* The 32-point Walsh-Hadamard transform of one block, in fp32, radix-2
 * butterflies with h = 1, 2, 4, 8, 16 in that order.  Each stage replaces
 * (x_i, x_{i+h}) by (x_i + x_{i+h}, x_i - x_{i+h}) for every i with i & h == 0.
 * The result is H32 x with H32 in Sylvester order. */
void vqo_fwht32_f32(float *x)
{
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; ++i)
            if ((i & h) == 0) {
                float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
}

/* H32 as an explicit +-1 matrix (Sylvester order), for checks. */
void vqo_h32_matrix(int8_t *h)
{
    for (int i = 0; i < 32; ++i)
        for (int j = 0; j < 32; ++j)
            h[i * 32 + j] = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* Per (row, 32-block): u = H32 x in fp32 (or u = x when rotate == 0),
 * amax = max |u|, d = fp16_rne(amax / qmax), q = clamp(rint(u / d), -qmax,
 * qmax).  qmax = 127 is the int8 quantizer, qmax = 7 the 4-bit one ([P4]
 * "Prompt processing": there the activations alone become 4-bit codes; read
 * here as the int8 rule with the symmetric 4-bit range, codes one per byte).
 * Returns 0, or -1 if some d overflows fp16 (then outputs are partial). */
int vqo_block_quant(const uint16_t *x, int x_dtype, int64_t N, int64_t K, int qmax, int rotate,
                    int8_t *q, uint16_t *d)
{
    int64_t nb = K / 32;
    int bad = 0;
    const float qm = (float)qmax;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            float u[32];
            for (int j = 0; j < 32; ++j)
                u[j] = (float)act_to_f64(x, x_dtype, n * K + 32 * b + j); /* exact */
            if (rotate)
                vqo_fwht32_f32(u);
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(u[j]);
                if (a > amax)
                    amax = a;
            }
            float d32 = amax / qm;
            uint16_t dh = vqo_f32_to_f16_rne(d32);
            if ((dh & 0x7c00u) == 0x7c00u)
                bad = 1;
            d[n * nb + b] = dh;
            float df = (float)vqo_f16_to_f64(dh);            /* exact */
            for (int j = 0; j < 32; ++j) {
                float r = 0.0f;
                if (df != 0.0f) {
                    r = nearbyintf(u[j] / df);                /* ties to even */
                    if (r > qm) r = qm;
                    if (r < -qm) r = -qm;
                }
                q[n * K + 32 * b + j] = (int8_t)r;
            }
        }
    }
    return bad ? -1 : 0;
}

/* The H32-rotated int8 quantizer (codes in [-127, 127]). */
int vqo_h32_quant_int8(const uint16_t *x, int x_dtype, int64_t N, int64_t K,
                       int8_t *q, uint16_t *d)
{
    return vqo_block_quant(x, x_dtype, N, K, 127, 1, q, d);
}

/* The H32-rotated 4-bit quantizer (codes in [-7, 7], one per byte). */
int vqo_h32_quant_int4(const uint16_t *x, int x_dtype, int64_t N, int64_t K,
                       int8_t *q, uint16_t *d)
{
    return vqo_block_quant(x, x_dtype, N, K, 7, 1, q, d);
}

/* ------------------------------------------------------------------ */
/* Greedy verification of a draft block                                */
/* ------------------------------------------------------------------ */

/* [P1] "A block-diffusion drafter, verified exactly" and "What 'lossless'
 * means here, precisely": the drafter proposes, the target checks every
 * position in one batched forward, and a proposal is committed only where the
 * target's own greedy choice is the same token, so the output is what plain
 * greedy decoding would produce.  logits: [n_rows][vocab] in dtype (VQO_F32,
 * VQO_F16 or VQO_BF16 bit patterns); draft: [n_rows - 1] proposed tokens.
 * Writes the target's choice of every row to target[] and returns the number
 * of committed tokens (accepted prefix + 1). */
int64_t vqo_greedy_verify(const void *logits, int dtype, int64_t n_rows, int64_t vocab,
                          const int32_t *draft, int32_t *target)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t best = -1;
        double bv = 0.0;
        for (int64_t v = 0; v < vocab; ++v) {
            const int64_t i = r * vocab + v;
            double x;
            if (dtype == VQO_F32) {
                float f;
                memcpy(&f, (const char *)logits + 4 * i, 4);
                x = (double)f;
            } else {
                x = act_to_f64((const uint16_t *)logits, dtype, i);
            }
            if (isnan(x)) {          /* a NaN is the choice: the first one */
                best = v;
                break;
            }
            if (best < 0 || x > bv) { /* strictly larger: ties keep the first */
                best = v;
                bv = x;
            }
        }
        target[r] = (int32_t)best;
    }
    int64_t a = 0;
    while (a < n_rows - 1 && draft[a] == target[a])
        ++a;
    return a + 1;
}

/* ------------------------------------------------------------------ */
/* Offline H32 rotation of Q4_0 weights                                */
/* ------------------------------------------------------------------ */

/* [P4] "Prompt processing: 4-bit activations, rotated first": the weights
 * are rotated once, offline, by the same 32-point Walsh-Hadamard transform
 * as the activations, so that the rotated product (divided by 32) equals the
 * plain one.  Input and output: Q4_0 codes [M][K/2] and fp16 scales [M][K/32]
 * in the layout read by vqo_q4_0_code.  Per block, in fp32: exact dequantized
 * values, the butterflies of vqo_fwht32_f32, then the Q4_0 rule stated in the
 * header (every step one IEEE fp32 operation; fp-contract is off). */
void vqo_q4_0_rotate_h32(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                         uint8_t *codes_out, uint16_t *scales_out)
{
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float d0 = (float)vqo_f16_to_f64(scales[m * nb + b]);
            float x[32];
            for (int j = 0; j < 32; ++j)
                x[j] = d0 * (float)(vqo_q4_0_code(codes, K, m, 32 * b + j) - 8); /* exact */
            vqo_fwht32_f32(x);
            float amax = 0.0f, mx = 0.0f;
            for (int j = 0; j < 32; ++j)
                if (fabsf(x[j]) > amax) {        /* strictly larger: the first on ties */
                    amax = fabsf(x[j]);
                    mx = x[j];
                }
            const float d = mx / -8.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            uint8_t q[32];
            for (int j = 0; j < 32; ++j) {
                const float t = x[j] * id;
                const float u = t + 8.5f;
                const int qi = (int)u;            /* u >= 0: truncation is floor */
                q[j] = (uint8_t)(qi > 15 ? 15 : qi);
            }
            /* byte i of the block: k = i in the low nibble, k = 16 + i in the high */
            for (int i = 0; i < 16; ++i)
                codes_out[m * (K / 2) + 16 * b + i] = (uint8_t)(q[i] | (q[16 + i] << 4));
            scales_out[m * nb + b] = vqo_f32_to_f16_rne(d);
        }
    }
}
