/*
 * W4A16 oracle: a plain, slow, obviously correct CPU implementation of what
 * the weight-only INT4 GEMM computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP library.
 *
 * Source of every definition: the page "GPU Kernels for INT4 Inference, in
 * depth" (aicassindra.com), sections "The job, stated precisely" and "The data
 * contract", and the paper "FuTransformer" (arXiv 2610.23796), section 2.1
 * (the Llama-style block, SwiGLU line) and section 3.3.4 (INT4 projection
 * weights).
 *
 * Readings of the pages that this file takes:
 *   - "round" in the quantizer is round-half-to-even (the data contract's
 *     packer uses torch.round, which rounds ties to even);
 *   - the quantizer divides by the fp32 scale; the stored scale is that fp32
 *     value rounded to fp16, which is what dequantization uses;
 *   - an all-zero group gets scale max(0, 1e-8f) = 1e-8f, which rounds to an
 *     fp16 zero; its nibbles are all 8;
 *   - the GEMM reference uses the exact dequantized weight (q-8)*s, with every
 *     product and the running sum in fp64; a second reference uses the
 *     fp16-rounded weight, as the page's test does;
 *   - bf16 activations (the bf16 models of FuTransformer and of the Swordfish
 *     page): the data contract's dequantize casts the exact (q-8)*s to the
 *     activation type, so for bf16 the weight is bf16((q-8)*s), rounded once
 *     to nearest even; the GEMM sums A * that weight in fp64;
 *   - the folded RMSNorm gain (FuTransformer, section 3.2.2) is applied to
 *     the fp32 weights before quantizing, one fp32 rounding per product; the
 *     row factor rho_m = (q_m / H + eps)^(-1/2) uses H = K, the length of the
 *     activation row the GEMM reads;
 *   - INT8 weights (Swordfish page, section "The packed format";
 *     "Making a Single GPU Go Fast", section 9.3.2): the int4 contract with
 *     8-bit codes, s = max|W| / 127, codes stored offset by 128, four per
 *     int32 along K;
 *   - zero points (Swordfish page, blog.alpindale.net, section "The packed
 *     format"): the prescaled row (8 - zp) * s is stored in the scales' type,
 *     fp16, rounded once; the weight (q - 8) * s + z is rounded once to the
 *     activation type (the page's fused multiply-add), and the zero-point
 *     GEMM references multiply A by those rounded weights.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no fast-math: the quantizer's decisions depend on IEEE fp32 division).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE -1
#define ORACLE_ERR_NONFINITE -3

/* ------------------------------------------------------------------------
 * IEEE 754 binary16, written out from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have
 * exponent field 0 and value frac * 2^-24; exponent field 31 is inf/NaN.
 * ---------------------------------------------------------------------- */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even. */
uint16_t oracle_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds up: overflow */
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; 1024 quanta is the smallest normal */
        double n = nearbyint(a / ldexp(1.0, -24)); /* exact scaling, RNE */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2);            /* a = frac * 2^e2, frac in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)), e in [-14, 15] */
    double n = nearbyint(a / ldexp(1.0, e - 10)); /* in [1024, 2048] */
    /* n == 2048 carries into the exponent field by plain addition */
    uint32_t code = ((uint32_t)(e + 15) << 10) + ((uint32_t)n - 1024u);
    return (uint16_t)(sign | code);
}

/* ------------------------------------------------------------------------
 * bfloat16, written out from the format's definition: the upper 16 bits of
 * an IEEE binary32 -- 1 sign bit, 8 exponent bits (bias 127), 7 fraction
 * bits; subnormals have exponent field 0 and value frac * 2^-133; exponent
 * field 255 is inf/NaN.
 * ---------------------------------------------------------------------- */

double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* Round a double to the nearest bfloat16 value, ties to even. */
uint16_t oracle_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0);
    /* the largest finite value is (2^8 - 1) * 2^120; halfway to 2^128 overflows */
    if (a >= ldexp(255.5, 120))
        return (uint16_t)(sign | 0x7f80);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: quantum 2^-133; 128 quanta is the smallest normal */
        double n = nearbyint(a / ldexp(1.0, -133));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2);            /* a = frac * 2^e2, frac in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)), e in [-126, 127] */
    double n = nearbyint(a / ldexp(1.0, e - 7)); /* in [128, 256] */
    /* n == 256 carries into the exponent field by plain addition */
    uint32_t code = ((uint32_t)(e + 127) << 7) + ((uint32_t)n - 128u);
    return (uint16_t)(sign | code);
}

/* ------------------------------------------------------------------------
 * Quantizer (data contract, quantize_pack): per group g of G rows along K
 * and column n,
 *   s   = max_k |W[k,n]| / 7       (fp32 division)
 *   s   = max(s, 1e-8)             (fp32 comparison against fl32(1e-8))
 *   q   = clamp(round(W/s), -8, 7) (fp32 division, ties to even)
 *   u   = q + 8                    (stored nibble, 0..15)
 *   s16 = fp16(s)                  (stored scale)
 * W is [K,N] row-major (K is the reduction axis).  u is [K,N], s16 [K/G,N].
 * ---------------------------------------------------------------------- */
int oracle_quantize(const float *W, int64_t K, int64_t N, int G,
                    uint8_t *u, uint16_t *s16)
{
    if (G <= 0 || K <= 0 || N <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < K * N; ++i)
        if (!isfinite(W[i]))
            return ORACLE_ERR_NONFINITE;
    fesetround(FE_TONEAREST);
    for (int64_t g = 0; g < K / G; ++g) {
        for (int64_t n = 0; n < N; ++n) {
            float amax = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float a = fabsf(W[k * N + n]);
                if (a > amax)
                    amax = a;
            }
            float s = amax / 7.0f;
            if (s < 1e-8f)
                s = 1e-8f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float r = W[k * N + n] / s;
                float q = nearbyintf(r); /* ties to even */
                if (q < -8.0f)
                    q = -8.0f;
                if (q > 7.0f)
                    q = 7.0f;
                u[k * N + n] = (uint8_t)((int)q + 8);
            }
            s16[g * N + n] = oracle_f64_to_f16((double)s);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Packing (data contract): eight values consecutive along K share one int32;
 * value k sits at bits 4(k mod 8) .. 4(k mod 8)+3 of word [k/8, n].
 * ---------------------------------------------------------------------- */
int oracle_pack(const uint8_t *u, int64_t K, int64_t N, int32_t *packed)
{
    if (K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t r = 0; r < K / 8; ++r) {
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = 0;
            for (int i = 0; i < 8; ++i)
                word |= ((uint32_t)(u[(8 * r + i) * N + n] & 0xF)) << (4 * i);
            packed[r * N + n] = (int32_t)word;
        }
    }
    return ORACLE_OK;
}

/* Unpack: shift, then mask with 0xF.  The shift is done on the unsigned
 * word, and the mask is applied regardless, so a top nibble >= 8 (which sets
 * the int32 sign bit) never leaks sign bits into the value. */
int oracle_unpack(const int32_t *packed, int64_t K, int64_t N, uint8_t *u)
{
    if (K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = (uint32_t)packed[(k / 8) * N + n];
            u[k * N + n] = (uint8_t)((word >> (4 * (k % 8))) & 0xFu);
        }
    return ORACLE_OK;
}

/* The exact dequantized weight (u - 8) * s16[k/G, n], as a double.  The
 * product of a 4-bit integer and an fp16 value is exact in double. */
static double exact_weight(const int32_t *packed, const uint16_t *s16,
                           int64_t N, int G, int64_t k, int64_t n)
{
    uint32_t word = (uint32_t)packed[(k / 8) * N + n];
    int uval = (int)((word >> (4 * (k % 8))) & 0xFu);
    return (double)(uval - 8) * oracle_f16_to_f64(s16[(k / G) * N + n]);
}

/* Dequantize (data contract, dequantize): W16[k,n] = fp16((u-8) * s16). */
int oracle_dequant(const int32_t *packed, const uint16_t *s16, int64_t K,
                   int64_t N, int G, uint16_t *W16)
{
    if (G <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            W16[k * N + n] = oracle_f64_to_f16(exact_weight(packed, s16, N, G, k, n));
    return ORACLE_OK;
}

/* Dequantize for bf16 activations: Wb[k,n] = bf16((u-8) * s16), the exact
 * product rounded once. */
int oracle_dequant_bf16(const int32_t *packed, const uint16_t *s16, int64_t K,
                        int64_t N, int G, uint16_t *Wb)
{
    if (G <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Wb[k * N + n] = oracle_f64_to_bf16(exact_weight(packed, s16, N, G, k, n));
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Zero points (Swordfish page, blog.alpindale.net, section "The packed
 * format").  Asymmetric (AWQ) checkpoints give each group and column a zero
 * point zp besides the scale, the weight being (q - zp) * s.  The kernel
 * receives them as a second tensor shaped like the scales, holding the
 * prescaled value (8 - zp) * s, so that the weight becomes
 * (q - 8) * s + (8 - zp) * s: the scale multiply and the zero-point add are
 * one fused multiply-add.
 * ---------------------------------------------------------------------- */

/* Prescaled zero rows: z16[g,n] = fp16((8 - zp[g,n]) * s16[g,n]), the exact
 * product (an 8-bit integer times an fp16 value) rounded once, stored in the
 * scales' type. */
int oracle_zero_rows(const uint16_t *s16, const uint8_t *zp, int64_t KG, int64_t N,
                     uint16_t *z16)
{
    if (KG < 0 || N < 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < KG * N; ++i)
        z16[i] = oracle_f64_to_f16((8.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]));
    return ORACLE_OK;
}

/* (q - 8) * s + z before its rounding.  Both terms are multiples of 2^-24
 * smaller than 2^20 in magnitude, so the double sum is exact. */
static double exact_weight_zp(const int32_t *packed, const uint16_t *s16, const uint16_t *z16,
                              int64_t N, int G, int64_t k, int64_t n)
{
    return exact_weight(packed, s16, N, G, k, n) + oracle_f16_to_f64(z16[(k / G) * N + n]);
}

/* Dequantize with zero rows: W[k,n] = round((q - 8) * s + z) with one
 * rounding (the fused multiply-add) to fp16, or to bf16 when bf16 != 0. */
int oracle_dequant_zp(const int32_t *packed, const uint16_t *s16, const uint16_t *z16,
                      int64_t K, int64_t N, int G, int bf16, uint16_t *W)
{
    if (G <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            double w = exact_weight_zp(packed, s16, z16, N, G, k, n);
            W[k * N + n] = bf16 ? oracle_f64_to_bf16(w) : oracle_f64_to_f16(w);
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * INT8 weights (W8A16).  The Swordfish page (blog.alpindale.net, section "The
 * packed format") runs an int8 variant of unsigned 8-bit codes with a bias of
 * 128 through the same dequantization idiom; "Making a Single GPU Go Fast"
 * (arunshar.com, chapter 9, section 9.3.2) recommends weight-only INT8 with
 * per-output-channel scales and gives the signed range [-128, 127].  Reading:
 * the int4 data contract with 8-bit codes.  Per group g of G rows along K
 * and column n:
 *   s   = max_k |W[k,n]| / 127      (fp32 division)
 *   s   = max(s, 1e-8)              (fp32 comparison against fl32(1e-8))
 *   q   = clamp(round(W/s), -128, 127)   (fp32 division, ties to even)
 *   u   = q + 128                   (stored byte, 0..255)
 *   s16 = fp16(s)
 * and four bytes consecutive along K share one int32, byte k at bits
 * 8(k mod 4) .. 8(k mod 4)+7 of word [k/4, n].  The weight is (u - 128) * s16.
 * Per-output-channel scales are G = K.
 * ---------------------------------------------------------------------- */
int oracle_quantize8(const float *W, int64_t K, int64_t N, int G, uint8_t *u, uint16_t *s16)
{
    if (G <= 0 || K <= 0 || N <= 0 || K % G != 0 || K % 4 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < K * N; ++i)
        if (!isfinite(W[i]))
            return ORACLE_ERR_NONFINITE;
    fesetround(FE_TONEAREST);
    for (int64_t g = 0; g < K / G; ++g) {
        for (int64_t n = 0; n < N; ++n) {
            float amax = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float a = fabsf(W[k * N + n]);
                if (a > amax)
                    amax = a;
            }
            float s = amax / 127.0f;
            if (s < 1e-8f)
                s = 1e-8f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float q = nearbyintf(W[k * N + n] / s); /* ties to even */
                if (q < -128.0f)
                    q = -128.0f;
                if (q > 127.0f)
                    q = 127.0f;
                u[k * N + n] = (uint8_t)((int)q + 128);
            }
            s16[g * N + n] = oracle_f64_to_f16((double)s);
        }
    }
    return ORACLE_OK;
}

int oracle_pack8(const uint8_t *u, int64_t K, int64_t N, int32_t *packed)
{
    if (K % 4 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t r = 0; r < K / 4; ++r)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = 0;
            for (int i = 0; i < 4; ++i)
                word |= (uint32_t)u[(4 * r + i) * N + n] << (8 * i);
            packed[r * N + n] = (int32_t)word;
        }
    return ORACLE_OK;
}

/* Unpack: shift the unsigned word, then mask with 0xFF. */
int oracle_unpack8(const int32_t *packed, int64_t K, int64_t N, uint8_t *u)
{
    if (K % 4 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = (uint32_t)packed[(k / 4) * N + n];
            u[k * N + n] = (uint8_t)((word >> (8 * (k % 4))) & 0xFFu);
        }
    return ORACLE_OK;
}

/* The exact weight (u - 128) * s16, a double (8-bit integer times fp16). */
static double exact_weight8(const int32_t *packed, const uint16_t *s16, int64_t N, int G,
                            int64_t k, int64_t n)
{
    uint32_t word = (uint32_t)packed[(k / 4) * N + n];
    int uval = (int)((word >> (8 * (k % 4))) & 0xFFu);
    return (double)(uval - 128) * oracle_f16_to_f64(s16[(k / G) * N + n]);
}

/* Dequantize: W[k,n] = round((u - 128) * s16), one rounding to fp16, or to
 * bf16 when bf16 != 0. */
int oracle_dequant8(const int32_t *packed, const uint16_t *s16, int64_t K, int64_t N, int G,
                    int bf16, uint16_t *W)
{
    if (G <= 0 || K % G != 0 || K % 4 != 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            double w = exact_weight8(packed, s16, N, G, k, n);
            W[k * N + n] = bf16 ? oracle_f64_to_bf16(w) : oracle_f64_to_f16(w);
        }
    return ORACLE_OK;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

#define NCHUNK 256

/* ------------------------------------------------------------------------
 * GEMM reference (the job, stated precisely): C = A * dequant(W),
 *   C[m,n] = sum_k A[m,k] * (u[k,n] - 8) * s16[k/G, n]
 * with A as fp16 bits [M,K] row-major, each product exact in fp64 and the sum
 * taken in fp64 in increasing k.  Output rows are independent, so threads
 * split the (row, column-chunk) pairs; no sum is reordered.
 * ---------------------------------------------------------------------- */
int oracle_gemm_f64(const uint16_t *A16, int64_t M, int64_t K,
                    const int32_t *packed, const uint16_t *s16, int64_t N,
                    int G, double *C, int nthreads)
{
    if (G <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    set_threads(nthreads);
    int64_t nchunks = (N + NCHUNK - 1) / NCHUNK;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NCHUNK;
            int64_t n1 = n0 + NCHUNK < N ? n0 + NCHUNK : N;
            double acc[NCHUNK];
            for (int64_t n = n0; n < n1; ++n)
                acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_f16_to_f64(A16[m * K + k]);
                for (int64_t n = n0; n < n1; ++n)
                    acc[n - n0] += a * exact_weight(packed, s16, N, G, k, n);
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * N + n] = acc[n - n0];
        }
    }
    return ORACLE_OK;
}

/* Second reference, as the page's test builds it: A times the fp16-rounded
 * dequantized weights W16 (bits, [K,N]), summed in fp64. */
int oracle_gemm_w16_f64(const uint16_t *A16, int64_t M, int64_t K,
                        const uint16_t *W16, int64_t N, double *C, int nthreads)
{
    set_threads(nthreads);
    int64_t nchunks = (N + NCHUNK - 1) / NCHUNK;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NCHUNK;
            int64_t n1 = n0 + NCHUNK < N ? n0 + NCHUNK : N;
            double acc[NCHUNK];
            for (int64_t n = n0; n < n1; ++n)
                acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_f16_to_f64(A16[m * K + k]);
                for (int64_t n = n0; n < n1; ++n)
                    acc[n - n0] += a * oracle_f16_to_f64(W16[k * N + n]);
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * N + n] = acc[n - n0];
        }
    }
    return 0;
}

/* The same for bf16: A times given bf16 weights Wb (bits, [K,N]), summed in
 * fp64 (the weights of a zero-point format with bf16 activations). */
int oracle_gemm_wb_f64(const uint16_t *Ab, int64_t M, int64_t K, const uint16_t *Wb,
                       int64_t N, double *C, int nthreads)
{
    set_threads(nthreads);
    int64_t nchunks = (N + NCHUNK - 1) / NCHUNK;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NCHUNK;
            int64_t n1 = n0 + NCHUNK < N ? n0 + NCHUNK : N;
            double acc[NCHUNK];
            for (int64_t n = n0; n < n1; ++n)
                acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_bf16_to_f64(Ab[m * K + k]);
                for (int64_t n = n0; n < n1; ++n)
                    acc[n - n0] += a * oracle_bf16_to_f64(Wb[k * N + n]);
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * N + n] = acc[n - n0];
        }
    }
    return 0;
}

/* GEMM reference for bf16 activations: Ab bf16 bits [M,K], weights
 * bf16((u-8) * s16) as oracle_dequant_bf16 defines them, each product exact
 * in fp64 (8-bit by 8-bit significands) and the sum in fp64 in increasing k. */
int oracle_gemm_bf16_f64(const uint16_t *Ab, int64_t M, int64_t K,
                         const int32_t *packed, const uint16_t *s16, int64_t N,
                         int G, double *C, int nthreads)
{
    if (G <= 0 || K % G != 0 || K % 8 != 0)
        return ORACLE_ERR_SHAPE;
    set_threads(nthreads);
    int64_t nchunks = (N + NCHUNK - 1) / NCHUNK;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NCHUNK;
            int64_t n1 = n0 + NCHUNK < N ? n0 + NCHUNK : N;
            double acc[NCHUNK];
            for (int64_t n = n0; n < n1; ++n)
                acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_bf16_to_f64(Ab[m * K + k]);
                for (int64_t n = n0; n < n1; ++n) {
                    double w = oracle_bf16_to_f64(
                        oracle_f64_to_bf16(exact_weight(packed, s16, N, G, k, n)));
                    acc[n - n0] += a * w;
                }
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * N + n] = acc[n - n0];
        }
    }
    return ORACLE_OK;
}

/* GEMM reference for INT8 weights: C[m,n] = sum_k A[m,k] * w[k,n] in fp64,
 * increasing k.  fp16 activations use the exact weight (u - 128) * s16 (as
 * the int4 reference does); bf16 activations (A as bf16 bits) use the weight
 * rounded once to bf16. */
int oracle_gemm8_f64(const uint16_t *A, int64_t M, int64_t K, const int32_t *packed,
                     const uint16_t *s16, int64_t N, int G, int bf16, double *C, int nthreads)
{
    if (G <= 0 || K % G != 0 || K % 4 != 0)
        return ORACLE_ERR_SHAPE;
    set_threads(nthreads);
    int64_t nchunks = (N + NCHUNK - 1) / NCHUNK;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NCHUNK;
            int64_t n1 = n0 + NCHUNK < N ? n0 + NCHUNK : N;
            double acc[NCHUNK];
            for (int64_t n = n0; n < n1; ++n)
                acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = bf16 ? oracle_bf16_to_f64(A[m * K + k]) : oracle_f16_to_f64(A[m * K + k]);
                for (int64_t n = n0; n < n1; ++n) {
                    double w = exact_weight8(packed, s16, N, G, k, n);
                    if (bf16)
                        w = oracle_bf16_to_f64(oracle_f64_to_bf16(w));
                    acc[n - n0] += a * w;
                }
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * N + n] = acc[n - n0];
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Folded RMSNorm gain (FuTransformer, section 3.2.2):
 *   C[m,n] = sum_h x[m,h] rho_m gamma_h W[h,n] = rho_m sum_h x[m,h] W'[h,n],
 *   W'[h,n] = gamma_h W[h,n],  rho_m = (q_m / H + eps)^(-1/2),
 *   q_m = sum_h x[m,h]^2.
 * ---------------------------------------------------------------------- */

/* W' = fp32(gamma[k] * W[k,n]): the double product of two floats is exact,
 * so converting it to float rounds once, as an IEEE fp32 multiply does. */
int oracle_fold_gain(const float *W, const float *gamma, int64_t K, int64_t N, float *Wf)
{
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Wf[k * N + n] = (float)((double)gamma[k] * (double)W[k * N + n]);
    return ORACLE_OK;
}

/* rho[m] in fp64 from fp16 (bf16 = 0) or bf16 (bf16 = 1) activation bits. */
int oracle_rms_rowscale_f64(const uint16_t *A, int64_t M, int64_t K, int bf16, double eps,
                            double *rho)
{
    if (K <= 0)
        return ORACLE_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m) {
        double q = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double x = bf16 ? oracle_bf16_to_f64(A[m * K + k]) : oracle_f16_to_f64(A[m * K + k]);
            q += x * x;
        }
        rho[m] = 1.0 / sqrt(q / (double)K + eps);
    }
    return ORACLE_OK;
}

/* The epilogue's row factor: out[m,n] = rho[m] * C[m,n]. */
int oracle_scale_rows(const double *C, int64_t M, int64_t N, const double *rho, double *out)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = rho[m] * C[m * N + n];
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * SwiGLU epilogue (FuTransformer, section 2.1: Z = SiLU(X W_g^T) * (X W_u^T),
 * gate and up sharing one GEMM).  C is [M,N] with columns [0,N/2) the gate
 * projection and [N/2,N) the up projection; Z is [M,N/2]:
 *   Z[m,j] = silu(C[m,j]) * C[m,j+N/2],   silu(x) = x / (1 + exp(-x)).
 * ---------------------------------------------------------------------- */
int oracle_swiglu_f64(const double *C, int64_t M, int64_t N, double *Z)
{
    if (N % 2 != 0)
        return ORACLE_ERR_SHAPE;
    int64_t I = N / 2;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < I; ++j) {
            double g = C[m * N + j];
            double up = C[m * N + I + j];
            Z[m * I + j] = g / (1.0 + exp(-g)) * up;
        }
    return ORACLE_OK;
}
