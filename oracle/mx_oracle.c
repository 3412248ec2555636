/*
 * mx_oracle.c — plain, slow CPU reference ("oracle") for the MX block-scaled linear layer
 *
 *     y[m, n] = sum_k dequant(x_q, s_x)[m, k] * dequant(W_q, s_w)[n, k]  (+ bias[n])
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only the test-suite, the package smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant with the HIP library; it is written from the
 * format definitions below, in fp64, one obvious step at a time.
 *
 * Sources (vLLM API pages):
 *  - compressed_tensors_w8a8_mxfp8 page, class CompressedTensorsW8A8Mxfp8 (docstring "MXFP8
 *    format" list and create_weights): values are float8_e4m3fn, one uint8 E8M0 scale per group
 *    of 32 along the input dimension; weight [N, K], weight_scale [N, K/32].
 *  - aiter_flydsl page, AiterFlyDSLMxfp8LinearKernel (class docstring, input_quant_key,
 *    apply_weights): activations are MXFP8-quantized with row-major E8M0 scales [M, K/32];
 *    the output is bf16; bias is added after the GEMM.
 *  - aiter_flydsl page, row_major_weight: the (16, 16) preshuffled weight stores the logical
 *    [N/16, 16, K/32, 2, 16] array as [N/16, K/32, 2, 16, 16].
 *  - mxfp6 page, MxFp6LinearLayerConfig: E2M3 / E3M2 weight formats, group size 32.
 *
 * The pages call the quantizer but do not define its arithmetic.  This file follows the OCP
 * Microscaling (MX) v1.0 conversion rule, which is the reading used throughout:
 *   shared scale X = 2^(floor(log2(amax)) - emax_elem), stored as the E8M0 byte
 *   floor(log2(amax)) - emax_elem + 127, clamped to [0, 254] (0 for an all-zero block,
 *   0xFF when the block holds Inf/NaN); each element is x / X rounded to the nearest
 *   representable element value (ties to the even code), saturating at the format maximum,
 *   sign kept (so negative values that round to zero give -0).
 *
 * Element formats (OCP MX v1.0 element types):
 *   E4M3 (fn): 1 sign | 4 exp | 3 mantissa, bias 7, max 448, S.1111.111 = NaN, no Inf.
 *   E2M3:      1 sign | 2 exp | 3 mantissa, bias 1, max 7.5, no NaN/Inf.
 *   E3M2:      1 sign | 3 exp | 2 mantissa, bias 3, max 28,  no NaN/Inf.
 * FP6 storage: four 6-bit codes per three bytes, little-endian along K
 *   (w24 = c0 | c1 << 6 | c2 << 12 | c3 << 18; bytes w24 & 255, (w24 >> 8) & 255, w24 >> 16).
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* format identifiers (the same numbers the public header uses, chosen independently here) */
#define ORC_E4M3 0
#define ORC_E2M3 2
#define ORC_E3M2 3

typedef struct {
    int mbits;      /* mantissa bits                                   */
    int emin;       /* exponent of the smallest normal (1 - bias)      */
    int emax;       /* exponent of the largest normal                  */
    double maxval;  /* largest finite magnitude                        */
    int maxcode;    /* its code (magnitude bits only)                  */
    int signbit;    /* position of the sign bit                        */
    int has_nan;    /* E4M3 only: S.1111.111                           */
} orc_fmt;

static int fmt_params(int fmt, orc_fmt* f)
{
    switch (fmt) {
    case ORC_E4M3: *f = (orc_fmt){3, -6, 8, 448.0, 0x7E, 7, 1}; return 0;
    case ORC_E2M3: *f = (orc_fmt){3, 0, 2, 7.5, 0x1F, 5, 0}; return 0;
    case ORC_E3M2: *f = (orc_fmt){2, -2, 4, 28.0, 0x1F, 5, 0}; return 0;
    default: return -1;
    }
}

/* ---------------------------------------------------------------- bf16 <-> fp64 */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* fp64 -> bf16, round to nearest even (used only to report the rounded reference).
 * Written on the fp64 value: find the bf16 spacing at |v| and round the quotient. */
uint16_t orc_double_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    int sign = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint32_t mag;
    if (a == 0.0) {
        mag = 0;
    } else {
        int p;
        frexp(a, &p);
        int e = p - 1;                          /* floor(log2 a)             */
        if (e < -126) e = -126;                 /* subnormal spacing 2^-133  */
        double q = nearbyint(a / ldexp(1.0, e - 7));   /* 8 significant bits */
        double r = q * ldexp(1.0, e - 7);
        if (r >= ldexp(1.0, 128)) {
            mag = 0x7F80;                       /* overflow to Inf           */
        } else {
            /* re-encode the exactly representable r */
            float rf = (float)r;
            uint32_t u;
            memcpy(&u, &rf, 4);
            mag = (u >> 16) & 0x7FFF;
        }
    }
    return (uint16_t)((sign << 15) | mag);
}

/* ---------------------------------------------------------------- element codec */

/* Value of one element code (sign included); NaN for the E4M3 NaN code. */
double orc_decode(int code, int fmt)
{
    orc_fmt f;
    if (fmt_params(fmt, &f)) return NAN;
    int sign = (code >> f.signbit) & 1;
    int mag = code & ((1 << f.signbit) - 1);
    if (f.has_nan && mag == 0x7F) return NAN;
    int field = mag >> f.mbits;
    int mant = mag & ((1 << f.mbits) - 1);
    double v;
    if (field == 0)   /* subnormal: mant * 2^(emin - mbits) */
        v = ldexp((double)mant, f.emin - f.mbits);
    else              /* normal: (2^mbits + mant) * 2^(field - 1 + emin - mbits) */
        v = ldexp((double)((1 << f.mbits) + mant), field - 1 + f.emin - f.mbits);
    return sign ? -v : v;
}

/* Code of the element nearest to v (v already divided by the block scale):
 * round to nearest, ties to the even code; magnitudes at or above the format maximum saturate;
 * the sign of v is kept even when the magnitude rounds to zero. */
int orc_encode(double v, int fmt)
{
    orc_fmt f;
    if (fmt_params(fmt, &f)) return -1;
    int sign = signbit(v) ? 1 : 0;
    if (isnan(v)) return f.has_nan ? ((sign << 7) | 0x7F) : (sign << f.signbit);
    double a = fabs(v);
    int mag;
    if (a >= f.maxval) {
        mag = f.maxcode;                       /* saturate (also +-Inf) */
    } else {
        /* binade of a: the spacing of representable values there is 2^(e - mbits),
         * with e = floor(log2 a) for normals and e = emin for the subnormal range. */
        int e = f.emin;
        if (a > 0.0) {
            int p;
            frexp(a, &p);                      /* a = m * 2^p, m in [0.5, 1) */
            if (p - 1 > e) e = p - 1;
        }
        double q = nearbyint(a / ldexp(1.0, e - f.mbits));   /* RNE on the integer grid */
        /* q counts spacings inside the binade starting at 2^e (or at 0 for subnormals):
         * subnormal range (e == emin): code = q (q == 2^mbits is the smallest normal);
         * normal: code = (e - emin + 1) << mbits | (q - 2^mbits); a carry (q == 2^(mbits+1))
         * moves to the next exponent with mantissa 0.  Both read as the single formula: */
        mag = (e - f.emin) * (1 << f.mbits) + (int)q;
        if (mag > f.maxcode) mag = f.maxcode;  /* cannot happen for a < maxval; kept as a guard */
    }
    return (sign << f.signbit) | mag;
}

/* orc_encode over an array (for the exhaustive sweeps in the tests). */
int orc_encode_many(const double* v, int64_t n, int fmt, uint8_t* out)
{
    orc_fmt f;
    if (fmt_params(fmt, &f)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_encode(v[i], fmt);
    return 0;
}

/* ---------------------------------------------------------------- E8M0 shared scale */

/* E8M0 byte for a block whose largest magnitude is amax (OCP MX rule, see header). */
int orc_scale_byte(double amax, int fmt)
{
    orc_fmt f;
    if (fmt_params(fmt, &f)) return -1;
    if (isnan(amax) || isinf(amax)) return 0xFF;
    if (amax == 0.0) return 0;                 /* 2^-127: the clamp of 2^-inf */
    int p;
    frexp(amax, &p);
    int e = (p - 1) - f.emax;                  /* floor(log2 amax) - emax_elem */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

double orc_scale_value(int byte)
{
    if (byte == 0xFF) return NAN;
    return ldexp(1.0, byte - 127);
}

/* ---------------------------------------------------------------- block quantizer */

/* Quantize a bf16 matrix [rows, K] (row stride ldx elements) along K in blocks of 32:
 * codes [rows, K] (one code per byte, row-major), scales [rows, K/32] row-major.
 * A block holding Inf/NaN gets scale 0xFF; its E4M3 codes are NaN (0x7F), FP6 codes 0.
 * Returns 0, or -1 for a bad format / K not a multiple of 32. */
int orc_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, int fmt,
                 uint8_t* codes, uint8_t* scales)
{
    orc_fmt f;
    if (fmt_params(fmt, &f) || K % 32 != 0) return -1;
    const int64_t KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint16_t* blk = x + r * ldx + kb * 32;
            /* step 1: block amax (Inf/NaN noted separately: fmax would skip a NaN) */
            double amax = 0.0;
            int nonfinite = 0;
            for (int j = 0; j < 32; ++j) {
                double v = orc_bf16_to_double(blk[j]);
                if (isnan(v) || isinf(v)) nonfinite = 1;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            /* step 2: shared E8M0 scale */
            int sb = nonfinite ? 0xFF : orc_scale_byte(amax, fmt);
            scales[r * KB + kb] = (uint8_t)sb;
            /* step 3: elements, x / 2^(sb - 127) exactly, then nearest code */
            for (int j = 0; j < 32; ++j) {
                int c;
                if (sb == 0xFF) {
                    c = f.has_nan ? 0x7F : 0;
                } else {
                    double v = ldexp(orc_bf16_to_double(blk[j]), 127 - sb);
                    c = orc_encode(v, fmt);
                }
                codes[r * K + kb * 32 + j] = (uint8_t)c;
            }
        }
    }
    return 0;
}

/* Dequantize codes [rows, K] with scales [rows, K/32] into fp64 [rows, K]. */
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                   int fmt, double* out)
{
    orc_fmt f;
    if (fmt_params(fmt, &f) || K % 32 != 0) return -1;
    const int64_t KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = orc_decode(codes[r * K + k], fmt) *
                             orc_scale_value(scales[r * KB + k / 32]);
    return 0;
}

/* ---------------------------------------------------------------- FP6 storage */

/* Pack 6-bit codes [rows, K] into [rows, 3K/4] bytes (four codes per three bytes). */
int orc_fp6_pack(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed)
{
    if (K % 4 != 0) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < K / 4; ++g) {
            const uint8_t* c = codes + r * K + 4 * g;
            uint32_t w24 = (uint32_t)(c[0] & 63) | (uint32_t)(c[1] & 63) << 6 |
                           (uint32_t)(c[2] & 63) << 12 | (uint32_t)(c[3] & 63) << 18;
            uint8_t* o = packed + r * (3 * K / 4) + 3 * g;
            o[0] = (uint8_t)(w24 & 255);
            o[1] = (uint8_t)((w24 >> 8) & 255);
            o[2] = (uint8_t)(w24 >> 16);
        }
    return 0;
}

int orc_fp6_unpack(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* codes)
{
    if (K % 4 != 0) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < K / 4; ++g) {
            const uint8_t* p = packed + r * (3 * K / 4) + 3 * g;
            uint32_t w24 = (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16;
            for (int j = 0; j < 4; ++j) codes[r * K + 4 * g + j] = (uint8_t)((w24 >> (6 * j)) & 63);
        }
    return 0;
}

/* ---------------------------------------------------------------- the pages' (16,16) shuffle */

/* aiter_flydsl page, row_major_weight: logical [N/16, 16, K/32, 2, 16] (row n = 16 n0 + n1,
 * column k = 32 k0 + 16 k1 + k2) is stored as [N/16, K/32, 2, 16, 16] indexed
 * [n0, k0, k1, n1, k2].  Forward: row-major W [N, K] bytes -> stored order. */
int orc_shuffle16(const uint8_t* w, int64_t N, int64_t K, uint8_t* out)
{
    if (N % 16 != 0 || K % 32 != 0) return -1;
    const int64_t KB = K / 32;
    for (int64_t n0 = 0; n0 < N / 16; ++n0)
        for (int64_t k0 = 0; k0 < KB; ++k0)
            for (int k1 = 0; k1 < 2; ++k1)
                for (int n1 = 0; n1 < 16; ++n1)
                    for (int k2 = 0; k2 < 16; ++k2) {
                        int64_t dst = (((n0 * KB + k0) * 2 + k1) * 16 + n1) * 16 + k2;
                        int64_t src = (16 * n0 + n1) * K + 32 * k0 + 16 * k1 + k2;
                        out[dst] = w[src];
                    }
    return 0;
}

/* Inverse: stored order -> row-major W [N, K]. */
int orc_unshuffle16(const uint8_t* s, int64_t N, int64_t K, uint8_t* w)
{
    if (N % 16 != 0 || K % 32 != 0) return -1;
    const int64_t KB = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t n0 = n / 16, n1 = n % 16, k0 = k / 32, k1 = (k % 32) / 16, k2 = k % 16;
            w[n * K + k] = s[(((n0 * KB + k0) * 2 + k1) * 16 + n1) * 16 + k2];
        }
    return 0;
}

/* ---------------------------------------------------------------- fp64 linear */

/* y[m, n] = sum_k xd[m, k] * wd[n, k] + (bias ? bias[n] : 0), all fp64, k ascending. */
void orc_matmul_nt(const double* xd, const double* wd, const double* bias,
                   int64_t M, int64_t N, int64_t K, double* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += xd[m * K + k] * wd[n * K + k];
            y[m * N + n] = s + (bias ? bias[n] : 0.0);
        }
}

/* The same sum for a list of (m, n) output positions, straight from the quantized operands
 * (codes one per byte + row-major E8M0 scales); used to check sampled outputs of large
 * problems without materialising the dequantized matrices. */
/* y[rows[i], cols[i]] from quantized operands, one code per byte.  The activation codes are
 * in format xfmt: E4M3 for the MXFP8 layer, or E2M3 / E3M2 when the mxfp6 page's
 * activation_quant_key names an MXFP6 activation format. */
int orc_linear_entries_fmt(const uint8_t* xq, const uint8_t* xs, int xfmt, int64_t K,
                           const uint8_t* wq, const uint8_t* ws, int wfmt, const double* bias,
                           const int64_t* rows, const int64_t* cols, int64_t count, double* out)
{
    orc_fmt f;
    if (fmt_params(wfmt, &f) || fmt_params(xfmt, &f) || K % 32 != 0) return -1;
    const int64_t KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = rows[i], n = cols[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = orc_decode(xq[m * K + k], xfmt) * orc_scale_value(xs[m * KB + k / 32]);
            double b = orc_decode(wq[n * K + k], wfmt) * orc_scale_value(ws[n * KB + k / 32]);
            s += a * b;
        }
        out[i] = s + (bias ? bias[n] : 0.0);
    }
    return 0;
}

int orc_linear_entries(const uint8_t* xq, const uint8_t* xs, int64_t K, const uint8_t* wq,
                       const uint8_t* ws, int wfmt, const double* bias, const int64_t* rows,
                       const int64_t* cols, int64_t count, double* out)
{
    return orc_linear_entries_fmt(xq, xs, ORC_E4M3, K, wq, ws, wfmt, bias, rows, cols, count, out);
}

/* Root-mean-square normalization of bf16 rows: the producer of a pre-quantized activation.
 * The Mxfp8LinearKernel page's input_quant_key lets a layer take activations quantized outside
 * the kernel (row-major [M, K/32] E8M0 scales); the pages name no producer, and the reading
 * here is the usual RMS norm with a bf16 weight, computed as a float norm does it:
 *     r   = 1 / sqrt(sum_k x_k^2 / K + eps)       (fp64), then r32 = fp32(r) (nearest even)
 *     p_k = fp32(x_k * r32)                       (the product is exact in fp64; one rounding)
 *     t_k = bf16(p_k),  y_k = bf16(t_k * gamma_k) (round to nearest even; t * gamma is exact)
 * pre (optional) receives p_k, the value the bf16 rounding of t acts on. */
int orc_rmsnorm(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* gamma,
                double eps, uint16_t* y, double* pre)
{
    if (K <= 0 || ldx < K || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; ++m) {
        const uint16_t* xr = x + m * ldx;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = orc_bf16_to_double(xr[k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        double r32 = (double)(float)r;
        for (int64_t k = 0; k < K; ++k) {
            double p = (double)(float)(orc_bf16_to_double(xr[k]) * r32);
            if (pre) pre[m * K + k] = p;
            uint16_t t = orc_double_to_bf16(p);
            y[m * K + k] = orc_double_to_bf16(orc_bf16_to_double(t) * orc_bf16_to_double(gamma[k]));
        }
    }
    return 0;
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
