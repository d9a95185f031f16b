/*
 * hqq_oracle.c -- plain, slow, single-threaded CPU oracle of the HQQ solve.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline, never by the library.  Build:
 *     gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction, no fast-math, IEEE fp32/fp64, denormals kept).
 *
 * What the pages say (the structure only):
 *   - HQQ is calibration-free: it needs the weights alone ([lnwmold] 2.1).
 *   - The quantization error is split through an auxiliary variable and the
 *     problem is solved by alternating between two simpler sub-problems
 *     ([lnwmold] 2.1, [devpress] 2, [ainews] technical deep dive).
 *   - The loss is non-convex and robust: small residuals are tolerated while
 *     large ones (outliers) are treated specially ([devpress] 2).
 *   - group_size consecutive weights share one scale and one zero point;
 *     nbits is the code width; axis picks the grouping direction
 *     ([devpress] 3.3, [lnwmold] 2.2).
 *
 * The solve implemented here, per group of gs weights w (b = nbits,
 * qmax = 2^b - 1):
 *   init     scale = qmax / (max w - min w),  zero = -(min w * scale)
 *   repeat iters times (beta starts at beta0):
 *     W_q  = clamp(round(w * scale + zero), 0, qmax)
 *     W_r  = (W_q - zero) / scale
 *     x    = w - W_r
 *     W_e  = sign(x) * max(|x| - |x|^(p-1) / beta, 0)       (lp shrinkage)
 *     zero = mean(W_q - (w - W_e) * scale)
 *     beta = beta * kappa
 *   output   codes = clamp(round(w * scale + zero), 0, qmax) with the final
 *            zero; scale never changes.
 *
 * Readings of points the pages leave open (all of them; each is also listed
 * in the design notes):
 *   R1 precision: every step is fp32 (the precision of the outputs and of the
 *      GPU kernel), so the integer codes are decided in the same precision on
 *      both sides.  w*scale+zero is one fused multiply-add (one rounding).
 *   R2 rounding: round half to even (rintf in the default mode).
 *   R3 constant group (max == min): scale = 1, zero = -min; every code is 0
 *      and the group is a fixed point (x = 0 so W_e = 0).
 *   R4 |x|^(p-1) is evaluated in fp64 and rounded once to fp32 (the correctly
 *      rounded fp32 power in all but astronomically rare cases); x = 0 with
 *      p < 1 gives +inf and so W_e = 0.
 *   R5 the mean is evaluated through linearity as
 *        (sum W_q - scale * (sum w - sum W_e)) / gs
 *      in fp64: sum W_q (small integers) and sum w (fp16 values) are exact in
 *      any order; sum W_e is the pairwise tree over adjacent elements (pairs
 *      (0,1), (2,3), ..., then pairs of those sums, and so on); the result is
 *      rounded once to fp32.
 *   R6 the first iteration uses beta0 and beta is multiplied by kappa after
 *      the zero update; exactly iters steps, no early stop; iters = 0 is RTN.
 *   R7 zero is neither rounded nor clamped.
 */
#include "hqq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32 conversions, written from the IEEE binary16 field layout    */
/* ------------------------------------------------------------------------ */

float hqq_ref_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    float mag;
    if (ex == 0)
        mag = ldexpf((float)man, -24);               /* subnormal: man * 2^-24 */
    else if (ex == 31)
        mag = man ? NAN : INFINITY;
    else
        mag = ldexpf((float)(man | 0x400), ex - 25); /* (1024 + man) * 2^(ex-25) */
    return sign ? -mag : mag;
}

uint16_t hqq_ref_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    float a = fabsf(f);
    if (isnan(a))
        return (uint16_t)(sign | 0x7e00u);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexpf(1.0f, -14)) {
        /* subnormal range, quantum 2^-24; 1024 quanta becomes the smallest normal */
        double m = nearbyint((double)a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    frexpf(a, &e);                                  /* a in [2^(e-1), 2^e) */
    double m = nearbyint(ldexp((double)a, 11 - e)); /* 11-bit significand in [1024, 2048] */
    int biased = e - 1 + 15;
    if (m == 2048.0) {
        m = 1024.0;
        biased += 1;
    }
    if (biased >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)m - 1024));
}

/* bfloat16 (1 sign, 8 exponent, 7 fraction bits; the top half of an IEEE
 * binary32), from its field layout: the models the pages quantize are often
 * loaded in bf16 (devpress.csdn.net tutorial, section 5). */
float hqq_ref_bf16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 7) & 0xff;
    int man = h & 0x7f;
    float mag;
    if (ex == 0)
        mag = ldexpf((float)man, -133);              /* subnormal: man * 2^-133 */
    else if (ex == 255)
        mag = man ? NAN : INFINITY;
    else
        mag = ldexpf((float)(man | 0x80), ex - 134); /* (128 + man) * 2^(ex-134) */
    return sign ? -mag : mag;
}

/* fp32 -> bf16, round to nearest, ties to even */
uint16_t hqq_ref_f32_to_bf16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    float a = fabsf(f);
    if (isnan(a))
        return (uint16_t)(sign | 0x7fc0u);
    if (isinf(a))
        return (uint16_t)(sign | 0x7f80u);
    if (a < ldexpf(1.0f, -126)) {
        /* subnormal range, quantum 2^-133; 128 quanta becomes the smallest normal */
        double m = nearbyint(ldexp((double)a, 133));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    frexpf(a, &e);                                  /* a in [2^(e-1), 2^e) */
    double m = nearbyint(ldexp((double)a, 8 - e));  /* 8-bit significand in [128, 256] */
    int biased = e - 1 + 127;
    if (m == 256.0) {
        m = 128.0;
        biased += 1;
    }
    if (biased >= 255)
        return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)m - 128));
}

static float widen16(uint16_t h, int dtype)
{
    return dtype == HQQ_REF_BF16 ? hqq_ref_bf16_to_f32(h) : hqq_ref_f16_to_f32(h);
}

/* ------------------------------------------------------------------------ */
/* the solve                                                                */
/* ------------------------------------------------------------------------ */

static float quantize_one(float w, float scale, float zero, float qmax)
{
    float q = rintf(fmaf(w, scale, zero));
    if (q < 0.0f)
        q = 0.0f;
    if (q > qmax)
        q = qmax;
    return q;
}

float hqq_ref_shrink(float x, float p, float beta)
{
    float pm1 = p - 1.0f;
    float a = fabsf(x);
    float pw = (float)pow((double)a, (double)pm1);
    float v = a - pw / beta;
    return v > 0.0f ? copysignf(v, x) : 0.0f;
}

int hqq_ref_solve_group(const float *w, int gs, int nbits, int iters,
                        float p, float beta0, float kappa,
                        uint8_t *codes, float *scale_out, float *zero_out,
                        float *tr_zero, float *tr_beta,
                        float *tr_q, float *tr_x, float *tr_e)
{
    if (!w || !codes || !scale_out || !zero_out || gs < 1 || nbits < 1 || nbits > 8 || iters < 0)
        return -1;
    const float qmax = (float)((1 << nbits) - 1);

    float mn = w[0], mx = w[0];
    for (int i = 1; i < gs; ++i) {
        if (w[i] < mn)
            mn = w[i];
        if (w[i] > mx)
            mx = w[i];
    }
    float rng = mx - mn;
    float scale, zero;
    if (rng == 0.0f) {
        scale = 1.0f;
        zero = -mn;
    } else {
        scale = qmax / rng;
        zero = -(mn * scale);
    }

    float *q = (float *)malloc(sizeof(float) * (size_t)gs);
    float *e = (float *)malloc(sizeof(float) * (size_t)gs);
    double *te = (double *)malloc(sizeof(double) * (size_t)gs);
    if (!q || !e || !te) {
        free(q);
        free(e);
        free(te);
        return -2;
    }

    float beta = beta0;
    if (tr_zero)
        tr_zero[0] = zero;
    for (int it = 0; it < iters; ++it) {
        /* W_q */
        for (int i = 0; i < gs; ++i)
            q[i] = quantize_one(w[i], scale, zero, qmax);
        /* W_r, x and W_e */
        for (int i = 0; i < gs; ++i) {
            float wr = (q[i] - zero) / scale;
            float x = w[i] - wr;
            e[i] = hqq_ref_shrink(x, p, beta);
            if (tr_x)
                tr_x[(size_t)it * gs + i] = x;
        }
        /* zero = mean(W_q - (w - W_e) * scale), reading R5 */
        double sum_q = 0.0, sum_w = 0.0;
        for (int i = 0; i < gs; ++i) {
            sum_q += (double)q[i];
            sum_w += (double)w[i];
            te[i] = (double)e[i];
        }
        for (int st = 1; st < gs; st *= 2)
            for (int i = 0; i + st < gs; i += 2 * st)
                te[i] += te[i + st];
        double sum_e = te[0];
        double num = sum_q - (double)scale * (sum_w - sum_e);
        zero = (float)(num / (double)gs);

        if (tr_beta)
            tr_beta[it] = beta;
        if (tr_q)
            memcpy(tr_q + (size_t)it * gs, q, sizeof(float) * (size_t)gs);
        if (tr_e)
            memcpy(tr_e + (size_t)it * gs, e, sizeof(float) * (size_t)gs);
        if (tr_zero)
            tr_zero[it + 1] = zero;
        beta = beta * kappa;
    }

    for (int i = 0; i < gs; ++i)
        codes[i] = (uint8_t)quantize_one(w[i], scale, zero, qmax);
    *scale_out = scale;
    *zero_out = zero;
    free(q);
    free(e);
    free(te);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* tensor-level entry points                                                */
/* ------------------------------------------------------------------------ */

static int codes_per_word(int nbits)
{
    switch (nbits) {
    case 8: return 4;
    case 4: return 8;
    case 3: return 10;
    case 2: return 16;
    case 1: return 32;
    default: return -1;
    }
}

static int check_shape(int64_t rows, int64_t cols, int nbits, int group_size, int axis)
{
    if (rows < 1 || cols < 1)
        return -4;
    if (codes_per_word(nbits) < 0)
        return -1;
    if (axis != 0 && axis != 1)
        return -2;
    int64_t line = axis == 1 ? cols : rows;
    if (group_size < 1 || line % group_size != 0)
        return -3;
    return 0;
}

int hqq_ref_quantize_codes(const uint16_t *W, int64_t rows, int64_t cols,
                           int nbits, int group_size, int axis, int iters,
                           float p, float beta0, float kappa,
                           uint8_t *codes, float *scale, float *zero)
{
    return hqq_ref_quantize_codes_dt(W, HQQ_REF_F16, rows, cols, nbits, group_size, axis, iters,
                                     p, beta0, kappa, codes, scale, zero);
}

int hqq_ref_quantize_codes_dt(const uint16_t *W, int dtype, int64_t rows, int64_t cols,
                              int nbits, int group_size, int axis, int iters,
                              float p, float beta0, float kappa,
                              uint8_t *codes, float *scale, float *zero)
{
    if (dtype != HQQ_REF_F16 && dtype != HQQ_REF_BF16)
        return -8;
    int st = check_shape(rows, cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!W || !codes || !scale || !zero)
        return -5;
    if (iters < 0)
        return -6;
    const int gs = group_size;
    float *w = (float *)malloc(sizeof(float) * (size_t)gs);
    uint8_t *c = (uint8_t *)malloc((size_t)gs);
    if (!w || !c) {
        free(w);
        free(c);
        return -2;
    }
    if (axis == 1) {
        const int64_t ng = cols / gs;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t g = 0; g < ng; ++g) {
                for (int j = 0; j < gs; ++j)
                    w[j] = widen16(W[r * cols + g * gs + j], dtype);
                float s, z;
                hqq_ref_solve_group(w, gs, nbits, iters, p, beta0, kappa, c, &s, &z,
                                    NULL, NULL, NULL, NULL, NULL);
                for (int j = 0; j < gs; ++j)
                    codes[r * cols + g * gs + j] = c[j];
                scale[r * ng + g] = s;
                zero[r * ng + g] = z;
            }
    } else {
        const int64_t ng = rows / gs;
        for (int64_t g = 0; g < ng; ++g)
            for (int64_t col = 0; col < cols; ++col) {
                for (int j = 0; j < gs; ++j)
                    w[j] = widen16(W[(g * gs + j) * cols + col], dtype);
                float s, z;
                hqq_ref_solve_group(w, gs, nbits, iters, p, beta0, kappa, c, &s, &z,
                                    NULL, NULL, NULL, NULL, NULL);
                for (int j = 0; j < gs; ++j)
                    codes[(g * gs + j) * cols + col] = c[j];
                scale[g * cols + col] = s;
                zero[g * cols + col] = z;
            }
    }
    free(w);
    free(c);
    return 0;
}

int64_t hqq_ref_packed_words(int64_t rows, int64_t cols, int nbits, int axis)
{
    int C = codes_per_word(nbits);
    if (C < 0 || rows < 1 || cols < 1 || (axis != 0 && axis != 1))
        return -1;
    if (axis == 1)
        return rows * ((cols + C - 1) / C);
    return ((rows + C - 1) / C) * cols;
}

/* Word k of a line holds codes k*C .. k*C+C-1 of that line, code j of the word
 * in bits [j*b, j*b+b); unused fields of a line's last word are zero. */
int hqq_ref_pack(const uint8_t *codes, int64_t rows, int64_t cols,
                 int nbits, int axis, uint32_t *packed)
{
    int C = codes_per_word(nbits);
    if (C < 0 || rows < 1 || cols < 1 || (axis != 0 && axis != 1) || !codes || !packed)
        return -1;
    const uint32_t mask = (1u << nbits) - 1u;
    if (axis == 1) {
        int64_t wpl = (cols + C - 1) / C;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < wpl; ++k) {
                uint32_t word = 0;
                for (int j = 0; j < C; ++j) {
                    int64_t col = k * C + j;
                    if (col < cols)
                        word |= ((uint32_t)codes[r * cols + col] & mask) << (j * nbits);
                }
                packed[r * wpl + k] = word;
            }
    } else {
        int64_t wrows = (rows + C - 1) / C;
        for (int64_t k = 0; k < wrows; ++k)
            for (int64_t col = 0; col < cols; ++col) {
                uint32_t word = 0;
                for (int j = 0; j < C; ++j) {
                    int64_t r = k * C + j;
                    if (r < rows)
                        word |= ((uint32_t)codes[r * cols + col] & mask) << (j * nbits);
                }
                packed[k * cols + col] = word;
            }
    }
    return 0;
}

int hqq_ref_unpack(const uint32_t *packed, int64_t rows, int64_t cols,
                   int nbits, int axis, uint8_t *codes)
{
    int C = codes_per_word(nbits);
    if (C < 0 || rows < 1 || cols < 1 || (axis != 0 && axis != 1) || !codes || !packed)
        return -1;
    const uint32_t mask = (1u << nbits) - 1u;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t col = 0; col < cols; ++col) {
            uint32_t word;
            int j;
            if (axis == 1) {
                int64_t wpl = (cols + C - 1) / C;
                word = packed[r * wpl + col / C];
                j = (int)(col % C);
            } else {
                word = packed[(r / C) * cols + col];
                j = (int)(r % C);
            }
            codes[r * cols + col] = (uint8_t)((word >> (j * nbits)) & mask);
        }
    return 0;
}

int hqq_ref_dequantize(const uint32_t *packed, const float *scale, const float *zero,
                       int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                       uint16_t *W_hat)
{
    return hqq_ref_dequantize_dt(packed, scale, zero, rows, cols, nbits, group_size, axis,
                                 HQQ_REF_F16, W_hat);
}

int hqq_ref_dequantize_dt(const uint32_t *packed, const float *scale, const float *zero,
                          int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                          int dtype, uint16_t *W_hat)
{
    if (dtype != HQQ_REF_F16 && dtype != HQQ_REF_BF16)
        return -8;
    int st = check_shape(rows, cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!packed || !scale || !zero || !W_hat)
        return -5;
    uint8_t *codes = (uint8_t *)malloc((size_t)(rows * cols));
    if (!codes)
        return -2;
    hqq_ref_unpack(packed, rows, cols, nbits, axis, codes);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t col = 0; col < cols; ++col) {
            int64_t gi = axis == 1 ? r * (cols / group_size) + col / group_size
                                   : (r / group_size) * cols + col;
            float q = (float)codes[r * cols + col];
            float wr = (q - zero[gi]) / scale[gi];
            W_hat[r * cols + col] = dtype == HQQ_REF_BF16 ? hqq_ref_f32_to_bf16(wr)
                                                          : hqq_ref_f32_to_f16(wr);
        }
    free(codes);
    return 0;
}

/* Metadata quantization (quant_scale / quant_zero: devpress.csdn.net
 * tutorial section 3.3 and its troubleshooting section: the scale and zero
 * arrays are themselves quantized at a higher precision such as 8 bits, and
 * kept in fp16 otherwise).  Reading: after the solve, a meta array of n fp32
 * values is cut into groups of group_size consecutive values (the last one
 * may be shorter) and each group is quantized by 8-bit min-max RTN -- the
 * solve above at iters = 0 -- giving uint8 codes and an fp32 scale and zero
 * per meta group.  Dequantization is (code - zero) / scale in fp32. */
int hqq_ref_quantize_meta(const float *meta, int64_t n, int group_size,
                          uint8_t *codes, float *mscale, float *mzero)
{
    if (n < 1 || group_size < 1 || group_size > 1024)
        return -4;
    if (!meta || !codes || !mscale || !mzero)
        return -5;
    const int64_t ng = (n + group_size - 1) / group_size;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t e0 = g * group_size;
        const int len = (int)(n - e0 < group_size ? n - e0 : group_size);
        float s, z;
        int st = hqq_ref_solve_group(meta + e0, len, 8, 0, 0.7f, 10.0f, 1.01f, codes + e0, &s, &z,
                                     NULL, NULL, NULL, NULL, NULL);
        if (st)
            return st;
        mscale[g] = s;
        mzero[g] = z;
    }
    return 0;
}

int hqq_ref_dequantize_meta(const uint8_t *codes, const float *mscale, const float *mzero,
                            int64_t n, int group_size, float *meta)
{
    if (n < 1 || group_size < 1 || group_size > 1024)
        return -4;
    if (!codes || !mscale || !mzero || !meta)
        return -5;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t g = i / group_size;
        meta[i] = ((float)codes[i] - mzero[g]) / mscale[g];
    }
    return 0;
}

int hqq_ref_linear(const uint16_t *X, int64_t M, int64_t K,
                   const uint32_t *packed, const float *scale, const float *zero,
                   int64_t N, int nbits, int group_size, double *Y, double *absY)
{
    return hqq_ref_linear_dt(X, HQQ_REF_F16, M, K, packed, scale, zero, N, nbits, group_size, Y, absY);
}

/* The quantized layer's forward in compute dtype fp16 or bf16: W_hat is the
 * dequantization into that dtype (lnwmold.com HQQ guide section 3.2, the
 * HQQLinear layer computes in compute_dtype), X is given in it, and each
 * output is the exact (fp64) sum of the products of the widened values. */
int hqq_ref_linear_dt(const uint16_t *X, int dtype, int64_t M, int64_t K,
                      const uint32_t *packed, const float *scale, const float *zero,
                      int64_t N, int nbits, int group_size, double *Y, double *absY)
{
    if (dtype != HQQ_REF_F16 && dtype != HQQ_REF_BF16)
        return -8;
    if (M < 1)
        return -4;
    int st = check_shape(N, K, nbits, group_size, 1);
    if (st)
        return st;
    if (!X || !packed || !scale || !zero || !Y)
        return -5;
    uint16_t *W_hat = (uint16_t *)malloc((size_t)(N * K) * sizeof(uint16_t));
    if (!W_hat)
        return -2;
    st = hqq_ref_dequantize_dt(packed, scale, zero, N, K, nbits, group_size, 1, dtype, W_hat);
    if (st == 0) {
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double prod = (double)widen16(X[m * K + k], dtype) *
                                  (double)widen16(W_hat[n * K + k], dtype);
                    acc += prod;
                    mag += fabs(prod);
                }
                Y[m * N + n] = acc;
                if (absY)
                    absY[m * N + n] = mag;
            }
    }
    free(W_hat);
    return st;
}

int hqq_ref_quantize(const uint16_t *W, int64_t rows, int64_t cols,
                     int nbits, int group_size, int axis, int iters,
                     float p, float beta0, float kappa,
                     uint32_t *packed, float *scale, float *zero)
{
    return hqq_ref_quantize_dt(W, HQQ_REF_F16, rows, cols, nbits, group_size, axis, iters,
                               p, beta0, kappa, packed, scale, zero);
}

int hqq_ref_quantize_dt(const uint16_t *W, int dtype, int64_t rows, int64_t cols,
                        int nbits, int group_size, int axis, int iters,
                        float p, float beta0, float kappa,
                        uint32_t *packed, float *scale, float *zero)
{
    if (!packed)
        return -5;
    uint8_t *codes = (uint8_t *)malloc((size_t)(rows > 0 && cols > 0 ? rows * cols : 1));
    if (!codes)
        return -2;
    int st = hqq_ref_quantize_codes_dt(W, dtype, rows, cols, nbits, group_size, axis, iters,
                                       p, beta0, kappa, codes, scale, zero);
    if (st == 0)
        st = hqq_ref_pack(codes, rows, cols, nbits, axis, packed);
    free(codes);
    return st;
}
