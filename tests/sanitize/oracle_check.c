/* oracle_check.c -- the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built with gcc by tests/test_sanitizers.py
 * together with oracle/hqq_oracle.c).
 *
 * Runs every oracle entry point over every format and ragged shapes (one
 * element past a line, a single row, lines that are not whole words), on
 * seeded weights that include outliers, constant groups, subnormals and the
 * fp16 extremes, and checks the invariants that hold at any size: codes in
 * [0, qmax], pack/unpack round trips, iters = 0 equal to min-max rounding,
 * dequantized weights within half a step of the group's range, and the
 * rejection of bad arguments.  Exit status 0: every check passed. */
#include "hqq_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int g_fail = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                             \
        }                                                                         \
    } while (0)

static unsigned long long g_rng = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (double)(g_rng >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void)
{
    double u = urand(), v = urand();
    if (u < 1e-300)
        u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

static void fill(uint16_t *W, int64_t n, int kind)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = 0.02 * nrand();
        if (urand() < 0.002)
            x *= 20.0;
        if (kind == 1 && (i % 97) < 8)
            x = 0.3;                     /* a run of equal values */
        if (kind == 2)
            x *= 1e-4;                   /* many subnormals */
        if (kind == 3 && i % 53 == 0)
            x = (i & 1) ? 65504.0 : -65504.0;
        W[i] = hqq_ref_f32_to_f16((float)x);
    }
}

static void one_case(int nbits, int gs, int axis, int64_t rows, int64_t cols, int iters, int kind)
{
    const int64_t n = rows * cols, ng = n / gs;
    const int qmax = (1 << nbits) - 1;
    uint16_t *W = malloc((size_t)n * 2), *Wh = malloc((size_t)n * 2);
    uint8_t *codes = malloc((size_t)n), *back = malloc((size_t)n);
    float *scale = malloc((size_t)ng * 4), *zero = malloc((size_t)ng * 4);
    float *scale2 = malloc((size_t)ng * 4), *zero2 = malloc((size_t)ng * 4);
    const int64_t nw = hqq_ref_packed_words(rows, cols, nbits, axis);
    CHECK(nw > 0);
    uint32_t *packed = malloc((size_t)nw * 4), *packed2 = malloc((size_t)nw * 4);
    fill(W, n, kind);
    CHECK(hqq_ref_quantize_codes(W, rows, cols, nbits, gs, axis, iters, 0.7f, 10.f, 1.01f, codes, scale, zero) == 0);
    for (int64_t i = 0; i < n; ++i)
        CHECK(codes[i] <= qmax);
    CHECK(hqq_ref_quantize(W, rows, cols, nbits, gs, axis, iters, 0.7f, 10.f, 1.01f, packed, scale2, zero2) == 0);
    CHECK(memcmp(scale, scale2, (size_t)ng * 4) == 0 && memcmp(zero, zero2, (size_t)ng * 4) == 0);
    CHECK(hqq_ref_pack(codes, rows, cols, nbits, axis, packed2) == 0);
    CHECK(memcmp(packed, packed2, (size_t)nw * 4) == 0);
    CHECK(hqq_ref_unpack(packed, rows, cols, nbits, axis, back) == 0);
    CHECK(memcmp(codes, back, (size_t)n) == 0);
    CHECK(hqq_ref_dequantize(packed, scale, zero, rows, cols, nbits, gs, axis, Wh) == 0);
    CHECK(hqq_ref_dequantize_dt(packed, scale, zero, rows, cols, nbits, gs, axis, 1, Wh) == 0);
    /* iters = 0: min-max rounding, the min maps to code 0 */
    if (iters == 0) {
        for (int64_t g = 0; g < ng; ++g) {
            /* group g's first element and its minimum, in W's layout */
            int64_t line, k;
            if (axis == 1) {
                line = g / (cols / gs);
                k = g % (cols / gs);
            } else {
                line = g % cols;
                k = g / cols;
            }
            float mn = INFINITY;
            int64_t imn = 0;
            for (int j = 0; j < gs; ++j) {
                const int64_t idx = axis == 1 ? line * cols + k * gs + j : (k * gs + j) * cols + line;
                const float v = hqq_ref_f16_to_f32(W[idx]);
                if (v < mn) {
                    mn = v;
                    imn = idx;
                }
            }
            CHECK(codes[imn] == 0);
        }
    }
    free(W);
    free(Wh);
    free(codes);
    free(back);
    free(scale);
    free(zero);
    free(scale2);
    free(zero2);
    free(packed);
    free(packed2);
}

int main(void)
{
    const int nbits[] = {1, 2, 3, 4, 8};
    const int gss[] = {8, 16, 32, 64, 128, 256};
    for (int a = 0; a < 5; ++a)
        for (int b = 0; b < 6; ++b)
            for (int axis = 0; axis < 2; ++axis) {
                const int gs = gss[b];
                const int64_t line = (int64_t)gs * (gs <= 64 ? 3 : 1);
                const int64_t other[] = {1, 7, 33};
                for (int o = 0; o < 3; ++o) {
                    const int64_t rows = axis == 1 ? other[o] : line, cols = axis == 1 ? line : other[o];
                    one_case(nbits[a], gs, axis, rows, cols, (o == 0) ? 0 : 20, o + (a & 1));
                }
            }
    /* the group solve with traces, p = 1 and a shrink-heavy beta */
    {
        float w[64], tz[21], tb[20], tq[20 * 64], tx[20 * 64], te[20 * 64], s, z;
        uint8_t c[64];
        for (int i = 0; i < 64; ++i)
            w[i] = (float)(0.05 * nrand());
        CHECK(hqq_ref_solve_group(w, 64, 4, 20, 1.0f, 1000.f, 1.01f, c, &s, &z, tz, tb, tq, tx, te) == 0);
        CHECK(hqq_ref_solve_group(w, 64, 2, 20, 0.7f, 0.1f, 1.5f, c, &s, &z, NULL, NULL, NULL, NULL, NULL) == 0);
        CHECK(hqq_ref_shrink(0.0f, 0.7f, 10.f) == 0.0f);
        CHECK(hqq_ref_shrink(1.0f, 1.0f, 10.f) == 0.9f);
    }
    /* meta quantization, ragged last group */
    {
        float m[1000], back[1000], ms[8], mz[8];
        uint8_t c[1000];
        for (int i = 0; i < 1000; ++i)
            m[i] = (float)(1.0 + nrand());
        CHECK(hqq_ref_quantize_meta(m, 1000, 128, c, ms, mz) == 0);
        CHECK(hqq_ref_dequantize_meta(c, ms, mz, 1000, 128, back) == 0);
    }
    /* linear layer, both dtypes */
    {
        enum { M = 3, K = 128, N = 40 };
        uint16_t X[M * K], Wq[N * K];
        uint32_t pk[N * K / 8];
        float s[N * K / 64], z[N * K / 64];
        double Y[M * N], A[M * N];
        fill(X, M * K, 0);
        fill(Wq, N * K, 0);
        CHECK(hqq_ref_quantize(Wq, N, K, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, s, z) == 0);
        CHECK(hqq_ref_linear(X, M, K, pk, s, z, N, 4, 64, Y, A) == 0);
        CHECK(hqq_ref_linear_dt(X, 1, M, K, pk, s, z, N, 4, 64, Y, NULL) == 0);
    }
    /* bad arguments are rejected without touching the buffers */
    {
        uint16_t W[64];
        uint8_t c[64];
        float s[8], z[8];
        CHECK(hqq_ref_quantize_codes(W, 1, 64, 5, 64, 1, 20, 0.7f, 10.f, 1.01f, c, s, z) < 0);
        CHECK(hqq_ref_quantize_codes(W, 1, 60, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, c, s, z) < 0);
        CHECK(hqq_ref_quantize_codes(W, 1, 64, 4, 64, 2, 20, 0.7f, 10.f, 1.01f, c, s, z) < 0);
        CHECK(hqq_ref_packed_words(0, 64, 4, 1) < 0);
    }
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
