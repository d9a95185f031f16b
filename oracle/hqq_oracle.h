/*
 * hqq_oracle.h -- CPU oracle for the HQQ group-wise weight quantization solve.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library product links, loads or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or helper with the
 * HIP path.
 *
 * Sources (the web pages this project is built from):
 *   [devpress]  devpress.csdn.net tutorial "dropbox/hqq", section 2 (core
 *               principle: auxiliary variable, alternating optimisation) and
 *               section 3.3 (nbits / group_size / axis meaning).
 *   [lnwmold]   lnwmold.com HQQ guide, section 2.1 (calibration-free
 *               half-quadratic splitting into two alternating sub-problems),
 *               section 2.2 (nbits, group_size, axis: axis=0 groups along the
 *               output dimension, axis=1 along the input dimension), section
 *               3.2 (HQQLinear: W_q, scale, zero, dequantize(), unpack()).
 *   [ainews]    ainews.cool Dropbox-HQQ analysis, "technical deep dive"
 *               (reconstruction objective, auxiliary variable, alternation).
 * The pages give the structure but no update equations; the equations this
 * oracle implements are the HQQ solve as fixed for this library and written
 * out in hqq_oracle.c.  Every reading of a point the pages leave open is
 * listed there.
 *
 * Conventions: W is fp16 bits, row-major [rows, cols] (rows = out_features,
 * cols = in_features).  axis=1: a group is gs consecutive elements of a row;
 * axis=0: gs consecutive rows of one column.  Codes are packed along the
 * group axis, LSB first, C = 4 (8b), 8 (4b), 10 (3b), 16 (2b), 32 (1b) per
 * uint32.
 * All functions return 0 on success, a negative value on invalid arguments.
 */
#ifndef HQQ_ORACLE_H
#define HQQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exact fp16 -> fp32 widening, computed from the fields' values */
float hqq_ref_f16_to_f32(uint16_t h);
/* bfloat16 <-> fp32 (round to nearest even), from the bf16 field layout */
float hqq_ref_bf16_to_f32(uint16_t h);
uint16_t hqq_ref_f32_to_bf16(float f);

/* element types of 16-bit weights / dequantized outputs */
#define HQQ_REF_F16 0
#define HQQ_REF_BF16 1
/* fp32 -> fp16, round to nearest even, subnormals and overflow handled */
uint16_t hqq_ref_f32_to_f16(float f);

/* the lp shrinkage W_e = sign(x) * max(|x| - |x|^(p-1) / beta, 0) for one residual */
float hqq_ref_shrink(float x, float p, float beta);

/* Solve one group of gs fp32 weights.  Optional traces (NULL to skip):
 *   tr_zero[iters+1]  zero before iteration 0 .. after the last iteration
 *   tr_beta[iters]    beta used in each iteration
 *   tr_q[iters*gs]    W_q computed in each iteration
 *   tr_x[iters*gs]    residual x = W - W_r in each iteration
 *   tr_e[iters*gs]    W_e in each iteration                                  */
int hqq_ref_solve_group(const float *w, int gs, int nbits, int iters,
                        float p, float beta0, float kappa,
                        uint8_t *codes, float *scale, float *zero,
                        float *tr_zero, float *tr_beta,
                        float *tr_q, float *tr_x, float *tr_e);

/* Whole-tensor solve: codes (uint8 [rows, cols], W's layout), scale and zero
 * (axis=1: [rows, cols/gs]; axis=0: [rows/gs, cols]). */
/* W of element type dtype (HQQ_REF_F16 / HQQ_REF_BF16; -8 otherwise), widened
 * exactly to fp32; everything after that is the same solve.  The group sum
 * of the mean is formed in fp64 in index order. */
int hqq_ref_quantize_codes_dt(const uint16_t *W, int dtype, int64_t rows, int64_t cols,
                              int nbits, int group_size, int axis, int iters,
                              float p, float beta0, float kappa,
                              uint8_t *codes, float *scale, float *zero);
int hqq_ref_quantize_dt(const uint16_t *W, int dtype, int64_t rows, int64_t cols,
                        int nbits, int group_size, int axis, int iters,
                        float p, float beta0, float kappa,
                        uint32_t *packed, float *scale, float *zero);
/* dequantize into dtype (fp16 or bf16, round half to even from the fp32 quotient) */
int hqq_ref_dequantize_dt(const uint32_t *packed, const float *scale, const float *zero,
                          int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                          int dtype, uint16_t *W_hat);
int hqq_ref_quantize_codes(const uint16_t *W, int64_t rows, int64_t cols,
                           int nbits, int group_size, int axis, int iters,
                           float p, float beta0, float kappa,
                           uint8_t *codes, float *scale, float *zero);

/* Whole-tensor solve with packed output. */
int hqq_ref_quantize(const uint16_t *W, int64_t rows, int64_t cols,
                     int nbits, int group_size, int axis, int iters,
                     float p, float beta0, float kappa,
                     uint32_t *packed, float *scale, float *zero);

/* number of uint32 words of the packed layout, <0 on bad arguments */
int64_t hqq_ref_packed_words(int64_t rows, int64_t cols, int nbits, int axis);

int hqq_ref_pack(const uint8_t *codes, int64_t rows, int64_t cols,
                 int nbits, int axis, uint32_t *packed);
int hqq_ref_unpack(const uint32_t *packed, int64_t rows, int64_t cols,
                   int nbits, int axis, uint8_t *codes);

/* W_hat = fp16_rne((W_q - zero) / scale), fp32 arithmetic */
int hqq_ref_dequantize(const uint32_t *packed, const float *scale, const float *zero,
                       int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                       uint16_t *W_hat);

/* 8-bit min-max RTN of a metadata array in groups of group_size (last one
 * shorter), and its dequantization (quant_scale / quant_zero). */
int hqq_ref_quantize_meta(const float *meta, int64_t n, int group_size,
                          uint8_t *codes, float *mscale, float *mzero);
int hqq_ref_dequantize_meta(const uint8_t *codes, const float *mscale, const float *mzero,
                            int64_t n, int group_size, float *meta);

/* Linear layer on quantized weights (the consumer of the codes: HQQLinear's
 * forward in the lnwmold.com HQQ guide, section 3.2, dequantizes W_q and
 * multiplies in the compute dtype).  W_hat = hqq_ref_dequantize(...) of an
 * axis = 1 weight [N, K]; X is fp16 bits [M, K].  Y[m, n] = sum_k X[m, k] *
 * W_hat[n, k], summed in fp64 in order k = 0..K-1 (Y [M, N] doubles); absY
 * [M, N] (optional) receives sum_k |X[m, k] * W_hat[n, k]| for error bounds.
 * Returns 0 or a negative status as above. */
int hqq_ref_linear(const uint16_t *X, int64_t M, int64_t K,
                   const uint32_t *packed, const float *scale, const float *zero,
                   int64_t N, int nbits, int group_size, double *Y, double *absY);

/* The same in compute dtype fp16 or bf16 (HQQ_REF_F16 / HQQ_REF_BF16): X is
 * given in that dtype and W_hat is the dequantization into it
 * (hqq_ref_dequantize_dt); -8 for another dtype. */
int hqq_ref_linear_dt(const uint16_t *X, int dtype, int64_t M, int64_t K,
                      const uint32_t *packed, const float *scale, const float *zero,
                      int64_t N, int nbits, int group_size, double *Y, double *absY);

#ifdef __cplusplus
}
#endif
#endif
