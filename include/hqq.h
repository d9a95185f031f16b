/*
 * hqq.h -- C ABI of the MI355X (gfx950) HQQ weight-quantization library.
 *
 * HQQ (half-quadratic quantization) quantizes each group of group_size
 * weights of an fp16 Linear weight matrix to nbits-bit integer codes that
 * share one fp32 scale and one fp32 zero point.  It needs no calibration data:
 * the error is split through an auxiliary variable W_e and the zero point is
 * refit by alternating minimisation.
 *   Sources: lnwmold.com HQQ guide, section 2.1 (calibration-free
 *   half-quadratic splitting into alternating sub-problems), section 2.2
 *   (nbits, group_size, axis), section 3.2 (HQQLinear state W_q / scale /
 *   zero, dequantize(), unpack()); devpress.csdn.net "dropbox/hqq" tutorial,
 *   section 2 (auxiliary variable, robust non-convex loss) and section 3.3
 *   (BaseQuantizeConfig).
 *
 * The solve, per group of gs weights w, with b = nbits and qmax = 2^b - 1:
 *   scale = qmax / (max w - min w),  zero = -(min w * scale)
 *   (a constant group has scale = 1, zero = -min w)
 *   repeat iters times, beta starting at beta0:
 *     W_q  = clamp(round_half_even(w * scale + zero), 0, qmax)
 *     W_r  = (W_q - zero) / scale,  x = w - W_r
 *     W_e  = sign(x) * max(|x| - |x|^(p-1) / beta, 0)
 *     zero = mean(W_q - (w - W_e) * scale)
 *     beta = beta * kappa
 *   codes = clamp(round_half_even(w * scale + zero), 0, qmax)
 * Defaults: p = 0.7, beta0 = 10, kappa = 1.01, iters = 20.  The result is
 * bit-for-bit the fp32 evaluation in which w*scale+zero is one fused
 * multiply-add and the mean is (sum W_q - scale*(sum w - sum W_e)) / gs in
 * fp64 (the two first sums exact, sum W_e in ascending element order), then
 * rounded once to fp32.
 *
 * Layout.  W is fp16 (IEEE binary16 bits; the _ex entry points also take
 * bf16), row-major [rows, cols] with rows = out_features and
 * cols = in_features.
 *   axis = 1: a group is group_size consecutive elements of one row
 *             (along in_features, contiguous); scale/zero are [rows, cols/gs].
 *   axis = 0: a group is group_size consecutive rows of one column
 *             (along out_features, strided); scale/zero are [rows/gs, cols].
 * Codes are packed along the group axis: C = 4 (8-bit), 8 (4-bit),
 * 10 (3-bit), 16 (2-bit) or 32 (1-bit) codes per uint32; word k of a line holds the
 * line's codes k*C .. k*C+C-1, code j in bits [j*b, j*b+b) (LSB first); the
 * unused fields of a line's last word, and bits 30-31 of 3-bit words, are 0.
 *   axis = 1: packed is [rows, ceil(cols/C)];  axis = 0: [ceil(rows/C), cols].
 * scale is codes per unit of weight: dequantization divides by it.
 *
 * Conventions for every entry point.
 *   - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *     owned by the caller; arrays of descriptors (the batched calls) and the
 *     weights of hqq_quantize_streamed are host memory, as their entries
 *     say.  The library allocates nothing and keeps no state, so calls are
 *     thread-safe.  Inputs are never written; outputs must not overlap
 *     inputs.  Tensor pointers must be 16-byte aligned unless the entry point
 *     states a weaker requirement (the meta calls).
 *   - stream is a hipStream_t passed as void*; NULL is the null stream.  Calls
 *     only enqueue work: results are ready when the stream reaches them.
 *   - Arguments are validated on the host before any HIP call; on failure
 *     nothing is enqueued and a negative HQQ_E* status is returned.
 *     HQQ_EHIP reports a failed kernel launch.  Contents of W that are NaN or
 *     Inf are a precondition violation and are not checked.
 *   - Supported: nbits in {1,2,3,4,8} (lnwmold.com HQQ guide, section 2.2
 *     lists 8/4/3/2/1 bits); group_size in {8,16,32,64,128,256},
 *     dividing the line length (cols for axis 1, rows for axis 0).
 */
#ifndef HQQ_H
#define HQQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef HQQ_API
#define HQQ_API __attribute__((visibility("default")))
#endif

#define HQQ_OK 0
#define HQQ_EINVAL_NBITS (-1) /* nbits not in {1,2,3,4,8}                            */
#define HQQ_EINVAL_AXIS (-2)  /* axis not in {0,1}                                   */
#define HQQ_EINVAL_GROUP (-3) /* group_size unsupported or not dividing the line     */
#define HQQ_EINVAL_SHAPE (-4) /* rows or cols < 1 or too large, or batch count < 0    */
#define HQQ_EINVAL_PTR (-5)   /* NULL or misaligned pointer                          */
#define HQQ_EINVAL_PARAM (-6) /* iters < 0, or p, beta0, kappa not finite and > 0    */
#define HQQ_EHIP (-7)         /* a HIP launch failed                                  */
#define HQQ_EINVAL_DTYPE (-8) /* dtype not HQQ_DTYPE_FP16 or HQQ_DTYPE_BF16           */
#define HQQ_ESCRATCH (-9)     /* a row block too large for the static staging array   */

/* Element types of 16-bit weight / dequantized tensors (the pages load models
 * in fp16 or bf16 and set compute_dtype to either: devpress.csdn.net tutorial
 * section 5, lnwmold.com HQQ guide sections 3.2 and 6.1). */
#define HQQ_DTYPE_FP16 0
#define HQQ_DTYPE_BF16 1

/* Quantize W with the HQQ solve above (lnwmold.com HQQ guide sections 2.1-2.2;
 * devpress.csdn.net tutorial section 2).
 *   W       fp16 bits [rows, cols], device, read only
 *   packed  uint32, hqq_packed_words(rows, cols, nbits, axis) words, written
 *   scale, zero  fp32, rows*cols/group_size values each, written
 * Returns HQQ_OK or a negative HQQ_E* status. */
HQQ_API int hqq_quantize(const uint16_t *W, int64_t rows, int64_t cols,
                 int nbits, int group_size, int axis,
                 int iters, float p, float beta0, float kappa,
                 uint32_t *packed, float *scale, float *zero, void *stream);

/* One tensor of a batched quantize call (all pointers device, 16-byte aligned;
 * layouts as for hqq_quantize). */
typedef struct hqq_tensor {
    const uint16_t *W;   /* fp16 bits [rows, cols], read only */
    int64_t rows, cols;
    uint32_t *packed;    /* hqq_packed_words(rows, cols, nbits, axis) words, written */
    float *scale;        /* rows*cols/group_size values, written */
    float *zero;         /* rows*cols/group_size values, written */
} hqq_tensor;

/* Quantize n tensors that share one format (nbits, group_size, axis) and one
 * set of solve parameters, with results identical to n hqq_quantize calls.
 * This is the pages' whole-model quantization (lnwmold.com HQQ guide section
 * 3.3, AutoHQQHFModel.quantize_model walks a model's Linear layers) in as few
 * kernel launches as possible: up to 48 tensors per launch (a call with more is
 * cut into launches of as even a size as that allows), so the GPU is not
 * idle between small launches and a wave's tail overlaps other tensors' work.
 *   tensors  HOST array of n descriptors (read during the call only)
 * Every descriptor is validated before anything is enqueued.  n = 0 is a
 * no-op.  Returns HQQ_OK or a negative HQQ_E* status. */
HQQ_API int hqq_quantize_batch(const hqq_tensor *tensors, int n,
                               int nbits, int group_size, int axis,
                               int iters, float p, float beta0, float kappa, void *stream);

/* hqq_quantize_batch for weights of element type wdtype: HQQ_DTYPE_FP16 (the
 * same call) or HQQ_DTYPE_BF16 (W holds bf16 bits; the devpress.csdn.net
 * tutorial's section 5 quantizes a model loaded in bf16).  bf16 widens to
 * fp32 exactly, so every later step is the fp16 path's; the group sum of the
 * mean is formed in fp64 in index order (exact for fp16 in any order, not
 * always for bf16's wider range).  Other wdtype: HQQ_EINVAL_DTYPE. */
HQQ_API int hqq_quantize_batch_ex(const hqq_tensor *tensors, int n, int wdtype,
                                  int nbits, int group_size, int axis,
                                  int iters, float p, float beta0, float kappa, void *stream);

/* Which solve kernel a batched launch runs (host query, no GPU call): for a
 * launch of `work_items` work items of this format (a work item is
 * lcm(group_size, codes per word) elements of one line; for the formats below
 * it is one group), HQQ_MAPPING_LANE: one lane per work item, the whole group
 * in its registers; HQQ_MAPPING_SEG: group_size / 8 lanes per group with 8
 * weights each, for axis 1, 32 <= group_size <= 128, fp16 weights and every
 * width but 3 bits; HQQ_MAPPING_SEG16: group_size / 16 lanes per group with
 * 16 weights each, for the same formats (1-bit codes from group_size 64).
 * The several-lanes kernels are taken for launches too small to fill the
 * device with one lane per group (a threshold per width): SEG16 for 4- and
 * 8-bit codes, SEG for 1 and 2 bits.  All give identical outputs.  The environment variable
 * HQQ_SOLVE_MAPPING=lane, =seg or =seg16, read at each call, forces one
 * (where the format lacks it: one lane per work item).  Invalid arguments: a
 * negative HQQ_E* status. */
#define HQQ_MAPPING_LANE 0
#define HQQ_MAPPING_SEG 1
#define HQQ_MAPPING_SEG16 2
HQQ_API int hqq_solve_mapping(int nbits, int group_size, int axis, int wdtype, int64_t work_items);

/* One tensor of a streamed quantize call: W in HOST memory, outputs on the
 * device (16-byte aligned; layouts as for hqq_quantize). */
typedef struct hqq_host_tensor {
    const uint16_t *W;   /* fp16 bits [rows, cols], host memory (page-locked for
                          * the copies to overlap the solve), read only */
    int64_t rows, cols;
    uint32_t *packed;    /* device, hqq_packed_words(rows, cols, nbits, axis) words, written */
    float *scale;        /* device, rows*cols/group_size values, written */
    float *zero;         /* device, rows*cols/group_size values, written */
} hqq_host_tensor;

/* Quantize weights that live in host memory (lnwmold.com HQQ guide section
 * 6.3: models too large for the device are quantized a batch of layers at a
 * time), with results identical to hqq_quantize on device copies of them.
 * The weights cross PCIe once, in chunks of whole row blocks (whole groups
 * and packed words) that fit half of the caller's device staging buffer:
 * chunk c is copied into half c % 2 on copy_stream while the solve of chunk
 * c - 1 runs on compute_stream.  The first copies wait for the work enqueued
 * on compute_stream before the call, so back-to-back calls may share one
 * staging buffer.  Everything is enqueued asynchronously; the results are
 * complete when compute_stream has finished, and the host weights and the
 * staging buffer must stay untouched until then.
 *   tensors        HOST array of n descriptors (read during the call only)
 *   staging        device buffer, 16-byte aligned, staging_bytes long; each
 *                  half must hold at least one block unit of every tensor
 *                  (lcm(group_size, codes per word) rows for axis 0, up to
 *                  16 rows for axis 1, times cols * 2 bytes), else
 *                  HQQ_EINVAL_SHAPE
 *   copy_stream, compute_stream  HIP streams (may be the same stream)
 * Every descriptor is validated before anything is enqueued.  n = 0 is a
 * no-op.  The call creates five HIP events and releases them before it
 * returns (pending ones when they complete); it allocates no memory. */
HQQ_API int hqq_quantize_streamed(const hqq_host_tensor *tensors, int n,
                                  int nbits, int group_size, int axis,
                                  int iters, float p, float beta0, float kappa,
                                  void *staging, int64_t staging_bytes,
                                  void *copy_stream, void *compute_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * hqq_quantize_streamed through the library's own staging buffer instead of
 * a caller's.  The buffer is a static device array of
 * HQQ_STATIC_STAGING_BYTES on each device the library runs on, held until the
 * process ends; at the first call on a device (with it current) the library
 * looks up the array's address there and creates five HIP events, which it
 * keeps and reuses.  No call allocates device memory.  Every call on a device
 * shares that device's array and events, which keep the last call's contents
 * (nothing needs to start at zero: each byte a solve reads was copied in by
 * the same call): calls that overlap on one device race, so a caller orders
 * them (one compute stream, or the previous call's compute stream completed
 * or waited on).  The first copies wait for the work enqueued on
 * compute_stream before the call, as in hqq_quantize_streamed.  A tensor
 * whose block unit (see hqq_quantize_streamed) exceeds half the array
 * returns HQQ_ESCRATCH before anything is enqueued; other arguments and
 * results as for hqq_quantize_streamed. */
#define HQQ_STATIC_STAGING_BYTES ((int64_t)64 << 20)
HQQ_API int hqq_quantize_streamed_static(const hqq_host_tensor *tensors, int n,
                                         int nbits, int group_size, int axis,
                                         int iters, float p, float beta0, float kappa,
                                         void *copy_stream, void *compute_stream);

/* Dequantize: W_hat = fp16_round_half_even((W_q - zero) / scale) with an
 * IEEE fp32 subtraction and division (lnwmold.com HQQ guide section 3.2,
 * HQQLinear.dequantize()).  W_hat is fp16 bits [rows, cols], written. */
HQQ_API int hqq_dequantize(const uint32_t *packed, const float *scale, const float *zero,
                   int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                   uint16_t *W_hat, void *stream);

/* hqq_dequantize into compute_dtype out_dtype (lnwmold.com HQQ guide section
 * 3.2: dequantize() returns the compute_dtype, fp16 or bf16): W_hat is the
 * same fp32 quotient rounded half to even to fp16 (HQQ_DTYPE_FP16, the same
 * call) or bf16 (HQQ_DTYPE_BF16).  Other out_dtype: HQQ_EINVAL_DTYPE. */
HQQ_API int hqq_dequantize_ex(const uint32_t *packed, const float *scale, const float *zero,
                              int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                              int out_dtype, uint16_t *W_hat, void *stream);

/* Pack uint8 codes [rows, cols] (W's layout; only the low nbits of each byte
 * are used) into the packed layout above (lnwmold.com HQQ guide section 3.2:
 * W_q is stored packed).  group_size is validated as for hqq_quantize but
 * does not change the layout. */
HQQ_API int hqq_pack(const uint8_t *codes, int64_t rows, int64_t cols,
             int nbits, int group_size, int axis, uint32_t *packed, void *stream);

/* Unpack to uint8 codes [rows, cols] (lnwmold.com HQQ guide section 3.2,
 * HQQLinear.unpack(dtype=uint8)). */
HQQ_API int hqq_unpack(const uint32_t *packed, int64_t rows, int64_t cols,
               int nbits, int group_size, int axis, uint8_t *codes, void *stream);

/* Metadata quantization (quant_scale / quant_zero: devpress.csdn.net
 * tutorial section 3.3 and its troubleshooting section -- the scale and zero
 * arrays themselves are quantized at a higher precision such as 8 bits).
 * The n fp32 values of meta (a scale or zero array of hqq_quantize, in its
 * layout, read flat) are cut into groups of group_size consecutive values
 * (the last one may be shorter) and each group is quantized by 8-bit min-max
 * round-to-nearest-even -- the solve at iters = 0:
 *   s = 255 / (max - min) (range 0: s = 1, z = -min), z = -(min * s),
 *   code = clamp(rint(fma(v, s, z)), 0, 255).
 *   meta    fp32 [n], device, read only (4-byte aligned)
 *   codes   uint8 [n], written
 *   mscale, mzero  fp32 [ceil(n / group_size)], written (4-byte aligned)
 * group_size in [1, 1024] (else HQQ_EINVAL_GROUP); n >= 1.  The weight codes
 * are unchanged: a caller that stores quantized meta dequantizes it with
 * hqq_dequantize_meta and passes the result to hqq_dequantize / hqq_linear. */
HQQ_API int hqq_quantize_meta(const float *meta, int64_t n, int group_size, uint8_t *codes,
                              float *mscale, float *mzero, void *stream);

/* meta[i] = (codes[i] - mzero[g]) / mscale[g], g = i / group_size, IEEE fp32;
 * arguments as for hqq_quantize_meta (meta written). */
HQQ_API int hqq_dequantize_meta(const uint8_t *codes, const float *mscale, const float *mzero,
                                int64_t n, int group_size, float *meta, void *stream);

/* One meta array of a batched meta call: the n values of meta and their
 * 8-bit codes and per-group mscale / mzero, as in hqq_quantize_meta (device
 * pointers, 4-byte aligned; codes any alignment). */
typedef struct hqq_meta_tensor {
    float *meta;         /* fp32 [n]: read by the quantize call, written by the dequantize call */
    int64_t n;
    uint8_t *codes;      /* uint8 [n] */
    float *mscale;       /* fp32 [ceil(n / group_size)] */
    float *mzero;        /* fp32 [ceil(n / group_size)] */
} hqq_meta_tensor;

/* hqq_quantize_meta over count arrays that share group_size, with results
 * identical to count single calls.  A model's scale and zero arrays are many
 * and each is small (a 4096 x 4096 layer at group size 64 has 1 MB of each),
 * so one launch per array is dominated by launch latency; here up to 64
 * arrays share a launch (descriptors passed by value, nothing allocated).
 *   items   host array of count descriptors, read during the call only
 * Every descriptor is checked before anything is enqueued (n < 1 or above
 * 2^40: HQQ_EINVAL_SHAPE; a null or misaligned pointer: HQQ_EINVAL_PTR);
 * count = 0 is a no-op, count < 0 HQQ_EINVAL_SHAPE.  Outputs of different
 * items must not overlap each other or any input. */
HQQ_API int hqq_quantize_meta_batch(const hqq_meta_tensor *items, int count, int group_size,
                                    void *stream);

/* hqq_dequantize_meta over count arrays (meta written); arguments and checks
 * as for hqq_quantize_meta_batch. */
HQQ_API int hqq_dequantize_meta_batch(const hqq_meta_tensor *items, int count, int group_size,
                                      void *stream);

/* Linear layer on quantized weights: Y = X . W_hat^T, the quantized layer's
 * forward pass (lnwmold.com HQQ guide section 3.2: the HQQLinear layer is
 * called like the Linear it replaces, computing in compute_dtype = fp16;
 * section 4.1: a backend fuses the dequantization and the matrix product
 * into one kernel, which requires axis = 1).
 *   X       fp16 bits [M, K] row-major, device, read only
 *   packed  the axis = 1 packed codes of W [N, K] (hqq_packed_words(N, K,
 *           nbits, 1) words, as written by hqq_quantize), read only
 *   scale, zero  fp32 [N, K / group_size], read only
 *   Y       fp16 bits [M, N] row-major, written (must not overlap the inputs)
 * W_hat is exactly what hqq_dequantize writes; each output is the fp32 sum
 * of the exact products X[m][k] * W_hat[n][k] (in an unspecified order)
 * rounded to fp16, round-half-even.
 * Supported: nbits in {1, 2, 4, 8} (a packed word holds whole 8-k runs);
 * group_size in {8, ..., 256} dividing K; K a multiple of 32; M, N >= 1;
 * X, the codes and the meta each below 2^31 bytes.
 * All pointers 16-byte aligned.  Invalid arguments return HQQ_EINVAL_* before
 * anything is enqueued (3-bit codes: HQQ_EINVAL_NBITS). */
HQQ_API int hqq_linear(const uint16_t *X, int64_t M, int64_t K,
                       const uint32_t *packed, const float *scale, const float *zero,
                       int64_t N, int nbits, int group_size, uint16_t *Y, void *stream);

/* hqq_linear in compute dtype fp16 or bf16 (HQQ_DTYPE_FP16 / HQQ_DTYPE_BF16;
 * lnwmold.com HQQ guide section 3.2: the layer computes in its
 * compute_dtype): X and Y hold that dtype's bits, W_hat is what
 * hqq_dequantize_ex writes for that dtype (the bf16 rounding of the same
 * fp32 quotient), the products are exact in fp32 and each output is rounded
 * to the dtype once, round-half-even.  Another dtype: HQQ_EINVAL_DTYPE.
 * Otherwise as hqq_linear (which is this call with HQQ_DTYPE_FP16). */
HQQ_API int hqq_linear_ex(const uint16_t *X, int64_t M, int64_t K,
                          const uint32_t *packed, const float *scale, const float *zero,
                          int64_t N, int nbits, int group_size, int dtype, uint16_t *Y,
                          void *stream);

/* One weight of hqq_linear_batch: its axis = 1 packed codes [N, K] and fp32
 * scale, zero [N, K / group_size] (read only), and its output Y [M, N] in the
 * compute dtype (written).  All pointers device, 16-byte aligned. */
typedef struct hqq_linear_weight {
    const uint32_t *packed;
    const float *scale;
    const float *zero;
    int64_t N;
    uint16_t *Y;
} hqq_linear_weight;

/* hqq_linear for count weights that share the input X (the projections of
 * one layer that read the same activations, such as q, k and v, or gate and
 * up), with results identical to count hqq_linear calls: Y_i = X . W_hat_i^T.
 * The weights share K, nbits and group_size; their N differ freely.  Up to 8
 * weights share one kernel launch, so a decode step pays the launch and
 * pipeline fill once per launch instead of once per weight.
 * Checks as for hqq_linear, per weight, before anything is enqueued; count =
 * 0 is a no-op, count < 0 HQQ_EINVAL_SHAPE, ws NULL with count > 0
 * HQQ_EINVAL_PTR.  dtype: the compute dtype of X and the Y, as for
 * hqq_linear_ex.  The Y of different weights must not overlap each other or
 * any input. */
HQQ_API int hqq_linear_batch(const uint16_t *X, int64_t M, int64_t K, const hqq_linear_weight *ws,
                             int count, int nbits, int group_size, int dtype, void *stream);

/* hqq_linear_batch with a caller's device workspace (16-byte aligned,
 * workspace_bytes long; NULL with 0 bytes is hqq_linear_batch).  Two uses,
 * for batches of many rows (prefill chunks, lnwmold.com HQQ guide section
 * 4.2; section 4.1: a backend fuses the dequantization into the product or
 * dequantizes and runs a dense GEMM):
 *  - where the workspace holds the largest weight's W_hat (N x K values of
 *    the compute dtype, rounded up to 256 bytes) and the batch has many rows
 *    (see hqq_linear_route), each weight is dequantized into it exactly as
 *    hqq_dequantize_ex writes W_hat, and one hipBLASLt GEMM with fp32
 *    accumulation forms Y = X . W_hat^T; the rest of the workspace is the
 *    GEMM's.  The first such call on a device creates a hipBLASLt handle and
 *    the call's plan (kept until the process ends; make it outside stream
 *    capture).  Where hipBLASLt offers no algorithm for a shape, the fused
 *    kernels run.
 *  - otherwise the fused kernels run; for output tiles too few to occupy the
 *    device the tiled kernel may split K in 2, 4 or 8 parts: each part's fp32
 *    partial products go to the workspace (splits x M x sum of N floats; the
 *    launcher takes the most splits the workspace holds when its time
 *    estimate is lower) and a second launch adds them in split order in fp32
 *    and rounds each output once to the compute dtype.
 * Either way the results stay within hqq_linear's bound (fp32 sums of the
 * exact products in some order, rounded once) but need not equal
 * hqq_linear_batch's bit for bit.  The environment variable
 * HQQ_LINEAR_PATH=fused or =gemm, read at each call, forces a route (gemm
 * only where the workspace holds W_hat).  The workspace is in use until the
 * stream reaches the end of the call's work.  A misaligned workspace,
 * negative bytes, or bytes with a NULL workspace: HQQ_EINVAL_PTR. */
HQQ_API int hqq_linear_batch_ws(const uint16_t *X, int64_t M, int64_t K, const hqq_linear_weight *ws,
                                int count, int nbits, int group_size, int dtype, void *workspace,
                                int64_t workspace_bytes, void *stream);

/* Which route hqq_linear_batch_ws takes (host query, no GPU call) for M rows,
 * depth K, count weights of at most n_max outputs and a workspace of
 * workspace_bytes: HQQ_ROUTE_GEMM (dequantize, then a hipBLASLt GEMM) where
 * the workspace holds n_max x K 2-byte values rounded up to 256 bytes and
 * M >= 2048, or count = 1, K <= 4096 and M >= 1024 (measured on MI355X at
 * the 7B shapes: there the dense GEMM on W_hat is the faster; below, the
 * fused kernels are as fast or faster), else HQQ_ROUTE_FUSED;
 * HQQ_LINEAR_PATH as for that call.  The call itself still runs the fused
 * kernels where hipBLASLt has no algorithm.  M, K, count or n_max < 1:
 * HQQ_EINVAL_SHAPE; workspace_bytes < 0: HQQ_EINVAL_PTR. */
#define HQQ_ROUTE_FUSED 0
#define HQQ_ROUTE_GEMM 1
HQQ_API int hqq_linear_route(int64_t M, int64_t K, int count, int64_t n_max, int64_t workspace_bytes);

/* Number of uint32 words of the packed layout; a negative HQQ_E* status for
 * invalid arguments.  Host only, no HIP call. */
HQQ_API int64_t hqq_packed_words(int64_t rows, int64_t cols, int nbits, int axis);

/* Static description of a status code.  Host only. */
HQQ_API const char *hqq_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* HQQ_H */
