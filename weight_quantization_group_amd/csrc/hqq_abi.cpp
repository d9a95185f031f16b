// hqq_abi.cpp -- the C ABI of include/hqq.h: argument validation on the host,
// the shrink certificate, and the kernel launches.  No allocation, no state.
#include "hqq.h"
#include "hqq_internal.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace {

constexpr int kMaxIters = 1 << 16;
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;

int check_common(int64_t rows, int64_t cols, int nbits, int group_size, int axis)
{
    if (!hqq::valid_nbits(nbits))
        return HQQ_EINVAL_NBITS;
    if (axis != 0 && axis != 1)
        return HQQ_EINVAL_AXIS;
    if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems)
        return HQQ_EINVAL_SHAPE;
    switch (group_size) {
    case 8: case 16: case 32: case 64: case 128: case 256: break;
    default: return HQQ_EINVAL_GROUP;
    }
    const int64_t line = axis == 1 ? cols : rows;
    if (line % group_size != 0)
        return HQQ_EINVAL_GROUP;
    return HQQ_OK;
}

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

bool finite_pos(float v) { return isfinite(v) && v > 0.0f; }

// HQQ_SOLVE_MAPPING=lane, =seg or =seg16 forces the solve's mapping where
// the format allows it (tests exercise each on the same inputs); otherwise the
// size of the launch decides.  -1: automatic, else the forced SolveMapping.
int mapping_override()
{
    const char *e = getenv("HQQ_SOLVE_MAPPING");
    if (!e)
        return -1;
    if (strcmp(e, "lane") == 0)
        return hqq::kMapLane;
    if (strcmp(e, "seg") == 0)
        return hqq::kMapSeg;
    if (strcmp(e, "seg16") == 0)
        return hqq::kMapSeg16;
    return -1;
}

// The solve's mapping for a launch of `items` work items of this format: one
// lane per work item from seg_max_items groups; below it 16 weights per lane
// for 4- and 8-bit codes and 8 for 1- and 2-bit codes (measured on lone
// tensors: 16 per lane halves the per-group work per weight, but low widths
// freeze many groups, whose exact finish runs a few groups at a time per wave,
// so they gain more from more, smaller waves).  A forced mapping the format
// lacks falls back to one lane per work item.
int pick_mapping(int nbits, int gs, int axis, bool bf16, int64_t items)
{
    const bool seg_ok = hqq::seg_format(nbits, gs, axis, bf16);
    const bool seg16_ok = hqq::seg16_format(nbits, gs, axis, bf16);
    const int force = mapping_override();
    if (force == hqq::kMapSeg)
        return seg_ok ? hqq::kMapSeg : hqq::kMapLane;
    if (force == hqq::kMapSeg16)
        return seg16_ok ? hqq::kMapSeg16 : hqq::kMapLane;
    if (force == hqq::kMapLane || !seg_ok || items >= hqq::seg_max_items(nbits))
        return hqq::kMapLane;
    return seg16_ok && nbits >= 4 ? hqq::kMapSeg16 : hqq::kMapSeg;
}

// Threshold below which the lp shrinkage is provably inactive in every
// iteration.  The shrink is nonzero iff |x|^(1-pm1) > 1/beta_k, i.e.
// |x| > tau_k = beta_k^(-1/(1-pm1)) when 1 - pm1 > 0; beta_k is the fp32
// sequence beta0 * kappa * ... * kappa exactly as the kernel forms it.  The
// returned thr is 2% below min_k tau_k; 0 disables the certificate (p - 1
// close to or above 1, where no such threshold exists).
void certificate(int iters, float pm1, float beta0, float kappa, float *thr, float *thr_m)
{
    *thr = 0.0f;
    *thr_m = 0.0f;
    const double ex = 1.0 - (double)pm1;
    if (iters == 0 || !(ex > 0.01))
        return;
    double tau_min = INFINITY;
    float b = beta0;
    for (int k = 0; k < iters; ++k) {
        const double tau = pow((double)b, -1.0 / ex);
        if (tau < tau_min)
            tau_min = tau;
        b = b * kappa;
    }
    const double t = 0.98 * tau_min;
    float f = (float)t;
    if ((double)f > t)
        f = nextafterf(f, 0.0f);
    if (!(f > 0.0f))
        return;
    *thr = f;
    *thr_m = f * 2048.0f;
}

}  // namespace

namespace hqq {

int check_params(int iters, float p, float beta0, float kappa)
{
    if (iters < 0 || iters > kMaxIters || !finite_pos(p) || !finite_pos(beta0) || !finite_pos(kappa))
        return HQQ_EINVAL_PARAM;
    return HQQ_OK;
}

int check_tensor(const hqq_tensor &t, int nbits, int group_size, int axis)
{
    const int st = check_common(t.rows, t.cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!aligned16(t.W) || !aligned16(t.packed) || !aligned16(t.scale) || !aligned16(t.zero))
        return HQQ_EINVAL_PTR;
    return HQQ_OK;
}

}  // namespace hqq

namespace {

// Workgroups of one meta array in the quantize or the dequantize grid.
int64_t meta_blocks(int64_t n, int gs, bool quant)
{
    if (quant) {
        const int gpb = hqq::meta_groups_per_block(gs);
        return ((n + gs - 1) / gs + gpb - 1) / gpb;
    }
    return (n + hqq::kMetaDequantBlock - 1) / hqq::kMetaDequantBlock;
}

// The meta calls: every descriptor checked, then launches of up to
// kMetaBatch arrays whose grid stays below 2^31 workgroups.
int meta_batch(const hqq_meta_tensor *items, int count, int gs, bool quant, void *stream)
{
    if (count < 0)
        return HQQ_EINVAL_SHAPE;
    if (count > 0 && !items)
        return HQQ_EINVAL_PTR;
    if (gs < 1 || gs > 1024)
        return HQQ_EINVAL_GROUP;
    const int64_t kMaxGrid = 0x7fffffff;
    for (int i = 0; i < count; ++i) {
        const hqq_meta_tensor &t = items[i];
        if (t.n < 1 || t.n > kMaxElems || meta_blocks(t.n, gs, quant) > kMaxGrid)
            return HQQ_EINVAL_SHAPE;
        if (!t.meta || !t.codes || !t.mscale || !t.mzero || ((uintptr_t)t.meta & 3u) ||
            ((uintptr_t)t.mscale & 3u) || ((uintptr_t)t.mzero & 3u))
            return HQQ_EINVAL_PTR;
    }
    hqq::MetaBatch b{};
    int64_t blocks = 0;
    auto flush = [&]() {
        const hipError_t e = quant ? hqq::launch_quantize_meta(b, gs, (hipStream_t)stream)
                                   : hqq::launch_dequantize_meta(b, gs, (hipStream_t)stream);
        b.count = 0;
        blocks = 0;
        return e == hipSuccess ? HQQ_OK : HQQ_EHIP;
    };
    for (int i = 0; i < count; ++i) {
        const hqq_meta_tensor &t = items[i];
        const int64_t nb = meta_blocks(t.n, gs, quant);
        if (b.count == hqq::kMetaBatch || blocks + nb > kMaxGrid)
            if (const int st = flush())
                return st;
        b.meta[b.count] = t.meta;
        b.n[b.count] = t.n;
        b.codes[b.count] = t.codes;
        b.mscale[b.count] = t.mscale;
        b.mzero[b.count] = t.mzero;
        ++b.count;
        blocks += nb;
    }
    return b.count ? flush() : HQQ_OK;
}

}  // namespace

extern "C" {

int64_t hqq_packed_words(int64_t rows, int64_t cols, int nbits, int axis)
{
    if (!hqq::valid_nbits(nbits))
        return HQQ_EINVAL_NBITS;
    if (axis != 0 && axis != 1)
        return HQQ_EINVAL_AXIS;
    if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems)
        return HQQ_EINVAL_SHAPE;
    const int64_t C = hqq::codes_per_word(nbits);
    return axis == 1 ? rows * ((cols + C - 1) / C) : ((rows + C - 1) / C) * cols;
}

const char *hqq_strerror(int status)
{
    switch (status) {
    case HQQ_OK: return "ok";
    case HQQ_EINVAL_NBITS: return "nbits must be 1, 2, 3, 4 or 8";
    case HQQ_EINVAL_AXIS: return "axis must be 0 or 1";
    case HQQ_EINVAL_GROUP: return "group_size must be 8, 16, 32, 64, 128 or 256 and divide the line length";
    case HQQ_EINVAL_SHAPE: return "rows and cols must be >= 1 (and rows, cols <= 2^31, rows*cols <= 2^40)";
    case HQQ_EINVAL_PTR: return "a pointer is NULL or not 16-byte aligned";
    case HQQ_EINVAL_PARAM: return "iters must be in [0, 65536] and p, beta0, kappa finite and > 0";
    case HQQ_EHIP: return "a HIP kernel launch failed";
    case HQQ_EINVAL_DTYPE: return "dtype must be HQQ_DTYPE_FP16 or HQQ_DTYPE_BF16";
    case HQQ_ESCRATCH: return "a tensor's row block does not fit half of the static staging array (HQQ_STATIC_STAGING_BYTES)";
    default: return "unknown status";
    }
}

int hqq_quantize_batch(const hqq_tensor *tensors, int n, int nbits, int group_size, int axis,
                       int iters, float p, float beta0, float kappa, void *stream)
{
    return hqq_quantize_batch_ex(tensors, n, HQQ_DTYPE_FP16, nbits, group_size, axis, iters, p, beta0,
                                 kappa, stream);
}

int hqq_quantize_batch_ex(const hqq_tensor *tensors, int n, int wdtype, int nbits, int group_size,
                          int axis, int iters, float p, float beta0, float kappa, void *stream)
{
    if (wdtype != HQQ_DTYPE_FP16 && wdtype != HQQ_DTYPE_BF16)
        return HQQ_EINVAL_DTYPE;
    if (n < 0)
        return HQQ_EINVAL_SHAPE;
    if (n > 0 && !tensors)
        return HQQ_EINVAL_PTR;
    if (const int st = hqq::check_params(iters, p, beta0, kappa))
        return st;
    for (int i = 0; i < n; ++i)
        if (const int st = hqq::check_tensor(tensors[i], nbits, group_size, axis))
            return st;
    if (n == 0)
        return HQQ_OK;

    hqq::SolveArgs a{};
    a.iters = iters;
    a.pm1 = p - 1.0f;
    a.beta0 = beta0;
    a.kappa = kappa;
    certificate(iters, a.pm1, beta0, kappa, &a.thr, &a.thr_m);
    const int C = hqq::codes_per_word(nbits);
    const int64_t lb = hqq::lcm_c(group_size, C);
    const int64_t kMaxBlocks = (int64_t(1) << 31) - 1;
    // launches of as even a number of tensors as kMaxBatch allows
    const int launches = (n + hqq::kMaxBatch - 1) / hqq::kMaxBatch;
    const int per_launch = (n + launches - 1) / launches;
    int i = 0;
    while (i < n) {
        // the tensors of this launch, and its work items
        a.n = 0;
        int64_t items = 0;
        while (i + a.n < n && a.n < per_launch) {
            const hqq_tensor &t = tensors[i + a.n];
            hqq::SolveTensor &d = a.t[a.n];
            const int64_t L = axis == 1 ? t.cols : t.rows;
            d.W = t.W;
            d.packed = t.packed;
            d.scale = t.scale;
            d.zero = t.zero;
            d.rows = t.rows;
            d.cols = t.cols;
            d.nblk = (L + lb - 1) / lb;
            d.n_items = d.nblk * (axis == 1 ? t.rows : t.cols);
            d.rdiv = 1.0 / (double)(axis == 1 ? d.nblk : t.cols);
            items += d.n_items;
            ++a.n;
        }
        // the mapping: one lane per work item, or several lanes per group
        // (8 or 16 weights each) for launches too small to fill the device
        // that way
        const int map = pick_mapping(nbits, group_size, axis, wdtype == HQQ_DTYPE_BF16, items);
        // work items per workgroup at depth 1 (one item per lane, or
        // seg_groups_per_wave groups per wave)
        const int64_t unit = map != hqq::kMapLane
                                 ? (int64_t)(hqq::kSolveBlock / 64) * hqq::seg_groups_per_wave(group_size, map)
                                 : (int64_t)hqq::kSolveBlock;
        // items per lane (or per wave's group slot): deep enough to overlap
        // each item's loads with the previous item's solve, shallow enough
        // to keep many workgroups
        int64_t depth = items / (unit * hqq::kTargetBlocks);
        a.depth = (int)(depth < 1 ? 1 : depth > hqq::kMaxDepth ? hqq::kMaxDepth : depth);
        const int64_t per_block = unit * a.depth;
        a.blocks = 0;
        int used = 0;
        for (; used < a.n; ++used) {
            const int64_t nb = (a.t[used].n_items + per_block - 1) / per_block;
            if (used > 0 && a.blocks + nb > kMaxBlocks)
                break;
            a.block0[used] = a.blocks;
            a.blocks += nb;
        }
        a.n = used;
        i += used;
        const hipError_t e = hqq::launch_solve(nbits, group_size, axis, wdtype == HQQ_DTYPE_BF16, map, a,
                                               (hipStream_t)stream);
        if (e != hipSuccess)
            return HQQ_EHIP;
    }
    return HQQ_OK;
}

int hqq_solve_mapping(int nbits, int group_size, int axis, int wdtype, int64_t work_items)
{
    if (wdtype != HQQ_DTYPE_FP16 && wdtype != HQQ_DTYPE_BF16)
        return HQQ_EINVAL_DTYPE;
    if (!hqq::valid_nbits(nbits))
        return HQQ_EINVAL_NBITS;
    if (axis != 0 && axis != 1)
        return HQQ_EINVAL_AXIS;
    if (group_size != 8 && group_size != 16 && group_size != 32 && group_size != 64 && group_size != 128 &&
        group_size != 256)
        return HQQ_EINVAL_GROUP;
    if (work_items < 0)
        return HQQ_EINVAL_SHAPE;
    switch (pick_mapping(nbits, group_size, axis, wdtype == HQQ_DTYPE_BF16, work_items)) {
    case hqq::kMapSeg: return HQQ_MAPPING_SEG;
    case hqq::kMapSeg16: return HQQ_MAPPING_SEG16;
    default: return HQQ_MAPPING_LANE;
    }
}

int hqq_quantize(const uint16_t *W, int64_t rows, int64_t cols, int nbits, int group_size,
                 int axis, int iters, float p, float beta0, float kappa, uint32_t *packed,
                 float *scale, float *zero, void *stream)
{
    const hqq_tensor t{W, rows, cols, packed, scale, zero};
    return hqq_quantize_batch(&t, 1, nbits, group_size, axis, iters, p, beta0, kappa, stream);
}

int hqq_dequantize(const uint32_t *packed, const float *scale, const float *zero, int64_t rows,
                   int64_t cols, int nbits, int group_size, int axis, uint16_t *W_hat, void *stream)
{
    return hqq_dequantize_ex(packed, scale, zero, rows, cols, nbits, group_size, axis, HQQ_DTYPE_FP16,
                             W_hat, stream);
}

int hqq_dequantize_ex(const uint32_t *packed, const float *scale, const float *zero, int64_t rows,
                      int64_t cols, int nbits, int group_size, int axis, int out_dtype, uint16_t *W_hat,
                      void *stream)
{
    if (out_dtype != HQQ_DTYPE_FP16 && out_dtype != HQQ_DTYPE_BF16)
        return HQQ_EINVAL_DTYPE;
    int st = check_common(rows, cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!aligned16(packed) || !aligned16(scale) || !aligned16(zero) || !aligned16(W_hat))
        return HQQ_EINVAL_PTR;
    hqq::CodecArgs a{};
    a.packed_in = packed;
    a.scale = scale;
    a.zero = zero;
    a.W_hat = W_hat;
    a.out_bf16 = out_dtype == HQQ_DTYPE_BF16;
    a.rows = rows;
    a.cols = cols;
    a.group_size = group_size;
    a.n_words = hqq_packed_words(rows, cols, nbits, axis);
    const hipError_t e = hqq::launch_dequantize(nbits, axis, a, (hipStream_t)stream);
    return e == hipSuccess ? HQQ_OK : HQQ_EHIP;
}

int hqq_pack(const uint8_t *codes, int64_t rows, int64_t cols, int nbits, int group_size, int axis,
             uint32_t *packed, void *stream)
{
    int st = check_common(rows, cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!aligned16(codes) || !aligned16(packed))
        return HQQ_EINVAL_PTR;
    hqq::CodecArgs a{};
    a.codes_in = codes;
    a.packed_out = packed;
    a.rows = rows;
    a.cols = cols;
    a.group_size = group_size;
    a.n_words = hqq_packed_words(rows, cols, nbits, axis);
    const hipError_t e = hqq::launch_pack(nbits, axis, a, (hipStream_t)stream);
    return e == hipSuccess ? HQQ_OK : HQQ_EHIP;
}

int hqq_unpack(const uint32_t *packed, int64_t rows, int64_t cols, int nbits, int group_size,
               int axis, uint8_t *codes, void *stream)
{
    int st = check_common(rows, cols, nbits, group_size, axis);
    if (st)
        return st;
    if (!aligned16(packed) || !aligned16(codes))
        return HQQ_EINVAL_PTR;
    hqq::CodecArgs a{};
    a.packed_in = packed;
    a.codes_out = codes;
    a.rows = rows;
    a.cols = cols;
    a.group_size = group_size;
    a.n_words = hqq_packed_words(rows, cols, nbits, axis);
    const hipError_t e = hqq::launch_unpack(nbits, axis, a, (hipStream_t)stream);
    return e == hipSuccess ? HQQ_OK : HQQ_EHIP;
}

int hqq_linear_batch(const uint16_t *X, int64_t M, int64_t K, const hqq_linear_weight *ws, int count,
                     int nbits, int group_size, int dtype, void *stream)
{
    return hqq_linear_batch_ws(X, M, K, ws, count, nbits, group_size, dtype, nullptr, 0, stream);
}

namespace {

// The linear layer's two routes: the fused kernels, or, where the caller's
// workspace holds the largest weight's W_hat (fp16 or bf16 [N, K], rounded up
// to 256 bytes), each weight dequantized into it and multiplied by one
// hipBLASLt GEMM (the rest of the workspace is the GEMM's).  Measured on
// MI355X (4-bit g64, the 7B shapes, graph-replayed calls), dequantize + GEMM
// is the faster route for every call from kGemmMinRows rows (one weight or a
// q/k/v or gate/up batch), and for one weight with K <= 4096 from
// kGemmMinRowsOne rows; below, the fused kernels (whose tiles span all weights
// of a batch) are as fast or faster.  HQQ_LINEAR_PATH=fused or =gemm forces a
// route (gemm only where the workspace allows it; tests run both on the same
// inputs).
constexpr int64_t kGemmMinRows = 2048;
constexpr int64_t kGemmMinRowsOne = 1024;

int64_t what_bytes(int64_t n_max, int64_t K) { return (n_max * K * 2 + 255) / 256 * 256; }

bool use_gemm_route(int64_t M, int64_t K, int count, int64_t n_max, const void *workspace, int64_t workspace_bytes)
{
    if (!workspace || workspace_bytes < what_bytes(n_max, K))
        return false;
    const char *e = getenv("HQQ_LINEAR_PATH");
    if (e && strcmp(e, "fused") == 0)
        return false;
    if (e && strcmp(e, "gemm") == 0)
        return true;
    return M >= kGemmMinRows || (count == 1 && K <= 4096 && M >= kGemmMinRowsOne);
}

}  // namespace

int hqq_linear_batch_ws(const uint16_t *X, int64_t M, int64_t K, const hqq_linear_weight *ws, int count,
                        int nbits, int group_size, int dtype, void *workspace, int64_t workspace_bytes,
                        void *stream)
{
    if (!hqq::valid_nbits(nbits) || nbits == 3)
        return HQQ_EINVAL_NBITS;
    if (dtype != HQQ_DTYPE_FP16 && dtype != HQQ_DTYPE_BF16)
        return HQQ_EINVAL_DTYPE;
    if (count < 0)
        return HQQ_EINVAL_SHAPE;
    if (count > 0 && !ws)
        return HQQ_EINVAL_PTR;
    if (M < 1 || K < 32 || K % 32 != 0 || M > kMaxDim || K > kMaxDim || M * K > kMaxElems)
        return HQQ_EINVAL_SHAPE;
    // gridDim.y = ceil(M / 32) must fit the launch limits, and the kernels
    // address X, the codes and the meta with 32-bit byte offsets
    const int64_t kMaxBytes = int64_t(1) << 31;
    if ((M + 31) / 32 > 0xffff || M * K * 2 >= kMaxBytes)
        return HQQ_EINVAL_SHAPE;
    for (int i = 0; i < count; ++i) {
        const int64_t N = ws[i].N;
        if (N < 1 || N > kMaxDim || N * K > kMaxElems || M * N > kMaxElems ||
            N * (K * nbits / 32) * 4 >= kMaxBytes || N * (K / 8) * 4 >= kMaxBytes)
            return HQQ_EINVAL_SHAPE;
    }
    int gshift = -1;
    for (int b = 3; b <= 8; ++b)
        if (group_size == (1 << b))
            gshift = b;
    if (gshift < 0 || K % group_size != 0)
        return HQQ_EINVAL_GROUP;
    if (!aligned16(X))
        return HQQ_EINVAL_PTR;
    for (int i = 0; i < count; ++i)
        if (!aligned16(ws[i].packed) || !aligned16(ws[i].scale) || !aligned16(ws[i].zero) ||
            !aligned16(ws[i].Y))
            return HQQ_EINVAL_PTR;
    if (workspace_bytes < 0 || (workspace && !aligned16(workspace)) || (!workspace && workspace_bytes > 0))
        return HQQ_EINVAL_PTR;
    const bool bf16 = dtype == HQQ_DTYPE_BF16;
    int64_t n_max = 0;
    for (int i = 0; i < count; ++i)
        n_max = ws[i].N > n_max ? ws[i].N : n_max;
    if (count > 0 && use_gemm_route(M, K, count, n_max, workspace, workspace_bytes)) {
        const int64_t wb = what_bytes(n_max, K);
        uint16_t *W_hat = reinterpret_cast<uint16_t *>(workspace);
        char *rest = reinterpret_cast<char *>(workspace) + wb;
        const size_t rest_bytes = (size_t)(workspace_bytes - wb);
        bool ok = true;
        for (int i = 0; i < count && ok; ++i)
            ok = hqq::gemm_available(M, ws[i].N, K, bf16, rest_bytes);
        if (ok) {
            for (int i = 0; i < count; ++i) {
                hqq::CodecArgs ca{};
                ca.packed_in = ws[i].packed;
                ca.scale = ws[i].scale;
                ca.zero = ws[i].zero;
                ca.W_hat = W_hat;
                ca.out_bf16 = bf16;
                ca.rows = ws[i].N;
                ca.cols = K;
                ca.group_size = group_size;
                ca.n_words = hqq_packed_words(ws[i].N, K, nbits, 1);
                if (hqq::launch_dequantize(nbits, 1, ca, (hipStream_t)stream) != hipSuccess ||
                    hqq::gemm_xwt(X, W_hat, ws[i].Y, M, ws[i].N, K, bf16, rest_bytes ? rest : nullptr, rest_bytes,
                                  (hipStream_t)stream) != hipSuccess)
                    return HQQ_EHIP;
            }
            return HQQ_OK;
        }
    }
    hqq::LinearBatch b{};
    b.work = reinterpret_cast<float *>(workspace);
    b.work_floats = workspace ? workspace_bytes / 4 : 0;
    b.a.X = X;
    b.a.M = M;
    b.a.K = K;
    b.a.wpr = K * nbits / 32;
    b.a.gpl = K / group_size;
    b.a.gs = group_size;
    b.a.gshift = gshift;
    // up to kLinBatch weights per launch (at most 8 x 2^27 column tiles: the
    // grid's x dimension stays below 2^31)
    for (int i0 = 0; i0 < count; i0 += hqq::kLinBatch) {
        b.count = count - i0 < hqq::kLinBatch ? count - i0 : hqq::kLinBatch;
        for (int j = 0; j < b.count; ++j) {
            const hqq_linear_weight &w = ws[i0 + j];
            b.packed[j] = w.packed;
            b.scale[j] = w.scale;
            b.zero[j] = w.zero;
            b.Y[j] = w.Y;
            b.N[j] = w.N;
        }
        if (hqq::launch_linear(nbits, dtype == HQQ_DTYPE_BF16, b, (hipStream_t)stream) != hipSuccess)
            return HQQ_EHIP;
    }
    return HQQ_OK;
}

int hqq_linear_route(int64_t M, int64_t K, int count, int64_t n_max, int64_t workspace_bytes)
{
    if (M < 1 || K < 1 || count < 1 || n_max < 1)
        return HQQ_EINVAL_SHAPE;
    if (workspace_bytes < 0)
        return HQQ_EINVAL_PTR;
    // the rule looks at the workspace's size only; any non-null stands in
    static const char stand_in = 0;
    return use_gemm_route(M, K, count, n_max, workspace_bytes ? &stand_in : nullptr, workspace_bytes)
               ? HQQ_ROUTE_GEMM
               : HQQ_ROUTE_FUSED;
}

int hqq_linear_ex(const uint16_t *X, int64_t M, int64_t K, const uint32_t *packed,
                  const float *scale, const float *zero, int64_t N, int nbits, int group_size,
                  int dtype, uint16_t *Y, void *stream)
{
    // null or misaligned pointers are rejected by the batch's alignment check
    const hqq_linear_weight w{packed, scale, zero, N, Y};
    return hqq_linear_batch(X, M, K, &w, 1, nbits, group_size, dtype, stream);
}

int hqq_linear(const uint16_t *X, int64_t M, int64_t K, const uint32_t *packed,
               const float *scale, const float *zero, int64_t N, int nbits, int group_size,
               uint16_t *Y, void *stream)
{
    return hqq_linear_ex(X, M, K, packed, scale, zero, N, nbits, group_size, HQQ_DTYPE_FP16, Y, stream);
}

int hqq_quantize_meta(const float *meta, int64_t n, int group_size, uint8_t *codes, float *mscale,
                      float *mzero, void *stream)
{
    if (n < 1 || n > kMaxElems)
        return HQQ_EINVAL_SHAPE;
    if (group_size < 1 || group_size > 1024)
        return HQQ_EINVAL_GROUP;
    const hqq_meta_tensor t{const_cast<float *>(meta), n, codes, mscale, mzero};
    return meta_batch(&t, 1, group_size, true, stream);
}

int hqq_dequantize_meta(const uint8_t *codes, const float *mscale, const float *mzero, int64_t n,
                        int group_size, float *meta, void *stream)
{
    if (n < 1 || n > kMaxElems)
        return HQQ_EINVAL_SHAPE;
    if (group_size < 1 || group_size > 1024)
        return HQQ_EINVAL_GROUP;
    const hqq_meta_tensor t{meta, n, const_cast<uint8_t *>(codes), const_cast<float *>(mscale),
                            const_cast<float *>(mzero)};
    return meta_batch(&t, 1, group_size, false, stream);
}

int hqq_quantize_meta_batch(const hqq_meta_tensor *items, int count, int group_size, void *stream)
{
    return meta_batch(items, count, group_size, true, stream);
}

int hqq_dequantize_meta_batch(const hqq_meta_tensor *items, int count, int group_size, void *stream)
{
    return meta_batch(items, count, group_size, false, stream);
}

}  // extern "C"
