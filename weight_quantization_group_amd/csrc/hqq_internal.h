// hqq_internal.h -- declarations shared by the library's own translation units.
#pragma once

#include "hqq.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

constexpr int codes_per_word(int nb) { return nb == 8 ? 4 : nb == 4 ? 8 : nb == 3 ? 10 : nb == 2 ? 16 : 32; }
constexpr bool valid_nbits(int nb) { return nb == 1 || nb == 2 || nb == 3 || nb == 4 || nb == 8; }
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// One tensor of a solve launch.
struct SolveTensor {
    const uint16_t *W;   // fp16 bits [rows, cols]
    uint32_t *packed;    // packed codes
    float *scale;        // per-group scale
    float *zero;         // per-group zero
    int64_t rows, cols;
    int64_t n_items;     // work items: one block of lcm(gs, C) elements of one line
    int64_t nblk;        // work items per line
    double rdiv;         // 1 / (axis 1: nblk, axis 0: cols), for the item -> (line, block) split
};

// Up to this many same-format tensors share one launch (kernel-argument size:
// SolveArgs stays within 4 KiB).  Fewer, larger launches leave fewer
// partially filled ends of a launch: on the 7B stack 48 tensors per launch
// ran 5.3% faster than 24.
constexpr int kMaxBatch = 48;
// Threads per workgroup of the solve kernels.
constexpr int kSolveBlock = 256;
// A workgroup solves depth * kSolveBlock work items (depth steps per lane);
// the host picks depth so that a launch still has about kTargetBlocks
// workgroups.  Deeper workgroups overlap more loads with solves but end a
// launch more raggedly: on the 7B stack's 44-tensor launches depth 4 ran 2%
// faster than 8, and 2 ran 0.7% slower than 4; depth 1 cost 6% on one 7B
// layer at 2 bits (axis 0).
constexpr int kMaxDepth = 4;
constexpr int64_t kTargetBlocks = 16384;

// The axis = 1 solve can also spread a group over several lanes: gs / 8 lanes
// with 8 weights each (kMapSeg, 512 / gs groups per wave) or gs / 16 lanes with
// 16 (kMapSeg16, 1024 / gs groups per wave): formats 32 <= gs <= 128, fp16
// weights, every code width but 3 bits (16 per lane: 1-bit codes from gs = 64).
// The host takes them for launches of fewer than seg_max_items groups
// (measured crossovers; 16 per lane for 4- and 8-bit codes, 8 for 1 and 2
// bits): below them one lane per group leaves most of the device idle and a
// wave waits for the slowest of its 64 groups.  1-bit groups
// often need the exact finish, which runs up to 64 / gs groups at a time per
// wave: many more waves win there at every size measured.
enum SolveMapping { kMapLane = 0, kMapSeg = 1, kMapSeg16 = 2 };
constexpr bool seg_format(int nbits, int gs, int axis, bool bf16)
{
    return axis == 1 && !bf16 && nbits != 3 && gs >= 32 && gs <= 128;
}
constexpr bool seg16_format(int nbits, int gs, int axis, bool bf16)
{
    return seg_format(nbits, gs, axis, bf16) && (nbits != 1 || gs >= 64);
}
constexpr int seg_groups_per_wave(int gs, int map) { return (map == kMapSeg16 ? 1024 : 512) / gs; }
constexpr int64_t seg_max_items(int nbits)
{
    // (4 bits: a lone 4096 x 1024 g64 tensor, 64 K groups, 12.3 us with 16
    // weights per lane against 16.4 with one lane per group; 4096 x 4096 g128,
    // 128 K groups, 29.9 us with one lane per group against 33.5)
    return nbits == 1   ? (int64_t(1) << 23)
           : nbits == 8 ? (int64_t(1) << 16)
           : nbits == 4 ? int64_t(96) << 10
                        : int64_t(320) << 10;
}

// Arguments of the solve kernels (passed by value as the kernel argument).
struct SolveArgs {
    int iters;
    float pm1;           // p - 1 (fp32)
    float beta0, kappa;
    // Shrink certificate: W_e is provably 0 for every residual |x| <= thr in
    // every iteration (thr = 0: no certificate).  thr_m bounds the group
    // magnitude for which the cheap residual estimate |t - q| / scale is
    // accurate enough to use it.
    float thr, thr_m;
    int n;               // tensors in this launch
    int depth;           // work items per lane
    int64_t blocks;      // workgroups of the launch
    int64_t block0[kMaxBatch];   // first workgroup of each tensor (increasing)
    SolveTensor t[kMaxBatch];
};
static_assert(sizeof(SolveArgs) <= 4096, "solve kernel arguments within 4 KiB");

struct CodecArgs {
    const uint32_t *packed_in;
    uint32_t *packed_out;
    const uint8_t *codes_in;
    uint8_t *codes_out;
    const float *scale;
    const float *zero;
    uint16_t *W_hat;     // fp16 or (out_bf16) bf16 bits
    int64_t rows, cols;
    int group_size;
    int64_t n_words;
    int out_bf16;
};

// Arguments of the fused dequantize + matmul kernels: Y[M, N] = X[M, K] .
// W_hat[N, K]^T with W in the axis = 1 packed layout.
struct LinearArgs {
    const uint16_t *X;       // fp16 (or bf16) bits [M, K]
    const uint32_t *packed;  // [N, wpr] words
    const float *scale;      // [N, gpl]
    const float *zero;       // [N, gpl]
    uint16_t *Y;             // fp16 (or bf16) bits [M, N]
    int64_t M, N, K;
    int64_t wpr;             // words per row of W: K * nbits / 32
    int64_t gpl;             // groups per row of W: K / gs
    int gs, gshift;          // group size and its log2
    float *part;             // split K: fp32 partial sums [splits, M, N], else null
};

// Several weights that share X (and K and the code format) in one launch:
// weight j's column tiles are grid columns tile0[j] .. tile0[j + 1] - 1.
constexpr int kLinBatch = 8;
struct LinearBatch {
    LinearArgs a;    // X, M, K, wpr, gpl, gs, gshift (its per-weight fields unused)
    int count;
    uint32_t tile0[kLinBatch + 1];   // filled by the launcher
    const uint32_t *packed[kLinBatch];
    const float *scale[kLinBatch];
    const float *zero[kLinBatch];
    uint16_t *Y[kLinBatch];
    int64_t N[kLinBatch];
    // split K (tiled kernel): a caller's workspace of work_floats fp32 values;
    // the launcher sets splits and part[j] (weight j's [splits, M, N] slice)
    float *work;
    int64_t work_floats;
    int splits;
    float *part[kLinBatch];
    uint32_t rblock0[kLinBatch + 1];   // reduction workgroups of each weight
};

// host-side argument checks shared by the entry points (HQQ_* status)
int check_params(int iters, float p, float beta0, float kappa);
int check_tensor(const ::hqq_tensor &t, int nbits, int group_size, int axis);

// launchers (return hipError_t of the launch)
// map: kMapLane, or a several-lanes-per-group kernel (kMapSeg for a format
// seg_format accepts, kMapSeg16 for one seg16_format accepts)
hipError_t launch_solve(int nbits, int group_size, int axis, bool bf16, int map, const SolveArgs &a,
                        hipStream_t s);
hipError_t launch_dequantize(int nbits, int axis, const CodecArgs &a, hipStream_t s);
hipError_t launch_pack(int nbits, int axis, const CodecArgs &a, hipStream_t s);
hipError_t launch_unpack(int nbits, int axis, const CodecArgs &a, hipStream_t s);
hipError_t launch_linear(int nbits, bool bf16, LinearBatch &b, hipStream_t s);
// Y [M, N] = X [M, K] . W [N, K]^T, row-major fp16 (or bf16) through hipBLASLt;
// ws: workspace the library's algorithm may use (hqq_gemm.cpp).  gemm_available:
// whether hipBLASLt has an algorithm for the shape within ws_bytes.
bool gemm_available(int64_t M, int64_t N, int64_t K, bool bf16, size_t ws_bytes);
hipError_t gemm_xwt(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, bool bf16,
                    void *ws, size_t ws_bytes, hipStream_t s);
// meta arrays per launch of the meta kernels (descriptors by value)
constexpr int kMetaBatch = 64;

struct MetaBatch {
    int count;
    int64_t block0[kMetaBatch + 1];   // first workgroup of each array; block0[count] = grid size
    float *meta[kMetaBatch];
    int64_t n[kMetaBatch];
    uint8_t *codes[kMetaBatch];
    float *mscale[kMetaBatch];
    float *mzero[kMetaBatch];
};

// Meta groups per workgroup of the quantize kernel: 16 slots of 64 lanes x 4
// values (one group per slot when gs >= 256).
constexpr int meta_groups_per_block(int gs)
{
    return gs >= 256 ? 16 : 16 * (256 / gs);
}
// Values per workgroup of the dequantize kernel.
constexpr int kMetaDequantBlock = 1024;

// up to kMetaBatch arrays per call; block0 is filled in here
hipError_t launch_quantize_meta(MetaBatch &b, int gs, hipStream_t s);
hipError_t launch_dequantize_meta(MetaBatch &b, int gs, hipStream_t s);

}  // namespace hqq
