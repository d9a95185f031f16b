// hqq_linear.hip -- Y = X . W_hat^T with W_hat dequantized from packed codes
// on the fly, on gfx950 matrix cores.
//
// This is the consumer of the codes: the HQQLinear forward of the lnwmold.com
// HQQ guide (section 3.2: the quantized layer is called like the Linear it
// replaces and computes in compute_dtype, fp16 or bf16 here; section 4.1: a
// backend fuses the dequantization and the matrix product into one kernel and
// needs axis = 1; section 4.2: axis = 1 4-bit layers with optimized kernels).  W is
// the axis = 1 layout, so a packed word holds C = 32 / nbits consecutive k of
// one output row n, and the group of gs consecutive k shares (scale, zero).
//
// Exact dequantization.  W_hat[n][k] is the fp16 (or bf16) rounding of the
// fp32 quotient (q - zero) / scale, both steps round-to-nearest-even, as the
// dequantize kernel computes it.  Here the quotient comes from one fp64 product instead
// of an fp32 division: with a = fl32(q - zero) and R = fl64(1 / scale),
// fl32(a * R) equals fl32(a / scale).  The fp64 product is within 2^-52 of
// a / scale (relative), while a quotient of two 24-bit significands is never
// a rounding midpoint of fp32 and never closer to one than 2^-49 relative, so
// both round to the same fp32 value.  Products of fp16 (or bf16) inputs are
// exact in the fp32 accumulators, so the kernel differs from an exact dot
// product of X with W_hat only by fp32 accumulation order and the final
// rounding to the compute dtype.
//
// Code tables (4-bit codes, groups of 32 or more).  A group has only 16
// distinct W_hat values, so a lane computes them once (16 exact quotients)
// and keeps them as two 16-byte tables, the low and the high bytes, in 8
// VGPRs.  A packed word then becomes 8 16-bit values with v_perm_b32 byte
// lookups (two 8-entry halves joined on bit 3 of each code with v_bfi_b32):
// about 3 VALU operations per weight instead of about 10 for the quotient.
// The lookups give the 8 k of a word in the order 0,2,4,6,1,3,5,7; the X run
// that meets it in the MFMA is permuted the same way (a dot product does not
// depend on the k order inside an MFMA), and the other code widths produce
// the same order.
//
// Skinny kernel (few rows of X: decode and small batches).  A workgroup owns
// 16 output columns n (an MFMA 16x16x32 tile) and its 4, 8 or 16 waves split
// K.  Lane
// l works on row n = l % 16 and, in each 256-wide step of k, on the 64
// consecutive k at 64 * (l / 16): one group (gs >= 64), the codes in 16 or 32
// bytes, dequantized in registers to the eight 8-half B operands of eight
// MFMAs.  When X fits (M * K * 2 bytes <= 64 KiB), the workgroup stages it in
// LDS once, in operand order, and the A operands are single ds_read_b128s;
// otherwise every lane reads its X runs from global memory (X is small and
// stays in cache).  The waves add their partial sums through LDS at the end.
#include "hqq_internal.h"

#include <stdlib.h>

namespace hqq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kLaneK = 64;                // consecutive k per lane per step
constexpr int kStepK = 4 * kLaneK;        // k per wave step
constexpr int kXldsMax = 64 * 1024;       // bytes of X staged in LDS, at most

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// an 8-k run of X (16-bit values, natural order) in operand order 0,2,4,6,1,3,5,7
__device__ __forceinline__ uint4 run_order(uint4 x)
{
    return uint4{perm(x.y, x.x, 0x05040100u), perm(x.w, x.z, 0x05040100u),
                 perm(x.y, x.x, 0x07060302u), perm(x.w, x.z, 0x07060302u)};
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// two fp32 -> packed fp16 pair, round-to-nearest-even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t f16x2(float lo, float hi)
{
    const half2v h = __builtin_convertvector(float2v{lo, hi}, half2v);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// two fp32 -> packed pair of the compute dtype (fp16, or BF: bf16), round to
// nearest even (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32)
template <bool BF>
__device__ __forceinline__ uint32_t out2(float lo, float hi)
{
    if constexpr (BF) {
        const bf2v h = __builtin_convertvector(float2v{lo, hi}, bf2v);
        uint32_t u;
        __builtin_memcpy(&u, &h, 4);
        return u;
    } else {
        return f16x2(lo, hi);
    }
}

// one fp32 -> 16-bit value of the compute dtype, round to nearest even
template <bool BF>
__device__ __forceinline__ uint16_t out1(float v)
{
    uint16_t u;
    if constexpr (BF) {
        const __bf16 h = (__bf16)v;
        __builtin_memcpy(&u, &h, 2);
    } else {
        const _Float16 h = (_Float16)v;
        __builtin_memcpy(&u, &h, 2);
    }
    return u;
}

// the exact dequantized value of code c (fp32, before the rounding to the
// compute dtype)
__device__ __forceinline__ float wq(float c, float z, double R)
{
    return (float)((double)(c - z) * R);
}

// The 16 values (fp16, or BF: bf16) of a 4-bit group as byte tables: L[q]
// holds the low bytes of codes 4q .. 4q+3, H[q] the high bytes.
struct Tab4 {
    uint32_t L[4], H[4];
};

template <bool BF>
__device__ __forceinline__ Tab4 make_tab4(float s, float z)
{
    const double R = 1.0 / (double)s;
    uint32_t P[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        P[i] = out2<BF>(wq((float)(2 * i), z, R), wq((float)(2 * i + 1), z, R));
    Tab4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        t.L[q] = perm(P[2 * q + 1], P[2 * q], 0x06040200u);
        t.H[q] = perm(P[2 * q + 1], P[2 * q], 0x07050301u);
    }
    return t;
}

// make_tab4 shared by two adjacent lanes that hold the same group: each lane
// evaluates 8 of the 16 values (the even lane codes 0-7, the odd lane codes
// 8-15) and takes the other 8 from its neighbour by a DPP quad permutation
// [1, 0, 3, 2].  The values are those of make_tab4, bit for bit.  Both lanes
// must be active.
template <bool BF>
__device__ __forceinline__ Tab4 make_tab4_pair(float s, float z, bool odd)
{
    const double R = 1.0 / (double)s;
    const float c0 = odd ? 8.0f : 0.0f;
    uint32_t P[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t mine = out2<BF>(wq(c0 + (float)(2 * j), z, R), wq(c0 + (float)(2 * j + 1), z, R));
        const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)mine, 0xB1, 0xF, 0xF, false);
        P[j] = odd ? other : mine;
        P[4 + j] = odd ? mine : other;
    }
    Tab4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        t.L[q] = perm(P[2 * q + 1], P[2 * q], 0x06040200u);
        t.H[q] = perm(P[2 * q + 1], P[2 * q], 0x07050301u);
    }
    return t;
}

// 8 codes of a 4-bit word -> 8 16-bit values in operand order (0,2,4,6,1,3,5,7)
__device__ __forceinline__ uint4 lookup4(const Tab4 &t, uint32_t w)
{
    // byte q of se / so: low 3 bits of the even / odd code of byte q; the
    // masks are 0xff where bit 3 of that code is set (v_perm replicates the
    // sign bit of a byte for selector values 8..11)
    const uint32_t se = w & 0x07070707u, so = (w >> 4) & 0x07070707u;
    const uint32_t me = perm(w << 12, w << 4, 0x090B080Au);
    const uint32_t mo = perm(w << 8, w, 0x090B080Au);
    auto pick = [](uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); };
    const uint32_t lo_e = pick(me, perm(t.L[3], t.L[2], se), perm(t.L[1], t.L[0], se));
    const uint32_t hi_e = pick(me, perm(t.H[3], t.H[2], se), perm(t.H[1], t.H[0], se));
    const uint32_t lo_o = pick(mo, perm(t.L[3], t.L[2], so), perm(t.L[1], t.L[0], so));
    const uint32_t hi_o = pick(mo, perm(t.H[3], t.H[2], so), perm(t.H[1], t.H[0], so));
    return uint4{perm(hi_e, lo_e, 0x05010400u), perm(hi_e, lo_e, 0x07030602u),
                 perm(hi_o, lo_o, 0x05010400u), perm(hi_o, lo_o, 0x07030602u)};
}

// Groups whose (scale, zero) a lane needs per step: 1 (gs >= 64), 2 (gs 32,
// one per 32 k) or 8 (gs 8 or 16, one per 8-k run).
constexpr int groups_per_chunk(int gs) { return gs >= 64 ? 1 : gs == 32 ? 2 : 8; }

// One wave step's codes and meta for one lane (its 64-k chunk), and the X
// runs of its m tiles when X is read from global memory.
template <int NB, int GPC>
struct StepBuf {
    uint32_t w[2 * NB];
    float s[GPC], z[GPC];
};

template <int MT>
struct XRuns {
    uint4 x[MT][8];
};

// Where a lane's chunk starts (k0) and where its second 32 k start (kh): k0
// + 32, or k0 again where that is K or beyond (K % 64 == 32; those products
// are masked to zero).  A chunk past K is moved to the last 32 k (in bounds;
// masked to zero as well).  Offsets are 32-bit: the host keeps every array
// below 2^31 bytes, so each load is a uniform base plus a lane offset.
struct Chunk {
    uint32_t k0, kh;
};

template <bool KT>
__device__ __forceinline__ Chunk lane_chunk(uint32_t kbase, int grp, uint32_t K)
{
    uint32_t k0 = kbase + kLaneK * grp;
    if constexpr (KT)
        k0 = k0 < K ? k0 : K - 32;
    const uint32_t kh = KT ? (k0 + 32 < K ? k0 + 32 : k0) : k0 + 32;
    return Chunk{k0, kh};
}

// The weight of a batch that grid column bx belongs to (uniform; count <=
// kLinBatch): the shared arguments with that weight's pointers and N; bx
// becomes the column tile within the weight.
__device__ __forceinline__ LinearArgs batch_item(const LinearBatch &b, uint32_t &bx)
{
    int j = 0;
#pragma unroll
    for (int k = 1; k < kLinBatch; ++k)
        j = k < b.count && bx >= b.tile0[k] ? k : j;
    LinearArgs a = b.a;
    a.packed = b.packed[j];
    a.scale = b.scale[j];
    a.zero = b.zero[j];
    a.Y = b.Y[j];
    a.N = b.N[j];
    a.part = b.splits > 1 ? b.part[j] : nullptr;
    bx -= b.tile0[j];
    return a;
}

template <typename T>
__device__ __forceinline__ const T *at(const void *base, uint32_t byte_off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

template <int NB, int GPC>
__device__ __forceinline__ void load_step(StepBuf<NB, GPC> &b, const LinearArgs &a, Chunk c,
                                          uint32_t nw, uint32_t ng)
{
    // nw: first word of the lane's row, ng: its first group
    const uint32_t wa = 4 * (nw + c.k0 * NB / 32), wb = 4 * (nw + c.kh * NB / 32);
    if constexpr (NB == 1) {
        b.w[0] = *at<uint32_t>(a.packed, wa);
        b.w[1] = *at<uint32_t>(a.packed, wb);
    } else if constexpr (NB == 2) {
        const uint2 u = *at<uint2>(a.packed, wa);
        const uint2 v = *at<uint2>(a.packed, wb);
        b.w[0] = u.x; b.w[1] = u.y; b.w[2] = v.x; b.w[3] = v.y;
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int q = 0; q < NB / 4; ++q) {
                const uint4 v = *at<uint4>(a.packed, (h ? wb : wa) + 16 * q);
                b.w[NB * h + 4 * q + 0] = v.x; b.w[NB * h + 4 * q + 1] = v.y;
                b.w[NB * h + 4 * q + 2] = v.z; b.w[NB * h + 4 * q + 3] = v.w;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < GPC; ++i) {
        const uint32_t kk = GPC == 1 ? c.k0 : GPC == 2 ? (i ? c.kh : c.k0) : (i < 4 ? c.k0 : c.kh) + 8 * (i & 3);
        const uint32_t g = 4 * (ng + (kk >> a.gshift));
        b.s[i] = *at<float>(a.scale, g);
        b.z[i] = *at<float>(a.zero, g);
    }
}

// xr: element index of the first X element of each of the lane's rows
template <int MT>
__device__ __forceinline__ void load_x(XRuns<MT> &b, const LinearArgs &a, Chunk c,
                                       const uint32_t (&xr)[MT])
{
#pragma unroll
    for (int u = 0; u < MT; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b.x[u][j] = *at<uint4>(a.X, 2 * (xr[u] + c.k0) + 16 * j);
            b.x[u][4 + j] = *at<uint4>(a.X, 2 * (xr[u] + c.kh) + 16 * j);
        }
    }
}

// B operand j (8-k run j of the chunk) by direct quotients, operand order
template <int NB, int GPC, bool BF>
__device__ __forceinline__ uint4 dequant_run(const uint32_t *w, int j, const float *s,
                                             const float *z)
{
    constexpr uint32_t MASK = (1u << NB) - 1u;
    constexpr int ord[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    const int gi = GPC == 1 ? 0 : GPC == 2 ? (j >> 2) : j;
    const double R = 1.0 / (double)s[gi];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int bit = (8 * j + ord[i]) * NB;
        v[i] = wq((float)((w[bit / 32] >> (bit % 32)) & MASK), z[gi], R);
    }
    return uint4{out2<BF>(v[0], v[1]), out2<BF>(v[2], v[3]), out2<BF>(v[4], v[5]), out2<BF>(v[6], v[7])};
}

__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m)
{
    return uint4{v.x & m, v.y & m, v.z & m, v.w & m};
}

// one 16x16x32 MFMA of the compute dtype (fp16, or BF: bf16), fp32 accumulation
template <bool BF>
__device__ __forceinline__ float4v mfma(uint4 A, uint4 B, float4v c)
{
    if constexpr (BF) {
        bf16x8 a, b;
        __builtin_memcpy(&a, &A, 16);
        __builtin_memcpy(&b, &B, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    } else {
        half8 a, b;
        __builtin_memcpy(&a, &A, 16);
        __builtin_memcpy(&b, &B, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
}

// X staged in LDS: row m of the workgroup's X rows at xs + m * xrow (uint4
// units), runs in operand order; the row pitch is K / 8 + 1 runs so that the
// 16 rows of an operand fall in different banks.
template <bool KT, int NB, int MT, int GPC, bool XL, bool BF>
__device__ __forceinline__ void compute_step(const StepBuf<NB, GPC> &b, const XRuns<XL ? 1 : MT> &xg,
                                             uint32_t km0, uint32_t km1, const uint4 *xs,
                                             const uint32_t (&xm)[MT], Chunk c,
                                             float4v (&acc)[MT])
{
    uint4 B[8];
    if constexpr (NB == 4 && GPC == 1) {
        const Tab4 t = make_tab4<BF>(b.s[0], b.z[0]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            B[j] = lookup4(t, b.w[j]);
    } else if constexpr (NB == 4 && GPC == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Tab4 t = make_tab4<BF>(b.s[h], b.z[h]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                B[4 * h + j] = lookup4(t, b.w[4 * h + j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            B[j] = dequant_run<NB, GPC, BF>(b.w, j, b.s, b.z);
    }
    // K % 256 != 0: a lane whose chunk (or its second half) lies past K adds
    // zeros; the operands are cleared with integer masks (a select would
    // become a branch that waits for every load in flight)
    if constexpr (KT) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            B[j] = and4(B[j], j < 4 ? km0 : km1);
    }
    const uint32_t r0 = c.k0 >> 3, r1 = c.kh >> 3;
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4 A;
            if constexpr (XL)
                A = xs[xm[u] + (j < 4 ? r0 + j : r1 + j - 4)];
            else
                A = run_order(xg.x[u][j]);
            if constexpr (KT)
                A = and4(A, j < 4 ? km0 : km1);
            acc[u] = mfma<BF>(A, B[j], acc[u]);
        }
}

// One K step in flight per wave: the next step's codes load while the
// current one is computed and other waves run in the meantime.  A second
// register buffer per wave costs more occupancy than it gains.
// resident waves per SIMD the register allocation must allow
constexpr int lin_waves_per_simd(int nb, int mt, int gpc, bool xl)
{
    return !xl ? (mt > 1 ? 3 : 4) : nb == 8 || mt > 1 || gpc == 8 ? 4 : 6;
}

template <bool KT, int NB, int MT, int GPC, bool XL, int WPB, bool BF>
__global__ __launch_bounds__(WPB * 64)
__attribute__((amdgpu_waves_per_eu(lin_waves_per_simd(NB, MT, GPC, XL)))) void linear_skinny_kernel(LinearBatch lb)
{
    uint32_t bx = blockIdx.x;
    const LinearArgs a = batch_item(lb, bx);
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane16 = lane & 15, grp = lane >> 4;
    const uint32_t K = (uint32_t)a.K;
    const int64_t n_raw = (int64_t)bx * 16 + lane16;
    const uint32_t n = (uint32_t)(n_raw < a.N ? n_raw : a.N - 1);
    const uint32_t nw = n * (uint32_t)a.wpr, ng = n * (uint32_t)a.gpl;
    const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
    const int mrows = (int)(a.M - m0 < 16 * MT ? a.M - m0 : 16 * MT);
    // X rows of the lane's m tiles (rows past M repeat the last; their
    // outputs are not stored): LDS run index, or element index of X
    const uint32_t xrow = K / 8 + 1;
    uint32_t xr[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int r = 16 * u + lane16 < mrows ? 16 * u + lane16 : mrows - 1;
        xr[u] = XL ? (uint32_t)r * xrow : (uint32_t)((m0 + r) * a.K);
    }

    // X rows of this workgroup into LDS, runs in operand order
    if constexpr (XL) {
        const uint32_t runs = K / 8;
        const uint4 *xg = reinterpret_cast<const uint4 *>(a.X + m0 * a.K);
        for (uint32_t c = threadIdx.x; c < (uint32_t)mrows * runs; c += WPB * 64) {
            const uint32_t m = c / runs, r = c - m * runs;
            lds[m * xrow + r] = run_order(xg[c]);
        }
        __syncthreads();
    }

    // this wave's K steps: wave, wave + WPB, ...
    const int n_steps = (int)((K + kStepK - 1) / kStepK);
    const int my = n_steps > wave ? (n_steps - wave + WPB - 1) / WPB : 0;
    auto kbase = [&](int i) { return (uint32_t)(wave + i * WPB) * kStepK; };

    float4v acc[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u)
        acc[u] = float4v{0.f, 0.f, 0.f, 0.f};

    // X from global memory: the step's X runs load before the next step's
    // codes, so that waiting for them does not wait for the codes
    StepBuf<NB, GPC> buf;
    XRuns<XL ? 1 : MT> xg;
    if (my > 0)
        load_step(buf, a, lane_chunk<KT>(kbase(0), grp, K), nw, ng);
    for (int i = 0; i < my; ++i) {
        const Chunk c = lane_chunk<KT>(kbase(i), grp, K);
        const uint32_t k0 = kbase(i) + kLaneK * grp;
        const uint32_t km0 = k0 < K ? 0xffffffffu : 0u;
        const uint32_t km1 = k0 + 32 < K ? 0xffffffffu : 0u;
        if constexpr (!XL)
            load_x(xg, a, c, xr);
        const StepBuf<NB, GPC> cur = buf;
        if (i + 1 < my)
            load_step(buf, a, lane_chunk<KT>(kbase(i + 1), grp, K), nw, ng);
        compute_step<KT, NB, MT, GPC, XL, BF>(cur, xg, km0, km1, lds, xr, c, acc);
    }

    // add the waves' partial sums: red[wave][u * 4 + r][lane]
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red[(wave * MT * 4 + u * 4 + r) * 64 + lane] = acc[u][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * 4 * 64; idx += WPB * 64) {
        const int v = idx >> 6, l = idx & 63;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WPB; ++w)
            s += red[(w * MT * 4 + v) * 64 + l];
        // accumulator r of lane l is D[4 * (l / 16) + r][l % 16] of tile u
        const int u = v >> 2, r = v & 3;
        const int64_t m = m0 + 16 * u + 4 * (l >> 4) + r;
        const int64_t nn = (int64_t)bx * 16 + (l & 15);
        if (m < a.M && nn < a.N)
            a.Y[m * a.N + nn] = out1<BF>(s);
    }
}

// Waves per workgroup (they split K): enough workgroups x waves to give every
// SIMD about four waves, but no more waves than K steps.
inline int lin_waves(int64_t blocks, int64_t K)
{
    const int64_t steps = (K + kStepK - 1) / kStepK;
    int w = blocks >= 1024 ? 4 : blocks >= 512 ? 8 : 16;
    while (w > 4 && w > steps)
        w /= 2;
    return w;
}

// grid columns of the batch: tile0[j] = first column tile of weight j
inline uint32_t fill_tiles(LinearBatch &b, int64_t cols_per_tile)
{
    uint32_t t = 0;
    for (int j = 0; j < b.count; ++j) {
        b.tile0[j] = t;
        t += (uint32_t)((b.N[j] + cols_per_tile - 1) / cols_per_tile);
    }
    b.tile0[b.count] = t;
    return t;
}

template <int NB, int MT, int GPC, bool XL, int WPB, bool BF>
hipError_t launch_wpb(const LinearBatch &b, dim3 grid, hipStream_t s)
{
    const LinearArgs &a = b.a;
    size_t lds = (size_t)WPB * MT * 4 * 64 * sizeof(float);
    if (XL) {
        const int64_t rows = a.M < 16 * MT ? a.M : 16 * MT;
        const size_t x = (size_t)rows * (size_t)(a.K / 8 + 1) * 16;
        lds = x > lds ? x : lds;
    }
    if (a.K % kStepK != 0)
        hipLaunchKernelGGL((linear_skinny_kernel<true, NB, MT, GPC, XL, WPB, BF>), grid, dim3(WPB * 64),
                           lds, s, b);
    else
        hipLaunchKernelGGL((linear_skinny_kernel<false, NB, MT, GPC, XL, WPB, BF>), grid, dim3(WPB * 64),
                           lds, s, b);
    return hipGetLastError();
}

template <int NB, int MT, int GPC, bool XL, bool BF>
hipError_t launch_one(LinearBatch &b, hipStream_t s)
{
    const LinearArgs &a = b.a;
    const dim3 grid(fill_tiles(b, 16), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)));
    switch (lin_waves((int64_t)grid.x * grid.y, a.K)) {
    case 4: return launch_wpb<NB, MT, GPC, XL, 4, BF>(b, grid, s);
    case 8: return launch_wpb<NB, MT, GPC, XL, 8, BF>(b, grid, s);
    default: return launch_wpb<NB, MT, GPC, XL, 16, BF>(b, grid, s);
    }
}

template <int NB, int MT, int GPC, bool BF>
hipError_t launch_xl(LinearBatch &b, hipStream_t s)
{
    const LinearArgs &a = b.a;
    const int64_t rows = a.M < 16 * MT ? a.M : 16 * MT;
    if (rows * (a.K / 8 + 1) * 16 <= kXldsMax)
        return launch_one<NB, MT, GPC, true, BF>(b, s);
    return launch_one<NB, MT, GPC, false, BF>(b, s);
}

template <int NB, int MT, bool BF>
hipError_t launch_gpc(LinearBatch &b, hipStream_t s)
{
    switch (groups_per_chunk(b.a.gs)) {
    case 1: return launch_xl<NB, MT, 1, BF>(b, s);
    case 2: return launch_xl<NB, MT, 2, BF>(b, s);
    default: return launch_xl<NB, MT, 8, BF>(b, s);
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel (many rows of X: prefill).  A workgroup computes a 256 x 128
// tile of Y (or 128 x 128 where that fills the CUs better) with eight waves in
// two roles, one of each on every SIMD:
//   * waves 0-3 (MFMA waves, 2 x 2, each 128 x 64 outputs as 8 x 4 MFMA
//     16x16x32 tiles, 64 x 64 as 4 x 4 with 128-row tiles) copy X's tile of
//     a 64-wide k step global ->
//     LDS by DMA (global_load_lds, no registers; runs of 8 k XOR-swizzled
//     by row so the MFMA reads of 16 rows spread over the banks) and run the
//     step's 64 MFMAs per wave from LDS;
//   * waves 4-7 (dequantization waves) turn W's 128 x 64 tile of the next
//     step into 16-bit values in LDS, in natural k order (two threads per
//     row, 32 k each; 4-bit codes through the group's code table, whose 16
//     values the two threads split when they share the group).
// The VALU work of the dequantization issues beside the other role's MFMAs
// on the same SIMD.  X goes through a ring of three LDS buffers (its DMA two
// steps ahead), W through two, with one barrier per step.  An MFMA wave
// reads all of a step's operands into registers before it issues the next
// DMA, so the wait the compiler places for the DMA before the next LDS read
// comes after a full step of matrix work.  The dequantization is shared by
// the 256 (or 128) rows of X.

constexpr int kTK = 64;              // k per step
constexpr int kTBM = 256, kTBN = 128;
constexpr int kWPitch = kTK / 8 + 1; // W tile row pitch in 8-k runs (uint4)

// End of a k step: this wave's LDS writes are complete (lgkmcnt(0)), then
// the workgroup barrier.  A plain __syncthreads() would also wait for every
// vector memory operation of the wave (it is a release fence: vmcnt(0)),
// including the loads just issued for later steps.  The empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 8 codes of a 4-bit word -> 8 16-bit values in natural k order
__device__ __forceinline__ uint4 lookup4n(const Tab4 &t, uint32_t w)
{
    const uint4 q = lookup4(t, w);   // (c0,c2) (c4,c6) (c1,c3) (c5,c7)
    return uint4{perm(q.z, q.x, 0x05040100u), perm(q.z, q.x, 0x07060302u),
                 perm(q.w, q.y, 0x05040100u), perm(q.w, q.y, 0x07060302u)};
}

// A thread's share of a W step: RW = 4 runs of 8 k of one row (its codes,
// and per run or per group the meta)
template <int NB, bool G1>
struct TileW {
    uint32_t w[NB];                  // 32 k x NB bits = NB words
    float s[G1 ? 1 : 4], z[G1 ? 1 : 4];
};

// PR: the two threads of a row hold the same group (gs >= 64) and share the
// code table
template <int NB, bool G1, bool BF, bool PR>
__device__ __forceinline__ void dequant_tile_runs(const TileW<NB, G1> &b, uint4 (&out)[4])
{
    if constexpr (NB == 4 && G1) {
        const Tab4 t = PR ? make_tab4_pair<BF>(b.s[0], b.z[0], (threadIdx.x & 1) != 0)
                          : make_tab4<BF>(b.s[0], b.z[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            out[j] = lookup4n(t, b.w[j]);
    } else {
        constexpr uint32_t MASK = (1u << NB) - 1u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = G1 ? 0 : j;
            const double R = 1.0 / (double)b.s[g];
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int bit = (8 * j + i) * NB;
                v[i] = wq((float)((b.w[bit / 32] >> (bit % 32)) & MASK), b.z[g], R);
            }
            out[j] = uint4{out2<BF>(v[0], v[1]), out2<BF>(v[2], v[3]), out2<BF>(v[4], v[5]),
                           out2<BF>(v[6], v[7])};
        }
    }
}


// BM: rows of the tile, 256 or 128 (per-thread arrays are sized for 256 and
// use the first BM / 32 entries)
template <int NB, bool G1, bool BF, bool PR, int BM>
__global__ __launch_bounds__(512, 1) void linear_tiled_kernel(LinearBatch lb)
{
    uint32_t bx = blockIdx.x;
    const LinearArgs a = batch_item(lb, bx);
    static_assert(BM == 256 || BM == 128, "tile rows");
    constexpr int TM = BM / 32, TN = kTBN / 32;     // MFMA tiles per MFMA wave (8 x 4 at BM = 256)
    constexpr int XI = BM / 32;                     // X DMA instructions per MFMA wave and step
    typedef __attribute__((address_space(3))) void *lds_ptr;
    __shared__ uint4 xs[3][kTBM * 8];
    __shared__ uint4 ws[2][kTBN * kWPitch];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)bx * kTBN;
    const uint32_t K = (uint32_t)a.K;
    // split K: workgroup z of gridDim.z takes steps s0 .. s0 + steps - 1 of
    // the K / 64 (the host keeps every split non-empty)
    const uint32_t all_steps = K / kTK, per = (all_steps + gridDim.z - 1) / gridDim.z;
    const uint32_t s0 = blockIdx.z * per;
    const uint32_t steps = all_steps - s0 < per ? all_steps - s0 : per;
    // past the last step the loads repeat it (in bounds, never used)
    auto clampk = [&](uint32_t s_) { return (s0 + (s_ < steps ? s_ : steps - 1)) * kTK; };

    if (wave < 4) {
        // MFMA wave: step st reads X from buffer st % 3 and W from st & 1
        const int wm = wave >> 1, wn = wave & 1;
        // X DMA: wave w moves rows BM/4 w .. BM/4 (w + 1) - 1, 8 rows (64
        // runs) per instruction; lane l fills slot (row 8 i + l / 8, column
        // l % 8), which holds run (l % 8) ^ (row % 8) of that row
        uint32_t xsrc[kTBM / 32];
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int r = (BM / 4) * wave + 8 * i + (lane >> 3);
            const int64_t m = m0 + r < a.M ? m0 + r : a.M - 1;
            xsrc[i] = (uint32_t)(m * a.K) + 8 * ((lane & 7) ^ (r & 7));      // halves
        }
        auto dma_x = [&](uint32_t k0, int b) {
#pragma unroll
            for (int i = 0; i < XI; ++i)
                __builtin_amdgcn_global_load_lds(a.X + xsrc[i] + k0,
                                                 (lds_ptr)&xs[b][((BM / 4) * wave + 8 * i) * 8], 16, 0, 0);
        };
        float4v acc[kTBM / 32][TN];
#pragma unroll
        for (int u = 0; u < TM; ++u)
#pragma unroll
            for (int t = 0; t < TN; ++t)
                acc[u][t] = float4v{0.f, 0.f, 0.f, 0.f};
        dma_x(clampk(0), 0);
        dma_x(clampk(1), 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): X(0) has landed
        lds_barrier();                        // and W(0) is in LDS
        for (uint32_t st = 0; st < steps; ++st) {
            const int bx_ = (int)(st % 3), bw = (int)(st & 1);
            uint4 A[2][kTBM / 32], B[2][TN];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int u = 0; u < TM; ++u) {
                    const int r = wm * (BM / 2) + 16 * u + (lane & 15);
                    A[ks][u] = xs[bx_][r * 8 + ((4 * ks + (lane >> 4)) ^ (r & 7))];
                }
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    B[ks][t] = ws[bw][(wn * (kTBN / 2) + 16 * t + (lane & 15)) * kWPitch + 4 * ks + (lane >> 4)];
            }
            dma_x(clampk(st + 2), (int)((st + 2) % 3));
            // all of the step's LDS reads are issued before the DMA
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int u = 0; u < TM; ++u)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[u][t] = mfma<BF>(A[ks][u], B[ks][t], acc[u][t]);
            lds_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA outlives the block

        // accumulator r of lane l in tile (u, t) is Y[m][n] with
        // m = 4 (l / 16) + r + 16 u, n = l % 16 + 16 t in the wave's quadrant
#pragma unroll
        for (int u = 0; u < TM; ++u)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm * (BM / 2) + 16 * u + 4 * (lane >> 4) + r;
                    const int64_t n = n0 + wn * (kTBN / 2) + 16 * t + (lane & 15);
                    if (m < a.M && n < a.N) {
                        if (a.part)
                            a.part[((int64_t)blockIdx.z * a.M + m) * a.N + n] = acc[u][t][r];
                        else
                            a.Y[m * a.N + n] = out1<BF>(acc[u][t][r]);
                    }
                }
    } else {
        // dequantization wave: thread p = tid - 256 dequantizes row p / 2,
        // runs 4 (p % 2) .. + 3; in step st it writes W(st + 1) and loads
        // the codes of step st + 3
        const int pt = tid - 256;
        const int wr = pt >> 1, wr0 = (pt & 1) * 4;
        const int64_t wn_ = n0 + wr < a.N ? n0 + wr : a.N - 1;
        const uint32_t wbase = (uint32_t)(wn_ * a.wpr) + (8 * wr0 * NB) / 32;
        const uint32_t gbase = (uint32_t)(wn_ * a.gpl);
        auto load_w = [&](uint32_t k0, TileW<NB, G1> &w) {
            const uint32_t wo = 4 * (wbase + (k0 * NB) / 32);
            if constexpr (NB == 8) {
                const uint4 u = *at<uint4>(a.packed, wo), v = *at<uint4>(a.packed, wo + 16);
                w.w[0] = u.x; w.w[1] = u.y; w.w[2] = u.z; w.w[3] = u.w;
                w.w[4] = v.x; w.w[5] = v.y; w.w[6] = v.z; w.w[7] = v.w;
            } else if constexpr (NB == 4) {
                const uint4 u = *at<uint4>(a.packed, wo);
                w.w[0] = u.x; w.w[1] = u.y; w.w[2] = u.z; w.w[3] = u.w;
            } else {
                const uint2 u = *at<uint2>(a.packed, wo);
                w.w[0] = u.x; w.w[1] = u.y;
            }
#pragma unroll
            for (int j = 0; j < (G1 ? 1 : 4); ++j) {
                const uint32_t g = 4 * (gbase + ((k0 + 8 * (wr0 + j)) >> a.gshift));
                w.s[j] = *at<float>(a.scale, g);
                w.z[j] = *at<float>(a.zero, g);
            }
        };
        auto store_w = [&](const TileW<NB, G1> &w, int b) {
            uint4 runs[4];
            dequant_tile_runs<NB, G1, BF, PR>(w, runs);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ws[b][wr * kWPitch + wr0 + j] = runs[j];
        };
        TileW<NB, G1> wb0, wb1;
        load_w(clampk(0), wb0);
        store_w(wb0, 0);
        load_w(clampk(1), wb1);
        load_w(clampk(2), wb0);
        lds_barrier();
        auto step = [&](uint32_t st, TileW<NB, G1> &wn1) {
            store_w(wn1, (int)(st & 1) ^ 1);
            load_w(clampk(st + 3), wn1);
            lds_barrier();
        };
        // two steps per trip, so that the register buffers are named statically
        for (uint32_t st = 0; st < steps; st += 2) {
            step(st, wb1);
            if (st + 1 < steps)
                step(st + 1, wb0);
        }
    }
}

// Split K, second pass: Y = the partial sums of the splits added in split
// order in fp32, rounded once to the compute dtype.  Four outputs per
// thread; workgroups rblock0[j] .. rblock0[j + 1] - 1 belong to weight j.
constexpr int kReduceBlock = 256;

template <bool BF>
__global__ __launch_bounds__(kReduceBlock) void linear_reduce_kernel(LinearBatch lb)
{
    const uint32_t bx = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int k = 1; k < kLinBatch; ++k)
        j = k < lb.count && bx >= lb.rblock0[k] ? k : j;
    const int64_t total = lb.a.M * lb.N[j];
    const int64_t i0 = ((int64_t)(bx - lb.rblock0[j]) * kReduceBlock + threadIdx.x) * 4;
    if (i0 >= total)
        return;
    const float *part = lb.part[j];
    uint16_t *Y = lb.Y[j];
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < lb.splits; ++z) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (i0 + e < total)
                v[e] += part[z * total + i0 + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (i0 + e < total)
            Y[i0 + e] = out1<BF>(v[e]);
}

// Time estimates of the two kernels (the row-block kernel re-derives W for
// every 32 rows of X, so its time grows with ceil(M / 32) * N * K; the tiled
// kernel's is its rounds of tiles over the 256 CUs times K / 64 steps), from
// times measured for 4-bit g64 codes at K = 4096 on MI355X: 9.1 us per
// 32-row block at N = 4096; a step of 0.92 us with 256-row tiles and 0.74 us
// with 128-row tiles.
inline double skinny_us(const LinearBatch &b)
{
    int64_t n = 0;
    for (int j = 0; j < b.count; ++j)
        n += b.N[j];
    return (double)((b.a.M + 31) / 32) * 9.1 * ((double)n * (double)b.a.K) / (4096.0 * 4096.0);
}

inline double tiled_us(const LinearBatch &b, int bm, int splits = 1)
{
    int64_t cols = 0, n = 0;
    for (int j = 0; j < b.count; ++j) {
        cols += (b.N[j] + kTBN - 1) / kTBN;
        n += b.N[j];
    }
    const int64_t tiles = cols * ((b.a.M + bm - 1) / bm) * splits;
    const int64_t steps = (b.a.K / kTK + splits - 1) / splits;
    double t = (double)((tiles + 255) / 256) * (double)steps * (bm == 128 ? 0.74 : 0.92);
    if (splits > 1)   // the second pass: read the partials, write Y, and its launch
        t += 3.0 + (double)b.a.M * (double)n * (4.0 * splits + 2.0) / 4.0e6;
    return t;
}

// The splits of K the workspace allows (every split non-empty): 1, 2, 4 or 8.
inline bool splits_ok(const LinearBatch &b, int splits)
{
    const int64_t steps = b.a.K / kTK;
    int64_t n = 0;
    for (int j = 0; j < b.count; ++j)
        n += b.N[j];
    const int64_t per = (steps + splits - 1) / splits;
    return splits == 1 || (b.work != nullptr && (splits - 1) * per < steps &&
                           (int64_t)splits * b.a.M * n <= b.work_floats);
}

// HQQ_LINEAR_SPLITS=1|2|4|8 in the environment forces that many K splits
// where the workspace allows them (tests use it to reach every split count);
// 0: the estimate decides.
inline int forced_splits()
{
    const char *e = getenv("HQQ_LINEAR_SPLITS");
    if (!e)
        return 0;
    const int v = atoi(e);
    return v == 1 || v == 2 || v == 4 || v == 8 ? v : 0;
}

// The tile height and split count of the smallest estimate.
inline double tiled_best(const LinearBatch &b, int &bm, int &splits)
{
    double best = 0.0;
    bm = 256;
    splits = 1;
    const int force = forced_splits();
    for (int sp : {1, 2, 4, 8}) {
        if (!splits_ok(b, sp) || (force && sp != force && splits_ok(b, force)))
            continue;
        for (int m : {256, 128}) {
            const double t = tiled_us(b, m, sp);
            if (best == 0.0 || t < best) {
                best = t;
                bm = m;
                splits = sp;
            }
        }
    }
    return best;
}

#define HQQ_LAUNCH_TILED(BMV)                                                                           \
    {                                                                                                   \
        const dim3 grid(cols, (unsigned)((b.a.M + BMV - 1) / BMV), (unsigned)b.splits);                 \
        if (NB == 4 && b.a.gs >= 64)                                                                    \
            hipLaunchKernelGGL((linear_tiled_kernel<NB, true, BF, NB == 4, BMV>), grid, dim3(512), 0, s, b); \
        else if (b.a.gs >= 32)                                                                          \
            hipLaunchKernelGGL((linear_tiled_kernel<NB, true, BF, false, BMV>), grid, dim3(512), 0, s, b);   \
        else                                                                                            \
            hipLaunchKernelGGL((linear_tiled_kernel<NB, false, BF, false, BMV>), grid, dim3(512), 0, s, b);  \
    }

// 128-row tiles where their estimate is the smaller (few 256-row tiles)
template <int NB, bool BF>
hipError_t launch_tiled(LinearBatch &b, hipStream_t s)
{
    const uint32_t cols = fill_tiles(b, kTBN);
    int bm, splits;
    tiled_best(b, bm, splits);
    b.splits = splits;
    if (splits > 1) {
        // weight j's partials: [splits, M, N_j], after those of weights < j
        int64_t off = 0;
        uint32_t rb = 0;
        for (int j = 0; j < b.count; ++j) {
            b.part[j] = b.work + off;
            off += (int64_t)splits * b.a.M * b.N[j];
            b.rblock0[j] = rb;
            rb += (uint32_t)((b.a.M * b.N[j] + 4 * kReduceBlock - 1) / (4 * kReduceBlock));
        }
        b.rblock0[b.count] = rb;
    }
    if (bm == 128)
        HQQ_LAUNCH_TILED(128)
    else
        HQQ_LAUNCH_TILED(256)
    if (splits > 1)
        hipLaunchKernelGGL((linear_reduce_kernel<BF>), dim3(b.rblock0[b.count]), dim3(kReduceBlock), 0, s, b);
    return hipGetLastError();
}
#undef HQQ_LAUNCH_TILED

// Kernel choice for M > 32 (K a multiple of 64; 2-, 4- and 8-bit codes): the
// smaller estimate; from 384 rows the tiled kernel whatever the shape (its
// estimate is the smaller one at every shape measured there).
constexpr int64_t kTiledMinRows = 384;

inline bool use_tiled(const LinearBatch &b)
{
    const LinearArgs &a = b.a;
    if (a.M <= 32 || a.K % kTK != 0)
        return false;
    if (a.M >= kTiledMinRows)
        return true;
    int bm, splits;
    return tiled_best(b, bm, splits) < skinny_us(b);
}

template <int NB, bool BF>
hipError_t launch_nb(LinearBatch &b, hipStream_t s)
{
    if constexpr (NB >= 2) {
        if (use_tiled(b))
            return launch_tiled<NB, BF>(b, s);
    }
    // skinny: M > 32 runs ceil(M / 32) row blocks of 32
    if (b.a.M <= 16)
        return launch_gpc<NB, 1, BF>(b, s);
    return launch_gpc<NB, 2, BF>(b, s);
}

template <bool BF>
hipError_t launch_bits(int nbits, LinearBatch &b, hipStream_t s)
{
    switch (nbits) {
    case 1: return launch_nb<1, BF>(b, s);
    case 2: return launch_nb<2, BF>(b, s);
    case 4: return launch_nb<4, BF>(b, s);
    case 8: return launch_nb<8, BF>(b, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_linear(int nbits, bool bf16, LinearBatch &b, hipStream_t s)
{
    return bf16 ? launch_bits<true>(nbits, b, s) : launch_bits<false>(nbits, b, s);
}

}  // namespace hqq
