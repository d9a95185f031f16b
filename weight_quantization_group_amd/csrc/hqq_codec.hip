// hqq_codec.hip -- dequantize (to fp16 or bf16), pack and unpack on gfx950.
//
// These are the HQQLinear state operations of the lnwmold.com HQQ guide,
// section 3.2 (W_q is kept bit-packed; dequantize() rebuilds the fp16 matrix
// from W_q, scale and zero; unpack(dtype=uint8) returns the codes).  All
// three are HBM-streaming: one lane per packed uint32 word, so the word is
// read or written once and its C codes are handled in registers.  axis = 1:
// lanes take consecutive words of a row (a row's words are contiguous);
// axis = 0: lanes take consecutive columns of one word-row, so every access
// of a wave covers 64 consecutive columns.
#include "hqq_internal.h"

namespace hqq {
namespace {

// element (row, col) of code j of word `wid`
template <int NB, int AXIS>
__device__ __forceinline__ void word_coords(int64_t wid, int64_t rows, int64_t cols,
                                            int64_t &r0, int64_t &c0, int64_t &wpl)
{
    constexpr int C = codes_per_word(NB);
    if constexpr (AXIS == 1) {
        wpl = (cols + C - 1) / C;
        r0 = wid / wpl;
        c0 = (wid - r0 * wpl) * C;
    } else {
        wpl = 0;
        const int64_t k = wid / cols;
        c0 = wid - k * cols;
        r0 = k * C;
    }
}

// fp32 -> fp16 (OB = false) or bf16 (OB = true) bits, round half to even
// (bf16: the low 16 bits rounded off with the carry; NaN stays a quiet NaN)
template <bool OB>
__device__ __forceinline__ uint16_t out16(float f)
{
    if constexpr (OB) {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            return (uint16_t)((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    } else {
        const _Float16 h = (_Float16)f;
        uint16_t b;
        __builtin_memcpy(&b, &h, 2);
        return b;
    }
}

template <int NB, int AXIS, bool OB>
__device__ __forceinline__ void dequant_body(const CodecArgs &a)
{
    constexpr int C = codes_per_word(NB);
    constexpr uint32_t MASK = (1u << NB) - 1u;
    const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wid >= a.n_words)
        return;
    int64_t r0, c0, wpl;
    word_coords<NB, AXIS>(wid, a.rows, a.cols, r0, c0, wpl);
    const uint32_t word = a.packed_in[wid];
    const int gs = a.group_size;
    if constexpr (AXIS == 1) {
        const int64_t gpl = a.cols / gs;
        if (NB == 4) {
            // 8 codes of one row, all in one group (gs is a multiple of 8)
            const int64_t gi = r0 * gpl + c0 / gs;
            const float s = a.scale[gi], z = a.zero[gi];
            uint16_t out[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q = (float)((word >> (j * NB)) & MASK);
                out[j] = out16<OB>((q - z) / s);
            }
            uint4 v;
            __builtin_memcpy(&v, out, 16);
            *reinterpret_cast<uint4 *>(a.W_hat + r0 * a.cols + c0) = v;
        } else {
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const int64_t c = c0 + j;
                if (c < a.cols) {
                    const int64_t gi = r0 * gpl + c / gs;
                    const float q = (float)((word >> (j * NB)) & MASK);
                    a.W_hat[r0 * a.cols + c] = out16<OB>((q - a.zero[gi]) / a.scale[gi]);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int64_t r = r0 + j;
            if (r < a.rows) {
                const int64_t gi = (r / gs) * a.cols + c0;
                const float q = (float)((word >> (j * NB)) & MASK);
                a.W_hat[r * a.cols + c0] = out16<OB>((q - a.zero[gi]) / a.scale[gi]);
            }
        }
    }
}

template <int NB, int AXIS>
__global__ __launch_bounds__(256) void dequant_kernel(CodecArgs a)
{
    dequant_body<NB, AXIS, false>(a);
}

template <int NB, int AXIS>
__global__ __launch_bounds__(256) void dequant_bf16_kernel(CodecArgs a)
{
    dequant_body<NB, AXIS, true>(a);
}

template <int NB, int AXIS>
__global__ __launch_bounds__(256) void pack_kernel(CodecArgs a)
{
    constexpr int C = codes_per_word(NB);
    constexpr uint32_t MASK = (1u << NB) - 1u;
    const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wid >= a.n_words)
        return;
    int64_t r0, c0, wpl;
    word_coords<NB, AXIS>(wid, a.rows, a.cols, r0, c0, wpl);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        if constexpr (AXIS == 1) {
            if (c0 + j < a.cols)
                word |= ((uint32_t)a.codes_in[r0 * a.cols + c0 + j] & MASK) << (j * NB);
        } else {
            if (r0 + j < a.rows)
                word |= ((uint32_t)a.codes_in[(r0 + j) * a.cols + c0] & MASK) << (j * NB);
        }
    }
    a.packed_out[wid] = word;
}

template <int NB, int AXIS>
__global__ __launch_bounds__(256) void unpack_kernel(CodecArgs a)
{
    constexpr int C = codes_per_word(NB);
    constexpr uint32_t MASK = (1u << NB) - 1u;
    const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wid >= a.n_words)
        return;
    int64_t r0, c0, wpl;
    word_coords<NB, AXIS>(wid, a.rows, a.cols, r0, c0, wpl);
    const uint32_t word = a.packed_in[wid];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const uint8_t v = (uint8_t)((word >> (j * NB)) & MASK);
        if constexpr (AXIS == 1) {
            if (c0 + j < a.cols)
                a.codes_out[r0 * a.cols + c0 + j] = v;
        } else {
            if (r0 + j < a.rows)
                a.codes_out[(r0 + j) * a.cols + c0] = v;
        }
    }
}

#define HQQ_DEFINE_LAUNCH(NAME, KERNEL)                                                   \
    template <int NB, int AXIS>                                                           \
    hipError_t NAME##_t(const CodecArgs &a, hipStream_t st)                               \
    {                                                                                     \
        const dim3 grid((unsigned)((a.n_words + 255) / 256));                             \
        hipLaunchKernelGGL((KERNEL<NB, AXIS>), grid, dim3(256), 0, st, a);                \
        return hipGetLastError();                                                         \
    }                                                                                     \
    hipError_t NAME##_any(int nbits, int axis, const CodecArgs &a, hipStream_t st)        \
    {                                                                                     \
        if (a.n_words == 0)                                                               \
            return hipSuccess;                                                            \
        switch (nbits * 2 + axis) {                                                       \
        case 2: return NAME##_t<1, 0>(a, st);                                             \
        case 3: return NAME##_t<1, 1>(a, st);                                             \
        case 4: return NAME##_t<2, 0>(a, st);                                             \
        case 5: return NAME##_t<2, 1>(a, st);                                             \
        case 6: return NAME##_t<3, 0>(a, st);                                             \
        case 7: return NAME##_t<3, 1>(a, st);                                             \
        case 8: return NAME##_t<4, 0>(a, st);                                             \
        case 9: return NAME##_t<4, 1>(a, st);                                             \
        case 16: return NAME##_t<8, 0>(a, st);                                            \
        case 17: return NAME##_t<8, 1>(a, st);                                            \
        default: return hipErrorInvalidValue;                                             \
        }                                                                                 \
    }

HQQ_DEFINE_LAUNCH(dequant, dequant_kernel)
HQQ_DEFINE_LAUNCH(dequant_bf16, dequant_bf16_kernel)
HQQ_DEFINE_LAUNCH(pack, pack_kernel)
HQQ_DEFINE_LAUNCH(unpack, unpack_kernel)

// Metadata quantization (quant_scale / quant_zero): 8-bit min-max RTN of a
// flattened fp32 array in groups of gs consecutive values (the last group
// may be shorter) -- the solve's set-up and final codes at iters = 0.  One
// wave per meta group; each lane takes every 64th value of the group.
__global__ __launch_bounds__(256) void meta_quant_kernel(const float *meta, int64_t n, int gs,
                                                         uint8_t *codes, float *mscale, float *mzero,
                                                         int64_t groups)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= groups)
        return;
    const int64_t e0 = g * gs;
    const int len = (int)(n - e0 < gs ? n - e0 : gs);
    float mn = meta[e0], mx = meta[e0];
    for (int i = lane; i < len; i += 64) {
        mn = fminf(mn, meta[e0 + i]);
        mx = fmaxf(mx, meta[e0 + i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const float rng = mx - mn;
    const float s = rng == 0.0f ? 1.0f : 255.0f / rng;
    const float z = rng == 0.0f ? -mn : -(mn * s);
    for (int i = lane; i < len; i += 64) {
        const float t = __builtin_rintf(__builtin_fmaf(meta[e0 + i], s, z));
        codes[e0 + i] = (uint8_t)__builtin_amdgcn_fmed3f(t, 0.0f, 255.0f);
    }
    if (lane == 0) {
        mscale[g] = s;
        mzero[g] = z;
    }
}

// meta[i] = (code - zero) / scale of its meta group, IEEE fp32
__global__ __launch_bounds__(256) void meta_dequant_kernel(const uint8_t *codes, const float *mscale,
                                                           const float *mzero, int64_t n, int gs,
                                                           float *meta)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const int64_t g = i / gs;
    meta[i] = ((float)codes[i] - mzero[g]) / mscale[g];
}

}  // namespace

hipError_t launch_quantize_meta(const float *meta, int64_t n, int gs, uint8_t *codes, float *mscale,
                                float *mzero, hipStream_t st)
{
    const int64_t groups = (n + gs - 1) / gs;
    hipLaunchKernelGGL(meta_quant_kernel, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, st, meta, n,
                       gs, codes, mscale, mzero, groups);
    return hipGetLastError();
}

hipError_t launch_dequantize_meta(const uint8_t *codes, const float *mscale, const float *mzero,
                                  int64_t n, int gs, float *meta, hipStream_t st)
{
    hipLaunchKernelGGL(meta_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, codes,
                       mscale, mzero, n, gs, meta);
    return hipGetLastError();
}

hipError_t launch_dequantize(int nbits, int axis, const CodecArgs &a, hipStream_t st)
{
    return a.out_bf16 ? dequant_bf16_any(nbits, axis, a, st) : dequant_any(nbits, axis, a, st);
}
hipError_t launch_pack(int nbits, int axis, const CodecArgs &a, hipStream_t st)
{
    return pack_any(nbits, axis, a, st);
}
hipError_t launch_unpack(int nbits, int axis, const CodecArgs &a, hipStream_t st)
{
    return unpack_any(nbits, axis, a, st);
}

}  // namespace hqq
