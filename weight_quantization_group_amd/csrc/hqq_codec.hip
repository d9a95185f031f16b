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

// Metadata quantization (quant_scale / quant_zero, devpress.csdn.net
// tutorial section 3.3): 8-bit min-max RTN of a flattened fp32 array in groups
// of gs consecutive values (the last group may be shorter) -- the solve's
// set-up and final codes at iters = 0.  The kernels take up to kMetaBatch
// arrays per launch: a model has two small meta arrays per layer, and one
// launch per array would cost more in launch latency than in memory time.

// Array of a meta batch that workgroup blk belongs to (uniform; count <= 64).
__device__ inline int meta_item(const MetaBatch &b, int64_t blk)
{
    // a launch has fewer than 2^31 workgroups: 32-bit scalar compares
    int j = 0;
    for (int k = 1; k < b.count; ++k)
        j = (uint32_t)blk >= (uint32_t)b.block0[k] ? k : j;
    return j;
}

// Code of value v in a group with scale s and zero z.
__device__ inline uint32_t meta_code(float v, float s, float z)
{
    return (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(__builtin_fmaf(v, s, z)), 0.0f, 255.0f);
}

// Scale and zero of a group from its minimum and maximum (range 0: s = 1).
__device__ inline void meta_scale_zero(float mn, float mx, float &s, float &z)
{
    const float rng = mx - mn;
    s = rng == 0.0f ? 1.0f : 255.0f / rng;
    z = rng == 0.0f ? -mn : -(mn * s);
}

// Generic path (any gs, any 4-byte alignment): one wave per group, each lane
// taking every 64th value; the wave walks its share of the block's groups.
__device__ void meta_quant_generic(const MetaBatch &b, int j, int gs, int64_t g0, int groups)
{
    const int lane = threadIdx.x & 63;
    const int64_t n = b.n[j];
    for (int k = threadIdx.x >> 6; k < groups; k += 4) {
        const int64_t g = g0 + k;
        const int64_t e0 = g * gs;
        if (e0 >= n)
            return;
        const float *meta = b.meta[j] + e0;
        uint8_t *codes = b.codes[j] + e0;
        const int len = (int)(n - e0 < gs ? n - e0 : gs);
        float mn = meta[0], mx = meta[0];
        for (int i = lane; i < len; i += 64) {
            mn = fminf(mn, meta[i]);
            mx = fmaxf(mx, meta[i]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        float s, z;
        meta_scale_zero(mn, mx, s, z);
        for (int i = lane; i < len; i += 64)
            codes[i] = (uint8_t)meta_code(meta[i], s, z);
        if (lane == 0) {
            b.mscale[j][g] = s;
            b.mzero[j][g] = z;
        }
    }
}

// Vector path (gs = 2^LG in [16, 1024], meta 16-byte and codes 4-byte
// aligned): L = min(64, gs / 4) lanes share a group and each loads F =
// max(1, gs / 256) float4 of it; a wave covers 64 / L groups per slot and its
// four slots' loads are all issued before the first reduction, so 4 KB per
// wave are in flight.  The group's last, shorter group is read value by value.
template <int LG>
__device__ void meta_quant_vec(const MetaBatch &b, int j, int64_t g0)
{
    constexpr int GS = 1 << LG;
    constexpr int L = GS / 4 < 64 ? GS / 4 : 64;
    constexpr int F = GS / 256 > 1 ? GS / 256 : 1;
    constexpr int PER = 64 / L;   // groups per slot
    const int lane = threadIdx.x & 63;
    const int sub = lane / L, r = lane % L;
    const int64_t n = b.n[j];
    const float *meta = b.meta[j];
    const int64_t gw = g0 + (int64_t)(threadIdx.x >> 6) * 4 * PER;   // the wave's first group
    float v[4][F][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t e0 = (gw + u * PER + sub) * GS;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int64_t e = e0 + (int64_t)(f * L + r) * 4;
            if (e0 + GS <= n) {
                const float4 q = *reinterpret_cast<const float4 *>(meta + e);
                v[u][f][0] = q.x, v[u][f][1] = q.y, v[u][f][2] = q.z, v[u][f][3] = q.w;
            } else if (e0 < n) {
                // the array's last group: values past n repeat its first value
                const float first = meta[e0];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    v[u][f][c] = e + c < n ? meta[e + c] : first;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    v[u][f][c] = 0.0f;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t g = gw + u * PER + sub;
        const int64_t e0 = g * GS;
        float mn = v[u][0][0], mx = v[u][0][0];
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mn = fminf(mn, v[u][f][c]);
                mx = fmaxf(mx, v[u][f][c]);
            }
#pragma unroll
        for (int o = L / 2; o > 0; o >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        if (e0 >= n)
            continue;
        float s, z;
        meta_scale_zero(mn, mx, s, z);
        uint8_t *codes = b.codes[j];
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int64_t e = e0 + (int64_t)(f * L + r) * 4;
            const uint32_t c0 = meta_code(v[u][f][0], s, z), c1 = meta_code(v[u][f][1], s, z);
            const uint32_t c2 = meta_code(v[u][f][2], s, z), c3 = meta_code(v[u][f][3], s, z);
            if (e0 + GS <= n) {
                *reinterpret_cast<uint32_t *>(codes + e) = c0 | c1 << 8 | c2 << 16 | c3 << 24;
            } else {
                const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (e + c < n)
                        codes[e + c] = (uint8_t)cs[c];
            }
        }
        if (r == 0) {
            b.mscale[j][g] = s;
            b.mzero[j][g] = z;
        }
    }
}

// LG = log2(gs) for the vector path's group sizes, 0 for any other gs.
template <int LG>
__global__ __launch_bounds__(256) void meta_quant_kernel(const MetaBatch b, int gs)
{
    const int64_t blk = blockIdx.x;
    const int j = meta_item(b, blk);
    const int gpb = meta_groups_per_block(gs);
    const int64_t g0 = (blk - b.block0[j]) * gpb;
    if constexpr (LG != 0) {
        if (((uintptr_t)b.meta[j] & 15u) == 0 && ((uintptr_t)b.codes[j] & 3u) == 0) {
            meta_quant_vec<LG>(b, j, g0);
            return;
        }
    }
    meta_quant_generic(b, j, gs, g0, gpb);
}

// meta[i] = (code - zero) / scale of its meta group, IEEE fp32.  A workgroup
// takes 1024 values of one array: four per lane (one uint32 of codes, one
// float4 out) when meta is 16-byte and codes 4-byte aligned, else one value
// at a time.
__global__ __launch_bounds__(256) void meta_dequant_kernel(const MetaBatch b, int gs)
{
    const int64_t blk = blockIdx.x;
    const int j = meta_item(b, blk);
    const int64_t n = b.n[j];
    const int64_t base = (blk - b.block0[j]) * kMetaDequantBlock;
    const uint8_t *codes = b.codes[j];
    const float *ms = b.mscale[j], *mz = b.mzero[j];
    float *meta = b.meta[j];
    if (((uintptr_t)meta & 15u) == 0 && ((uintptr_t)codes & 3u) == 0) {
        const int64_t i = base + threadIdx.x * 4;
        if (i + 4 <= n) {
            const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + i);
            float o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t g = (i + k) / gs;
                o[k] = ((float)((c >> (8 * k)) & 255u) - mz[g]) / ms[g];
            }
            *reinterpret_cast<float4 *>(meta + i) = make_float4(o[0], o[1], o[2], o[3]);
            return;
        }
        for (int64_t e = i; e < n && e < i + 4; ++e)
            meta[e] = ((float)codes[e] - mz[e / gs]) / ms[e / gs];
        return;
    }
    for (int k = 0; k < kMetaDequantBlock; k += 256) {
        const int64_t e = base + k + threadIdx.x;
        if (e < n)
            meta[e] = ((float)codes[e] - mz[e / gs]) / ms[e / gs];
    }
}

}  // namespace

hipError_t launch_quantize_meta(MetaBatch &b, int gs, hipStream_t st)
{
    const int gpb = meta_groups_per_block(gs);
    int64_t blocks = 0;
    for (int j = 0; j < b.count; ++j) {
        b.block0[j] = blocks;
        blocks += ((b.n[j] + gs - 1) / gs + gpb - 1) / gpb;
    }
    b.block0[b.count] = blocks;
    const dim3 grid((unsigned)blocks), block(256);
    switch (gs) {
    case 16: hipLaunchKernelGGL(meta_quant_kernel<4>, grid, block, 0, st, b, gs); break;
    case 32: hipLaunchKernelGGL(meta_quant_kernel<5>, grid, block, 0, st, b, gs); break;
    case 64: hipLaunchKernelGGL(meta_quant_kernel<6>, grid, block, 0, st, b, gs); break;
    case 128: hipLaunchKernelGGL(meta_quant_kernel<7>, grid, block, 0, st, b, gs); break;
    case 256: hipLaunchKernelGGL(meta_quant_kernel<8>, grid, block, 0, st, b, gs); break;
    case 512: hipLaunchKernelGGL(meta_quant_kernel<9>, grid, block, 0, st, b, gs); break;
    case 1024: hipLaunchKernelGGL(meta_quant_kernel<10>, grid, block, 0, st, b, gs); break;
    default: hipLaunchKernelGGL(meta_quant_kernel<0>, grid, block, 0, st, b, gs); break;
    }
    return hipGetLastError();
}

hipError_t launch_dequantize_meta(MetaBatch &b, int gs, hipStream_t st)
{
    int64_t blocks = 0;
    for (int j = 0; j < b.count; ++j) {
        b.block0[j] = blocks;
        blocks += (b.n[j] + kMetaDequantBlock - 1) / kMetaDequantBlock;
    }
    b.block0[b.count] = blocks;
    hipLaunchKernelGGL(meta_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, b, gs);
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
