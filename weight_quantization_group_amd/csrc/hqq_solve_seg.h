// hqq_solve_seg.h -- the axis = 1 solve with several lanes per group, for
// launches too small to fill the device with one lane per group.
//
// Included by hqq_solve_impl.h after the lane-per-group kernel, whose
// helpers it uses (widen8, seg_sum, FrozenGroup, Finish, finish_staged,
// wave_sync, Item).  Formats: axis = 1, 32 <= gs <= 128, fp16 weights, every
// code width whose words tile a group (all but 3 bits).
//
// Layout: a lane holds CH chunks of 8 consecutive weights of one group (CH = 1
// or 2), SEG = gs / (8 CH) lanes hold a group, and a wave holds B = 64 / SEG
// consecutive groups of the tensor.  Chunk k of lane j is the group's chunk
// k SEG + j, so that every 16-byte load, every store of packed words and the
// staging of frozen groups are contiguous across the wave's lanes (along axis
// 1 the groups of a tensor follow each other in memory: cols is a multiple of
// gs).  Loads are issued a step ahead.  The per-group quantities of the HQQ
// solve (lnwmold.com HQQ guide, section 2.1: alternating W_q / W_e / zero
// updates; section 2.2: nbits, group_size, axis) are formed across the
// group's lanes with DPP: min and max, the exact fp64 sum of the weights
// (every partial sum of at most 128 fp16 values is exact in fp64, so the lane
// order cannot change it), and the sum of the codes (integers).  The
// certificate, the fixed-point stop and the exact finish of frozen groups are
// the lane-per-group kernel's, so every output is identical bit for bit.  The
// wave runs until its slowest of B groups is done instead of its slowest of
// 64; two chunks per lane halve the per-group work (certificate, zero update,
// reductions) per weight, for twice the groups per wave.
#pragma once

namespace hqq {
namespace {

template <int GS, int CH>
struct Seg {
    static constexpr int SEG = GS / (8 * CH);   // lanes per group
    static constexpr int B = 64 / SEG;          // groups per wave
};

template <int GS>
struct SegFinish {
    alignas(16) uint16_t w[64 * Finish<GS>::EPL];   // staged frozen groups (fp16 bits)
    FrozenGroup g[Finish<GS>::B];
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Reductions over the SEG lanes of a group (aligned blocks of 2, 4, 8 or 16
// lanes): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror; every lane of the block gets the result.  All 64 lanes must be
// active.
template <int SEG>
__device__ __forceinline__ float seg_min(float v)
{
    v = fminf(v, dpp_f32<0xB1>(v));
    if constexpr (SEG >= 4)
        v = fminf(v, dpp_f32<0x4E>(v));
    if constexpr (SEG >= 8)
        v = fminf(v, dpp_f32<0x141>(v));
    if constexpr (SEG >= 16)
        v = fminf(v, dpp_f32<0x140>(v));
    return v;
}

template <int SEG>
__device__ __forceinline__ float seg_max(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v));
    if constexpr (SEG >= 4)
        v = fmaxf(v, dpp_f32<0x4E>(v));
    if constexpr (SEG >= 8)
        v = fmaxf(v, dpp_f32<0x141>(v));
    if constexpr (SEG >= 16)
        v = fmaxf(v, dpp_f32<0x140>(v));
    return v;
}

// Occupancy target: the largest at which the kernel needs no scratch (the
// out-of-line power of the frozen finish sets the register count; a spill
// would make the wave wait for the next step's load at once).
constexpr int seg_waves_per_simd(int gs, int ch)
{
    return ch == 1 ? (gs == 64 ? 6 : 5) : (gs == 128 ? 4 : 5);
}

// A workgroup owns kWaves * B * depth consecutive groups of one tensor, its
// waves B * depth each; a step of a wave solves B groups.
template <int NB, int GS, int CH>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(seg_waves_per_simd(GS, CH))))
void solve_seg_kernel(SolveArgs a)
{
    using S = Seg<GS, CH>;
    using F = Finish<GS>;
    constexpr int C = codes_per_word(NB);
    constexpr float QMAX = (float)((1 << NB) - 1);
    constexpr uint32_t QB = (uint32_t)((1 << NB) - 1) * 0x01010101u;
    constexpr double INV_GS = 1.0 / GS;
    static_assert(GS >= 32 && GS <= 128 && GS % C == 0 && NB != 3 && (CH == 1 || CH == 2) && S::SEG >= 2,
                  "format of the multi-lane kernel");
    // a word of 1-bit codes is 4 chunks: those of 4 consecutive lanes of a group
    static_assert(NB != 1 || S::SEG % 4 == 0, "1-bit codes need 4 lanes per word");
    __shared__ SegFinish<GS> finish[kWaves];

    int ti = 0;
#pragma unroll
    for (int j = 1; j < kMaxBatch; ++j)
        ti = (j < a.n && blockIdx.x >= (uint32_t)a.block0[j]) ? j : ti;
    ti = __builtin_amdgcn_readfirstlane(ti);
    const SolveTensor &T = a.t[ti];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    SegFinish<GS> &wf = finish[wave];
    const int lane = (int)(threadIdx.x & 63);
    const int b = lane / S::SEG;     // the lane's group in the step
    const int j = lane % S::SEG;     // its chunks: k SEG + j of the group, k < CH
    const int64_t per_wave = (int64_t)S::B * a.depth;
    const int64_t g0 = ((int64_t)blockIdx.x - a.block0[ti]) * kWaves * per_wave + wave * per_wave;
    const int64_t gend = g0 + per_wave < T.n_items ? g0 + per_wave : T.n_items;
    if (g0 >= gend)
        return;

    // lanes past the tensor's last group read that group (in bounds) and
    // store nothing
    auto load = [&](int64_t gbase, u32x4 (&out)[CH]) {
        int64_t gi = gbase + b;
        gi = gi < T.n_items ? gi : T.n_items - 1;
#pragma unroll
        for (int k = 0; k < CH; ++k)
            out[k] = *reinterpret_cast<const u32x4 *>(T.W + gi * GS + 8 * (k * S::SEG + j));
    };
    u32x4 next[CH];
    load(g0, next);
    for (int64_t gb = g0; gb < gend; gb += S::B) {
        u32x4 raw[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k)
            raw[k] = next[k];
        if (gb + S::B < gend)
            load(gb + S::B, next);
        const int64_t gi = gb + b;
        const bool valid = gi < gend;
        float we[8 * CH];
#pragma unroll
        for (int k = 0; k < CH; ++k)
            widen8<false>(raw[k], &we[8 * k]);

        // set-up: the lane-per-group kernel's min, max, scale, zero and sum
        float mn = we[0], mx = we[0];
        double sw = (double)we[0];
#pragma unroll
        for (int k = 1; k < 8 * CH; ++k) {
            mn = fminf(mn, we[k]);
            mx = fmaxf(mx, we[k]);
            sw += (double)we[k];
        }
        mn = seg_min<S::SEG>(mn);
        mx = seg_max<S::SEG>(mx);
        sw = seg_sum_f64<S::SEG>(sw);
        const float rng = mx - mn;
        float s, z;
        if (rng == 0.0f) {
            s = 1.0f;
            z = -mn;
        } else {
            s = QMAX / rng;
            z = -(mn * s);
        }
        const float amag = fmaxf(fabsf(mn), fabsf(mx));
        const float thr_s = a.thr * s;
        const float lim = a.thr_m * s;
        const double ssw = (double)s * sw;

        // iterations under the certificate, as in the lane-per-group kernel.
        // The loop is divergent: a group's lanes take every decision from the
        // same sums, so they leave it together, and the DPP sums only read
        // lanes of the group, which are then all still in it.
        float beta = a.beta0;
        int it = 0;
        bool frozen = false;
        if (valid && a.iters > 0) {
            while (true) {
                const float tmin = __builtin_fmaf(mn, s, z);
                const float tmax = __builtin_fmaf(mx, s, z);
                const float bound = fmaxf(0.5f, fmaxf(-tmin, tmax - QMAX));
                const bool est_ok = __builtin_fmaf(amag, s, fabsf(z)) + QMAX <= lim;
                if (!(est_ok && bound <= thr_s)) {
                    frozen = true;
                    break;
                }
                uint32_t c = 0u, q = 0u;
#pragma unroll
                for (int h = 0; h < 2 * CH; ++h) {
                    uint32_t d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[4 * h], s, z), 0, 0u);
#pragma unroll
                    for (int k = 1; k < 4; ++k)
                        d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[4 * h + k], s, z), k, d);
                    c = __builtin_amdgcn_sad_u8(d, 0u, c);
                    q = __builtin_amdgcn_sad_u8(d, QB, q);
                }
                const int tot = seg_sum<S::SEG>((int)c - (int)q);
                const uint32_t sq = (uint32_t)(tot + GS * ((1 << NB) - 1)) >> 1;
                const float zn = (float)(((double)sq - ssw) * INV_GS);
                it = zn == z ? a.iters : it + 1;
                beta = beta * a.kappa;
                z = zn;
                if (it >= a.iters)
                    break;
            }
        }

        // frozen groups: staged by their lanes, finished F::B at a time with
        // the exact residual and shrink
        {
            const int lead = lane - j;   // the group's first lane
            uint64_t pending = __ballot(frozen && j == 0);
            while (pending) {
                uint64_t take = 0;
#pragma unroll
                for (int k = 0; k < F::B; ++k) {
                    if (pending & ~take)
                        take |= (pending & ~take) & (~(pending & ~take) + 1ull);
                }
                pending &= ~take;
                const int nb = __popcll(take);
                const bool mine = (take >> lead) & 1ull;
                const int slot = __popcll(take & ((1ull << lead) - 1ull));
                if (mine) {
#pragma unroll
                    for (int k = 0; k < CH; ++k)
                        *reinterpret_cast<u32x4 *>(&wf.w[slot * GS + 8 * (k * S::SEG + j)]) = raw[k];
                    if (j == 0)
                        wf.g[slot] = FrozenGroup{s, z, beta, mn, mx, amag, it, 0, sw};
                }
                wave_sync();
                finish_staged<NB, GS, false>(a, wf, nb);
                if (mine)
                    z = wf.g[slot].z;
                wave_sync();
            }
        }

        // final codes at the final zero, packed and stored chunk by chunk: chunk
        // p = k SEG + j of the group holds codes 8p .. 8p + 7
        uint32_t *gw = T.packed + gi * (GS / C);   // the group's words (axis 1: groups are contiguous)
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int p = k * S::SEG + j;
            auto code = [&](int e) { return __builtin_amdgcn_fmed3f(__builtin_fmaf(we[8 * k + e], s, z), 0.0f, QMAX); };
            // the chunk's eight codes packed LSB first (8 bits: two words of
            // bytes; else R = 8 / nbits byte words, byte i of word r holding
            // code R i + r, joined by R - 1 shift-ors)
            uint32_t d0 = 0, d1 = 0, h = 0;
            if constexpr (NB == 8) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    d0 = __builtin_amdgcn_cvt_pk_u8_f32(code(e), e, d0);
                    d1 = __builtin_amdgcn_cvt_pk_u8_f32(code(4 + e), e, d1);
                }
            } else {
                constexpr int R = 8 / NB;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t d = 0;
#pragma unroll
                    for (int i = 0; i < 8 / R; ++i)
                        d = __builtin_amdgcn_cvt_pk_u8_f32(code(R * i + r), i, d);
                    h = r == 0 ? d : (d << (NB * r)) | h;
                }
            }
            if constexpr (NB == 8) {
                if (valid)
                    *reinterpret_cast<uint2 *>(gw + 2 * p) = uint2{d0, d1};
            } else if constexpr (NB == 4) {
                if (valid)
                    gw[p] = h;
            } else if constexpr (NB == 2) {
                // a word holds the 16 codes of chunks p, p + 1 (lanes j, j + 1, j even)
                const uint32_t w = h | ((uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0xB1, 0xF, 0xF, false) << 16);
                if (valid && (j & 1) == 0)
                    gw[p >> 1] = w;
            } else {
                // a word holds the 32 codes of chunks p .. p + 3 (lanes j .. j + 3, j % 4 == 0)
                const uint32_t w = h | ((uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x55, 0xF, 0xF, false) << 8) |
                                   ((uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0xAA, 0xF, 0xF, false) << 16) |
                                   ((uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0xFF, 0xF, 0xF, false) << 24);
                if (valid && (j & 3) == 0)
                    gw[p >> 2] = w;
            }
        }
        if (valid && j == 0) {
            T.scale[gi] = s;
            T.zero[gi] = z;
        }
    }
}

}  // namespace
}  // namespace hqq
