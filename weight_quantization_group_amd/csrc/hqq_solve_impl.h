// hqq_solve_impl.h -- the HQQ solve kernels for gfx950 (included by the
// per-bit-width translation units hqq_solve_b{1,2,3,4}.hip).
//
// Method (lnwmold.com HQQ guide, section 2.1: calibration-free half-quadratic
// splitting into alternating sub-problems; devpress.csdn.net "dropbox/hqq"
// tutorial, section 2: auxiliary error variable, robust non-convex loss;
// section 2.2 of the guide and section 3.3 of the tutorial: nbits,
// group_size, axis).  Per group of gs weights w, qmax = 2^b - 1:
//   scale = qmax / (max - min), zero = -(min * scale)
//   iters times: W_q = clamp(rne(w*scale + zero), 0, qmax)
//                W_e = shrink_p(w - (W_q - zero)/scale, beta)
//                zero = (sum W_q - scale * (sum w - sum W_e)) / gs
//                beta *= kappa
//   codes = clamp(rne(w*scale + zero), 0, qmax)
//
// Mapping to CDNA4.  The solve is elementwise work plus per-group sums: no
// dense contraction, so no MFMA.  One lane owns a whole group: its gs weights
// cross HBM once (DMA into LDS one group ahead of the solve, then into VGPRs),
// are widened exactly to fp32 and stay in VGPRs for all iterations; min, max
// and the sums are in-lane, so the 64 lanes of a wave run 64 independent
// groups with no cross-lane traffic.  Where C (codes per uint32) and gs do
// not divide each other (3-bit, or gs < C) a lane owns lcm(gs, C) consecutive
// elements of a line (several groups, solved one after the other), so every
// packed word is assembled in-register by one lane and written once.
// axis = 1: lanes take consecutive blocks of a row; axis = 0: lanes take
// consecutive columns, so each access of a wave covers 64 consecutive columns.
//
// Exactness.  The arithmetic is the fp32 evaluation with w*scale+zero as one
// fma and the mean in fp64: sum W_q (small integers) and sum w (fp16 values)
// are exact in fp64 in any order; sum W_e is the pairwise tree over adjacent
// elements.  W_e = 0 exactly when |x| <= tau_k = beta_k^(-1/(1-(p-1))); the
// host passes thr <= 0.98 * min_k tau_k.  |x_i| * scale is within a tiny,
// bounded error of |t_i - q_i|, t_i = w_i*scale + zero, and
// max_i |t_i - q_i| <= max(0.5, -t(min w), t(max w) - qmax) because the fma
// is monotone in w.
//   fast loop:  while that bound is below thr*scale (and the group's
//               magnitude keeps the estimate's error far below the 2% margin)
//               every W_e of the group is 0 and the update is
//               (sum W_q - scale * sum w) / gs: per weight one fma and one
//               round-and-pack to a byte (v_cvt_pk_u8_f32), and two byte-sums
//               per four weights that apply the clamp to the sum.  That update
//               reads the zero only through the codes and no later iteration
//               can fail the test (thr bounds every iteration), so once an
//               update returns the zero it was given, every later one does:
//               the group stops there with the result of all iterations.
//   freeze:     a group that fails the test stops in its lane (the lane idles
//               while the wave's other groups finish their iterations).
//   finish:     the wave then completes its frozen groups together, one lane
//               per element (64/gs groups at a time): every residual the
//               estimate cannot clear is evaluated exactly (IEEE division,
//               |x|^(p-1) in fp64 rounded once to fp32) and the sums are
//               butterflies across the group's lanes -- for sum W_e exactly
//               the pairwise tree.  Rare, outlier-heavy groups therefore cost
//               a short SIMD phase instead of a long serial tail.
#pragma once
#include <type_traits>

#include "hqq_internal.h"

namespace hqq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = kSolveBlock;
constexpr int kWaves = kBlock / 64;

__device__ __forceinline__ float quant(float w, float s, float z, float qmax)
{
    return __builtin_amdgcn_fmed3f(__builtin_rintf(__builtin_fmaf(w, s, z)), 0.0f, qmax);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b)
{
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f)   // exact for fp16 values
{
    const _Float16 h = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// Input weights are fp16 (BF = false) or bf16 (BF = true) bits; both widen
// to fp32 exactly, and an fp32 value that came from them narrows back
// exactly (bf16: the top 16 bits).
template <bool BF>
__device__ __forceinline__ float widen(uint16_t b)
{
    if constexpr (BF)
        return __uint_as_float((uint32_t)b << 16);
    else
        return half_bits_to_float(b);
}

template <bool BF>
__device__ __forceinline__ uint16_t narrow(float f)
{
    if constexpr (BF)
        return (uint16_t)(__float_as_uint(f) >> 16);
    else
        return float_to_half_bits(f);
}

// Two values that came from 16-bit weights, narrowed back into one word (lo
// in the low half).  fp16: v_cvt_pkrtz_f16_f32, whose rounding toward zero
// is exact on fp16 values (subnormals included: fp16 denormals are not
// flushed), one instruction per pair.
template <bool BF>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi)
{
    if constexpr (BF) {
        return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    } else {
        const auto h = __builtin_amdgcn_cvt_pkrtz(lo, hi);
        uint32_t u;
        __builtin_memcpy(&u, &h, 4);
        return u;
    }
}

// eight 16-bit values of a 16-byte vector, widened to fp32
template <bool BF>
__device__ __forceinline__ void widen8(u32x4 v, float *out)
{
    if constexpr (BF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    } else {
        _Float16 h[8];
        __builtin_memcpy(h, &v, 16);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i] = (float)h[i];
    }
}

// Column line of rows eg..eg+gs-1, widened to fp32.  The pointer advances one
// row per load (the empty asm keeps the compiler from holding gs addresses).
template <int GS, bool BF>
__device__ __forceinline__ void load_column(const uint16_t *__restrict__ W, int64_t cols, int64_t line,
                                            int64_t eg, float (&w)[GS])
{
    const uint16_t *q = W + eg * cols + line;
#pragma unroll
    for (int i = 0; i < GS; ++i) {
        w[i] = widen<BF>(__builtin_nontemporal_load(q));
        q += cols;
        asm volatile("" : "+v"(q));
    }
}

// Load one group (gs fp16 values) directly from global memory and widen
// exactly to fp32.
template <int GS, int AXIS, bool BF>
__device__ __forceinline__ void load_group(const uint16_t *__restrict__ W, int64_t cols,
                                           int64_t line, int64_t e0, float (&w)[GS])
{
    if constexpr (AXIS == 1) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(W + line * cols + e0);
#pragma unroll
        for (int j = 0; j < GS / 8; ++j) {
            u32x4 v = __builtin_nontemporal_load(src + j);
            widen8<BF>(v, &w[j * 8]);
        }
    } else {
        load_column<GS, BF>(W, cols, line, e0, w);
    }
}

// Sum of the group's weights in fp64.  fp16 values are multiples of 2^-24
// below 2^16, so any partial sum of <= 256 of them is an integer multiple of
// 2^-24 below 2^24, exactly representable in fp64: the order is free.  bf16
// values span a far wider range, so their sum is formed in index order (the
// order the method's mean states), rounding where it must.
template <int GS, bool BF>
__device__ __forceinline__ double exact_sum(const float (&w)[GS])
{
    if constexpr (BF) {
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < GS; ++i)
            acc += (double)w[i];
        return acc;
    }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < GS; ++i)
        acc[i & 3] += (double)w[i];
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// |x|^(p-1) evaluated in fp64 and rounded once to fp32 (x > 0 finite).
// exp((p-1) ln x): ln x = k ln2 + 2 atanh(u), u = (m-1)/(m+1) for the
// significand m in [sqrt(1/2), sqrt(2)) (the atanh power series to u^21);
// exp by reduction y = j ln2 + r, |r| <= ln2/2, and its Taylor polynomial to
// r^13.  Relative error ~1e-15, far below the fp32 rounding it feeds.
// Kept out of line: it runs only for the residuals of frozen groups, and
// inlined its fp64 temporaries would set the register budget of the whole
// kernel (149 VGPRs instead of 121 at gs = 64).
__device__ __attribute__((noinline)) float pow_rounded(float xf, float pm1f)
{
    int e;
    double m = frexp((double)xf, &e);
    if (m < 0.70710678118654752440) {
        m *= 2.0;
        e -= 1;
    }
    const double f = m - 1.0;
    const double u = f / (2.0 + f);
    const double u2 = u * u;
    double p = 1.0 / 21;
    p = __builtin_fma(p, u2, 1.0 / 19);
    p = __builtin_fma(p, u2, 1.0 / 17);
    p = __builtin_fma(p, u2, 1.0 / 15);
    p = __builtin_fma(p, u2, 1.0 / 13);
    p = __builtin_fma(p, u2, 1.0 / 11);
    p = __builtin_fma(p, u2, 1.0 / 9);
    p = __builtin_fma(p, u2, 1.0 / 7);
    p = __builtin_fma(p, u2, 1.0 / 5);
    p = __builtin_fma(p, u2, 1.0 / 3);
    const double lnm = __builtin_fma(2.0 * u, u2 * p, 2.0 * u);
    const double lnx = __builtin_fma((double)e, 0.69314718055994530942, lnm);
    double y = (double)pm1f * lnx;
    y = fmin(fmax(y, -800.0), 800.0);
    const double j = rint(y * 1.44269504088896340736);
    double r = __builtin_fma(-j, 0.69314718055994530942, y);
    r = __builtin_fma(-j, 2.319046813846299558e-17, r);
    double q = 1.0 / 6227020800.0;
    q = __builtin_fma(q, r, 1.0 / 479001600.0);
    q = __builtin_fma(q, r, 1.0 / 39916800.0);
    q = __builtin_fma(q, r, 1.0 / 3628800.0);
    q = __builtin_fma(q, r, 1.0 / 362880.0);
    q = __builtin_fma(q, r, 1.0 / 40320.0);
    q = __builtin_fma(q, r, 1.0 / 5040.0);
    q = __builtin_fma(q, r, 1.0 / 720.0);
    q = __builtin_fma(q, r, 1.0 / 120.0);
    q = __builtin_fma(q, r, 1.0 / 24.0);
    q = __builtin_fma(q, r, 1.0 / 6.0);
    q = __builtin_fma(q, r, 0.5);
    q = __builtin_fma(q, r, 1.0);
    q = __builtin_fma(q, r, 1.0);
    return (float)ldexp(q, (int)j);
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Layout of the finish phase: a frozen group is spread over SEG lanes with EPL
// consecutive elements each; B groups are finished at once.
template <int GS>
struct Finish {
    static constexpr int SEG = GS < 64 ? GS : 64;
    static constexpr int EPL = GS / SEG;
    static constexpr int B = 64 / SEG;
};

struct FrozenGroup {   // state of a frozen group handed to the finish phase
    float s, z, beta, mn, mx, amag;
    int it;
    int pad;
    double sw;
};

// Compact mode of the fast loop (32 <= gs <= 128): once at most B groups of a
// wave still iterate, they are spread over SEG = gs/8 lanes each (8 elements
// per lane) and the wave advances all of them in one pass per iteration.
template <int GS>
struct Compact {
    static constexpr bool ON = GS >= 32 && GS <= 128;
    static constexpr int SEG = ON ? GS / 8 : 1;
    static constexpr int B = 64 / SEG;
};

struct CompactGroup {   // a group in compact mode: LaneRun and GroupInit fields
    float s, z, mn, mx, amag, beta;
    int it, frozen;
    double sw;
};

template <int GS>
struct WaveFinish {
    uint16_t w[64 * Finish<GS>::EPL];    // B groups x GS fp16 weights
    FrozenGroup g[Finish<GS>::B];
    u32x4 cw[Compact<GS>::ON ? 64 : 1];                       // slot b, chunk j at [b SEG + j]
    CompactGroup cg[Compact<GS>::ON ? Compact<GS>::B : 1];
};

// Pack a group's final codes into the work item's words.  8-bit: a word is
// four clamped bytes.  4-, 2- and 1-bit groups of whole bytes: the codes as
// bytes (v_cvt_pk_u8_f32 of the clamped value: round half to even of
// clamp(t) equals clamp of the rounded t) in R = 8 / nbits byte words whose
// byte k holds code R k + r of the word's run, so the packed word (or the
// group's part of one) is (R - 1) shift-ors of them, LSB first.  Other
// formats: code by code.  TOP = false: the caller has shown that no t of the
// group rounds above qmax and that t is never NaN; the conversion's
// saturation at 0 is then the whole clamp.
template <int NB, int GS, int G, int WPB, bool TOP = true>
__device__ __forceinline__ void pack_codes(const float (&w)[GS], float s, float z,
                                           uint32_t (&words)[WPB])
{
    constexpr int C = codes_per_word(NB);
    constexpr float QMAX = (float)((1 << NB) - 1);
    auto clamped = [&](float x) {
        const float t = __builtin_fmaf(x, s, z);
        return TOP ? __builtin_amdgcn_fmed3f(t, 0.0f, QMAX) : t;
    };
    if constexpr ((NB == 4 || NB == 2 || NB == 1) && GS % 8 == 0 && (G * GS) % (C < GS ? C : GS) == 0) {
        constexpr int R = 8 / NB;                       // byte words per packed word
        constexpr int RUN = C < GS ? C : GS;            // codes per run (a word, or the group's part of one)
        constexpr int NBYTE = RUN / R;                  // bytes per byte word
#pragma unroll
        for (int q = 0; q < GS / RUN; ++q) {
            uint32_t x = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t d = 0;
#pragma unroll
                for (int k = 0; k < NBYTE; ++k)
                    d = __builtin_amdgcn_cvt_pk_u8_f32(clamped(w[RUN * q + R * k + r]), k, d);
                x = r == 0 ? d : (d << (NB * r)) | x;
            }
            const int n0 = G * GS + RUN * q;
            words[n0 / C] |= x << ((n0 % C) * NB);
        }
    } else if constexpr (NB == 8) {
        // four codes per word: the word is the four clamped bytes
#pragma unroll
        for (int q = 0; q < GS / 4; ++q) {
            uint32_t d = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d = __builtin_amdgcn_cvt_pk_u8_f32(clamped(w[4 * q + j]), j, d);
            words[(G * GS) / 4 + q] = d;
        }
    } else {
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const int n = G * GS + i;
            words[n / C] |= (uint32_t)quant(w[i], s, z, QMAX) << ((n % C) * NB);
        }
    }
}

// Sum over the SEG lanes of a group (aligned blocks of 2, 4, 8 or 16
// lanes) with DPP row permutations; every lane gets the total.
template <int SEG>
__device__ __forceinline__ int seg_sum(int v)
{
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);          // quad_perm [1,0,3,2]
    if constexpr (SEG >= 4)
        v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);      // quad_perm [2,3,0,1]
    if constexpr (SEG >= 8)
        v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);     // row_half_mirror
    if constexpr (SEG >= 16)
        v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);     // row_mirror
    return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

// The same block sums in fp64: each level adds the sibling block's sum, as
// a butterfly does (fp64 addition commutes, so the result is the pairwise
// tree's, bit for bit).
template <int SEG>
__device__ __forceinline__ double seg_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);
    if constexpr (SEG >= 4)
        v += dpp_f64<0x4E>(v);
    if constexpr (SEG >= 8)
        v += dpp_f64<0x141>(v);
    if constexpr (SEG >= 16)
        v += dpp_f64<0x140>(v);
    return v;
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

// Finish the nb frozen groups staged in an area with fields w (B groups x GS
// 16-bit weights) and g (their FrozenGroup states): one lane per element (EPL
// consecutive elements per lane), every remaining iteration with the exact
// residual and shrink; each group's final zero is written back to g[slot].z.
template <int NB, int GS, bool BF, typename A>
__device__ __forceinline__ void finish_staged(const SolveArgs &a, A &wf, int nb)
{
    using F = Finish<GS>;
    constexpr float QMAX = (float)((1 << NB) - 1);
    constexpr double INV_GS = 1.0 / GS;
    const uint32_t lane = __lane_id();
    const int slot = (int)lane / F::SEG;
    const int pos = (int)lane % F::SEG;
    const bool ok = slot < nb;
    const FrozenGroup st = wf.g[ok ? slot : 0];
    float we[F::EPL];
#pragma unroll
    for (int k = 0; k < F::EPL; ++k)
        we[k] = widen<BF>(wf.w[(ok ? slot : 0) * GS + pos * F::EPL + k]);
    const float gs_s = st.s;
    const float thr_s = a.thr * gs_s;
    const float lim = a.thr_m * gs_s;
    float gz = st.z, gbeta = st.beta;
    int it = ok ? st.it : a.iters;
    while (__any(it < a.iters)) {
        const bool act = it < a.iters;
        // certificate of the group for the current zero
        const float tmin = __builtin_fmaf(st.mn, gs_s, gz);
        const float tmax = __builtin_fmaf(st.mx, gs_s, gz);
        const float bound = fmaxf(0.5f, fmaxf(-tmin, tmax - QMAX));
        const bool est_ok = __builtin_fmaf(st.amag, gs_s, fabsf(gz)) + QMAX <= lim;
        const bool cand = !(est_ok && bound <= thr_s);
        uint32_t ck[F::EPL];
        double te[F::EPL];
#pragma unroll
        for (int k = 0; k < F::EPL; ++k) {
            const float t = __builtin_fmaf(we[k], gs_s, gz);
            const float qk = __builtin_amdgcn_fmed3f(__builtin_rintf(t), 0.0f, QMAX);
            ck[k] = (uint32_t)qk;
            float e = 0.0f;
            if (act && cand && !(est_ok && fabsf(t - qk) <= thr_s)) {
                const float wr = (qk - gz) / gs_s;
                const float x = we[k] - wr;
                const float ax = fabsf(x);
                if (ax > a.thr) {
                    const float pw = pow_rounded(ax, a.pm1);
                    const float v = ax - pw / gbeta;
                    if (v > 0.0f)
                        e = copysignf(v, x);
                }
            }
            te[k] = (double)e;
        }
        // in-lane levels of W_e's pairwise tree
#pragma unroll
        for (int st2 = 1; st2 < F::EPL; st2 *= 2)
#pragma unroll
            for (int k = 0; k + st2 < F::EPL; k += 2 * st2)
                te[k] += te[k + st2];
        double se = te[0];
        int sqi;
        if constexpr (F::EPL > 2) {
            // gs = 256 (four elements per lane, every register in use): the
            // butterfly through LDS for both sums
            float sf = 0.0f;
#pragma unroll
            for (int k = 0; k < F::EPL; ++k)
                sf += (float)ck[k];
#pragma unroll
            for (int m = 1; m < F::SEG; m *= 2) {
                sf += __shfl_xor(sf, m);
                se += __shfl_xor(se, m);
            }
            sqi = (int)sf;
        } else if constexpr (F::SEG == 64) {
            // one group per pass.  sum W_q: the codes are integers (exact in
            // any order), counted bit by bit with ballots.  sum W_e: where at
            // most two lanes hold a nonzero partial sum, the tree's result is
            // their sum (every other term is an exact +0), read with
            // readlane; otherwise the butterfly.
            sqi = 0;
#pragma unroll
            for (int bit = 0; bit < NB; ++bit) {
#pragma unroll
                for (int k = 0; k < F::EPL; ++k)
                    sqi += __popcll(__ballot((ck[k] >> bit) & 1u)) << bit;
            }
            const uint64_t nz = __ballot(se != 0.0);
            if (__popcll(nz) <= 2) {
                double v = 0.0;
                if (nz) {
                    v = readlane_f64(se, __builtin_ctzll(nz));
                    if (nz & (nz - 1ull))
                        v = v + readlane_f64(se, 63 - __builtin_clzll(nz));
                }
                se = v;
            } else {
                se = seg_sum_f64<16>(se);
                se += __shfl_xor(se, 16);
                se += __shfl_xor(se, 32);
            }
        } else {
            // the butterfly across the group's lanes, by DPP within rows of
            // 16 lanes (and one exchange between rows at gs = 32)
            int cs = 0;
#pragma unroll
            for (int k = 0; k < F::EPL; ++k)
                cs += (int)ck[k];
            constexpr int R = F::SEG < 16 ? F::SEG : 16;
            sqi = seg_sum<R>(cs);
            se = seg_sum_f64<R>(se);
            if constexpr (F::SEG == 32) {
                sqi += __shfl_xor(sqi, 16);
                se += __shfl_xor(se, 16);
            }
        }
        const float sq = (float)sqi;
        const float zn = (float)(((double)sq - (double)gs_s * (st.sw - se)) * INV_GS);
        if (act) {
            // where the certificate holds every W_e is 0 and the update is
            // the fast one: a returned zero is then a fixed point
            const bool fixed = !cand && zn == gz;
            gz = zn;
            gbeta = gbeta * a.kappa;
            it = fixed ? a.iters : it + 1;
        }
    }
    if (ok && pos == 0)
        wf.g[slot].z = gz;
    wave_sync();
}

// The frozen lanes' groups (one group per lane) through finish_staged, up to
// Finish::B at a time in lane order; z returns each group's final zero.
template <int NB, int GS, bool BF>
__device__ __forceinline__ void finish_frozen(const SolveArgs &a, WaveFinish<GS> &wf, bool frozen,
                                              const float (&w)[GS], float s, float &z, float beta,
                                              float mn, float mx, float amag, int it_f, double sw)
{
    using F = Finish<GS>;
    const uint32_t lane = __lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    uint64_t pending = __ballot(frozen);
    while (pending) {
        // the next (up to) B frozen groups, in lane order
        uint64_t take = 0;
#pragma unroll
        for (int b = 0; b < F::B; ++b) {
            if (pending & ~take)
                take |= (pending & ~take) & (~(pending & ~take) + 1ull);
        }
        pending &= ~take;
        const int nb = __popcll(take);
        const bool mine = (take >> lane) & 1ull;
        if (mine) {
            const int slot = __popcll(take & below);
#pragma unroll
            for (int i = 0; i < GS; ++i)
                wf.w[slot * GS + i] = narrow<BF>(w[i]);
            wf.g[slot] = FrozenGroup{s, z, beta, mn, mx, amag, it_f, 0, sw};
        }
        wave_sync();
        finish_staged<NB, GS, BF>(a, wf, nb);
        if (mine)
            z = wf.g[__popcll(take & below)].z;
        wave_sync();
    }
}

// Occupancy target (waves per SIMD): the largest at which the kernel needs
// no scratch.  A spill reload is a vector memory load, and the in-order
// vmcnt would make it wait for the DMA of the next group as well.
constexpr int waves_per_simd(int nb, int gs)
{
    return nb == 3   ? (gs == 8 ? 5 : gs <= 32 ? 4 : gs == 64 ? 3 : 1)
           : nb == 8 ? (gs == 8 ? 6 : gs == 16 ? 5 : gs == 32 ? 4 : gs == 64 ? 3 : gs == 128 ? 2 : 1)
           : nb == 1 && gs == 8 ? 5
                              : (gs <= 16 ? 6 : gs == 32 ? 5 : gs == 64 ? 4 : gs == 128 ? 2 : 1);
}

// Per-group set-up: min, max, scale, initial zero, exact sum of the weights.
struct GroupInit {
    float mn, mx, s, z, amag;
    double sw;
};

template <int NB, int GS, bool BF>
__device__ __forceinline__ GroupInit group_init(const float (&w)[GS])
{
    constexpr float QMAX = (float)((1 << NB) - 1);
    GroupInit g;
    g.mn = w[0];
    g.mx = w[0];
#pragma unroll
    for (int i = 1; i < GS; ++i) {
        g.mn = fminf(g.mn, w[i]);
        g.mx = fmaxf(g.mx, w[i]);
    }
    const float rng = g.mx - g.mn;
    if (rng == 0.0f) {
        g.s = 1.0f;
        g.z = -g.mn;
    } else {
        g.s = QMAX / rng;
        g.z = -(g.mn * g.s);
    }
    g.sw = exact_sum<GS, BF>(w);
    g.amag = fmaxf(fabsf(g.mn), fabsf(g.mx));
    return g;
}

// Where a lane's group stands in the fast loop.
struct LaneRun {
    float z;        // current zero
    float beta;     // beta of iteration `it`
    int it;         // next iteration
    bool run;       // still iterating
    bool frozen;    // certificate failed at iteration it (beta is its beta)
};

// Compact mode: the running lanes' groups (at most B) move to LDS, SEG lanes
// per group iterate them with the same update as the fast loop (codes by
// v_cvt_pk_u8_f32, sums by v_sad_u8, the lanes' partial sums added exactly),
// and the owners take back zero, iteration, beta and frozen.
template <int NB, int GS, bool BF>
__device__ __forceinline__ void compact_iters(const SolveArgs &a, WaveFinish<GS> &wf, const float (&w)[GS],
                                           const GroupInit &g, LaneRun &r)
{
    using K = Compact<GS>;
    constexpr double INV_GS = 1.0 / GS;
    constexpr float QMAX = (float)((1 << NB) - 1);
    constexpr uint32_t QB = (uint32_t)((1 << NB) - 1) * 0x01010101u;
    const uint32_t lane = __lane_id();
    const uint64_t run_m = __ballot(r.run);
    const int nrun = __popcll(run_m);
    const int mine = __popcll(run_m & ((1ull << lane) - 1ull));
    if (r.run) {
#pragma unroll
        for (int j = 0; j < GS / 8; ++j) {
            uint32_t hw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hw[i] = narrow2<BF>(w[8 * j + 2 * i], w[8 * j + 2 * i + 1]);
            wf.cw[mine * K::SEG + j] = u32x4{hw[0], hw[1], hw[2], hw[3]};
        }
        wf.cg[mine] = CompactGroup{g.s, r.z, g.mn, g.mx, g.amag, r.beta, r.it, 0, g.sw};
    }
    wave_sync();
    const int b = (int)lane / K::SEG;
    const bool act = b < nrun;
    const CompactGroup st = wf.cg[act ? b : 0];
    float we[8];
    {
        const u32x4 v = wf.cw[(act ? b : 0) * K::SEG + (int)lane % K::SEG];
        widen8<BF>(v, we);
    }
    const float s = st.s;
    const float thr_s = a.thr * s;
    const float lim = a.thr_m * s;
    const double ssw = (double)s * st.sw;
    float z = st.z, beta = st.beta;
    int it = st.it;
    bool frozen = false;
    // a divergent loop: a group's SEG lanes take every decision from the
    // same sums, so they leave it together, and the DPP sums only read lanes
    // of the group, which are then all still in it
    if (act) {
        while (true) {
            const float tmin = __builtin_fmaf(st.mn, s, z);
            const float tmax = __builtin_fmaf(st.mx, s, z);
            const float bound = fmaxf(0.5f, fmaxf(-tmin, tmax - QMAX));
            const bool est_ok = __builtin_fmaf(st.amag, s, fabsf(z)) + QMAX <= lim;
            if (!(est_ok && bound <= thr_s)) {
                frozen = true;
                break;
            }
            uint32_t d0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[0], s, z), 0, 0u);
            uint32_t d1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[4], s, z), 0, 0u);
#pragma unroll
            for (int j = 1; j < 4; ++j) {
                d0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[j], s, z), j, d0);
                d1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(we[4 + j], s, z), j, d1);
            }
            const uint32_t c = __builtin_amdgcn_sad_u8(d1, 0u, __builtin_amdgcn_sad_u8(d0, 0u, 0u));
            const uint32_t q = __builtin_amdgcn_sad_u8(d1, QB, __builtin_amdgcn_sad_u8(d0, QB, 0u));
            const int tot = seg_sum<K::SEG>((int)c - (int)q);
            const uint32_t sq = (uint32_t)(tot + GS * ((1 << NB) - 1)) >> 1;
            const float zn = (float)(((double)sq - ssw) * INV_GS);
            it = zn == z ? a.iters : it + 1;
            beta = beta * a.kappa;
            z = zn;
            if (it >= a.iters)
                break;
        }
    }
    wave_sync();
    if (act && (int)lane % K::SEG == 0) {
        wf.cg[b].z = z;
        wf.cg[b].beta = beta;
        wf.cg[b].it = it;
        wf.cg[b].frozen = frozen ? 1 : 0;
    }
    wave_sync();
    if (r.run) {
        const CompactGroup o = wf.cg[mine];
        r.z = o.z;
        r.beta = o.beta;
        r.it = o.it;
        r.frozen = o.frozen != 0;
        r.run = false;
    }
    wave_sync();
}

// sum W_q of one fast iteration.  v_cvt_pk_u8_f32 rounds half to even and
// saturates to [0, 255] (the clamp at 0), four codes to a word; v_sad_u8
// against 0 adds a word's four codes c.  TOP: also against qmax in every
// byte, giving sum |c - qmax|, and min(c, qmax) = (c + qmax - |c - qmax|) / 2:
// 2.5 VALU ops per weight, 2 without.
template <int NB, int GS, bool TOP>
__device__ __forceinline__ uint32_t code_sum(const float (&w)[GS], float s, float z)
{
    static_assert(GS % 8 == 0, "two byte-sum chains of whole words");
    constexpr uint32_t QB = (uint32_t)((1 << NB) - 1) * 0x01010101u;
    uint32_t c0 = 0, c1 = 0, a0 = 0, a1 = 0;
#pragma unroll
    for (int k = 0; k < GS / 4; k += 2) {
        uint32_t d0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(w[4 * k + 0], s, z), 0, 0u);
        uint32_t d1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(w[4 * k + 4], s, z), 0, 0u);
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            d0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(w[4 * k + j], s, z), j, d0);
            d1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(w[4 * k + 4 + j], s, z), j, d1);
        }
        c0 = __builtin_amdgcn_sad_u8(d0, 0u, c0);
        c1 = __builtin_amdgcn_sad_u8(d1, 0u, c1);
        if constexpr (TOP) {
            a0 = __builtin_amdgcn_sad_u8(d0, QB, a0);
            a1 = __builtin_amdgcn_sad_u8(d1, QB, a1);
        }
    }
    if constexpr (TOP)
        return ((c0 + c1) + (uint32_t)(GS * ((1 << NB) - 1)) - (a0 + a1)) >> 1;
    return c0 + c1;
}

// Fast iterations of the lanes with r.run, up to iters: a lane freezes its
// group at the first iteration whose certificate fails, and stops once its
// zero is a fixed point (r.it = iters then).  With wf: compact mode once at
// most Compact::B groups of the wave still iterate.  The loop is divergent:
// a lane leaves it when its group freezes or is done (the hardware's exec
// mask carries that state, so the loop keeps no per-lane flags), and the
// wave-wide choices -- compact mode, the clamp at qmax -- are ballots over
// the lanes still in it.
template <int NB, int GS, bool BF>
__device__ __forceinline__ void fast_iters(const SolveArgs &a, const float (&w)[GS], const GroupInit &g,
                                           LaneRun &r, WaveFinish<GS> *wf = nullptr)
{
    constexpr float QMAX = (float)((1 << NB) - 1);
    constexpr double INV_GS = 1.0 / GS;
    const float s = g.s;
    const float thr_s = a.thr * s;
    const float lim = a.thr_m * s;
    const double ssw = (double)s * g.sw;
    float z = r.z, beta = r.beta;
    int it = r.it;
    bool frozen = false, compact = false;
    if (r.run && a.iters > 0) {
        while (true) {
            if constexpr (Compact<GS>::ON) {
                if (wf != nullptr && __popcll(__ballot(1)) <= Compact<GS>::B) {
                    compact = true;
                    break;
                }
            }
            const float tmin = __builtin_fmaf(g.mn, s, z);
            const float tmax = __builtin_fmaf(g.mx, s, z);
            const float bound = fmaxf(0.5f, fmaxf(-tmin, tmax - QMAX));
            const bool est_ok = __builtin_fmaf(g.amag, s, fabsf(z)) + QMAX <= lim;
            if (!(est_ok && bound <= thr_s)) {
                frozen = true;
                break;
            }
            // The clamp at qmax can bind only where the largest weight's t
            // rounds above qmax (the fma is monotone in w); when no lane of
            // the wave still iterating is there (uniform branch), the codes
            // are summed without it.  8-bit codes never need it: the
            // conversion saturates at 255.
            const bool top = NB < 8 && __any(!(tmax < QMAX + 0.5f));
            // (the clamped variant adds +0 to the zero, which changes no
            // code -- t = +-0 gives code 0 either way -- and keeps the two
            // variants' fmas apart: merged above the branch, their gs
            // results would all be live at once)
            uint32_t sq;
            if (top)
                sq = code_sum<NB, GS, true>(w, s, z + 0.0f);
            else
                sq = code_sum<NB, GS, false>(w, s, z);
            const float zn = (float)(((double)sq - ssw) * INV_GS);
            // Fixed point: the next zero depends on the current one only
            // through the codes, which are equal for equal zeros (+0 and -0
            // included), and the certificate is the same for every remaining
            // iteration; so every later iteration returns zn again, bit for
            // bit, and the group is done.
            it = zn == z ? a.iters : it + 1;
            beta = beta * a.kappa;
            z = zn;
            if (it >= a.iters)
                break;
        }
    }
    r.z = z;
    r.beta = beta;
    r.it = it;
    r.frozen = frozen;
    r.run = compact;
    if constexpr (Compact<GS>::ON) {
        if (__any(compact))
            compact_iters<NB, GS, BF>(a, *wf, w, g, r);
    }
}

// Finish: frozen lanes complete their iterations together (one lane per
// element); then every valid lane packs its final codes.
template <int NB, int GS, int G, int AXIS, int WPB, bool BF>
__device__ __forceinline__ void finish_group(const SolveArgs &a, const SolveTensor &T, WaveFinish<GS> &wf,
                                             bool valid, int64_t line, int64_t eg, const float (&w)[GS],
                                             const GroupInit &g, LaneRun &r, uint32_t (&words)[WPB])
{
    // uniform choice of the packing without the clamp at qmax: every packing
    // lane's largest t rounds to at most qmax and its group holds no NaN
    // (the exact sum would be NaN)
    constexpr float QMAX = (float)((1 << NB) - 1);
    const bool packing = valid && !r.frozen;
    const bool top = __any(packing && !(__builtin_fmaf(g.mx, g.s, r.z) < QMAX + 0.5f && g.sw == g.sw));
    if (top) {
        if (packing)
            pack_codes<NB, GS, G, WPB, true>(w, g.s, r.z, words);
    } else {
        if (packing)
            pack_codes<NB, GS, G, WPB, false>(w, g.s, r.z, words);
    }
    if (__any(r.frozen)) {
        finish_frozen<NB, GS, BF>(a, wf, r.frozen, w, g.s, r.z, r.beta, g.mn, g.mx, g.amag, r.it, g.sw);
        if (r.frozen) {
            float w2[GS];
            load_group<GS, AXIS, BF>(T.W, T.cols, line, eg, w2);
            pack_codes<NB, GS, G>(w2, g.s, r.z, words);
        }
    }
}

template <int NB, int GS, int G, int AXIS, int WPB, bool BF>
__device__ __forceinline__ void solve_one(const SolveArgs &a, const SolveTensor &T,
                                          WaveFinish<GS> &wf, bool valid, int64_t line, int64_t eg,
                                          const float (&w)[GS], uint32_t (&words)[WPB],
                                          float &s_out, float &z_out)
{
    // Lanes without a valid group hold in-bounds weights (staged from the
    // item's first group) and run the set-up on them; they never enter the
    // loop and their results are not stored.
    const GroupInit g = group_init<NB, GS, BF>(w);
    LaneRun r{g.z, a.beta0, 0, valid, false};
    fast_iters<NB, GS, BF>(a, w, g, r, &wf);
    finish_group<NB, GS, G, AXIS, WPB, BF>(a, T, wf, valid, line, eg, w, g, r, words);
    s_out = g.s;
    z_out = r.z;
}

// Shape of the work item of a kernel: lcm(gs, C) consecutive elements of a
// line, so that whole words belong to one lane.
template <int NB, int GS, int AXIS>
struct Item {
    static constexpr int C = codes_per_word(NB);
    static constexpr int LB = lcm_c(GS, C);      // elements per work item
    static constexpr int GSEQ = LB / GS;         // groups per work item
    static constexpr int WPB = LB / C;           // words per work item
};

// Where a work item lies: its line, first element and valid groups.
struct ItemPos {
    int64_t line, e0;
    int ng;
};

template <int NB, int GS, int AXIS>
__device__ __forceinline__ ItemPos item_pos(const SolveTensor &T, int64_t item)
{
    using I = Item<NB, GS, AXIS>;
    const bool live = item < T.n_items;
    const int64_t it_c = live ? item : 0;
    ItemPos p;
    // quotient by the tensor's divisor through its fp64 reciprocal: the
    // product is within one of the quotient (item < 2^53), the remainder
    // test corrects it; the quotient is a row or block index (< 2^31)
    const int64_t dv = AXIS == 1 ? T.nblk : T.cols;
    int64_t q = (int64_t)(uint32_t)((double)it_c * T.rdiv);
    int64_t r = it_c - q * dv;
    if (r < 0) {
        q -= 1;
        r += dv;
    } else if (r >= dv) {
        q += 1;
        r -= dv;
    }
    int64_t blk;
    if constexpr (AXIS == 1) {
        p.line = q;
        blk = r;
    } else {
        blk = q;
        p.line = r;
    }
    const int64_t L = AXIS == 1 ? T.cols : T.rows;
    p.e0 = blk * I::LB;
    const int64_t rem = (L - p.e0) / GS;
    p.ng = live ? (rem < I::GSEQ ? (int)rem : I::GSEQ) : 0;
    return p;
}

// Staging of one group per wave in LDS, filled by DMA one group ahead:
// gs rows of 64 lanes x 2 bytes (row i of lane l at [i][l]).  axis = 1: lane
// l's group is gs consecutive halves, fetched as gs/8 16-byte chunks
// (global_load_lds_dwordx4 puts lane l's 16 bytes at base + 16 l, so chunk j
// of lane l lands at [8j..8j+7][l] read as 16-byte rows).  axis = 0: lane l's
// group is column line_l of rows eg..eg+gs-1; when the wave's 64 columns are
// consecutive and 16-byte aligned (cols % 64 == 0), 8 lanes fetch one row's
// 128 bytes, so a 16-byte DMA moves 8 rows and the data lands row-major.
// Other axis = 0 shapes are read directly from global memory when the group
// is solved (a sub-dword DMA gives every lane a whole dword, which would
// double the staging area).  Every address is inside the tensor.
template <int GS, int AXIS>
struct Stage {
    u32x4 v[GS / 8][64];
};

template <int GS, int AXIS>
__device__ __forceinline__ void stage_group(const SolveTensor &T, int64_t line, int64_t eg, bool rows64,
                                            Stage<GS, AXIS> &st)
{
    typedef __attribute__((address_space(3))) void *lds_ptr;
    const int lane = (int)(threadIdx.x & 63);
    if constexpr (AXIS == 1) {
        const uint16_t *src = T.W + line * T.cols + eg;
#pragma unroll
        for (int j = 0; j < GS / 8; ++j)
            __builtin_amdgcn_global_load_lds(src + 8 * j, (lds_ptr)&st.v[j][0], 16, 0, 0);
    } else {
        if (rows64) {
            const int64_t c0 = line - lane;                  // the wave's first column
            const uint16_t *src = T.W + (eg + (lane >> 3)) * T.cols + c0 + 8 * (lane & 7);
            const int64_t step = 8 * T.cols;
#pragma unroll
            for (int j = 0; j < GS / 8; ++j)
                __builtin_amdgcn_global_load_lds(src + j * step, (lds_ptr)&st.v[j][0], 16, 0, 0);
        }
    }
}

// Read this lane's staged group (or, for axis = 0 shapes that are not
// staged, load it) and widen it exactly to fp32.
template <int GS, int AXIS, bool BF>
__device__ __forceinline__ void read_group(const Stage<GS, AXIS> &st, const SolveTensor &T, int64_t line,
                                           int64_t eg, bool rows64, float (&w)[GS])
{
    const int lane = (int)(threadIdx.x & 63);
    if constexpr (AXIS == 1) {
#pragma unroll
        for (int j = 0; j < GS / 8; ++j) {
            const u32x4 v = st.v[j][lane];
            widen8<BF>(v, &w[8 * j]);
        }
    } else {
        if (rows64) {
            const uint16_t(*rows)[64] = reinterpret_cast<const uint16_t(*)[64]>(&st.v[0][0]);
#pragma unroll
            for (int i = 0; i < GS; ++i)
                w[i] = widen<BF>(rows[i][lane]);
        } else {
            load_column<GS, BF>(T.W, T.cols, line, eg, w);
        }
    }
    // The group stays resident as fp32 only: without this the compiler keeps
    // the fp16 originals alive too (to fold the widening into later fmas),
    // which doubles the group's registers.
#pragma unroll
    for (int i = 0; i < GS; ++i)
        asm volatile("" : "+v"(w[i]));
}

// Write a finished work item: packed words, then scale and zero per group.
template <int NB, int GS, int AXIS>
__device__ __forceinline__ void store_item(const SolveTensor &T, const ItemPos &p,
                                           const uint32_t (&words)[Item<NB, GS, AXIS>::WPB],
                                           const float (&sv)[Item<NB, GS, AXIS>::GSEQ],
                                           const float (&zv)[Item<NB, GS, AXIS>::GSEQ])
{
    using I = Item<NB, GS, AXIS>;
    constexpr int C = I::C, WPB = I::WPB;
    const int64_t L = AXIS == 1 ? T.cols : T.rows;
    const int64_t words_per_line = (L + C - 1) / C;
    const int64_t k0 = p.e0 / C;
#pragma unroll
    for (int g = 0; g < I::GSEQ; ++g) {
        if (g < p.ng) {
            const int64_t eg = p.e0 + (int64_t)g * GS;
            const int64_t gi = AXIS == 1 ? p.line * (L / GS) + eg / GS : (eg / GS) * T.cols + p.line;
            T.scale[gi] = sv[g];
            T.zero[gi] = zv[g];
        }
    }
    // Words go out through L2 (ordinary stores) so that lanes' partial lines
    // merge before reaching HBM.  axis = 1: a lane's words are contiguous and
    // leave as 16-byte stores when the row pitch allows; axis = 0: each word
    // store of the wave covers 64 consecutive columns.
    if constexpr (AXIS == 1 && WPB % 4 == 0) {
        if ((words_per_line & 3) == 0 && p.ng == I::GSEQ) {
            u32x4 *dst = reinterpret_cast<u32x4 *>(T.packed + p.line * words_per_line + k0);
#pragma unroll
            for (int k = 0; k < WPB / 4; ++k)
                dst[k] = u32x4{words[4 * k], words[4 * k + 1], words[4 * k + 2], words[4 * k + 3]};
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < WPB; ++k) {
        if (k * C < p.ng * GS && k0 + k < words_per_line) {
            const int64_t addr = AXIS == 1 ? p.line * words_per_line + k0 + k : (k0 + k) * T.cols + p.line;
            T.packed[addr] = words[k];
        }
    }
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;     // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, F, I + 1>(static_cast<F &&>(f));
    }
}

// A workgroup owns depth * 256 consecutive work items of one tensor; at step m
// lane l of the workgroup takes item base + 256 m + l and solves its groups
// in order.  Per group: wait for its DMA, read it into registers, start the
// DMA of the lane's next group, solve the group; a finished item is stored.
// The loads of a group thus overlap the solve of the one before.
template <int NB, int GS, int AXIS, bool BF>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(waves_per_simd(NB, GS))))
void solve_kernel(SolveArgs a)
{
    using I = Item<NB, GS, AXIS>;
    constexpr int GSEQ = I::GSEQ, WPB = I::WPB;
    __shared__ WaveFinish<GS> finish[kWaves];
    __shared__ Stage<GS, AXIS> stage[kWaves];

    // the launch's tensor of this workgroup: block0 is increasing and
    // tensors start on workgroup boundaries (uniform, no dependent loads;
    // a launch has fewer than 2^31 workgroups, so 32-bit scalar compares)
    int ti = 0;
#pragma unroll
    for (int j = 1; j < kMaxBatch; ++j)
        ti = (j < a.n && blockIdx.x >= (uint32_t)a.block0[j]) ? j : ti;
    const SolveTensor &T = a.t[ti];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    Stage<GS, AXIS> &st = stage[wave];
    WaveFinish<GS> &wf = finish[wave];
    const int64_t first = ((int64_t)blockIdx.x - a.block0[ti]) * kBlock * a.depth + threadIdx.x;
    const int64_t wave_first = first - (threadIdx.x & 63);
    // axis = 0 waves cover 64 consecutive, 16-byte aligned columns of one
    // row block exactly when cols % 64 == 0 (items start at multiples of 64)
    const bool rows64 = AXIS == 0 && (T.cols & 63) == 0;

    // first element of group G of item q, or of the item's first group when
    // G is not valid (always inside the tensor)
    auto group_e = [](const ItemPos &q, int G) { return q.e0 + (int64_t)(G < q.ng ? G : 0) * GS; };
    auto stage_of = [&](const ItemPos &q, int G) { stage_group<GS, AXIS>(T, q.line, group_e(q, G), rows64, st); };
    if (wave_first < T.n_items)
        stage_of(item_pos<NB, GS, AXIS>(T, first), 0);
    for (int m = 0; m < a.depth; ++m) {
        // every lane of a wave with work stays to the end of the step: lanes
        // past the last item own no group but take part in the finish phases
        if (wave_first + (int64_t)m * kBlock >= T.n_items)
            break;
        const ItemPos p = item_pos<NB, GS, AXIS>(T, first + (int64_t)m * kBlock);
        const bool more = m + 1 < a.depth && wave_first + (int64_t)(m + 1) * kBlock < T.n_items;
        uint32_t words[WPB];
#pragma unroll
        for (int k = 0; k < WPB; ++k)
            words[k] = 0;
        float sv[GSEQ], zv[GSEQ];
        static_for<GSEQ>([&](auto Gc) {
            constexpr int G = decltype(Gc)::value;
            float w[GS];
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            read_group<GS, AXIS, BF>(st, T, p.line, group_e(p, G), rows64, w);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            if constexpr (G + 1 < GSEQ)
                stage_of(p, G + 1);
            else if (more)
                stage_of(item_pos<NB, GS, AXIS>(T, first + (int64_t)(m + 1) * kBlock), 0);
            solve_one<NB, GS, G, AXIS, I::WPB, BF>(a, T, wf, G < p.ng, p.line, p.e0 + (int64_t)G * GS, w, words,
                                       sv[G], zv[G]);
        });
        store_item<NB, GS, AXIS>(T, p, words, sv, zv);
    }
}

}  // namespace
}  // namespace hqq

#include "hqq_solve_seg.h"

namespace hqq {
namespace {

template <int NB, int GS, int AXIS, bool BF>
void launch_one(dim3 grid, dim3 block, const SolveArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((solve_kernel<NB, GS, AXIS, BF>), grid, block, 0, st, a);
}

template <int NB, int AXIS, bool BF>
hipError_t launch_gs(int group_size, const SolveArgs &a, hipStream_t st)
{
    const dim3 block(kBlock);
    const dim3 grid((unsigned)a.blocks);
    switch (group_size) {
    case 8: launch_one<NB, 8, AXIS, BF>(grid, block, a, st); break;
    case 16: launch_one<NB, 16, AXIS, BF>(grid, block, a, st); break;
    case 32: launch_one<NB, 32, AXIS, BF>(grid, block, a, st); break;
    case 64: launch_one<NB, 64, AXIS, BF>(grid, block, a, st); break;
    case 128: launch_one<NB, 128, AXIS, BF>(grid, block, a, st); break;
    case 256: launch_one<NB, 256, AXIS, BF>(grid, block, a, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// launcher of the NB-bit solve kernels for fp16 (BF = false) or bf16 inputs
// (defined in hqq_solve_b<NB>.hip and hqq_solve_b<NB>_bf16.hip)
template <int NB, bool BF>
hipError_t launch_solve_nb(int group_size, int axis, int map, const SolveArgs &a, hipStream_t st)
{
    if (map != kMapLane) {
        if constexpr (NB != 3 && !BF) {
            const dim3 block(kBlock);
            const dim3 grid((unsigned)a.blocks);
            if (map == kMapSeg) {
                switch (group_size) {
                case 32: hipLaunchKernelGGL((solve_seg_kernel<NB, 32, 1>), grid, block, 0, st, a); break;
                case 64: hipLaunchKernelGGL((solve_seg_kernel<NB, 64, 1>), grid, block, 0, st, a); break;
                case 128: hipLaunchKernelGGL((solve_seg_kernel<NB, 128, 1>), grid, block, 0, st, a); break;
                default: return hipErrorInvalidValue;
                }
            } else {
                switch (group_size) {
                case 32:
                    if constexpr (NB != 1)
                        hipLaunchKernelGGL((solve_seg_kernel<NB, 32, 2>), grid, block, 0, st, a);
                    else
                        return hipErrorInvalidValue;
                    break;
                case 64: hipLaunchKernelGGL((solve_seg_kernel<NB, 64, 2>), grid, block, 0, st, a); break;
                case 128: hipLaunchKernelGGL((solve_seg_kernel<NB, 128, 2>), grid, block, 0, st, a); break;
                default: return hipErrorInvalidValue;
                }
            }
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    return axis == 1 ? launch_gs<NB, 1, BF>(group_size, a, st) : launch_gs<NB, 0, BF>(group_size, a, st);
}

}  // namespace hqq
