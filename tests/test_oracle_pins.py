"""Pins of the CPU oracle to facts other than its own code.

Each test pins one part of the solve to something the method or the
mathematics fixes independently of how the oracle is written:
  - iters = 0 is min-max round-to-nearest (RTN), a textbook closed form
    (ainews.cool Dropbox-HQQ analysis, benchmark table: RTN as the
    iteration-free baseline);
  - p = 1 turns the lp shrinkage into soft thresholding (textbook);
  - each zero update is the minimiser of a quadratic, found here by brute
    force over a grid (lnwmold.com HQQ guide, section 2.1: each alternating
    sub-problem is solved exactly);
  - codes stay in [0, 2^b - 1]; pack/unpack round-trips and matches
    hand-derived words; weights on the quantization grid are a fixed point;
  - with W_e = 0 the alternation never increases the quadratic objective;
  - fp16 <-> fp32 conversions equal numpy's (a library routine).
"""
import math

import numpy as np
import pytest

from helpers import f16_bits_to_f32, fma_f32, random_f16

QMAX = {1: 1, 2: 3, 3: 7, 4: 15, 8: 255}


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------

def test_f16_to_f32_all_patterns(oracle_mod):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_rne(oracle_mod):
    rng = np.random.RandomState(1)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 70000.0, -1e9,
                     2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25,
                     2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                     1.0 + 3 * 2.0 ** -11, 1e-8, np.inf, -np.inf], dtype=np.float32)
    rand = np.concatenate([
        (rng.randn(40000) * 0.05).astype(np.float32),
        (rng.randn(20000) * 1e-5).astype(np.float32),
        np.exp(rng.uniform(-20, 11.5, 20000)).astype(np.float32),
        # halfway points between neighbouring fp16 values: ties must go to even
        ((np.arange(1, 10001, dtype=np.float32).astype(np.float16).astype(np.float32)
          + np.float32(0.5))),
    ])
    x = np.concatenate([edge, rand])
    got = oracle_mod.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# RTN at iters = 0
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_iters0_is_minmax_rtn(oracle_mod, nbits):
    rng = np.random.RandomState(10 + nbits)
    qmax = QMAX[nbits]
    for gs in (8, 16, 64):
        W16 = random_f16(rng, (32, gs), std=0.02, outlier_frac=0.01)
        w = f16_bits_to_f32(W16)
        codes, scale, zero = oracle_mod.quantize_codes(W16, nbits, gs, 1, iters=0)
        mn = w.min(axis=1)
        mx = w.max(axis=1)
        s = np.float32(qmax) / (mx - mn)                  # fp32 division
        z = -(mn * s)                                     # fp32 multiply, negated
        assert np.array_equal(scale[:, 0], s)
        assert np.array_equal(zero[:, 0], z)
        t = fma_f32(w, s[:, None], z[:, None])
        ref = np.clip(np.rint(t), 0, qmax).astype(np.uint8)
        assert np.array_equal(codes, ref)
        # textbook RTN in exact rational arithmetic: code = round((w - min) / (max - min) * qmax);
        # equal except where fp32 rounding of the scale moves a value across a .5 boundary
        exact = (w.astype(np.float64) - mn[:, None]) / (mx - mn)[:, None].astype(np.float64) * qmax
        frac = np.abs(exact - np.floor(exact) - 0.5)
        sure = frac > 1e-4
        assert np.array_equal(codes[sure], np.rint(exact[sure]).astype(np.uint8))
        # the min element gets code 0 and the max element qmax
        assert np.all(codes[np.arange(32), w.argmin(axis=1)] == 0)
        assert np.all(codes[np.arange(32), w.argmax(axis=1)] == qmax)


def test_constant_group(oracle_mod):
    for v in (0.0, 0.125, -3.5):
        w = np.full(16, v, np.float32)
        r = oracle_mod.solve_group(w, 4, iters=20)
        assert r["scale"] == 1.0
        assert r["zero"] == -v
        assert np.all(r["codes"] == 0)


# --------------------------------------------------------------------------
# the shrinkage
# --------------------------------------------------------------------------

def test_p1_is_soft_threshold(oracle_mod):
    for beta in (10.0, 12.08, 0.5, 1e3):
        b = np.float32(beta)
        thr = np.float32(1.0) / b
        base = [0.0, -0.0, 1e-40, -1e-40, 1e-30, 0.5, -0.5, 2.0, -7.0, 123.0]
        near = [float(thr), float(-thr),
                float(np.nextafter(thr, np.float32(1))), float(np.nextafter(thr, np.float32(0))),
                float(-np.nextafter(thr, np.float32(1))), float(-np.nextafter(thr, np.float32(0)))]
        rng = np.random.RandomState(3)
        xs = np.array(base + near + list(rng.randn(200) * 3 * thr), dtype=np.float32)
        for x in xs:
            got = oracle_mod.shrink(float(x), 1.0, float(b))
            a = np.float32(abs(x))
            v = np.float32(a - thr)
            ref = float(np.copysign(v, x)) if v > 0 else 0.0
            assert got == ref, (x, beta, got, ref)


def test_shrink_matches_fp64_formula(oracle_mod):
    """W_e = sign(x) max(|x| - |x|^(p-1)/beta, 0) against an fp64 evaluation."""
    rng = np.random.RandomState(4)
    xs = np.concatenate([rng.randn(2000) * 0.3, rng.randn(500) * 3]).astype(np.float32)
    for p in (0.7, 0.5, 0.9, 1.3):
        for beta in (10.0, 2.0, 0.01):
            for x in xs:
                got = oracle_mod.shrink(float(x), p, beta)
                a = abs(float(x))
                v = a - (a ** (float(np.float32(p) - np.float32(1.0))) if a > 0 else math.inf) / beta
                ref = math.copysign(v, x) if v > 0 else 0.0
                tol = 4 * np.spacing(np.float32(max(a, 1e-30))) + 1e-6 * abs(ref)
                assert abs(got - ref) <= tol, (x, p, beta, got, ref)


def test_shrink_zero_residual(oracle_mod):
    # |x|^(p-1) at x = 0 is +inf for p < 1 and 1 for p = 1; W_e must be 0, never NaN
    for p in (0.3, 0.7, 1.0, 1.5):
        assert oracle_mod.shrink(0.0, p, 10.0) == 0.0
        assert oracle_mod.shrink(-0.0, p, 10.0) == 0.0


# --------------------------------------------------------------------------
# per-iteration pins on traces
# --------------------------------------------------------------------------

def _grid_argmin(c: np.ndarray, lo, hi) -> float:
    """argmin_z sum((c - z)^2) by brute force: coarse grid, then two refinements."""
    step = (hi - lo) / 20000.0
    for _ in range(3):
        z = np.arange(lo, hi + step, step)
        f = ((c[None, :] - z[:, None]) ** 2).sum(axis=1)
        k = int(np.argmin(f))
        lo, hi = z[max(k - 2, 0)], z[min(k + 2, len(z) - 1)]
        step = (hi - lo) / 2000.0
    return float(z[k])


@pytest.mark.parametrize("beta0", [10.0, 1000.0])
def test_zero_update_is_quadratic_argmin(oracle_mod, beta0):
    """8-element 2-bit groups: every new zero minimises sum((W_q - (w - W_e) s - z)^2)."""
    rng = np.random.RandomState(5)
    qmax = 3
    nz_e = 0
    for trial in range(30):
        w = (rng.randn(8) * 0.4).astype(np.float16).astype(np.float32)
        if trial % 3 == 0:
            w[rng.randint(8)] *= 8
        r = oracle_mod.solve_group(w, 2, iters=6, beta0=beta0, kappa=1.01, trace=True)
        s = r["scale"]
        for k in range(6):
            q, e = r["q"][k].astype(np.float64), r["e"][k].astype(np.float64)
            nz_e += int(np.count_nonzero(e))
            c = q - (w.astype(np.float64) - e) * s
            zg = _grid_argmin(c, -2 * qmax, 3 * qmax)
            zn = float(r["zero_trace"][k + 1])
            assert abs(zn - zg) <= 1e-5 + 1e-6 * abs(zg), (trial, k, zn, zg)
    if beta0 > 100:
        assert nz_e > 50   # the shrink was really exercised


def test_codes_follow_current_zero(oracle_mod):
    """W_q of iteration k is RTN at the zero left by iteration k-1 (and the
    output codes are RTN at the final zero)."""
    rng = np.random.RandomState(6)
    for nbits, gs in ((4, 64), (3, 64), (2, 16), (1, 16)):
        qmax = QMAX[nbits]
        for _ in range(10):
            w = f16_bits_to_f32(random_f16(rng, (gs,), std=0.03, outlier_frac=0.05))
            r = oracle_mod.solve_group(w, nbits, iters=8, beta0=1.0, trace=True)
            s = np.float32(r["scale"])
            for k in range(8):
                z = np.float32(r["zero_trace"][k])
                ref = np.clip(np.rint(fma_f32(w, s, z)), 0, qmax)
                assert np.array_equal(r["q"][k], ref)
            ref = np.clip(np.rint(fma_f32(w, s, np.float32(r["zero"]))), 0, qmax)
            assert np.array_equal(r["codes"], ref.astype(np.uint8))


def test_residual_and_beta_schedule(oracle_mod):
    """x = w - (W_q - zero)/scale within fp32 rounding, and with p = 1 the
    shrink of iteration k removes exactly 1/beta_k with beta_k = beta0 kappa^k."""
    rng = np.random.RandomState(7)
    beta0, kappa = 4.0, 1.3
    seen = set()
    for _ in range(20):
        w = f16_bits_to_f32(random_f16(rng, (16,), std=0.5))
        r = oracle_mod.solve_group(w, 2, iters=6, p=1.0, beta0=beta0, kappa=kappa, trace=True)
        s = float(r["scale"])
        for k in range(6):
            z = float(r["zero_trace"][k])
            x64 = w.astype(np.float64) - (r["q"][k].astype(np.float64) - z) / s
            assert np.all(np.abs(r["x"][k] - x64) <= 4e-7 * (np.abs(w) + 1.0))
            e, x = r["e"][k], r["x"][k]
            act = e != 0
            if act.any():
                seen.add(k)
                removed = np.abs(x[act].astype(np.float64)) - np.abs(e[act].astype(np.float64))
                beta_k = beta0 * kappa ** k
                assert np.allclose(removed, 1.0 / beta_k, rtol=1e-5, atol=1e-6), (k, removed)
                assert np.all(np.sign(e[act]) == np.sign(x[act]))
    assert len(seen) >= 4


# --------------------------------------------------------------------------
# fixed point, clamp, descent, symmetry, determinism
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nbits,gs", [(4, 64), (3, 64), (2, 16), (1, 16), (4, 8)])
def test_grid_weights_are_a_fixed_point(oracle_mod, nbits, gs):
    rng = np.random.RandomState(8 + nbits)
    qmax = QMAX[nbits]
    for k in (4, 6, 9):
        d = 2.0 ** -k
        m = rng.randint(-40, 40) * d
        q = rng.randint(0, qmax + 1, size=gs)
        q[rng.randint(gs)] = 0
        q[(rng.randint(gs - 1) + 1 + int(np.argmin(q))) % gs] = qmax
        w = (m + q * d).astype(np.float32)
        assert np.array_equal(w.astype(np.float16).astype(np.float32), w)
        for iters in (0, 1, 20):
            r = oracle_mod.solve_group(w, nbits, iters=iters)
            assert r["scale"] == 1.0 / d
            assert r["zero"] == -m / d
            assert np.array_equal(r["codes"], q.astype(np.uint8))
        # and the whole-tensor path dequantizes them back bit for bit
        W16 = w.astype(np.float16).view(np.uint16).reshape(1, gs)
        packed, scale, zero = oracle_mod.quantize(W16, nbits, gs, 1, iters=20)
        back = oracle_mod.dequantize(packed, scale, zero, 1, gs, nbits, gs, 1)
        assert np.array_equal(back, W16)


@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_codes_in_range_and_axis_layout(oracle_mod, nbits):
    rng = np.random.RandomState(20 + nbits)
    W16 = random_f16(rng, (64, 48), std=0.05, outlier_frac=0.02)
    for axis in (0, 1):
        codes, scale, zero = oracle_mod.quantize_codes(W16, nbits, 16, axis, iters=5)
        assert codes.max() <= QMAX[nbits]
        # axis=0 on W equals axis=1 on W transposed (groups of consecutive rows of a column)
        cT, sT, zT = oracle_mod.quantize_codes(np.ascontiguousarray(W16.T), nbits, 16, 1 - axis,
                                               iters=5)
        assert np.array_equal(codes, cT.T)
        assert np.array_equal(scale, sT.T)
        assert np.array_equal(zero, zT.T)


def _objective(w, s, z, q):
    return float(np.sum((w.astype(np.float64) * s + z - q) ** 2))


@pytest.mark.parametrize("nbits,gs", [(4, 64), (3, 64), (2, 16), (1, 16), (4, 8)])
def test_zero_sequence_monotone_and_settles(oracle_mod, nbits, gs):
    """While every W_e is 0 the zero update reads the zero only through the
    codes, and the codes are a non-decreasing function of the zero (fma, round
    and clamp are monotone): so the zero sequence is monotone, and once an
    update returns the zero it was given, every later one does too, bit for
    bit.  The solve kernels stop a group at that point."""
    rng = np.random.RandomState(70 + nbits * 10 + gs)
    settled = 0
    for _ in range(60):
        w = f16_bits_to_f32(random_f16(rng, (gs,), std=0.02, outlier_frac=0.01))
        r = oracle_mod.solve_group(w, nbits, iters=30, trace=True)   # default p, beta0, kappa
        if np.any(r["e"] != 0):
            continue
        zt = r["zero_trace"].astype(np.float64)
        d = np.diff(zt)
        assert np.all(d >= 0) or np.all(d <= 0), zt
        bits = r["zero_trace"].view(np.uint32)
        rep = np.nonzero(bits[1:] == bits[:-1])[0]
        if rep.size:
            k = int(rep[0])
            assert np.all(bits[k:] == bits[k]), zt
            settled += 1
    assert settled >= 30


@pytest.mark.parametrize("nbits,gs", [(4, 64), (3, 64), (2, 16), (1, 16)])
def test_alternation_descends_when_we_zero(oracle_mod, nbits, gs):
    """With W_e = 0 (beta0 tiny, so the shrink threshold is huge) each half-step minimises J(q, z) = sum (w s + z - q)^2
    over one variable, so J never increases and the result is no worse than RTN."""
    rng = np.random.RandomState(30 + nbits)
    qmax = QMAX[nbits]
    for _ in range(20):
        w = f16_bits_to_f32(random_f16(rng, (gs,), std=0.02, outlier_frac=0.02))
        r = oracle_mod.solve_group(w, nbits, iters=20, beta0=1e-30, kappa=1.0, trace=True)
        assert np.all(r["e"] == 0)
        s = r["scale"]
        zt = r["zero_trace"]
        prev = None
        for k in range(20):
            jq = _objective(w, s, zt[k], r["q"][k])       # after the q-step
            jz = _objective(w, s, zt[k + 1], r["q"][k])   # after the z-step
            slack = 1e-5 * (jq + 1e-12) + 1e-9
            assert jz <= jq + slack
            if prev is not None:
                assert jq <= prev + slack
            prev = jz
        j_rtn = _objective(w, s, zt[0], np.clip(np.rint(fma_f32(w, np.float32(s), np.float32(zt[0]))), 0, qmax))
        j_fin = _objective(w, s, r["zero"], r["codes"].astype(np.float64))
        assert j_fin <= j_rtn * (1 + 1e-5) + 1e-9


def test_symmetry_under_negation(oracle_mod):
    rng = np.random.RandomState(40)
    W16 = random_f16(rng, (128, 256), std=0.02, outlier_frac=0.001)
    Wn = (W16 ^ np.uint16(0x8000)).astype(np.uint16)
    c, s, z = oracle_mod.quantize_codes(W16, 4, 64, 1)
    cn, sn, zn = oracle_mod.quantize_codes(Wn, 4, 64, 1)
    assert np.array_equal(s, sn)
    assert np.allclose(zn, 15 - z, atol=0.2)
    mism = np.mean(cn != 15 - c.astype(np.int32))
    assert mism < 2e-3, mism


def test_determinism(oracle_mod):
    rng = np.random.RandomState(41)
    W16 = random_f16(rng, (64, 128), outlier_frac=0.01)
    a = oracle_mod.quantize(W16, 3, 64, 0)
    b = oracle_mod.quantize(W16, 3, 64, 0)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------

def test_pack_hand_derived_words(oracle_mod):
    # 4-bit: codes 1..8 along a row -> nibbles LSB first
    codes = np.arange(1, 9, dtype=np.uint8).reshape(1, 8)
    assert oracle_mod.pack(codes, 4, 1)[0, 0] == 0x87654321
    # 8-bit: four bytes per word, LSB first; a 6-wide row pads its 2nd word with zeros
    codes = np.array([[0x11, 0xA2, 0x03, 0xFF, 0x7E, 0x80]], dtype=np.uint8)
    words = oracle_mod.pack(codes, 8, 1)
    assert words.shape == (1, 2) and words[0, 0] == 0xFF03A211 and words[0, 1] == 0x0000807E
    # 8-bit along axis 0: word k of column c holds rows 4k..4k+3
    colw = oracle_mod.pack(codes.reshape(6, 1), 8, 0)
    assert colw.shape == (2, 1) and colw[0, 0] == 0xFF03A211 and colw[1, 0] == 0x0000807E
    # 3-bit: ten codes per word in bits 0..29, bits 30-31 zero; a 12-wide row pads its 2nd word
    codes = np.array([[7, 0, 1, 2, 3, 4, 5, 6, 7, 7, 5, 1]], dtype=np.uint8)
    words = oracle_mod.pack(codes, 3, 1)
    ref0 = sum(int(c) << (3 * j) for j, c in enumerate(codes[0, :10]))
    assert words.shape == (1, 2)
    assert words[0, 0] == ref0 and words[0, 0] < 2 ** 30
    assert words[0, 1] == (5 | (1 << 3))
    # 2-bit along a column (axis=0): word (k, c) holds rows 16k .. 16k+15 of column c
    codes = np.zeros((17, 2), np.uint8)
    codes[:, 0] = np.arange(17) % 4
    codes[16, 1] = 3
    words = oracle_mod.pack(codes, 2, 0)
    assert words.shape == (2, 2)
    assert words[0, 0] == sum((r % 4) << (2 * r) for r in range(16))
    assert words[1, 0] == 0 and words[1, 1] == 3 and words[0, 1] == 0
    # 1-bit: 32 per word
    codes = np.zeros((1, 33), np.uint8)
    codes[0, [0, 5, 31, 32]] = 1
    words = oracle_mod.pack(codes, 1, 1)
    assert words[0, 0] == (1 | (1 << 5) | (1 << 31)) and words[0, 1] == 1


@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("axis", [0, 1])
def test_pack_unpack_roundtrip(oracle_mod, nbits, axis):
    C = oracle_mod.CODES_PER_WORD[nbits]
    rng = np.random.RandomState(50 + nbits)
    for L in (C - 1, C, C + 1, 4096, 11008):
        shape = (3, L) if axis == 1 else (L, 3)
        codes = rng.randint(0, QMAX[nbits] + 1, size=shape).astype(np.uint8)
        packed = oracle_mod.pack(codes, nbits, axis)
        assert packed.size == oracle_mod.packed_words(shape[0], shape[1], nbits, axis)
        assert np.array_equal(oracle_mod.unpack(packed, shape[0], shape[1], nbits, axis), codes)
        # pack(unpack(words)) == words for words whose unused fields are zero
        back = oracle_mod.pack(oracle_mod.unpack(packed, shape[0], shape[1], nbits, axis), nbits, axis)
        assert np.array_equal(back, packed)


def test_dequantize_definition(oracle_mod):
    rng = np.random.RandomState(60)
    W16 = random_f16(rng, (16, 128), std=0.03)
    packed, scale, zero = oracle_mod.quantize(W16, 4, 64, 1)
    back = oracle_mod.dequantize(packed, scale, zero, 16, 128, 4, 64, 1)
    codes = oracle_mod.unpack(packed, 16, 128, 4, 1)
    s = np.repeat(scale, 64, axis=1)
    z = np.repeat(zero, 64, axis=1)
    ref = ((codes.astype(np.float32) - z) / s).astype(np.float16).view(np.uint16)
    assert np.array_equal(back, ref)


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_rtn_ties_go_to_even(oracle_mod, nbits):
    """Weights exactly half-way between two grid levels round to the even code."""
    qmax = QMAX[nbits]
    d = 2.0 ** -6
    m = -5 * d
    half = [k + 0.5 for k in range(qmax)]
    vals = [0.0, float(qmax)] + half
    w = np.array([m + v * d for v in vals], np.float32)
    gs = 8 if len(w) <= 8 else 16 if len(w) <= 16 else 32
    w = np.concatenate([w, np.full(gs - len(w), m, np.float32)])
    r = oracle_mod.solve_group(w, nbits, iters=0)
    assert r["scale"] == 1.0 / d and r["zero"] == -m / d
    ref = [0, qmax] + [int(np.rint(v)) for v in half] + [0] * (gs - 2 - len(half))
    assert [int(c) for c in r["codes"]] == ref
    assert any(int(np.floor(v)) % 2 == 1 for v in half)   # some ties round up, some down


@pytest.mark.parametrize("nbits,gs,p,beta0,kappa,side,seed", [
    (3, 64, 1.0, 0.1, 1.5, "up", 2),
    (1, 16, 1.5, 0.1, 1.5, "up", 49),
    (2, 16, 0.7, 0.1, 1.5, "lo", 23),
    (3, 64, 0.3, 1.0, 1.01, "lo", 5),
])
def test_clamp_engaged(oracle_mod, nbits, gs, p, beta0, kappa, side, seed):
    """Trajectories whose zero drifts far enough that w*scale+zero rounds
    outside [0, qmax]: W_q must be the clamped rounding (the clamp is part of
    the quantization step), and the clamp must really be engaged here."""
    qmax = QMAX[nbits]
    rng = np.random.RandomState(seed)   # a seed whose groups reach the clamp
    engaged = 0
    for _ in range(120):
        w = f16_bits_to_f32(random_f16(rng, (gs,), std=0.03, outlier_frac=0.05))
        r = oracle_mod.solve_group(w, nbits, iters=20, p=p, beta0=beta0, kappa=kappa, trace=True)
        s = np.float32(r["scale"])
        for k in range(20):
            t = np.rint(fma_f32(w, s, np.float32(r["zero_trace"][k])))
            engaged += int(np.sum(t > qmax) if side == "up" else np.sum(t < 0))
            assert np.array_equal(r["q"][k], np.clip(t, 0, qmax))
        assert r["codes"].max() <= qmax
    assert engaged > 0
