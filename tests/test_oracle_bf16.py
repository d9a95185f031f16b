"""Pins of the oracle's bf16 paths: weights of a model loaded in bf16 and
dequantization into compute_dtype bf16 (devpress.csdn.net tutorial, section
5; lnwmold.com HQQ guide, sections 3.2 and 6.1).  None of these reuse the
oracle's own conversion code."""
import numpy as np
import pytest

from helpers import fma_f32

QMAX = {1: 1, 2: 3, 3: 7, 4: 15, 8: 255}


def bf16_via_bits(h: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: widen by a 16-bit shift."""
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


def rne_bf16_by_neighbours(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 by comparing the two bf16 neighbours of x exactly in fp64;
    ties to the even significand; from the midpoint between the largest finite
    bf16 and 2^128 on, infinity."""
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)                 # truncation toward zero
    hi = lo + 1                                      # next bf16 away from zero
    vlo = bf16_via_bits(lo).astype(np.float64)
    # past the largest finite bf16 the next value is 2^128 (IEEE rounding with
    # an unbounded exponent; choosing it means overflow to infinity)
    vhi = np.where((hi & 0x7fff) == 0x7f80, 2.0 ** 128, bf16_via_bits(hi).astype(np.float64))
    ax = np.abs(x.astype(np.float64))
    dlo = ax - np.abs(vlo)
    dhi = np.abs(vhi) - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    out = np.where(pick_hi, hi, lo).astype(np.uint16)
    return out


def test_bf16_widening_all_patterns(oracle_mod):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.bf16_to_f32(h)
    ref = bf16_via_bits(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_rounding_nearest_even(oracle_mod):
    rng = np.random.RandomState(3)
    # random fp32 bit patterns over the finite range, exact ties, values next
    # to ties, subnormals and the overflow boundary
    u = rng.randint(0, 0x7f7fffff, size=20000, dtype=np.int64).astype(np.uint32)
    ties = (rng.randint(0, 0x7f7f, size=2000).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    sub = rng.randint(0, 0x00800000, size=2000).astype(np.uint32)
    edge = np.array([0x7f7f7fff, 0x7f7f8000, 0x7f7f8001, 0x7f7fffff, 0x00000000, 0x00008000,
                     0x00018000, 0x3f808000, 0x3f818000], np.uint32)
    bits = np.concatenate([u, ties, near, sub, edge])
    for sign in (0, 0x80000000):
        x = (bits | np.uint32(sign)).view(np.float32)
        got = oracle_mod.f32_to_bf16(x)
        assert np.array_equal(got, rne_bf16_by_neighbours(x)), "bf16 rounding"


def _both_exact(rng, shape, std):
    """Weights exact in fp16 and in bf16 (8 significant bits, normal fp16
    range): their fp16 bits and bf16 bits."""
    w = rng.randn(*shape) * std
    w = np.where(np.abs(w) < 2.0 ** -13, 2.0 ** -13, w)
    e = np.floor(np.log2(np.abs(w)))
    w = np.round(w / 2.0 ** (e - 7)) * 2.0 ** (e - 7)
    f32 = w.astype(np.float32)
    h16 = f32.astype(np.float16)
    assert np.array_equal(h16.astype(np.float32), f32)
    bf = (f32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_via_bits(bf), f32)
    return h16.view(np.uint16), bf


@pytest.mark.parametrize("nbits,gs,axis", [(4, 64, 1), (3, 64, 0), (2, 16, 0), (8, 128, 1), (1, 32, 1)])
def test_bf16_weights_equal_to_fp16_weights_quantize_alike(oracle_mod, nbits, gs, axis):
    rng = np.random.RandomState(nbits * 7 + gs + axis)
    W16, WB = _both_exact(rng, (128, 256), 0.02)
    a = oracle_mod.quantize(W16, nbits, gs, axis, iters=20)
    b = oracle_mod.quantize(WB, nbits, gs, axis, iters=20, dtype="bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_bf16_dequantize_is_rne_of_fp32_quotient(oracle_mod):
    rng = np.random.RandomState(5)
    rows, cols, gs, nbits = 40, 256, 64, 4
    codes = rng.randint(0, 16, size=(rows, cols)).astype(np.uint8)
    scale = (rng.uniform(1, 2, (rows, cols // gs)) * 2.0 ** rng.randint(-10, 40, (rows, cols // gs))).astype(np.float32)
    zero = rng.uniform(-50, 50, (rows, cols // gs)).astype(np.float32)
    packed = oracle_mod.pack(codes, nbits, 1)
    got = oracle_mod.dequantize(packed, scale, zero, rows, cols, nbits, gs, 1, dtype="bf16")
    s = np.repeat(scale, gs, axis=1)
    z = np.repeat(zero, gs, axis=1)
    q = (codes.astype(np.float32) - z) / s              # IEEE fp32 subtract and divide
    assert np.array_equal(got, rne_bf16_by_neighbours(q.astype(np.float32)))


@pytest.mark.parametrize("nbits", [2, 4, 8])
def test_bf16_iters0_is_minmax_rtn_wide_range(oracle_mod, nbits):
    """bf16 weights far outside fp16's range (1e-30 .. 1e8): RTN from min/max."""
    rng = np.random.RandomState(20 + nbits)
    qmax = QMAX[nbits]
    gs = 32
    mag = 10.0 ** rng.uniform(-30, 8, size=(16, gs))
    w = (mag * rng.choice([-1, 1], size=(16, gs))).astype(np.float32)
    WB = (w.view(np.uint32) >> 16).astype(np.uint16)
    w = bf16_via_bits(WB)
    codes, scale, zero = oracle_mod.quantize_codes(WB, nbits, gs, 1, iters=0, dtype="bf16")
    mn, mx = w.min(axis=1), w.max(axis=1)
    s = np.float32(qmax) / (mx - mn)
    z = -(mn * s)
    assert np.array_equal(scale[:, 0], s)
    assert np.array_equal(zero[:, 0], z)
    ref = np.clip(np.rint(fma_f32(w, s[:, None], z[:, None])), 0, qmax).astype(np.uint8)
    assert np.array_equal(codes, ref)


def test_bf16_dtype_rejected_when_unknown(oracle_mod):
    lib = oracle_mod.lib()
    W = np.zeros((8, 8), np.uint16)
    out = np.zeros((8, 8), np.uint8)
    m = np.zeros((8, 1), np.float32)
    st = lib.hqq_ref_quantize_codes_dt(oracle_mod._ptr(W), 5, 8, 8, 4, 8, 1, 0, 0.7, 10.0, 1.01,
                                       oracle_mod._ptr(out), oracle_mod._ptr(m), oracle_mod._ptr(m))
    assert st == -8
