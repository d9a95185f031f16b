"""Pins of the oracle's metadata quantization (quant_scale / quant_zero:
devpress.csdn.net tutorial, section 3.3 and troubleshooting: the scale and
zero arrays are quantized at a higher precision such as 8 bits).  Reading:
8-bit min-max RTN in groups of consecutive values, the last group shorter."""
import numpy as np
import pytest

from helpers import fma_f32, random_f16


def closed_form(v: np.ndarray):
    mn, mx = np.float32(v.min()), np.float32(v.max())
    rng = np.float32(mx - mn)
    if rng == 0:
        s, z = np.float32(1.0), np.float32(-mn)
    else:
        s = np.float32(np.float32(255.0) / rng)
        z = np.float32(-(mn * s))
    c = np.clip(np.rint(fma_f32(v, s, z)), 0, 255).astype(np.uint8)
    return c, s, z


@pytest.mark.parametrize("n,gs", [(1000, 128), (4096, 128), (77, 16), (5, 1), (300, 1024), (129, 64)])
def test_meta_rtn_closed_form(oracle_mod, n, gs):
    rng = np.random.RandomState(n + gs)
    m = rng.uniform(50, 400, n).astype(np.float32)
    codes, s, z = oracle_mod.quantize_meta(m, gs)
    assert len(s) == -(-n // gs)
    for g in range(len(s)):
        v = m[g * gs:(g + 1) * gs]
        c, sg, zg = closed_form(v)
        assert s[g] == sg and z[g] == zg
        assert np.array_equal(codes[g * gs:(g + 1) * gs], c)
        # min -> 0, max -> 255 (for a group with range)
        if len(v) > 1 and v.max() > v.min():
            assert codes[g * gs + v.argmin()] == 0 and codes[g * gs + v.argmax()] == 255


def test_meta_reconstruction_within_half_step(oracle_mod):
    rng = np.random.RandomState(1)
    W16 = random_f16(rng, (64, 1024), std=0.02, outlier_frac=0.002)
    _, scale, zero = oracle_mod.quantize(W16, 4, 64, 1, iters=5)
    for meta in (scale.ravel(), zero.ravel()):
        codes, s, z = oracle_mod.quantize_meta(meta, 128)
        back = oracle_mod.dequantize_meta(codes, s, z, 128)
        for g in range(len(s)):
            v = meta[g * 128:(g + 1) * 128].astype(np.float64)
            half = 0.5 * (v.max() - v.min()) / 255.0
            err = np.abs(back[g * 128:(g + 1) * 128] - v)
            assert np.all(err <= half * (1 + 1e-5) + 1e-6 * np.abs(v).max())


def test_meta_constant_group_is_exact(oracle_mod):
    m = np.array([3.25] * 128 + [7.0] * 5, np.float32)
    codes, s, z = oracle_mod.quantize_meta(m, 128)
    assert np.all(codes == 0) and list(s) == [1.0, 1.0] and list(z) == [-3.25, -7.0]
    assert np.array_equal(oracle_mod.dequantize_meta(codes, s, z, 128), m)


def test_meta_dequantize_formula(oracle_mod):
    rng = np.random.RandomState(2)
    codes = rng.randint(0, 256, 300).astype(np.uint8)
    s = rng.uniform(0.5, 3, 3).astype(np.float32)
    z = rng.uniform(-100, 100, 3).astype(np.float32)
    got = oracle_mod.dequantize_meta(codes, s, z, 128)
    ref = (codes.astype(np.float32) - np.repeat(z, 128)[:300]) / np.repeat(s, 128)[:300]
    assert np.array_equal(got, ref)
