"""Pins of the oracle's linear layer on quantized weights (X @ W_hat^T with
W_hat the exact dequantization of an axis = 1 weight [N, K]).  The consumer of
the codes is HQQLinear's forward (lnwmold.com HQQ guide, section 3.2):
dequantize, then multiply in the compute dtype."""
import numpy as np
import pytest

from helpers import f16_bits_to_f32, random_f16


def _quantized(oracle_mod, rng, N, K, gs, nbits=4):
    W16 = random_f16(rng, (N, K), std=0.02, outlier_frac=0.002)
    packed, scale, zero = oracle_mod.quantize(W16, nbits, gs, 1, iters=3)
    return packed, scale, zero


def test_identity_input_returns_w_hat_transposed(oracle_mod):
    """X = I (M = K): every output is one dequantized weight, exactly."""
    rng = np.random.RandomState(1)
    N, K, gs = 48, 128, 64
    packed, scale, zero = _quantized(oracle_mod, rng, N, K, gs)
    X = np.zeros((K, K), np.float16)
    np.fill_diagonal(X, 1.0)
    Y = oracle_mod.linear(X.view(np.uint16), packed, scale, zero, N, 4, gs)
    W_hat = f16_bits_to_f32(oracle_mod.dequantize(packed, scale, zero, N, K, 4, gs, 1))
    assert Y.shape == (K, N)
    assert np.array_equal(Y, W_hat.T.astype(np.float64))


def test_hand_derived_outputs(oracle_mod):
    """K = 8, one group per row; scale 2, zero 1 -> W_hat = (q - 1) / 2."""
    codes = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [15, 15, 0, 0, 1, 1, 3, 9]], np.uint8)
    packed = oracle_mod.pack(codes, 4, 1)
    scale = np.full((2, 1), 2.0, np.float32)
    zero = np.full((2, 1), 1.0, np.float32)
    X = np.array([[1, 1, 1, 1, 1, 1, 1, 1], [1, -1, 2, 0, 0, 0, 0.5, 0.25]], np.float16)
    Y = oracle_mod.linear(X.view(np.uint16), packed, scale, zero, 2, 4, 8)
    # row 0 weights: -0.5 0 0.5 1 1.5 2 2.5 3 ; row 1: 7 7 -0.5 -0.5 0 0 1 4
    assert Y[0, 0] == 10.0 and Y[0, 1] == 18.0
    assert Y[1, 0] == -0.5 - 0 + 1.0 + 1.25 + 0.75 and Y[1, 1] == 7 - 7 - 1.0 + 0.5 + 1.0


def test_power_of_two_scaling_and_additivity(oracle_mod):
    rng = np.random.RandomState(2)
    N, K, M, gs = 40, 256, 6, 32
    packed, scale, zero = _quantized(oracle_mod, rng, N, K, gs)
    X = random_f16(rng, (M, K), std=0.5)
    Y = oracle_mod.linear(X, packed, scale, zero, N, 4, gs)
    X2 = (f16_bits_to_f32(X) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle_mod.linear(X2, packed, scale, zero, N, 4, gs), 2 * Y)
    # split X into two fp16 parts whose sum is exact: the outputs add (to fp64 rounding)
    Xf = f16_bits_to_f32(X)
    A = np.where(np.arange(K) % 2 == 0, Xf, 0).astype(np.float16)
    B = np.where(np.arange(K) % 2 == 1, Xf, 0).astype(np.float16)
    YA = oracle_mod.linear(A.view(np.uint16), packed, scale, zero, N, 4, gs)
    YB = oracle_mod.linear(B.view(np.uint16), packed, scale, zero, N, 4, gs)
    assert np.allclose(YA + YB, Y, rtol=1e-14, atol=1e-14)


def test_matches_fp64_product_of_dequantized(oracle_mod):
    rng = np.random.RandomState(3)
    N, K, M, gs = 24, 128, 5, 64
    packed, scale, zero = _quantized(oracle_mod, rng, N, K, gs, nbits=4)
    X = random_f16(rng, (M, K), std=1.0)
    Y, A = oracle_mod.linear(X, packed, scale, zero, N, 4, gs, with_abs=True)
    W_hat = f16_bits_to_f32(oracle_mod.dequantize(packed, scale, zero, N, K, 4, gs, 1)).astype(np.float64)
    ref = f16_bits_to_f32(X).astype(np.float64) @ W_hat.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)
    assert np.all(A >= np.abs(Y))


def test_linear_rejects(oracle_mod):
    X = np.zeros((2, 64), np.uint16)
    packed = np.zeros((4, 8), np.uint32)
    s = np.ones((4, 1), np.float32)
    with pytest.raises(ValueError):
        oracle_mod.linear(X, packed, s, s, 4, 4, 48)     # group size does not divide K
    with pytest.raises(ValueError):
        oracle_mod.linear(X, packed, s, s, 4, 5, 64)     # nbits


# compute dtype bf16 (lnwmold.com HQQ guide section 3.2: HQQLinear computes in
# compute_dtype, fp16 or bf16); bf16 values are checked by widening the bits
# with a 16-bit shift, independently of the oracle's own conversions


def _bf16_f32(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


def _f32_bf16_exact(x):
    """bf16 bits of fp32 values that bf16 represents exactly."""
    f = np.asarray(x, np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_bf16_f32(b), f)
    return b


def test_bf16_identity_input_returns_bf16_w_hat(oracle_mod):
    rng = np.random.RandomState(11)
    N, K, gs = 40, 128, 32
    packed, scale, zero = _quantized(oracle_mod, rng, N, K, gs)
    X = _f32_bf16_exact(np.eye(K, dtype=np.float32))
    Y = oracle_mod.linear(X, packed, scale, zero, N, 4, gs, dtype="bf16")
    W_hat = _bf16_f32(oracle_mod.dequantize(packed, scale, zero, N, K, 4, gs, 1, dtype="bf16"))
    assert np.array_equal(Y, W_hat.T.astype(np.float64))


def test_bf16_hand_derived_outputs(oracle_mod):
    """As the fp16 case: every weight and input is exact in bf16."""
    codes = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [15, 15, 0, 0, 1, 1, 3, 9]], np.uint8)
    packed = oracle_mod.pack(codes, 4, 1)
    scale = np.full((2, 1), 2.0, np.float32)
    zero = np.full((2, 1), 1.0, np.float32)
    X = _f32_bf16_exact(np.array([[1, 1, 1, 1, 1, 1, 1, 1], [1, -1, 2, 0, 0, 0, 0.5, 0.25]], np.float32))
    Y = oracle_mod.linear(X, packed, scale, zero, 2, 4, 8, dtype="bf16")
    assert Y[0, 0] == 10.0 and Y[0, 1] == 18.0
    assert Y[1, 0] == -0.5 - 0 + 1.0 + 1.25 + 0.75 and Y[1, 1] == 7 - 7 - 1.0 + 0.5 + 1.0


def test_bf16_w_hat_is_rne_of_quotient_in_products(oracle_mod):
    """Y equals the fp64 product of X (bf16) with the bf16 rounding of the
    fp32 quotients (q - z) / s, rounded here by comparing both neighbours."""
    rng = np.random.RandomState(12)
    N, K, M, gs = 16, 64, 3, 32
    codes = rng.randint(0, 16, size=(N, K)).astype(np.uint8)
    packed = oracle_mod.pack(codes, 4, 1)
    scale = (rng.uniform(1, 2, (N, K // gs)) * 2.0 ** rng.randint(0, 12, (N, K // gs))).astype(np.float32)
    zero = rng.uniform(0, 15, (N, K // gs)).astype(np.float32)
    q = (codes.astype(np.float32) - np.repeat(zero, gs, axis=1)) / np.repeat(scale, gs, axis=1)
    u = q.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    vlo, vhi = _bf16_f32(lo).astype(np.float64), _bf16_f32(lo + 1).astype(np.float64)
    ax = np.abs(q.astype(np.float64))
    dlo, dhi = ax - np.abs(vlo), np.abs(vhi) - ax
    wb = np.where((dhi < dlo) | ((dhi == dlo) & (lo & 1 == 1)), lo + 1, lo)
    Xf = rng.uniform(-2, 2, (M, K)).astype(np.float32)
    X = (Xf.view(np.uint32) >> 16).astype(np.uint16)          # truncation: exact bf16 inputs
    ref = _bf16_f32(X).astype(np.float64) @ _bf16_f32(wb).astype(np.float64).T
    Y = oracle_mod.linear(X, packed, scale, zero, N, 4, gs, dtype="bf16")
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def test_bf16_and_fp16_agree_where_both_are_exact(oracle_mod):
    """Codes and meta whose W_hat is exact in both dtypes (scale a power of
    two, integer zero) and inputs exact in both: identical outputs."""
    rng = np.random.RandomState(13)
    N, K, M, gs = 12, 64, 4, 16
    codes = rng.randint(0, 16, size=(N, K)).astype(np.uint8)
    packed = oracle_mod.pack(codes, 4, 1)
    scale = (2.0 ** rng.randint(-2, 4, (N, K // gs))).astype(np.float32)
    zero = rng.randint(0, 15, (N, K // gs)).astype(np.float32)
    Xf = (rng.randint(-64, 64, (M, K)) / 16.0).astype(np.float32)     # 7 significant bits
    Y16 = oracle_mod.linear(Xf.astype(np.float16).view(np.uint16), packed, scale, zero, N, 4, gs)
    Yb = oracle_mod.linear(_f32_bf16_exact(Xf), packed, scale, zero, N, 4, gs, dtype="bf16")
    assert np.array_equal(Y16, Yb)


def test_linear_rejects_unknown_dtype(oracle_mod):
    lib = oracle_mod.lib()
    X = np.zeros((2, 64), np.uint16)
    packed = np.zeros((4, 8), np.uint32)
    s = np.ones((4, 1), np.float32)
    Y = np.zeros((2, 4), np.float64)
    st = lib.hqq_ref_linear_dt(oracle_mod._ptr(X), 7, 2, 64, oracle_mod._ptr(packed), oracle_mod._ptr(s),
                               oracle_mod._ptr(s), 4, 4, 64, oracle_mod._ptr(Y), None)
    assert st == -8
