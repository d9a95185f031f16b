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
