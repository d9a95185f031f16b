"""Host-side helpers shared by the tests (evaluation only, no quantization)."""
from __future__ import annotations

import numpy as np


def f16_bits_to_f32(W16: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(W16, dtype=np.uint16).view(np.float16).astype(np.float32)


def random_f16(rng: np.random.RandomState, shape, std=0.02, outlier_frac=0.0) -> np.ndarray:
    w = rng.randn(*shape) * std
    if outlier_frac:
        m = rng.rand(*shape) < outlier_frac
        w = np.where(m, w * 20.0, w)
    return w.astype(np.float16).view(np.uint16)


def expand_meta(meta: np.ndarray, rows, cols, group_size, axis) -> np.ndarray:
    """Broadcast per-group values to the [rows, cols] layout."""
    if axis == 1:
        return np.repeat(meta, group_size, axis=1)
    return np.repeat(meta, group_size, axis=0)


def recon_mse(W16, codes, scale, zero, group_size, axis) -> float:
    """Per-tensor reconstruction MSE: mean((W - W_r)^2) with W_r = (q - zero) / scale
    evaluated in fp32, accumulated in fp64.  Runs unchanged on the oracle's and
    on the GPU's outputs."""
    rows, cols = codes.shape
    w = f16_bits_to_f32(W16)
    s = expand_meta(scale, rows, cols, group_size, axis).astype(np.float32)
    z = expand_meta(zero, rows, cols, group_size, axis).astype(np.float32)
    wr = (codes.astype(np.float32) - z) / s
    d = (w - wr).astype(np.float64)
    return float(np.mean(d * d))


def fma_f32(a, b, c) -> np.ndarray:
    """Correctly rounded fp32 fused multiply-add via x87 extended precision:
    for fp16 a, fp32 b, c of moderate range the long-double value a*b+c is
    exact, and the conversion to fp32 rounds it once."""
    a = np.asarray(a, dtype=np.float32).astype(np.longdouble)
    b = np.asarray(b, dtype=np.float32).astype(np.longdouble)
    c = np.asarray(c, dtype=np.float32).astype(np.longdouble)
    return (a * b + c).astype(np.float32)
