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


def oracle_threads() -> int:
    """Worker threads for the oracle: the host's cores, at most 16 (a GPU machine's
    CPU share)."""
    import os

    return max(1, min(16, os.cpu_count() or 1))


def oracle_codes_parallel(oracle_mod, W16, nbits, group_size, axis, threads=None, **kw):
    """The oracle's (codes, scale, zero) of a whole tensor, computed as
    independent row slices on worker threads.  Each slice holds whole groups
    (axis 0: a multiple of group_size rows), so every group is solved by the
    single-threaded oracle exactly as in one call over the tensor; the
    oracle's C entry point runs without the GIL."""
    import concurrent.futures as cf

    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    rows, cols = W16.shape
    P = threads or oracle_threads()
    unit = group_size if axis == 0 else 1
    per = max(unit, -(-rows // (4 * P)) // unit * unit)
    cuts = list(range(0, rows, per)) + [rows]
    codes = np.empty((rows, cols), np.uint8)
    ms = oracle_mod.meta_shape(rows, cols, group_size, axis)
    scale = np.empty(ms, np.float32)
    zero = np.empty(ms, np.float32)

    def job(k):
        r0, r1 = cuts[k], cuts[k + 1]
        c, s, z = oracle_mod.quantize_codes(W16[r0:r1], nbits, group_size, axis, **kw)
        codes[r0:r1] = c
        m0, m1 = (r0, r1) if axis == 1 else (r0 // group_size, r1 // group_size)
        scale[m0:m1] = s
        zero[m0:m1] = z

    with cf.ThreadPoolExecutor(P) as ex:
        list(ex.map(job, range(len(cuts) - 1)))
    return codes, scale, zero


def recon_mse_chunked(W16, codes, scale, zero, group_size, axis, rows_per_chunk=1024) -> float:
    """recon_mse over row blocks (whole groups per block), for tensors too large
    to expand at once; the same per-element arithmetic and fp64 accumulation."""
    rows, cols = codes.shape
    step = rows_per_chunk if axis == 1 else max(group_size, rows_per_chunk // group_size * group_size)
    total = 0.0
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        m0, m1 = (r0, r1) if axis == 1 else (r0 // group_size, r1 // group_size)
        w = f16_bits_to_f32(W16[r0:r1])
        s = expand_meta(scale[m0:m1], r1 - r0, cols, group_size, axis).astype(np.float32)
        z = expand_meta(zero[m0:m1], r1 - r0, cols, group_size, axis).astype(np.float32)
        wr = (codes[r0:r1].astype(np.float32) - z) / s
        d = (w - wr).astype(np.float64)
        total += float(np.sum(d * d))
    return total / codes.size
