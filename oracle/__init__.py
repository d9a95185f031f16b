"""CPU oracle of the HQQ solve -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library product never does.

This module is a numpy/ctypes wrapper around ``hqq_oracle.c`` (plain,
single-threaded C, no FMA contraction, no fast-math).  See that file's header
for the solve it implements, the pages' passages it follows and the reading
taken of every point the pages leave open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hqq_oracle.c")
_LIB = os.path.join(_HERE, "libhqq_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

# solve defaults (p, beta0, kappa, iters)
P_DEFAULT = 0.7
BETA0_DEFAULT = 10.0
KAPPA_DEFAULT = 1.01
ITERS_DEFAULT = 20

CODES_PER_WORD = {8: 4, 4: 8, 3: 10, 2: 16, 1: 32}

# element types of 16-bit weights and dequantized outputs
DTYPES = {"f16": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libhqq_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(L):
    P = ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.hqq_ref_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.hqq_ref_f16_to_f32.restype = f32
    L.hqq_ref_f32_to_f16.argtypes = [f32]
    L.hqq_ref_f32_to_f16.restype = ctypes.c_uint16
    L.hqq_ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.hqq_ref_bf16_to_f32.restype = f32
    L.hqq_ref_f32_to_bf16.argtypes = [f32]
    L.hqq_ref_f32_to_bf16.restype = ctypes.c_uint16
    L.hqq_ref_quantize_dt.argtypes = [P, i32, i64, i64, i32, i32, i32, i32, f32, f32, f32, P, P, P]
    L.hqq_ref_quantize_dt.restype = i32
    L.hqq_ref_quantize_codes_dt.argtypes = [P, i32, i64, i64, i32, i32, i32, i32, f32, f32, f32, P, P, P]
    L.hqq_ref_quantize_codes_dt.restype = i32
    L.hqq_ref_dequantize_dt.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32, P]
    L.hqq_ref_dequantize_dt.restype = i32
    L.hqq_ref_quantize_meta.argtypes = [P, i64, i32, P, P, P]
    L.hqq_ref_quantize_meta.restype = i32
    L.hqq_ref_dequantize_meta.argtypes = [P, P, P, i64, i32, P]
    L.hqq_ref_dequantize_meta.restype = i32
    L.hqq_ref_shrink.argtypes = [f32, f32, f32]
    L.hqq_ref_shrink.restype = f32
    L.hqq_ref_solve_group.argtypes = [P, i32, i32, i32, f32, f32, f32, P, P, P, P, P, P, P, P]
    L.hqq_ref_solve_group.restype = i32
    L.hqq_ref_quantize_codes.argtypes = [P, i64, i64, i32, i32, i32, i32, f32, f32, f32, P, P, P]
    L.hqq_ref_quantize_codes.restype = i32
    L.hqq_ref_quantize.argtypes = [P, i64, i64, i32, i32, i32, i32, f32, f32, f32, P, P, P]
    L.hqq_ref_quantize.restype = i32
    L.hqq_ref_packed_words.argtypes = [i64, i64, i32, i32]
    L.hqq_ref_packed_words.restype = i64
    L.hqq_ref_pack.argtypes = [P, i64, i64, i32, i32, P]
    L.hqq_ref_pack.restype = i32
    L.hqq_ref_unpack.argtypes = [P, i64, i64, i32, i32, P]
    L.hqq_ref_unpack.restype = i32
    L.hqq_ref_dequantize.argtypes = [P, P, P, i64, i64, i32, i32, i32, P]
    L.hqq_ref_dequantize.restype = i32
    L.hqq_ref_linear.argtypes = [P, i64, i64, P, P, P, i64, i32, i32, P, P]
    L.hqq_ref_linear.restype = i32
    L.hqq_ref_linear_dt.argtypes = [P, i32, i64, i64, P, P, P, i64, i32, i32, P, P]
    L.hqq_ref_linear_dt.restype = i32
    return L


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {st})")


# --------------------------------------------------------------------------
# wrappers
# --------------------------------------------------------------------------

def f16_to_f32(h: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    return np.array([L.hqq_ref_f16_to_f32(int(v)) for v in flat], dtype=np.float32).reshape(np.shape(h))


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    return np.array([L.hqq_ref_f32_to_f16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    return np.array([L.hqq_ref_bf16_to_f32(int(v)) for v in flat], dtype=np.float32).reshape(np.shape(h))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    return np.array([L.hqq_ref_f32_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def shrink(x: float, p: float, beta: float) -> float:
    return float(lib().hqq_ref_shrink(x, p, beta))


def solve_group(w, nbits, iters=ITERS_DEFAULT, p=P_DEFAULT, beta0=BETA0_DEFAULT,
                kappa=KAPPA_DEFAULT, trace=False):
    """Solve one group of fp32 weights.  Returns a dict with codes, scale, zero
    and (trace=True) the per-iteration zero, beta, W_q, x and W_e."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    gs = w.size
    codes = np.zeros(gs, np.uint8)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    out = {}
    if trace:
        tz = np.zeros(iters + 1, np.float32)
        tb = np.zeros(max(iters, 1), np.float32)
        tq = np.zeros((max(iters, 1), gs), np.float32)
        tx = np.zeros((max(iters, 1), gs), np.float32)
        te = np.zeros((max(iters, 1), gs), np.float32)
        args = [_ptr(tz), _ptr(tb), _ptr(tq), _ptr(tx), _ptr(te)]
    else:
        args = [None] * 5
    st = lib().hqq_ref_solve_group(_ptr(w), gs, nbits, iters, p, beta0, kappa,
                                   _ptr(codes), _ptr(s), _ptr(z), *args)
    _check(st, "solve_group")
    out.update(codes=codes, scale=float(s[0]), zero=float(z[0]))
    if trace:
        out.update(zero_trace=tz, beta=tb[:iters], q=tq[:iters], x=tx[:iters], e=te[:iters])
    return out


def meta_shape(rows, cols, group_size, axis):
    return (rows, cols // group_size) if axis == 1 else (rows // group_size, cols)


def quantize_codes(W16: np.ndarray, nbits, group_size, axis, iters=ITERS_DEFAULT,
                   p=P_DEFAULT, beta0=BETA0_DEFAULT, kappa=KAPPA_DEFAULT, dtype="f16"):
    """W16: uint16 (fp16 or, dtype="bf16", bf16 bits) [rows, cols].
    Returns (codes uint8, scale, zero)."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    rows, cols = W16.shape
    codes = np.zeros((rows, cols), np.uint8)
    ms = meta_shape(rows, cols, group_size, axis)
    scale = np.zeros(ms, np.float32)
    zero = np.zeros(ms, np.float32)
    st = lib().hqq_ref_quantize_codes_dt(_ptr(W16), DTYPES[dtype], rows, cols, nbits, group_size,
                                         axis, iters, p, beta0, kappa, _ptr(codes), _ptr(scale),
                                         _ptr(zero))
    _check(st, "quantize_codes")
    return codes, scale, zero


def packed_shape(rows, cols, nbits, axis):
    C = CODES_PER_WORD[nbits]
    return (rows, -(-cols // C)) if axis == 1 else (-(-rows // C), cols)


def quantize(W16: np.ndarray, nbits, group_size, axis, iters=ITERS_DEFAULT,
             p=P_DEFAULT, beta0=BETA0_DEFAULT, kappa=KAPPA_DEFAULT, dtype="f16"):
    """W16: fp16 (or dtype="bf16": bf16) bits.  Returns (packed uint32, scale, zero)."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    rows, cols = W16.shape
    packed = np.zeros(packed_shape(rows, cols, nbits, axis), np.uint32)
    ms = meta_shape(rows, cols, group_size, axis)
    scale = np.zeros(ms, np.float32)
    zero = np.zeros(ms, np.float32)
    st = lib().hqq_ref_quantize_dt(_ptr(W16), DTYPES[dtype], rows, cols, nbits, group_size, axis,
                                   iters, p, beta0, kappa, _ptr(packed), _ptr(scale), _ptr(zero))
    _check(st, "quantize")
    return packed, scale, zero


def packed_words(rows, cols, nbits, axis) -> int:
    return int(lib().hqq_ref_packed_words(rows, cols, nbits, axis))


def pack(codes: np.ndarray, nbits, axis) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    packed = np.zeros(packed_shape(rows, cols, nbits, axis), np.uint32)
    _check(lib().hqq_ref_pack(_ptr(codes), rows, cols, nbits, axis, _ptr(packed)), "pack")
    return packed


def unpack(packed: np.ndarray, rows, cols, nbits, axis) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    codes = np.zeros((rows, cols), np.uint8)
    _check(lib().hqq_ref_unpack(_ptr(packed), rows, cols, nbits, axis, _ptr(codes)), "unpack")
    return codes


def dequantize(packed, scale, zero, rows, cols, nbits, group_size, axis, dtype="f16") -> np.ndarray:
    """Returns W_hat as uint16 fp16 (or dtype="bf16": bf16) bits [rows, cols]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    zero = np.ascontiguousarray(zero, dtype=np.float32)
    out = np.zeros((rows, cols), np.uint16)
    st = lib().hqq_ref_dequantize_dt(_ptr(packed), _ptr(scale), _ptr(zero), rows, cols,
                                     nbits, group_size, axis, DTYPES[dtype], _ptr(out))
    _check(st, "dequantize")
    return out


def linear(X16: np.ndarray, packed, scale, zero, N, nbits, group_size, with_abs=False, dtype="f16"):
    """Y = X @ W_hat^T in fp64 (X fp16 or, dtype="bf16", bf16 bits [M, K];
    axis = 1 weight [N, K], W_hat dequantized into the same dtype).
    Returns Y [M, N] (and sum |x w| per output with with_abs)."""
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    M, K = X16.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    zero = np.ascontiguousarray(zero, dtype=np.float32)
    Y = np.zeros((M, N), np.float64)
    A = np.zeros((M, N), np.float64)
    st = lib().hqq_ref_linear_dt(_ptr(X16), DTYPES[dtype], M, K, _ptr(packed), _ptr(scale), _ptr(zero),
                                 N, nbits, group_size, _ptr(Y), _ptr(A))
    _check(st, "linear")
    return (Y, A) if with_abs else Y


class Oracle:
    """The wrappers above bound to another build of the oracle source (used by
    the tests that plant mistakes in the oracle to show the pins catch them)."""

    CODES_PER_WORD = CODES_PER_WORD

    def __init__(self, libpath: str):
        self._L = _bind(ctypes.CDLL(libpath))

    def __getattr__(self, name):
        fn = globals()[name]
        if not callable(fn):
            return fn

        def call(*a, **k):
            global _lib
            saved = _lib
            _lib = self._L
            try:
                return fn(*a, **k)
            finally:
                _lib = saved
        return call


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a modified oracle source (test use only) with the oracle's flags."""
    cpath = out_path + ".c"
    with open(cpath, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, "-I", _HERE, "-o", out_path, cpath, "-lm"])
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def quantize_meta(meta: np.ndarray, group_size: int = 128):
    """8-bit RTN of a metadata array (flattened, groups of group_size).
    Returns (codes uint8 [n], scale fp32 [ceil(n/gs)], zero fp32 [ceil(n/gs)])."""
    m = np.ascontiguousarray(meta, dtype=np.float32).ravel()
    ng = -(-m.size // group_size)
    codes = np.zeros(m.size, np.uint8)
    s = np.zeros(ng, np.float32)
    z = np.zeros(ng, np.float32)
    _check(lib().hqq_ref_quantize_meta(_ptr(m), m.size, group_size, _ptr(codes), _ptr(s), _ptr(z)),
           "quantize_meta")
    return codes, s, z


def dequantize_meta(codes, mscale, mzero, group_size: int = 128) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    mscale = np.ascontiguousarray(mscale, dtype=np.float32)
    mzero = np.ascontiguousarray(mzero, dtype=np.float32)
    out = np.zeros(codes.size, np.float32)
    _check(lib().hqq_ref_dequantize_meta(_ptr(codes), _ptr(mscale), _ptr(mzero), codes.size,
                                         group_size, _ptr(out)), "dequantize_meta")
    return out
