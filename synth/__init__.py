"""Seeded synthetic fp16 Linear weights for the HQQ workloads.

This module holds the input generator shared by the tests and the benchmark
(and nothing of the quantization method).  The pages quantize real
checkpoints (Llama-2-7B, Llama-7B, Llama-3-8B, a 70B): those trained weights
are not available, so seeded synthetic weights of the same Linear shapes
stand in for them.

Distribution (per tensor, element (r, c), idx = r * cols + c):
    z      ~ N(0, 1)                    Box-Muller, stream 0, counter idx
    f_r    = exp(0.5 * z_r)             z_r ~ N(0, 1) from stream 1, counter r
                                        (a lognormal(0, 0.5) factor per output row)
    o      = 20 if u < 0.001 else 1     u ~ U(0, 1) from stream 2, counter idx
                                        (0.1% outliers at uniform positions)
    W[r,c] = fp16_rne(((0.02 * z) * f_r) * o)    (fp64 arithmetic, one rounding)

Random bits: the SplitMix64 finaliser applied to a counter,
    key  = mix(mix(mix(seed) ^ (layer + 1)) ^ (tensor_id + 1))
    h    = mix(key ^ (stream << 56) ^ counter)
    u(a) = (a + 0.5) / 2^24 for a 24-bit field a of h: a1 = h >> 40,
           a2 = (h >> 16) & 0xFFFFFF
    z    = sqrt(-2 ln u(a1)) * cos(2 pi u(a2))
The GPU generator (synth.hip) computes the same definition in fp64; its
output is identical except where the two fp64 libms differ by an ulp right at
an fp16 rounding boundary.  Parity tests always hand the *same* fp16 bits to
the oracle and to the HIP path, so generator differences cannot enter parity.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.hip")
_LIB = os.path.join(_HERE, "libhqq_synth.so")

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}

SEED_SINGLE = 0x48515101   # the single-Linear workload
SEED_7B = 0x48515107       # 7B-shaped layer / stack (shared so they can cross-check)
SEED_70B = 0x48515170      # 70B-shaped stack


# ---------------------------------------------------------------------------
# workloads (shapes and quantization settings; no arithmetic of the method)
# ---------------------------------------------------------------------------

def _layer_7b():
    return [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
            ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]


def _layer_70b():
    return [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
            ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]


def workload(name: str):
    """List of tensors: dicts with layer, name, tensor_id, rows, cols, nbits,
    group_size, axis, seed.  Names: 'linear_4096x1024_4b_g64',
    'llama7b_layer_4b_g64', 'llama7b_layer_3b2b_axis0', 'llama7b_stack32_4b_g64',
    'llama7b_stack32_8b_g128' (the same weights at 8 bits, group 128),
    'llama70b_stack80_mixed', and 'llama7b_stack<L>_<b>b_g<gs>[_axis0]' (L layers
    of the 7B shapes in one format)."""
    out = []
    if name == "linear_4096x1024_4b_g64":
        out.append(dict(layer=0, name="q", tensor_id=0, rows=4096, cols=1024, nbits=4,
                        group_size=64, axis=1, seed=SEED_SINGLE))
    elif name == "llama7b_layer_4b_g64":
        for n, r, c in _layer_7b():
            out.append(dict(layer=0, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c, nbits=4,
                            group_size=64, axis=1, seed=SEED_7B))
    elif name == "llama7b_layer_3b2b_axis0":
        for n, r, c in _layer_7b():
            attn = n in ("q", "k", "v", "o")
            out.append(dict(layer=0, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c,
                            nbits=3 if attn else 2, group_size=64 if attn else 16, axis=0,
                            seed=SEED_7B))
    elif name == "llama7b_stack32_4b_g64":
        for layer in range(32):
            for n, r, c in _layer_7b():
                out.append(dict(layer=layer, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c,
                                nbits=4, group_size=64, axis=1, seed=SEED_7B))
    elif name == "llama7b_stack32_8b_g128":
        for layer in range(32):
            for n, r, c in _layer_7b():
                out.append(dict(layer=layer, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c,
                                nbits=8, group_size=128, axis=1, seed=SEED_7B))
    elif name == "llama70b_stack80_mixed":
        for layer in range(80):
            for n, r, c in _layer_70b():
                attn = n in ("q", "k", "v", "o")
                nb, gs = (4, 64) if attn else (2, 16)
                if layer == 0 and n == "down":
                    nb, gs = 1, 16
                out.append(dict(layer=layer, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c,
                                nbits=nb, group_size=gs, axis=1, seed=SEED_70B))
    else:
        # llama7b_stack<L>_<b>b_g<gs>[_axis0]: L decoder layers of the 7B shapes,
        # every tensor in one format (axis 1 unless the suffix says 0)
        m = re.fullmatch(r"llama7b_stack(\d+)_([12348])b_g(\d+)(_axis0)?", name)
        if not m:
            raise KeyError(name)
        L, nb, gs, ax = int(m.group(1)), int(m.group(2)), int(m.group(3)), 0 if m.group(4) else 1
        for layer in range(L):
            for n, r, c in _layer_7b():
                out.append(dict(layer=layer, name=n, tensor_id=TENSOR_IDS[n], rows=r, cols=c,
                                nbits=nb, group_size=gs, axis=ax, seed=SEED_7B))
    return out


WORKLOADS = ["linear_4096x1024_4b_g64", "llama7b_layer_4b_g64", "llama7b_layer_3b2b_axis0",
             "llama7b_stack32_4b_g64", "llama7b_stack32_8b_g128", "llama70b_stack80_mixed"]


# ---------------------------------------------------------------------------
# CPU generator (numpy)
# ---------------------------------------------------------------------------

def _mix_int(x: int) -> int:
    z = (x + GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def tensor_key(seed: int, layer: int, tensor_id: int) -> int:
    return _mix_int(_mix_int(_mix_int(seed) ^ (layer + 1)) ^ (tensor_id + 1))


def _mix_np(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = x + np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def _bits(key: int, stream: int, counter: np.ndarray) -> np.ndarray:
    base = np.uint64(key ^ (stream << 56))
    return _mix_np(base ^ counter.astype(np.uint64))


def _unit(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.float64) + 0.5) / 16777216.0


def _normal(h: np.ndarray) -> np.ndarray:
    a1 = h >> np.uint64(40)
    a2 = (h >> np.uint64(16)) & np.uint64(0xFFFFFF)
    return np.sqrt(-2.0 * np.log(_unit(a1))) * np.cos(2.0 * np.pi * _unit(a2))


def generate_np(seed: int, layer: int, tensor_id: int, rows: int, cols: int,
                row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """fp16 bits (uint16) of rows [row0, row0 + nrows) of the tensor."""
    if nrows is None:
        nrows = rows - row0
    key = tensor_key(seed, layer, tensor_id)
    r = np.arange(row0, row0 + nrows, dtype=np.uint64)
    f = np.exp(0.5 * _normal(_bits(key, 1, r)))
    idx = (r[:, None] * np.uint64(cols) + np.arange(cols, dtype=np.uint64)[None, :]).ravel()
    z = _normal(_bits(key, 0, idx)).reshape(nrows, cols)
    u = _unit(_bits(key, 2, idx) >> np.uint64(40)).reshape(nrows, cols)
    o = np.where(u < 0.001, 20.0, 1.0)
    w = ((0.02 * z) * f[:, None]) * o
    return w.astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# GPU generator (synth.hip), for workloads too large to build on the host
# ---------------------------------------------------------------------------

HIPCC_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
               "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["hipcc", *HIPCC_FLAGS, "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _gpu_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        L.hqq_synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p]
        L.hqq_synth_fill.restype = ctypes.c_int
        _lib = L
    return _lib


def generate_gpu(out, seed: int, layer: int, tensor_id: int, row0: int = 0):
    """Fill the torch fp16/int16 CUDA tensor ``out`` [nrows, cols] with rows
    row0.. of the tensor, on torch's current stream."""
    import torch
    assert out.is_cuda and out.is_contiguous() and out.dim() == 2 and out.element_size() == 2
    nrows, cols = out.shape
    key = tensor_key(seed, layer, tensor_id)
    st = _gpu_lib().hqq_synth_fill(ctypes.c_void_p(out.data_ptr()), row0, nrows, cols,
                                   ctypes.c_uint64(key),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(f"hqq_synth_fill failed with status {st}")
    return out
