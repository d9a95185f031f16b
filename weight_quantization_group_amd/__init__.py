"""Python binding of the MI355X HQQ library (``libhqq.so``, C ABI in include/hqq.h).

Argument marshalling only: every step of quantize / dequantize / pack / unpack
/ linear runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is not built, or a
tensor is not on the GPU, the call raises.

Tensor conventions (all CUDA tensors, contiguous):
    W        fp16 (or int16/uint16 holding fp16 bits) [rows, cols]
    packed   int32 (bit pattern of the uint32 words), shape
             [rows, ceil(cols/C)] for axis=1, [ceil(rows/C), cols] for axis=0
    scale    float32, [rows, cols/gs] (axis=1) or [rows/gs, cols] (axis=0)
    zero     float32, same shape as scale
    codes    uint8 [rows, cols]
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhqq.so")

CODES_PER_WORD = {8: 4, 4: 8, 3: 10, 2: 16, 1: 32}
P_DEFAULT, BETA0_DEFAULT, KAPPA_DEFAULT, ITERS_DEFAULT = 0.7, 10.0, 1.01, 20

# exported symbols, in include/hqq.h order
EXPORTS = ("hqq_quantize", "hqq_quantize_batch", "hqq_quantize_batch_ex", "hqq_quantize_streamed",
           "hqq_quantize_streamed_static",
           "hqq_dequantize", "hqq_dequantize_ex", "hqq_pack", "hqq_unpack", "hqq_quantize_meta",
           "hqq_dequantize_meta", "hqq_quantize_meta_batch", "hqq_dequantize_meta_batch", "hqq_linear", "hqq_linear_ex", "hqq_linear_batch",
           "hqq_linear_batch_ws", "hqq_solve_mapping", "hqq_linear_route", "hqq_packed_words", "hqq_strerror")

# element types of include/hqq.h
DTYPE_FP16, DTYPE_BF16 = 0, 1

# tensors per kernel launch of hqq_quantize_batch
MAX_BATCH = 48
# weights per kernel launch of hqq_linear_batch
LINEAR_BATCH = 8
# meta arrays per kernel launch of hqq_quantize_meta_batch / hqq_dequantize_meta_batch
META_BATCH = 64


class HqqTensor(ctypes.Structure):
    """struct hqq_tensor of include/hqq.h"""
    _fields_ = [("W", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p)]


class HqqMetaTensor(ctypes.Structure):
    """struct hqq_meta_tensor of include/hqq.h"""
    _fields_ = [("meta", ctypes.c_void_p), ("n", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("mscale", ctypes.c_void_p), ("mzero", ctypes.c_void_p)]


class HqqLinearWeight(ctypes.Structure):
    """struct hqq_linear_weight of include/hqq.h"""
    _fields_ = [("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("Y", ctypes.c_void_p)]


class HqqHostTensor(ctypes.Structure):
    """struct hqq_host_tensor of include/hqq.h (W in host memory)"""
    _fields_ = HqqTensor._fields_


_lib = None


class HQQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {hqq_strerror(status)} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libhqq.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m weight_quantization_group_amd.build`")
    L = ctypes.CDLL(path)
    P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.hqq_quantize.argtypes = [P, i64, i64, i32, i32, i32, i32, f32, f32, f32, P, P, P, P]
    L.hqq_quantize.restype = i32
    L.hqq_quantize_batch.argtypes = [P, i32, i32, i32, i32, i32, f32, f32, f32, P]
    L.hqq_quantize_batch.restype = i32
    L.hqq_quantize_batch_ex.argtypes = [P, i32, i32, i32, i32, i32, i32, f32, f32, f32, P]
    L.hqq_quantize_batch_ex.restype = i32
    L.hqq_dequantize_ex.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32, P, P]
    L.hqq_dequantize_ex.restype = i32
    L.hqq_dequantize.argtypes = [P, P, P, i64, i64, i32, i32, i32, P, P]
    L.hqq_dequantize.restype = i32
    L.hqq_pack.argtypes = [P, i64, i64, i32, i32, i32, P, P]
    L.hqq_pack.restype = i32
    L.hqq_unpack.argtypes = [P, i64, i64, i32, i32, i32, P, P]
    L.hqq_unpack.restype = i32
    L.hqq_quantize_streamed.argtypes = [P, i32, i32, i32, i32, i32, f32, f32, f32, P, i64, P, P]
    L.hqq_quantize_streamed.restype = i32
    L.hqq_quantize_streamed_static.argtypes = [P, i32, i32, i32, i32, i32, f32, f32, f32, P, P]
    L.hqq_quantize_streamed_static.restype = i32
    L.hqq_quantize_meta.argtypes = [P, i64, i32, P, P, P, P]
    L.hqq_quantize_meta.restype = i32
    L.hqq_dequantize_meta.argtypes = [P, P, P, i64, i32, P, P]
    L.hqq_dequantize_meta.restype = i32
    L.hqq_quantize_meta_batch.argtypes = [P, i32, i32, P]
    L.hqq_quantize_meta_batch.restype = i32
    L.hqq_dequantize_meta_batch.argtypes = [P, i32, i32, P]
    L.hqq_dequantize_meta_batch.restype = i32
    L.hqq_linear.argtypes = [P, i64, i64, P, P, P, i64, i32, i32, P, P]
    L.hqq_linear.restype = i32
    L.hqq_linear_ex.argtypes = [P, i64, i64, P, P, P, i64, i32, i32, i32, P, P]
    L.hqq_linear_ex.restype = i32
    L.hqq_linear_batch.argtypes = [P, i64, i64, P, i32, i32, i32, i32, P]
    L.hqq_linear_batch.restype = i32
    L.hqq_linear_batch_ws.argtypes = [P, i64, i64, P, i32, i32, i32, i32, P, i64, P]
    L.hqq_linear_batch_ws.restype = i32
    L.hqq_solve_mapping.argtypes = [i32, i32, i32, i32, i64]
    L.hqq_solve_mapping.restype = i32
    L.hqq_linear_route.argtypes = [i64, i64, i32, i64, i64]
    L.hqq_linear_route.restype = i32
    L.hqq_packed_words.argtypes = [i64, i64, i32, i32]
    L.hqq_packed_words.restype = i64
    L.hqq_strerror.argtypes = [i32]
    L.hqq_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def hqq_strerror(status: int) -> str:
    return load_library().hqq_strerror(int(status)).decode()


def hqq_solve_mapping(nbits: int, group_size: int, axis: int, wdtype: int, work_items: int) -> int:
    """MAPPING_LANE, MAPPING_SEG or MAPPING_SEG16: the solve kernel a launch
    of work_items work items of this format runs."""
    m = load_library().hqq_solve_mapping(nbits, group_size, axis, wdtype, work_items)
    if m < 0:
        raise HQQError("hqq_solve_mapping", m)
    return int(m)


MAPPING_LANE, MAPPING_SEG, MAPPING_SEG16 = 0, 1, 2


def hqq_linear_route(M: int, K: int, count: int, n_max: int, workspace_bytes: int) -> int:
    """ROUTE_FUSED or ROUTE_GEMM: the route hqq_linear_batch_ws takes for M
    rows, depth K, count weights of at most n_max outputs and the workspace
    size."""
    r = load_library().hqq_linear_route(M, K, count, n_max, workspace_bytes)
    if r < 0:
        raise HQQError("hqq_linear_route", r)
    return int(r)


ROUTE_FUSED, ROUTE_GEMM = 0, 1


def hqq_packed_words(rows: int, cols: int, nbits: int, axis: int) -> int:
    n = load_library().hqq_packed_words(rows, cols, nbits, axis)
    if n < 0:
        raise HQQError("hqq_packed_words", n)
    return int(n)


def packed_shape(rows, cols, nbits, axis):
    C = CODES_PER_WORD[nbits]
    return (rows, -(-cols // C)) if axis == 1 else (-(-rows // C), cols)


def meta_shape(rows, cols, group_size, axis):
    return (rows, cols // group_size) if axis == 1 else (rows // group_size, cols)


def _dev_ptr(t: torch.Tensor, name: str, dtypes) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_F16 = (torch.float16, torch.int16)
try:
    _F16 = _F16 + (torch.uint16,)
except AttributeError:  # pragma: no cover
    pass
_U32 = (torch.int32,) + ((torch.uint32,) if hasattr(torch, "uint32") else ())


def hqq_quantize(W: torch.Tensor, nbits: int, group_size: int, axis: int,
                 iters: int = ITERS_DEFAULT, p: float = P_DEFAULT, beta0: float = BETA0_DEFAULT,
                 kappa: float = KAPPA_DEFAULT, packed=None, scale=None, zero=None):
    """HQQ-quantize W [rows, cols] (fp16, or bf16).  Returns (packed, scale, zero)."""
    L = load_library()
    if isinstance(W, torch.Tensor) and W.dtype == torch.bfloat16:
        rows, cols = W.shape
        dev = W.device
        if packed is None:
            packed = torch.empty(packed_shape(rows, cols, nbits, axis), dtype=torch.int32, device=dev)
        line = cols if axis == 1 else rows
        ms = meta_shape(rows, cols, group_size, axis) if group_size > 0 and line % group_size == 0 else (1,)
        if scale is None:
            scale = torch.empty(ms, dtype=torch.float32, device=dev)
        if zero is None:
            zero = torch.empty(ms, dtype=torch.float32, device=dev)
        QuantizeBatch([(W, packed, scale, zero)], nbits, group_size, axis, iters, p, beta0, kappa).run()
        return packed, scale, zero
    rows, cols = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_shape(rows, cols, nbits, axis), dtype=torch.int32, device=dev)
    line = cols if axis == 1 else rows
    ms = meta_shape(rows, cols, group_size, axis) if group_size > 0 and line % group_size == 0 else (1,)
    if scale is None:
        scale = torch.empty(ms, dtype=torch.float32, device=dev)
    if zero is None:
        zero = torch.empty(ms, dtype=torch.float32, device=dev)
    st = L.hqq_quantize(_dev_ptr(W, "W", _F16), rows, cols, nbits, group_size, axis, iters,
                        p, beta0, kappa, _dev_ptr(packed, "packed", _U32),
                        _dev_ptr(scale, "scale", (torch.float32,)),
                        _dev_ptr(zero, "zero", (torch.float32,)), _stream(dev))
    if st != 0:
        raise HQQError("hqq_quantize", st)
    return packed, scale, zero


class QuantizeBatch:
    """Several same-format tensors for hqq_quantize_batch, validated and
    marshalled into the C descriptor array once; run() is then a single
    C-ABI call (one launch per 48 tensors) on the current stream.
    items: list of (W, packed, scale, zero) CUDA tensors (outputs
    preallocated); the tensors are kept alive by the object."""

    def __init__(self, items, nbits: int, group_size: int, axis: int,
                 iters: int = ITERS_DEFAULT, p: float = P_DEFAULT,
                 beta0: float = BETA0_DEFAULT, kappa: float = KAPPA_DEFAULT):
        self._lib = load_library()
        self._items = [tuple(it) for it in items]
        n = len(self._items)
        # the weights' element type: bf16 tensors, else fp16 bits
        bf = [it[0].dtype == torch.bfloat16 for it in self._items]
        if any(bf) and not all(bf):
            raise TypeError("a batch holds fp16 or bf16 weights, not both")
        self._wdtype = DTYPE_BF16 if n and bf[0] else DTYPE_FP16
        self._arr = (HqqTensor * max(n, 1))()
        for i, (W, pk, sc, ze) in enumerate(self._items):
            rows, cols = W.shape
            self._arr[i] = HqqTensor(_dev_ptr(W, "W", _F16 + (torch.bfloat16,)).value, rows, cols,
                                     _dev_ptr(pk, "packed", _U32).value,
                                     _dev_ptr(sc, "scale", (torch.float32,)).value,
                                     _dev_ptr(ze, "zero", (torch.float32,)).value)
        self._n = n
        self._ptr = ctypes.cast(self._arr, ctypes.c_void_p)
        self._dev = self._items[0][0].device if n else torch.device("cuda", torch.cuda.current_device())
        self._args = (nbits, group_size, axis, iters, p, beta0, kappa)

    def run(self):
        st = self._lib.hqq_quantize_batch_ex(self._ptr, self._n, self._wdtype, *self._args,
                                             _stream(self._dev))
        if st != 0:
            raise HQQError("hqq_quantize_batch_ex", st)


def hqq_quantize_batch(items, nbits: int, group_size: int, axis: int,
                       iters: int = ITERS_DEFAULT, p: float = P_DEFAULT,
                       beta0: float = BETA0_DEFAULT, kappa: float = KAPPA_DEFAULT):
    """Quantize several same-format tensors in as few launches as possible.
    items: list of (W, packed, scale, zero) CUDA tensors (outputs preallocated)."""
    QuantizeBatch(items, nbits, group_size, axis, iters, p, beta0, kappa).run()


def hqq_dequantize(packed, scale, zero, rows: int, cols: int, nbits: int, group_size: int,
                   axis: int, out=None, dtype=torch.float16) -> torch.Tensor:
    """W_hat = round((W_q - zero) / scale) to dtype (torch.float16 or
    torch.bfloat16; out's dtype when out is given) as a tensor [rows, cols]."""
    L = load_library()
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=packed.device)
    odt = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_FP16
    st = L.hqq_dequantize_ex(_dev_ptr(packed, "packed", _U32), _dev_ptr(scale, "scale", (torch.float32,)),
                             _dev_ptr(zero, "zero", (torch.float32,)), rows, cols, nbits, group_size,
                             axis, odt, _dev_ptr(out, "out", _F16 + (torch.bfloat16,)),
                             _stream(packed.device))
    if st != 0:
        raise HQQError("hqq_dequantize_ex", st)
    return out


def hqq_pack(codes: torch.Tensor, nbits: int, group_size: int, axis: int, out=None) -> torch.Tensor:
    L = load_library()
    rows, cols = codes.shape
    if out is None:
        out = torch.empty(packed_shape(rows, cols, nbits, axis), dtype=torch.int32, device=codes.device)
    st = L.hqq_pack(_dev_ptr(codes, "codes", (torch.uint8,)), rows, cols, nbits, group_size, axis,
                    _dev_ptr(out, "out", _U32), _stream(codes.device))
    if st != 0:
        raise HQQError("hqq_pack", st)
    return out


def hqq_unpack(packed: torch.Tensor, rows: int, cols: int, nbits: int, group_size: int, axis: int,
               out=None) -> torch.Tensor:
    L = load_library()
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=packed.device)
    st = L.hqq_unpack(_dev_ptr(packed, "packed", _U32), rows, cols, nbits, group_size, axis,
                      _dev_ptr(out, "out", (torch.uint8,)), _stream(packed.device))
    if st != 0:
        raise HQQError("hqq_unpack", st)
    return out


def _compute_dtype(X: torch.Tensor):
    """(C dtype code, torch dtype, accepted tensor dtypes) of an activation."""
    if X.dtype == torch.bfloat16:
        return DTYPE_BF16, torch.bfloat16, (torch.bfloat16,)
    return DTYPE_FP16, torch.float16, _F16


def hqq_linear(X: torch.Tensor, packed, scale, zero, N: int, nbits: int, group_size: int,
               out=None) -> torch.Tensor:
    """Y = X . W_hat^T ([M, N]) for X [M, K] and the axis = 1 quantized weight
    W [N, K] given by (packed, scale, zero).  The compute dtype is X's: fp16
    (or int16 / uint16 fp16 bits), or bfloat16."""
    L = load_library()
    M, K = X.shape
    code, tdt, ok = _compute_dtype(X)
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=X.device)
    st = L.hqq_linear_ex(_dev_ptr(X, "X", ok), M, K, _dev_ptr(packed, "packed", _U32),
                         _dev_ptr(scale, "scale", (torch.float32,)),
                         _dev_ptr(zero, "zero", (torch.float32,)), N, nbits, group_size, code,
                         _dev_ptr(out, "out", ok), _stream(X.device))
    if st != 0:
        raise HQQError("hqq_linear_ex", st)
    return out


class LinearBatch:
    """Weights that share the input X, for hqq_linear_batch, marshalled into
    the C descriptor array once; run(X) is then a single C-ABI call (one
    launch per 8 weights) on the current stream.  weights: list of (packed,
    scale, zero, N, Y) with Y a preallocated fp16 [M, N] CUDA tensor; the
    tensors are kept alive by the object.  workspace: an optional CUDA tensor
    for hqq_linear_batch_ws (the tiled kernel's K splits, or W_hat and the
    GEMM of the dequantize-then-GEMM route); see linear_workspace_bytes."""

    def __init__(self, weights, nbits: int, group_size: int, dtype=torch.float16, workspace=None):
        self._lib = load_library()
        self._ws = workspace
        if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
            raise TypeError("workspace must be a contiguous CUDA tensor")
        self._items = [tuple(w) for w in weights]
        self.nbits, self.group_size = nbits, group_size
        self._code, _, ok = _compute_dtype(torch.empty(0, dtype=dtype))
        self._ok = ok
        arr = (HqqLinearWeight * max(1, len(self._items)))()
        for i, (pk, sc, ze, N, Y) in enumerate(self._items):
            arr[i] = HqqLinearWeight(_dev_ptr(pk, "packed", _U32).value,
                                     _dev_ptr(sc, "scale", (torch.float32,)).value,
                                     _dev_ptr(ze, "zero", (torch.float32,)).value, N,
                                     _dev_ptr(Y, "Y", ok).value)
        self._arr = arr

    def run(self, X: torch.Tensor):
        M, K = X.shape
        for (_, _, _, N, Y) in self._items:
            if tuple(Y.shape) != (M, N):
                raise ValueError(f"Y must be [{M}, {N}], got {tuple(Y.shape)}")
        ws = self._ws
        st = self._lib.hqq_linear_batch_ws(_dev_ptr(X, "X", self._ok), M, K, self._arr, len(self._items),
                                           self.nbits, self.group_size, self._code,
                                           ctypes.c_void_p(ws.data_ptr() if ws is not None else None),
                                           ws.numel() * ws.element_size() if ws is not None else 0,
                                           _stream(X.device))
        if st != 0:
            raise HQQError("hqq_linear_batch_ws", st)
        if ws is not None and not torch.cuda.is_current_stream_capturing():
            ws.record_stream(torch.cuda.current_stream(X.device))
        return [it[4] for it in self._items]


GEMM_WORKSPACE_BYTES = 32 << 20


def linear_workspace_bytes(M: int, Ns, K: int | None = None) -> int:
    """Workspace for hqq_linear_batch_ws over weights of output sizes Ns on M
    rows: the most K splits (8) of the fused kernels, and, given K, room for
    the dequantize-then-GEMM route (the largest W_hat, max(Ns) x K 2-byte
    values rounded up to 256 bytes, plus GEMM_WORKSPACE_BYTES for the GEMM)."""
    split = 8 * M * sum(Ns) * 4
    if K is None:
        return split
    what = -(-max(Ns) * K * 2 // 256) * 256
    return max(split, what + GEMM_WORKSPACE_BYTES)


def hqq_linear_batch(X: torch.Tensor, weights, nbits: int, group_size: int, workspace=None):
    """[X . W_hat_i^T] for weights [(packed, scale, zero, N), ...] sharing X,
    in one C-ABI call, in X's compute dtype (fp16 or bfloat16).  Returns the
    outputs.  workspace: see LinearBatch."""
    M = X.shape[0]
    _, tdt, _ = _compute_dtype(X)
    items = [(pk, sc, ze, N, torch.empty((M, N), dtype=tdt, device=X.device))
             for (pk, sc, ze, N) in weights]
    return LinearBatch(items, nbits, group_size, dtype=tdt, workspace=workspace).run(X)


def hqq_quantize_streamed(items, nbits: int, group_size: int, axis: int, staging: torch.Tensor,
                          copy_stream=None, compute_stream=None, iters: int = ITERS_DEFAULT,
                          p: float = P_DEFAULT, beta0: float = BETA0_DEFAULT,
                          kappa: float = KAPPA_DEFAULT):
    """Quantize weights held in host memory.  items: list of (W, packed, scale,
    zero) with W a CPU fp16 tensor (pinned for the copies to overlap) and the
    outputs CUDA tensors; staging: a CUDA buffer (any dtype) split in two
    halves.  Everything is enqueued on the two streams (default: the current
    stream for both); the results are complete when compute_stream is."""
    L = load_library()
    n = len(items)
    arr = (HqqHostTensor * max(n, 1))()
    for i, (W, pk, sc, ze) in enumerate(items):
        if not isinstance(W, torch.Tensor) or W.is_cuda or W.dtype not in _F16 or not W.is_contiguous():
            raise TypeError("W must be a contiguous CPU fp16 tensor")
        rows, cols = W.shape
        arr[i] = HqqHostTensor(W.data_ptr(), rows, cols, _dev_ptr(pk, "packed", _U32).value,
                               _dev_ptr(sc, "scale", (torch.float32,)).value,
                               _dev_ptr(ze, "zero", (torch.float32,)).value)
    if not isinstance(staging, torch.Tensor) or not staging.is_cuda or not staging.is_contiguous():
        raise TypeError("staging must be a contiguous CUDA tensor")
    dev = staging.device
    cs = copy_stream if copy_stream is not None else torch.cuda.current_stream(dev)
    ks = compute_stream if compute_stream is not None else torch.cuda.current_stream(dev)
    st = L.hqq_quantize_streamed(ctypes.cast(arr, ctypes.c_void_p), n, nbits, group_size, axis, iters,
                                 p, beta0, kappa, ctypes.c_void_p(staging.data_ptr()),
                                 staging.numel() * staging.element_size(),
                                 ctypes.c_void_p(cs.cuda_stream), ctypes.c_void_p(ks.cuda_stream))
    if st != 0:
        raise HQQError("hqq_quantize_streamed", st)
    # the staging buffer is in use on both streams until compute_stream
    # completes: keep torch's allocator from handing it out earlier
    staging.record_stream(cs)
    staging.record_stream(ks)


def _host_items(items):
    n = len(items)
    arr = (HqqHostTensor * max(n, 1))()
    for i, (W, pk, sc, ze) in enumerate(items):
        if not isinstance(W, torch.Tensor) or W.is_cuda or W.dtype not in _F16 or not W.is_contiguous():
            raise TypeError("W must be a contiguous CPU fp16 tensor")
        rows, cols = W.shape
        arr[i] = HqqHostTensor(W.data_ptr(), rows, cols, _dev_ptr(pk, "packed", _U32).value,
                               _dev_ptr(sc, "scale", (torch.float32,)).value,
                               _dev_ptr(ze, "zero", (torch.float32,)).value)
    return arr, n


STATIC_STAGING_BYTES = 64 << 20


def hqq_quantize_streamed_static(items, nbits: int, group_size: int, axis: int, copy_stream=None,
                                 compute_stream=None, iters: int = ITERS_DEFAULT,
                                 p: float = P_DEFAULT, beta0: float = BETA0_DEFAULT,
                                 kappa: float = KAPPA_DEFAULT, device=None):
    """hqq_quantize_streamed through the library's static staging array
    (STATIC_STAGING_BYTES per device): no device allocation in the call.
    Calls on one device must not overlap (they share the array)."""
    L = load_library()
    arr, n = _host_items(items)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    cs = copy_stream if copy_stream is not None else torch.cuda.current_stream(dev)
    ks = compute_stream if compute_stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = L.hqq_quantize_streamed_static(ctypes.cast(arr, ctypes.c_void_p), n, nbits, group_size, axis,
                                            iters, p, beta0, kappa, ctypes.c_void_p(cs.cuda_stream),
                                            ctypes.c_void_p(ks.cuda_stream))
    if st != 0:
        raise HQQError("hqq_quantize_streamed_static", st)


def hqq_quantize_meta(meta: torch.Tensor, group_size: int = 128):
    """8-bit RTN of a scale or zero array (quant_scale / quant_zero), read flat
    in groups of group_size.  Returns (codes uint8 [n], mscale, mzero)."""
    L = load_library()
    n = meta.numel()
    ng = -(-n // group_size)
    codes = torch.empty(n, dtype=torch.uint8, device=meta.device)
    ms = torch.empty(ng, dtype=torch.float32, device=meta.device)
    mz = torch.empty(ng, dtype=torch.float32, device=meta.device)
    st = L.hqq_quantize_meta(_dev_ptr(meta, "meta", (torch.float32,)), n, group_size,
                             _dev_ptr(codes, "codes", (torch.uint8,)), _dev_ptr(ms, "mscale", (torch.float32,)),
                             _dev_ptr(mz, "mzero", (torch.float32,)), _stream(meta.device))
    if st != 0:
        raise HQQError("hqq_quantize_meta", st)
    return codes, ms, mz


def hqq_dequantize_meta(codes: torch.Tensor, mscale, mzero, group_size: int = 128, out=None):
    """fp32 meta [n] from its 8-bit codes."""
    L = load_library()
    n = codes.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    st = L.hqq_dequantize_meta(_dev_ptr(codes, "codes", (torch.uint8,)),
                               _dev_ptr(mscale, "mscale", (torch.float32,)),
                               _dev_ptr(mzero, "mzero", (torch.float32,)), n, group_size,
                               _dev_ptr(out, "out", (torch.float32,)), _stream(codes.device))
    if st != 0:
        raise HQQError("hqq_dequantize_meta", st)
    return out


class MetaBatch:
    """Several meta arrays for hqq_quantize_meta_batch / hqq_dequantize_meta_batch,
    marshalled into the C descriptor array once; quantize() and dequantize()
    are then single C-ABI calls (one launch per 64 arrays) on the current
    stream.  items: list of (meta fp32, codes uint8, mscale fp32, mzero fp32)
    CUDA tensors, kept alive by the object."""

    def __init__(self, items, group_size: int = 128):
        self._lib = load_library()
        self._items = [tuple(it) for it in items]
        self.group_size = group_size
        arr = (HqqMetaTensor * max(1, len(self._items)))()
        for i, (m, c, ms, mz) in enumerate(self._items):
            n = m.numel()
            if c.numel() != n:
                raise ValueError(f"item {i}: codes has {c.numel()} values for {n} meta values")
            ng = -(-n // group_size)
            if ms.numel() != ng or mz.numel() != ng:
                raise ValueError(f"item {i}: mscale / mzero need {ng} values")
            arr[i] = HqqMetaTensor(_dev_ptr(m, "meta", (torch.float32,)).value, n,
                                   _dev_ptr(c, "codes", (torch.uint8,)).value,
                                   _dev_ptr(ms, "mscale", (torch.float32,)).value,
                                   _dev_ptr(mz, "mzero", (torch.float32,)).value)
        self._arr = arr
        self._device = self._items[0][0].device if self._items else None

    def quantize(self, stream=None):
        st = self._lib.hqq_quantize_meta_batch(self._arr, len(self._items), self.group_size,
                                               stream if stream is not None else self._stream())
        if st != 0:
            raise HQQError("hqq_quantize_meta_batch", st)

    def dequantize(self, stream=None):
        st = self._lib.hqq_dequantize_meta_batch(self._arr, len(self._items), self.group_size,
                                                 stream if stream is not None else self._stream())
        if st != 0:
            raise HQQError("hqq_dequantize_meta_batch", st)

    def _stream(self):
        return _stream(self._device) if self._device is not None else None


def hqq_quantize_meta_batch(metas, group_size: int = 128):
    """hqq_quantize_meta over a list of fp32 arrays in one call.  Returns a list
    of (codes, mscale, mzero)."""
    outs = []
    for m in metas:
        ng = -(-m.numel() // group_size)
        outs.append((torch.empty(m.numel(), dtype=torch.uint8, device=m.device),
                     torch.empty(ng, dtype=torch.float32, device=m.device),
                     torch.empty(ng, dtype=torch.float32, device=m.device)))
    MetaBatch([(m, *o) for m, o in zip(metas, outs)], group_size).quantize()
    return outs


def hqq_dequantize_meta_batch(quantized, group_size: int = 128):
    """hqq_dequantize_meta over a list of (codes, mscale, mzero) in one call.
    Returns the fp32 arrays."""
    outs = [torch.empty(c.numel(), dtype=torch.float32, device=c.device) for c, _, _ in quantized]
    MetaBatch([(o, c, ms, mz) for o, (c, ms, mz) in zip(outs, quantized)], group_size).dequantize()
    return outs
