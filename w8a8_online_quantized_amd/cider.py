"""Python binding of libcider (include/cider.h): argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU (PyTorch is used for device memory and
the current stream, nothing else). Every step of the computation runs in the
HIP kernels of libcider.so; if the library is missing, or the device is not a
gfx950, the call raises instead of computing anything some other way.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcider.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "cider.h")

CIDER_SUCCESS = 0
CIDER_ERROR_INVALID_VALUE = 1
CIDER_ERROR_NOT_SUPPORTED = 2
CIDER_ERROR_LAUNCH = 3
CIDER_ERROR_SCRATCH_LIMIT = 4
NOALLOC_SCRATCH_BYTES = 48 * 1024 * 1024

_c_i64, _c_i32, _c_p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p

# (restype, argtypes) of every entry point declared in include/cider.h
SIGNATURES = {
    "cider_is_available": (ctypes.c_int, []),
    "cider_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cider_version": (ctypes.c_int, []),
    "cider_quant_act": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "cider_quant_weight": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "cider_w8a8_gemm": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p]),
    "cider_w4a8_gemm": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "cider_gemm_acc_i32": (ctypes.c_int, [_c_i32, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p]),
    "cider_w8a8_gemm_token_group": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p,
                                                   _c_p, _c_i64, _c_p]),
    "cider_w8a8_gemm_token_group_dt": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p,
                                                      _c_i32, _c_p, _c_i64, _c_p]),
    "cider_w8a8_gemm_split": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "cider_w8a8_gemm_split_dt": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_i32,
                                                _c_p]),
    "cider_linear_workspace_size": (ctypes.c_int64, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "cider_gemm_workspace_size": (ctypes.c_int64, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "cider_w8a8_gemm_ex": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_i32, _c_p,
                                         _c_i64, _c_p]),
    "cider_w8a8_gemm_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_i32,
                                              _c_p]),
    "cider_w4a8_gemm_ex": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i32, _c_p, _c_i64,
                                         _c_p]),
    "cider_linear": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_p, _c_i64, _c_p,
                                    _c_p]),
    "cider_linear_dt": (ctypes.c_int, [_c_p, _c_i32, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_p,
                                       _c_i64, _c_p, _c_p]),
    "cider_quant_weight_clip": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32, ctypes.c_double, _c_p,
                                               _c_p, _c_p]),
    "cider_quant_act_dt": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "cider_quant_weight_dt": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "cider_w8a8_gemm_dt": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_i32, _c_p]),
    "cider_w4a8_gemm_dt": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
    "cider_read_probe": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p]),
    "cider_int8_mv": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p]),
    "cider_stack_workspace_layout": (ctypes.c_int64, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                      ctypes.POINTER(ctypes.c_int64)]),
    "cider_stack_forward": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p,
                                           _c_i64, _c_p, _c_p]),
    "cider_stack_forward_dt": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p,
                                              _c_p, _c_i64, _c_p, _c_p]),
}

STACK_PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")
STACK_REGIONS = ("codes", "scales", "q", "k", "v", "o", "gate", "up", "h")


class StackLayer(ctypes.Structure):
    """cider_stack_layer_t: device pointers of one layer's 7 weight matrices."""
    _fields_ = [("w", ctypes.c_void_p * 7), ("s", ctypes.c_void_p * 7)]

_lib = None


class CiderError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def header_entry_points(path: str = HEADER_PATH):
    """Names of the functions include/cider.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cider_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Load libcider.so (built in-tree by w8a8_online_quantized_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m w8a8_online_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().cider_status_string(status).decode()


def _check(fn: str, status: int):
    if status != CIDER_SUCCESS:
        raise CiderError(fn, status, status_string(status))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run the wrapped call with `stream` (when given) as torch's current
    stream, so that every output and temporary it allocates belongs to the
    stream its kernels run on: torch's caching allocator then reuses a freed
    temporary only for later work on that same stream, never while a kernel
    of the call may still read it."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        import torch
        ctx = torch.cuda.stream(stream) if stream != torch.cuda.current_stream() else contextlib.nullcontext()
        with ctx:
            return fn(*args, stream=stream, **kw)
    return wrapper


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _carg(a):
    """A call argument in C form: a tensor as its device pointer, a stream as
    its handle, anything else as given (ctypes converts ints and None)."""
    import torch
    if isinstance(a, torch.Tensor):
        return ctypes.c_void_p(a.data_ptr())
    if isinstance(a, torch.cuda.Stream):
        return ctypes.c_void_p(a.cuda_stream)
    return a


def prepared(fn_name: str, *args):
    """A zero-argument callable that calls the C entry point `fn_name` with
    its arguments already in C form (tensors as device pointers, the stream
    as its handle) and raises on a non-zero status. Timing loops use it so
    that back-to-back launches of short kernels are not paced by Python-side
    argument checking; the caller keeps the tensors alive."""
    f = getattr(lib(), fn_name)
    cargs = tuple(_carg(a) for a in args)

    def call():
        st = f(*cargs)
        if st != CIDER_SUCCESS:
            _check(fn_name, st)
    return call


def cider_is_available() -> bool:
    return bool(lib().cider_is_available())


def cider_version() -> int:
    return int(lib().cider_version())


CIDER_DTYPE_F16, CIDER_DTYPE_BF16 = 0, 1


def _fp_code(t, name):
    """cider_dtype_t of an fp16 / bf16 tensor."""
    import torch
    if t.dtype == torch.float16:
        return CIDER_DTYPE_F16
    if t.dtype == torch.bfloat16:
        return CIDER_DTYPE_BF16
    raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")


def _scale_shape(rows, K, group_size):
    return (rows,) if group_size == 0 else (rows, K // group_size)


@_on_stream
def cider_quant_act(x, group_size: int = 0, x_q=None, x_scale=None, stream=None):
    """fp16 or bf16 [M, K] -> (int8 codes [M, K], fp32 scales [M] or [M, K/gs])."""
    import torch
    M, K = x.shape
    dt = _fp_code(x, "x")
    _need(x, x.dtype, (M, K), "x")
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(_scale_shape(M, K, group_size), dtype=torch.float32, device=x.device)
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(x_scale, torch.float32, _scale_shape(M, K, group_size), "x_scale")
    _check("cider_quant_act_dt", lib().cider_quant_act_dt(_ptr(x), dt, M, K, group_size, _ptr(x_q), _ptr(x_scale),
                                                          _stream(stream)))
    return x_q, x_scale


@_on_stream
def cider_quant_weight(w, bits: int = 8, group_size: int = 0, w_q=None, w_scale=None, stream=None):
    """fp16 or bf16 [N, K] -> (int8 [N, K] or packed uint8 [N, K/2], fp32 scales)."""
    import torch
    N, K = w.shape
    dt = _fp_code(w, "w")
    _need(w, w.dtype, (N, K), "w")
    qshape = (N, K) if bits == 8 else (N, K // 2)
    qdtype = torch.int8 if bits == 8 else torch.uint8
    if w_q is None:
        w_q = torch.empty(qshape, dtype=qdtype, device=w.device)
    if w_scale is None:
        w_scale = torch.empty(_scale_shape(N, K, group_size), dtype=torch.float32, device=w.device)
    _need(w_q, qdtype, qshape, "w_q")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    _check("cider_quant_weight_dt", lib().cider_quant_weight_dt(_ptr(w), dt, N, K, bits, group_size, _ptr(w_q),
                                                                _ptr(w_scale), _stream(stream)))
    return w_q, w_scale


@_on_stream
def cider_quant_weight_clip(w, bits: int = 8, group_size: int = 0, percentile: float = 99.9, w_q=None,
                            w_scale=None, stream=None):
    """cider_quant_weight with percentile-clipped scales (same outputs)."""
    import torch
    N, K = w.shape
    dt = _fp_code(w, "w")
    _need(w, w.dtype, (N, K), "w")
    qshape = (N, K) if bits == 8 else (N, K // 2)
    qdtype = torch.int8 if bits == 8 else torch.uint8
    if w_q is None:
        w_q = torch.empty(qshape, dtype=qdtype, device=w.device)
    if w_scale is None:
        w_scale = torch.empty(_scale_shape(N, K, group_size), dtype=torch.float32, device=w.device)
    _need(w_q, qdtype, qshape, "w_q")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    _check("cider_quant_weight_clip",
           lib().cider_quant_weight_clip(_ptr(w), dt, N, K, bits, group_size, float(percentile), _ptr(w_q),
                                         _ptr(w_scale), _stream(stream)))
    return w_q, w_scale


def cider_gemm_workspace_size(M: int, N: int, K: int, bits: int = 8, group_size: int = 0) -> int:
    """Split-K workspace bytes the GEMM dispatch uses at this shape (0: none)."""
    n = int(lib().cider_gemm_workspace_size(M, N, K, bits, group_size))
    if n < 0:
        raise ValueError("invalid GEMM sizes")
    return n


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


@_on_stream
def cider_w8a8_gemm(x_q, x_scale, w_q, w_scale, group_size: int = 0, y=None, stream=None, out_dtype=None,
                    workspace=None):
    """int8 codes + scales -> y [M, N] (fused dequant): fp16, or bf16 when
    out_dtype (or a given y) is bfloat16. A workspace of at least
    cider_gemm_workspace_size bytes enables split-K where the plan uses it."""
    import torch
    M, K = x_q.shape
    N = w_q.shape[0]
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(w_q, torch.int8, (N, K), "w_q")
    if group_size and K % group_size:
        raise ValueError("K must be a multiple of group_size")
    _need(x_scale, torch.float32, _scale_shape(M, K, group_size), "x_scale")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float16, device=x_q.device)
    dt = _fp_code(y, "y")
    _need(y, y.dtype, (M, N), "y")
    wsp, wsb = _ws_args(workspace)
    _check("cider_w8a8_gemm_ex", lib().cider_w8a8_gemm_ex(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                                                          M, N, K, group_size, _ptr(y), dt, wsp, wsb,
                                                          _stream(stream)))
    return y


@_on_stream
def cider_w8a8_gemm_noalloc(x_q, x_scale, w_q, w_scale, group_size: int = 0, y=None, stream=None, out_dtype=None):
    """cider_w8a8_gemm with the split-K scratch in the library's own device
    array (the C call allocates nothing; pass y to allocate nothing here
    either). Calls that overlap in time on one GPU race on that array."""
    import torch
    M, K = x_q.shape
    N = w_q.shape[0]
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(w_q, torch.int8, (N, K), "w_q")
    if group_size and K % group_size:
        raise ValueError("K must be a multiple of group_size")
    _need(x_scale, torch.float32, _scale_shape(M, K, group_size), "x_scale")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float16, device=x_q.device)
    dt = _fp_code(y, "y")
    _need(y, y.dtype, (M, N), "y")
    _check("cider_w8a8_gemm_noalloc", lib().cider_w8a8_gemm_noalloc(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                                                                    M, N, K, group_size, _ptr(y), dt, _stream(stream)))
    return y


@_on_stream
def cider_w8a8_gemm_token_group(x_q, x_scale, w_q, w_scale, group_size: int, y=None, stream=None, workspace=None,
                                out_dtype=None):
    """Per-token activation codes (x_scale [M]) times per-group weight codes
    (w_scale [N, K/group_size], group_size 64 or 128) -> y [M, N]: fp16, or
    bf16 when out_dtype (or a given y) is bfloat16."""
    import torch
    M, K = x_q.shape
    N = w_q.shape[0]
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(w_q, torch.int8, (N, K), "w_q")
    if group_size not in (64, 128) or K % group_size:
        raise ValueError("group_size must be 64 or 128 and divide K")
    _need(x_scale, torch.float32, (M,), "x_scale")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float16, device=x_q.device)
    dt = _fp_code(y, "y")
    _need(y, y.dtype, (M, N), "y")
    _check("cider_w8a8_gemm_token_group_dt",
           lib().cider_w8a8_gemm_token_group_dt(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale), M, N, K,
                                                group_size, _ptr(y), dt, *_ws_args(workspace), _stream(stream)))
    return y


@_on_stream
def cider_w8a8_gemm_split(x_q, x_scale, w_q, w_scale, part_n, ys=None, stream=None, out_dtype=None):
    """Per-channel GEMM of x_q against row-concatenated weights w_q [sum(part_n), K];
    returns one [M, part_n[i]] output per part: fp16, or bf16 when out_dtype
    (or the given ys) is bfloat16."""
    import torch
    M, K = x_q.shape
    N = w_q.shape[0]
    part_n = [int(n) for n in part_n]
    if sum(part_n) != N:
        raise ValueError("part widths must add up to the weight rows")
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(w_q, torch.int8, (N, K), "w_q")
    _need(x_scale, torch.float32, (M,), "x_scale")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if ys is None:
        ys = [torch.empty((M, n), dtype=out_dtype or torch.float16, device=x_q.device) for n in part_n]
    dt = _fp_code(ys[0], "ys[0]")
    for i, (y, n) in enumerate(zip(ys, part_n)):
        _need(y, ys[0].dtype, (M, n), f"ys[{i}]")
    arr_n = (ctypes.c_int64 * len(part_n))(*part_n)
    arr_y = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    _check("cider_w8a8_gemm_split_dt",
           lib().cider_w8a8_gemm_split_dt(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale), M, K, len(part_n),
                                          ctypes.cast(arr_n, ctypes.c_void_p), ctypes.cast(arr_y, ctypes.c_void_p),
                                          dt, _stream(stream)))
    return ys


def cider_linear_workspace_size(M: int, N: int, K: int, bits: int = 8, group_size: int = 0) -> int:
    """Workspace bytes cider_linear needs (0: one launch, no workspace)."""
    n = int(lib().cider_linear_workspace_size(M, N, K, bits, group_size))
    if n < 0:
        raise ValueError("invalid linear sizes")
    return n


@_on_stream
def cider_linear(x, w, w_scale, bits: int = 8, group_size: int = 0, workspace=None, y=None, stream=None):
    """x [M, K] -> y [M, N] of the same dtype (fp16 or bf16) through the
    quantized linear (w: int8 codes [N, K] for bits 8, packed uint8 [N, K/2]
    for bits 4)."""
    import torch
    M, K = x.shape
    N = w.shape[0]
    dt = _fp_code(x, "x")
    _need(x, x.dtype, (M, K), "x")
    if bits == 8:
        _need(w, torch.int8, (N, K), "w")
    else:
        _need(w, torch.uint8, (N, K // 2), "w")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    need = cider_linear_workspace_size(M, N, K, bits, group_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _need(y, x.dtype, (M, N), "y")
    wsp = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("cider_linear_dt", lib().cider_linear_dt(_ptr(x), dt, _ptr(w), _ptr(w_scale), M, N, K, bits, group_size,
                                                    wsp, wsb, _ptr(y), _stream(stream)))
    return y


@_on_stream
def cider_int8_mv(x, w_q, w_scale, group_size: int = 0, y=None, stream=None):
    """Decode MV: fp16 x [M, K] (M <= 4) times int8 weights dequantized on the
    fly -> fp16 y [M, N]; no activation quantization."""
    import torch
    M, K = x.shape
    N = w_q.shape[0]
    _need(x, torch.float16, (M, K), "x")
    _need(w_q, torch.int8, (N, K), "w_q")
    if group_size and K % group_size:
        raise ValueError("K must be a multiple of group_size")
    _need(w_scale, torch.float32, _scale_shape(N, K, group_size), "w_scale")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _need(y, torch.float16, (M, N), "y")
    _check("cider_int8_mv", lib().cider_int8_mv(_ptr(x), _ptr(w_q), _ptr(w_scale), M, N, K, group_size,
                                                _ptr(y), _stream(stream)))
    return y


def cider_read_probe(buf, sink, stream=None):
    """One pass over a device buffer (measurement helper: the single-launch
    read ceiling); `sink` is a small int32 device tensor."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _need(sink, torch.int32, tuple(sink.shape), "sink")
    _check("cider_read_probe", lib().cider_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                      _stream(stream)))


@_on_stream
def cider_w4a8_gemm(x_q, x_scale, w_packed, w_scale, y=None, stream=None, out_dtype=None, workspace=None):
    """int8 activation codes x packed int4 weights -> y [M, N] (fp16 or bf16)."""
    import torch
    M, K = x_q.shape
    N = w_packed.shape[0]
    _need(x_q, torch.int8, (M, K), "x_q")
    _need(w_packed, torch.uint8, (N, K // 2), "w_packed")
    _need(x_scale, torch.float32, (M,), "x_scale")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float16, device=x_q.device)
    dt = _fp_code(y, "y")
    _need(y, y.dtype, (M, N), "y")
    wsp, wsb = _ws_args(workspace)
    _check("cider_w4a8_gemm_ex", lib().cider_w4a8_gemm_ex(_ptr(x_q), _ptr(x_scale), _ptr(w_packed), _ptr(w_scale),
                                                          M, N, K, _ptr(y), dt, wsp, wsb, _stream(stream)))
    return y


@_on_stream
def cider_gemm_acc_i32(mode: int, x_q, w, group_size: int = 0, acc=None, stream=None):
    """int32 accumulators of the GEMM main loop: [M, N], or [G, M, N] per group."""
    import torch
    M, K = x_q.shape
    N = w.shape[0]
    _need(x_q, torch.int8, (M, K), "x_q")
    if mode == 0:
        _need(w, torch.int8, (N, K), "w")
    else:
        _need(w, torch.uint8, (N, K // 2), "w")
    shape = (M, N) if group_size == 0 else (K // group_size, M, N)
    if acc is None:
        acc = torch.empty(shape, dtype=torch.int32, device=x_q.device)
    _need(acc, torch.int32, shape, "acc")
    _check("cider_gemm_acc_i32", lib().cider_gemm_acc_i32(mode, _ptr(x_q), _ptr(w), M, N, K, group_size,
                                                          _ptr(acc), _stream(stream)))
    return acc


@_on_stream
def w8a8_linear(x, w_q, w_scale, group_size: int = 0, stream=None):
    """The README's per-channel / per-group linear: quantize x, then the fused
    GEMM; the output has x's type (fp16 or bf16)."""
    x_q, x_scale = cider_quant_act(x, group_size, stream=stream)
    return cider_w8a8_gemm(x_q, x_scale, w_q, w_scale, group_size, stream=stream, out_dtype=x.dtype)


@_on_stream
def w8a8_linear_token_group(x, w_q, w_scale, group_size: int, stream=None):
    """Per-token activation quantization, then the per-group-weight GEMM."""
    x_q, x_scale = cider_quant_act(x, 0, stream=stream)
    return cider_w8a8_gemm_token_group(x_q, x_scale, w_q, w_scale, group_size, stream=stream)


@_on_stream
def w4a8_linear(x, w_packed, w_scale, stream=None):
    """The README's W4A8 linear: per-token int8 activations times packed int4
    weights; the output has x's type (fp16 or bf16)."""
    x_q, x_scale = cider_quant_act(x, 0, stream=stream)
    return cider_w4a8_gemm(x_q, x_scale, w_packed, w_scale, stream=stream, out_dtype=x.dtype)


def cider_stack_workspace_layout(M: int, hidden: int, q_dim: int, kv_dim: int, mlp_dim: int):
    """(total bytes, {region: byte offset}) of the stack driver's workspace."""
    offs = (ctypes.c_int64 * 9)()
    total = int(lib().cider_stack_workspace_layout(M, hidden, q_dim, kv_dim, mlp_dim, offs))
    return total, dict(zip(STACK_REGIONS, list(offs)))


def stack_region(workspace, offsets, name, M, hidden, q_dim, kv_dim, mlp_dim, dtype=None):
    """A torch view of one workspace region (for checking intermediates);
    dtype: torch.float16 (default) or torch.bfloat16 for a bf16 chain."""
    import torch
    dims = {"q": q_dim, "k": kv_dim, "v": kv_dim, "o": hidden, "gate": mlp_dim, "up": mlp_dim, "h": hidden}
    n = dims[name]
    start = offsets[name]
    return workspace[start:start + 2 * M * n].view(dtype or torch.float16).view(M, n)


def fuse_stack_layer(layer):
    """A copy of one stack layer ({name: (codes, scales)}) whose q/k/v and
    gate/up codes and scales live back to back in one allocation each, so
    that cider_stack_forward runs each group as one GEMM."""
    import torch
    out = dict(layer)
    for group in (("q", "k", "v"), ("gate", "up")):
        wcat = torch.cat([layer[n][0] for n in group])
        scat = torch.cat([layer[n][1] for n in group])
        r = 0
        for n in group:
            rows = layer[n][0].shape[0]
            out[n] = (wcat[r:r + rows], scat[r:r + rows])
            r += rows
    return out


@_on_stream
def cider_stack_forward(x, layers, dims, workspace=None, y=None, stream=None):
    """Runs the chained linear stack. `layers`: list of dicts {name: (codes, scales)}
    for the seven projections; dims = (hidden, q_dim, kv_dim, mlp_dim)."""
    import torch
    hidden, q_dim, kv_dim, mlp_dim = dims
    M = x.shape[0]
    dt = _fp_code(x, "x")
    _need(x, x.dtype, (M, hidden), "x")
    total, _ = cider_stack_workspace_layout(M, hidden, q_dim, kv_dim, mlp_dim)
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, hidden), dtype=x.dtype, device=x.device)
    _need(y, x.dtype, (M, hidden), "y")
    arr = (StackLayer * len(layers))()
    for i, L in enumerate(layers):
        for j, name in enumerate(STACK_PROJECTIONS):
            wq, ws = L[name]
            arr[i].w[j] = wq.data_ptr()
            arr[i].s[j] = ws.data_ptr()
    _check("cider_stack_forward_dt", lib().cider_stack_forward_dt(
        _ptr(x), dt, M, hidden, q_dim, kv_dim, mlp_dim, len(layers), ctypes.cast(arr, ctypes.c_void_p),
        _ptr(workspace), workspace.numel(), _ptr(y), _stream(stream)))
    return y, workspace
