"""Python binding of the HQQ C-ABI library (``libhqq.so``, HIP kernels for gfx950).

The functions here only marshal arguments: torch tensors provide device memory and the
current HIP stream; every step of the quantizer, the dequantisation and the fused
product runs in the library's kernels.  There is no fallback: when the library is missing
the import of a compute function raises.

Names follow the C ABI (``include/hqq.h``): ``hqq_quantize``, ``hqq_dequantize``,
``hqq_gemv_w4a16``, ``hqq_gemv`` (the other stored formats), plus the size queries.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhqq.so")
PROBE_LIB_PATH = os.path.join(HERE, "libhqq_probe.so")

HQQ_OK = 0
HQQ_ERR_INVALID_ARGUMENT = 1
HQQ_ERR_UNSUPPORTED = 2
HQQ_ERR_WORKSPACE = 3
HQQ_ERR_DEVICE = 4
HQQ_META_F16, HQQ_META_F32, HQQ_META_F64 = 0, 1, 2
HQQ_OUT_F16, HQQ_OUT_F32 = 0, 1
HQQ_MAX_ITERS = 64
HQQ_TINY_RANGE = 1e-4
HQQ_STOP_BEST, HQQ_STOP_FAILED, HQQ_STOP_NONE, HQQ_STOP_MEASURED_END = 0, 1, 2, 4
HQQ_DEBUG_NO_FROZEN_SKIP, HQQ_DEBUG_SLOW_SHRINK, HQQ_DEBUG_SYNC = 1, 2, 4
HQQ_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol the header declares.
EXPORTS = ("hqq_packed_bytes", "hqq_num_groups", "hqq_quantize_workspace_bytes", "hqq_quantize", "hqq_quantize_ex",
           "hqq_quantize_noalloc",
           "hqq_quantize_v2", "hqq_quantize_v2_workspace_bytes",
           "hqq_dequantize", "hqq_gemv_w4a16", "hqq_gemm_workspace_bytes", "hqq_gemm_w4a16",
           "hqq_gemm_dx_workspace_bytes", "hqq_gemm_w4a16_dx", "hqq_gemm_dx", "hqq_gemv", "hqq_gemm",
           "hqq_release_workspaces", "hqq_status_string", "hqq_last_error")

_lib = None


class HQQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_string(status) if _lib else status, message))
        self.status = status


def load(path: str = LIB_PATH):
    """Load libhqq.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libhqq.so not built (run `python -m weight_only_quantization_amd.build`): %s" % path)
    lib = ctypes.CDLL(path)
    i64, i32, dbl, p, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
    lib.hqq_packed_bytes.argtypes = [i64, i64, i32]
    lib.hqq_packed_bytes.restype = sz
    lib.hqq_num_groups.argtypes = [i64, i64, i32]
    lib.hqq_num_groups.restype = i64
    lib.hqq_quantize_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    lib.hqq_quantize_workspace_bytes.restype = sz
    lib.hqq_quantize.argtypes = [p, i64, i64, i32, i32, i32, i32, dbl, dbl, dbl, p, p, p, i32, p, sz, p, p, p]
    lib.hqq_quantize.restype = i32
    lib.hqq_quantize_noalloc.argtypes = [p, i64, i64, i32, i32, i32, i32, dbl, dbl, dbl, p, p, p, i32, p, p, p]
    lib.hqq_quantize_noalloc.restype = i32
    lib.hqq_quantize_ex.argtypes = [ctypes.POINTER(QuantArgs)]
    lib.hqq_quantize_ex.restype = i32
    lib.hqq_quantize_v2.argtypes = [ctypes.POINTER(QuantV2Args)]
    lib.hqq_quantize_v2.restype = i32
    lib.hqq_quantize_v2_workspace_bytes.argtypes = [i64, i64, i32]
    lib.hqq_quantize_v2_workspace_bytes.restype = sz
    lib.hqq_dequantize.argtypes = [p, p, p, i32, i64, i64, i32, i32, i32, p, p]
    lib.hqq_dequantize.restype = i32
    lib.hqq_gemv_w4a16.argtypes = [p, p, p, i64, i64, i32, p, i64, p, i32, p]
    lib.hqq_gemv_w4a16.restype = i32
    lib.hqq_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.hqq_gemm_workspace_bytes.restype = sz
    lib.hqq_gemm_w4a16.argtypes = [p, p, p, i64, i64, i32, p, i64, p, i32, p, sz, p]
    lib.hqq_gemm_w4a16.restype = i32
    lib.hqq_gemm_dx_workspace_bytes.argtypes = [i64, i64, i64]
    lib.hqq_gemm_dx_workspace_bytes.restype = sz
    lib.hqq_gemm_w4a16_dx.argtypes = [p, p, p, i64, i64, i32, p, i64, p, i32, p, sz, p]
    lib.hqq_gemm_w4a16_dx.restype = i32
    lib.hqq_gemm_dx.argtypes = [p, p, p, i64, i64, i32, i32, i32, p, i64, p, i32, p, sz, p]
    lib.hqq_gemm_dx.restype = i32
    lib.hqq_gemv.argtypes = [p, p, p, i64, i64, i32, i32, i32, p, i64, p, i32, p]
    lib.hqq_gemv.restype = i32
    lib.hqq_gemm.argtypes = [p, p, p, i64, i64, i32, i32, i32, p, i64, p, i32, p, sz, p]
    lib.hqq_gemm.restype = i32
    lib.hqq_status_string.argtypes = [i32]
    lib.hqq_status_string.restype = ctypes.c_char_p
    lib.hqq_release_workspaces.argtypes = []
    lib.hqq_release_workspaces.restype = i32
    lib.hqq_last_error.argtypes = []
    lib.hqq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().hqq_status_string(status).decode()


def last_error() -> str:
    return load().hqq_last_error().decode()


def _check(status: int):
    if status != HQQ_OK:
        raise HQQError(status, last_error())


# ------------------------------------------------------------------------------ size queries

def hqq_packed_bytes(rows: int, cols: int, nbits: int) -> int:
    return load().hqq_packed_bytes(rows, cols, nbits)


def hqq_num_groups(rows: int, cols: int, group_size: int) -> int:
    return load().hqq_num_groups(rows, cols, group_size)


def hqq_quantize_workspace_bytes(rows, cols, nbits, group_size, axis, iters) -> int:
    return load().hqq_quantize_workspace_bytes(rows, cols, nbits, group_size, axis, iters)


# ------------------------------------------------------------------------------ compute calls

def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for the tensors a call allocates: the caching allocator ties a block to the stream
    that is current when it is allocated, so temporaries (workspaces) and outputs are allocated
    on the stream the kernels run on; a block freed on return is then reused only by work
    ordered after those kernels."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(t, name, dtype=None, numel=None, min_bytes=None, shape=None, device=True):
    """Check a tensor operand before its pointer crosses the ABI (the C side reads raw memory of
    the type the format implies, so a wrong dtype or size would be read silently).  With
    device=False only the values are checked (the caller checks placement after all operands)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, %d needed" % (name, t.numel(), numel))
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, t.numel() * t.element_size(), min_bytes))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device:
        _placed(t, name)


def _placed(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _product_operands(packed, delta, zero, N, K, nbits, group_size, x, xname="x", out=None, out_cols=None):
    """Checks shared by the fused products: codes and fp16 metadata of W [N, K] and fp16 x [batch, *]."""
    import torch
    lib = load()
    if group_size <= 0 or (N * K) % group_size:
        raise ValueError("group_size must divide N*K")
    _need(packed, "packed", torch.uint8, min_bytes=lib.hqq_packed_bytes(N, K, nbits), device=False)
    _need(delta, "delta", torch.float16, numel=N * K // group_size, device=False)
    _need(zero, "zero", torch.float16, numel=N * K // group_size, device=False)
    _need(x, xname, torch.float16, device=False)
    if x.dim() != 2:
        raise ValueError("%s must be 2-D [batch, K]" % xname)
    if x.shape[1] != (K if xname == "x" else N):
        raise ValueError("%s must be [batch, %d], got %s" % (xname, K if xname == "x" else N, tuple(x.shape)))
    if out is not None:
        _need(out, "out", (torch.float16, torch.float32), shape=(x.shape[0], out_cols), device=False)
    for t, name in ((packed, "packed"), (delta, "delta"), (zero, "zero"), (x, xname), (out, "out")):
        if t is not None:
            _placed(t, name)


_META = {}


def _meta_code(dtype) -> int:
    import torch
    if not _META:
        _META.update({torch.float16: HQQ_META_F16, torch.float32: HQQ_META_F32, torch.float64: HQQ_META_F64})
    return _META[dtype]


@dataclass
class Quantized:
    """Result of hqq_quantize: packed codes plus per-group step and zero, and the solver's
    device-side stop index and MAE trace."""
    packed: "object"
    delta: "object"
    zero: "object"
    rows: int
    cols: int
    nbits: int
    group_size: int
    axis: int
    stop_iter: "object"
    mae_trace: "object"


class QuantArgs(ctypes.Structure):
    """hqq_quant_args of include/hqq.h (field order and C types as declared there)."""
    _fields_ = [("W_fp16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("nbits", ctypes.c_int), ("group_size", ctypes.c_int), ("axis", ctypes.c_int), ("iters", ctypes.c_int),
                ("p", ctypes.c_double), ("beta0", ctypes.c_double), ("kappa", ctypes.c_double),
                ("packed", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("zero", ctypes.c_void_p),
                ("meta_dtype", ctypes.c_int), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stop_iter_dev", ctypes.c_void_p), ("mae_trace_dev", ctypes.c_void_p), ("stream", ctypes.c_void_p),
                ("stop_rule", ctypes.c_int), ("tiny_range", ctypes.c_double), ("debug_flags", ctypes.c_int)]


class QuantV2Args(ctypes.Structure):
    """hqq_quant_v2_args of include/hqq.h (field order and C types as declared there)."""
    _fields_ = [("W_fp16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("nbits", ctypes.c_int), ("group_size", ctypes.c_int), ("axis", ctypes.c_int), ("iters", ctypes.c_int),
                ("p", ctypes.c_double), ("beta0", ctypes.c_double), ("kappa", ctypes.c_double),
                ("tiny_range", ctypes.c_double), ("scale_grid", ctypes.c_void_p), ("n_candidates", ctypes.c_int),
                ("packed", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("zero", ctypes.c_void_p),
                ("meta_dtype", ctypes.c_int), ("choice_dev", ctypes.c_void_p), ("stream", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


def hqq_quantize(W, nbits: int = 4, group_size: int = 64, axis: int = 1, iters: int = 20, p: float = 0.7,
                 beta0: float = 10.0, kappa: float = 1.01, meta_dtype=None, workspace=None, out=None,
                 stream=None, stop_rule: int = HQQ_STOP_BEST, tiny_range: float | None = None,
                 debug_flags: int = 0) -> Quantized:
    """HQQ quantisation of a 2-D fp16 CUDA tensor.  Output buffers are torch tensors (or the
    ones passed in `out` as (packed, delta, zero, stop_iter, mae_trace)).  A stop rule, tiny
    range or debug flag other than the defaults goes through hqq_quantize_ex."""
    import torch
    lib = load()
    _need(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    rows, cols = W.shape
    meta_dtype = meta_dtype or torch.float16
    G = lib.hqq_num_groups(rows, cols, group_size)
    dev = W.device
    with _on(stream):
        if out is None:
            packed = torch.empty(max(lib.hqq_packed_bytes(rows, cols, nbits), 1), dtype=torch.uint8, device=dev)
            delta = torch.empty(max(G, 1), dtype=meta_dtype, device=dev)
            zero = torch.empty(max(G, 1), dtype=meta_dtype, device=dev)
            stop_iter = torch.empty(1, dtype=torch.int32, device=dev)
            mae_trace = torch.empty(max(iters, 1), dtype=torch.float64, device=dev)
        else:
            packed, delta, zero, stop_iter, mae_trace = out
            _need(packed, "packed", torch.uint8, min_bytes=lib.hqq_packed_bytes(rows, cols, nbits))
            for t, n in ((delta, "delta"), (zero, "zero")):
                _need(t, n, meta_dtype, numel=max(G, 1))
            _need(stop_iter, "stop_iter", torch.int32, numel=1)
            _need(mae_trace, "mae_trace", torch.float64, numel=iters)
        ws_bytes = lib.hqq_quantize_workspace_bytes(rows, cols, nbits, group_size, axis, iters)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        else:
            _need(workspace, "workspace", torch.uint8)
    if stop_rule == HQQ_STOP_BEST and tiny_range is None and debug_flags == 0:
        st = lib.hqq_quantize(ctypes.c_void_p(W.data_ptr()), rows, cols, nbits, group_size, axis, iters, p, beta0,
                              kappa, ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                              ctypes.c_void_p(zero.data_ptr()), _meta_code(meta_dtype),
                              ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                              ctypes.c_void_p(stop_iter.data_ptr()), ctypes.c_void_p(mae_trace.data_ptr()),
                              _stream_ptr(stream))
    else:
        args = QuantArgs(W.data_ptr(), rows, cols, nbits, group_size, axis, iters, p, beta0, kappa, packed.data_ptr(),
                         delta.data_ptr(), zero.data_ptr(), _meta_code(meta_dtype), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), stop_iter.data_ptr(), mae_trace.data_ptr(),
                         _stream_ptr(stream).value, stop_rule, HQQ_TINY_RANGE if tiny_range is None else tiny_range,
                         debug_flags)
        st = lib.hqq_quantize_ex(ctypes.byref(args))
    _check(st)
    return Quantized(packed, delta, zero, rows, cols, nbits, group_size, axis, stop_iter, mae_trace)


def hqq_quantize_noalloc(W, out, nbits: int = 4, group_size: int = 64, axis: int = 1, iters: int = 20,
                         p: float = 0.7, beta0: float = 10.0, kappa: float = 1.01, stream=None) -> Quantized:
    """hqq_quantize into caller-given outputs `out` = (packed, delta, zero, stop_iter, mae_trace)
    with the library's own scratch array: the call allocates nothing (no torch allocation either),
    so it may run where allocation is not allowed.  Calls on one GPU share its scratch array and
    must not overlap."""
    import torch
    lib = load()
    _need(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    rows, cols = W.shape
    packed, delta, zero, stop_iter, mae_trace = out
    G = lib.hqq_num_groups(rows, cols, group_size)
    _need(packed, "packed", torch.uint8, min_bytes=lib.hqq_packed_bytes(rows, cols, nbits))
    _need(delta, "delta", (torch.float16, torch.float32, torch.float64), numel=max(G, 1))
    _need(zero, "zero", delta.dtype, numel=max(G, 1))
    _need(stop_iter, "stop_iter", torch.int32, numel=1)
    _need(mae_trace, "mae_trace", torch.float64, numel=iters)
    st = lib.hqq_quantize_noalloc(ctypes.c_void_p(W.data_ptr()), rows, cols, nbits, group_size, axis, iters, p, beta0,
                                  kappa, ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                                  ctypes.c_void_p(zero.data_ptr()), _meta_code(delta.dtype),
                                  ctypes.c_void_p(stop_iter.data_ptr()), ctypes.c_void_p(mae_trace.data_ptr()),
                                  _stream_ptr(stream))
    _check(st)
    return Quantized(packed, delta, zero, rows, cols, nbits, group_size, axis, stop_iter, mae_trace)


def hqq_quantize_v2(W, scale_grid, nbits: int = 4, group_size: int = 64, iters: int = 20, p: float = 0.7,
                    beta0: float = 10.0, kappa: float = 1.01, tiny_range: float | None = None, meta_dtype=None,
                    out=None, workspace=None, stream=None, axis: int = 1):
    """Scale search (either axis, 2/3/4-bit) over the multipliers `scale_grid` of the min-max scale.
    Returns (Quantized, choice): the packed codes, delta and zero as hqq_quantize (no stop index
    or MAE trace: the stop is per group) and the chosen multiplier's index per group (uint8).
    `out` may give (packed, delta, zero, choice)."""
    import numpy as np
    import torch
    lib = load()
    _need(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    rows, cols = W.shape
    meta_dtype = meta_dtype or torch.float16
    G = lib.hqq_num_groups(rows, cols, group_size)
    dev = W.device
    grid = np.ascontiguousarray(scale_grid, dtype=np.float64)
    with _on(stream):
        if out is None:
            packed = torch.empty(max(lib.hqq_packed_bytes(rows, cols, nbits), 1), dtype=torch.uint8, device=dev)
            delta = torch.empty(max(G, 1), dtype=meta_dtype, device=dev)
            zero = torch.empty(max(G, 1), dtype=meta_dtype, device=dev)
            choice = torch.empty(max(G, 1), dtype=torch.uint8, device=dev)
        else:
            packed, delta, zero, choice = out
            _need(packed, "packed", torch.uint8, min_bytes=lib.hqq_packed_bytes(rows, cols, nbits))
            for t, n in ((delta, "delta"), (zero, "zero")):
                _need(t, n, meta_dtype, numel=max(G, 1))
            if choice is not None:
                _need(choice, "choice", torch.uint8, numel=max(G, 1))
        ws_bytes = lib.hqq_quantize_v2_workspace_bytes(rows, cols, nbits)
        if workspace is None and ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    args = QuantV2Args(W.data_ptr(), rows, cols, nbits, group_size, axis, iters, p, beta0, kappa,
                       HQQ_TINY_RANGE if tiny_range is None else tiny_range, grid.ctypes.data, grid.size,
                       packed.data_ptr(), delta.data_ptr(), zero.data_ptr(), _meta_code(meta_dtype),
                       choice.data_ptr() if choice is not None else None, _stream_ptr(stream).value,
                       workspace.data_ptr() if workspace is not None else None,
                       workspace.numel() * workspace.element_size() if workspace is not None else 0)
    _check(lib.hqq_quantize_v2(ctypes.byref(args)))
    return Quantized(packed, delta, zero, rows, cols, nbits, group_size, axis, None, None), choice


def hqq_dequantize(packed, delta, zero, rows: int, cols: int, nbits: int, group_size: int, axis: int, out=None,
                   stream=None):
    """fp16 [rows, cols] W_hat = (q - zero) * delta."""
    import torch
    lib = load()
    if group_size <= 0 or (rows * cols) % group_size:
        raise ValueError("group_size must divide rows*cols")
    _need(packed, "packed", torch.uint8, min_bytes=lib.hqq_packed_bytes(rows, cols, nbits), device=False)
    _need(delta, "delta", (torch.float16, torch.float32), numel=rows * cols // group_size, device=False)
    _need(zero, "zero", delta.dtype, numel=rows * cols // group_size, device=False)
    for t, name in ((packed, "packed"), (delta, "delta"), (zero, "zero")):
        _placed(t, name)
    with _on(stream):
        if out is None:
            out = torch.empty((rows, cols), dtype=torch.float16, device=packed.device)
    _need(out, "out", torch.float16, numel=rows * cols)
    st = lib.hqq_dequantize(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                            ctypes.c_void_p(zero.data_ptr()), _meta_code(delta.dtype), rows, cols, nbits, group_size,
                            axis, ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream))
    _check(st)
    return out


def hqq_gemv_w4a16(packed, delta, zero, N: int, K: int, group_size: int, x, out_dtype=None, out=None,
                   stream=None):
    """y [batch, N] = x [batch, K] @ W_hat^T for a 4-bit axis=1 weight W [N, K].  Above batch 8
    (past 2^26 weights up to batch 16) the library runs its split GEMM on a workspace it keeps per
    stream (hqq_release_workspaces frees them)."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, 4, group_size, x, out=out, out_cols=N)
    batch = x.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((batch, N), dtype=out_dtype, device=x.device)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemv_w4a16(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                            ctypes.c_void_p(zero.data_ptr()), N, K, group_size, ctypes.c_void_p(x.data_ptr()), batch,
                            ctypes.c_void_p(out.data_ptr()), code, _stream_ptr(stream))
    _check(st)
    return out


def hqq_release_workspaces():
    """Frees the workspaces hqq_gemv_w4a16 keeps per stream above batch 8."""
    _check(load().hqq_release_workspaces())


def hqq_gemm_workspace_bytes(N: int, K: int, batch: int) -> int:
    return load().hqq_gemm_workspace_bytes(N, K, batch)


def hqq_gemm_w4a16(packed, delta, zero, N: int, K: int, group_size: int, x, out_dtype=None, out=None, workspace=None,
                   stream=None):
    """Batched y [batch, N] = x [batch, K] @ W_hat^T (4-bit, axis=1) with a workspace (a torch
    uint8 CUDA tensor of at least hqq_gemm_workspace_bytes(N, K, batch) bytes; allocated here
    when not given)."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, 4, group_size, x, out=out, out_cols=N)
    batch = x.shape[0]
    need = lib.hqq_gemm_workspace_bytes(N, K, batch)
    with _on(stream):
        if out is None:
            out = torch.empty((batch, N), dtype=out_dtype, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemm_w4a16(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                            ctypes.c_void_p(zero.data_ptr()), N, K, group_size, ctypes.c_void_p(x.data_ptr()), batch,
                            ctypes.c_void_p(out.data_ptr()), code, ctypes.c_void_p(workspace.data_ptr()),
                            workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check(st)
    return out


def hqq_gemm(packed, delta, zero, N: int, K: int, nbits: int, group_size: int, axis: int, x, out_dtype=None,
             out=None, workspace=None, stream=None):
    """Batched y [batch, N] = x [batch, K] @ W_hat^T for 2-, 3- or 4-bit codes with axis-1 groups
    and 4-bit codes with axis-0 groups, with a workspace as hqq_gemm_w4a16
    (hqq_gemm_workspace_bytes(N, K, batch) bytes)."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, nbits, group_size, x, out=out, out_cols=N)
    batch = x.shape[0]
    need = lib.hqq_gemm_workspace_bytes(N, K, batch)
    with _on(stream):
        if out is None:
            out = torch.empty((batch, N), dtype=out_dtype, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemm(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                      ctypes.c_void_p(zero.data_ptr()), N, K, nbits, group_size, axis, ctypes.c_void_p(x.data_ptr()),
                      batch, ctypes.c_void_p(out.data_ptr()), code, ctypes.c_void_p(workspace.data_ptr()),
                      workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check(st)
    return out


def hqq_gemm_dx_workspace_bytes(N: int, K: int, batch: int) -> int:
    return load().hqq_gemm_dx_workspace_bytes(N, K, batch)


def hqq_gemm_w4a16_dx(packed, delta, zero, N: int, K: int, group_size: int, dy, out_dtype=None, out=None,
                      workspace=None, stream=None):
    """Input gradient dX [batch, K] = dY [batch, N] @ W_hat for a 4-bit axis=1 weight W [N, K]
    (workspace as hqq_gemm_w4a16, sized by hqq_gemm_dx_workspace_bytes)."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, 4, group_size, dy, xname="dy", out=out, out_cols=K)
    batch = dy.shape[0]
    need = lib.hqq_gemm_dx_workspace_bytes(N, K, batch)
    with _on(stream):
        if out is None:
            out = torch.empty((batch, K), dtype=out_dtype, device=dy.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dy.device)
    _need(workspace, "workspace", torch.uint8)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemm_w4a16_dx(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                               ctypes.c_void_p(zero.data_ptr()), N, K, group_size, ctypes.c_void_p(dy.data_ptr()),
                               batch, ctypes.c_void_p(out.data_ptr()), code, ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check(st)
    return out


def hqq_gemm_dx(packed, delta, zero, N: int, K: int, nbits: int, group_size: int, axis: int, dy, out_dtype=None,
                out=None, workspace=None, stream=None):
    """Input gradient dX [batch, K] = dY [batch, N] @ W_hat for the formats of hqq_gemm (2-, 3- or
    4-bit codes of W [N, K] with axis-1 groups, 4-bit with axis-0 groups); workspace as
    hqq_gemm_w4a16, sized by hqq_gemm_dx_workspace_bytes."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, nbits, group_size, dy, xname="dy", out=out, out_cols=K)
    batch = dy.shape[0]
    need = lib.hqq_gemm_dx_workspace_bytes(N, K, batch)
    with _on(stream):
        if out is None:
            out = torch.empty((batch, K), dtype=out_dtype, device=dy.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dy.device)
    _need(workspace, "workspace", torch.uint8)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemm_dx(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                         ctypes.c_void_p(zero.data_ptr()), N, K, nbits, group_size, axis,
                         ctypes.c_void_p(dy.data_ptr()), batch, ctypes.c_void_p(out.data_ptr()), code,
                         ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                         _stream_ptr(stream))
    _check(st)
    return out


def hqq_gemv(packed, delta, zero, N: int, K: int, nbits: int, group_size: int, axis: int, x, out_dtype=None,
             out=None, stream=None):
    """y [batch, N] = x [batch, K] @ W_hat^T for any stored format the library fuses
    (4-bit axis 1 or 0 at batch 1-8, 3-bit axis 1 and 2-bit axis 1 with groups of 16 at batch 1-16;
    larger batches: hqq_gemm)."""
    import torch
    lib = load()
    out_dtype = out_dtype or torch.float16
    _product_operands(packed, delta, zero, N, K, nbits, group_size, x, out=out, out_cols=N)
    batch = x.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((batch, N), dtype=out_dtype, device=x.device)
    code = HQQ_OUT_F16 if out.dtype == torch.float16 else HQQ_OUT_F32
    st = lib.hqq_gemv(ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                      ctypes.c_void_p(zero.data_ptr()), N, K, nbits, group_size, axis, ctypes.c_void_p(x.data_ptr()),
                      batch, ctypes.c_void_p(out.data_ptr()), code, _stream_ptr(stream))
    _check(st)
    return out


# ------------------------------------------------------------------------------ HBM probes

PROBE_EXPORTS = ("hqq_probe_copy", "hqq_probe_read")
_probe = None


def load_probe(path: str = PROBE_LIB_PATH):
    """Load libhqq_probe.so (include/hqq_probe.h): a streaming copy and read of known byte counts,
    used by the measurements; no part of the method."""
    global _probe
    if _probe is None:
        if not os.path.exists(path):
            raise OSError("libhqq_probe.so not built (run `python -m weight_only_quantization_amd.build`): %s" % path)
        lib = ctypes.CDLL(path)
        p, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.hqq_probe_copy.argtypes = [p, p, sz, i32, p]
        lib.hqq_probe_copy.restype = i32
        lib.hqq_probe_read.argtypes = [ctypes.POINTER(p), ctypes.POINTER(sz), i32, p, i32, p]
        lib.hqq_probe_read.restype = i32
        _probe = lib
    return _probe


def probe_copy(src, dst, unroll: int = 4, stream=None):
    """dst[:] = src[:] (same byte count) with the streaming copy kernel."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    if load_probe().hqq_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, unroll,
                                   _stream_ptr(stream)) != 0:
        raise RuntimeError("hqq_probe_copy failed")


def probe_read(bufs, sink, unroll: int = 4, stream=None) -> int:
    """Stream the tensors in `bufs` (1-3) once; `sink` is a 16-byte device tensor.  Each buffer is
    read up to the last whole 16-byte block (a packed 3-bit buffer may end inside one); returns
    the bytes read."""
    n = len(bufs)
    ptrs = (ctypes.c_void_p * n)(*[b.data_ptr() for b in bufs])
    nb = [(b.numel() * b.element_size()) & ~15 for b in bufs]
    sizes = (ctypes.c_size_t * n)(*nb)
    if load_probe().hqq_probe_read(ptrs, sizes, n, ctypes.c_void_p(sink.data_ptr()), unroll,
                                   _stream_ptr(stream)) != 0:
        raise RuntimeError("hqq_probe_read failed")
    return sum(nb)
