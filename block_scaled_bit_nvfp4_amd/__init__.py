"""NVFP4 weight x bf16 activation matrix-vector products on MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so``, whose C ABI is declared in
``include/nvfp4.h``.  Every function below has the name of the C entry point
it calls and only marshals arguments: torch tensors in device memory become
raw pointers, and the current torch stream of the tensors' device becomes
the HIP stream.  All arithmetic runs in the library's HIP kernels; if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "NVFP4Error", "library_path", "load",
    "nvfp4_strerror", "nvfp4_repacked_code_bytes", "nvfp4_repacked_scale_bytes",
    "nvfp4_quantize", "nvfp4_repack", "nvfp4_dequant", "nvfp4_gemv",
    "nvfp4_gemv_argmax_workspace_bytes", "nvfp4_gemv_argmax", "nvfp4_gemv_argmax_noalloc", "nvfp4_swiglu",
    "nvfp4_gemv_swiglu", "nvfp4_gemv_batch", "nvfp4_gemv_batch_workspace_bytes", "NVFP4_MAX_BATCH",
    "mxfp4_repacked_code_bytes", "mxfp4_repacked_scale_bytes", "mxfp4_quantize", "mxfp4_repack",
    "mxfp4_dequant", "mxfp4_gemv",
    "alloc_repacked", "alloc_mx_repacked",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libnvfp4.so")
_lock = threading.Lock()
_lib = None

NVFP4_MAX_N = 65536
NVFP4_MAX_BATCH = 4


class _Product(ctypes.Structure):
    """struct nvfp4_product of nvfp4.h."""
    _fields_ = [("wq", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("tscale", ctypes.c_float),
                ("rows", ctypes.c_int64), ("y", ctypes.c_void_p), ("argmax", ctypes.c_void_p)]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, nvfp4_strerror(status), status))


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libnvfp4.so (built by ``python -m block_scaled_bit_nvfp4_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libnvfp4.so is not built (%s); run "
                               "`python -m block_scaled_bit_nvfp4_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                ctypes.c_size_t)
        sigs = {
            "nvfp4_strerror": (ctypes.c_char_p, [i32]),
            "nvfp4_repacked_code_bytes": (sz, [i64, i64]),
            "nvfp4_repacked_scale_bytes": (sz, [i64, i64]),
            "nvfp4_quantize": (i32, [P, i64, i64, f32, P, P, P]),
            "nvfp4_repack": (i32, [P, P, i64, i64, P, P, P]),
            "nvfp4_dequant": (i32, [P, P, f32, i64, i64, P, P, P]),
            "nvfp4_gemv": (i32, [P, P, f32, i64, i64, P, i32, P, P]),
            "nvfp4_gemv_argmax_workspace_bytes": (sz, [i64, i64, i32]),
            "nvfp4_gemv_argmax": (i32, [P, P, f32, i64, i64, P, i32, P, P, P, sz, P]),
            "nvfp4_gemv_argmax_noalloc": (i32, [P, P, f32, i64, i64, P, i32, P, P, P]),
            "nvfp4_swiglu": (i32, [P, i64, i32, P, P]),
            "nvfp4_gemv_swiglu": (i32, [P, P, f32, i64, i64, P, i32, P, P, P]),
            "nvfp4_gemv_batch_workspace_bytes": (sz, [P, i32, i64, i32]),
            "nvfp4_gemv_batch": (i32, [P, i32, i64, P, i32, P, sz, P]),
            "mxfp4_repacked_code_bytes": (sz, [i64, i64]),
            "mxfp4_repacked_scale_bytes": (sz, [i64, i64]),
            "mxfp4_quantize": (i32, [P, i64, i64, f32, P, P, P]),
            "mxfp4_repack": (i32, [P, P, i64, i64, P, P, P]),
            "mxfp4_dequant": (i32, [P, P, f32, i64, i64, P, P, P]),
            "mxfp4_gemv": (i32, [P, P, f32, i64, i64, P, i32, P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16, torch.int16)      # bf16 values or their bit patterns
_I32 = (torch.int32,)
_ANY = None


def _checked(*specs):
    """Validate the tensors of one call before any pointer reaches the
    library: each spec is (name, tensor, allowed dtypes or None, least byte
    count, may be None).  A tensor must be a contiguous torch.Tensor of an
    allowed dtype holding at least the bytes the call's shape implies, and all
    tensors must sit on one GPU (checked after the rest).  Raises TypeError or
    ValueError; does no arithmetic on the data."""
    device = None
    for name, t, dtypes, nbytes, optional in specs:
        if t is None:
            if optional:
                continue
            raise ValueError("%s is required" % name)
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: expected a torch.Tensor, got %r" % (name, type(t)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if dtypes is not None and t.dtype not in dtypes:
            raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, " or ".join(map(str, dtypes))))
        have = t.numel() * t.element_size()
        if nbytes > 0 and have < nbytes:
            raise ValueError("%s holds %d bytes, the call needs %d" % (name, have, nbytes))
    for name, t, _, _, _ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be in GPU memory (is on %s)" % (name, t.device))
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError("%s is on %s, other arguments on %s" % (name, t.device, device))


def _prod(*v):
    out = 1
    for x in v:
        out *= int(x)
    return out


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise NVFP4Error(status, where)


def nvfp4_strerror(status: int) -> str:
    return load().nvfp4_strerror(int(status)).decode()


def nvfp4_repacked_code_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_repacked_code_bytes(rows, cols))


def nvfp4_repacked_scale_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_repacked_scale_bytes(rows, cols))


def nvfp4_gemv_argmax_workspace_bytes(rows: int, cols: int, n: int) -> int:
    return int(load().nvfp4_gemv_argmax_workspace_bytes(rows, cols, n))


def _planes(wq, ws, rows, cols, mx=False):
    nq = (mxfp4_repacked_code_bytes if mx else nvfp4_repacked_code_bytes)(rows, cols)
    ns = (mxfp4_repacked_scale_bytes if mx else nvfp4_repacked_scale_bytes)(rows, cols)
    return ("wq", wq, _U8, nq, False), ("ws", ws, _U8, ns, False)


def nvfp4_quantize(W, rows, cols, tscale, codes, scales, stream=None):
    _checked(("W", W, _F32, 4 * _prod(rows, cols), False),
             ("codes", codes, _U8, _prod(rows, cols) // 2, False),
             ("scales", scales, _U8, _prod(rows, cols) // 16, False))
    _check(load().nvfp4_quantize(_ptr(W), rows, cols, float(tscale), _ptr(codes), _ptr(scales),
                                 _stream(stream, W)), "nvfp4_quantize")


def nvfp4_repack(codes, scales, rows, cols, wq, ws, stream=None):
    _checked(("codes", codes, _U8, _prod(rows, cols) // 2, False),
             ("scales", scales, _U8, _prod(rows, cols) // 16, False), *_planes(wq, ws, rows, cols))
    _check(load().nvfp4_repack(_ptr(codes), _ptr(scales), rows, cols, _ptr(wq), _ptr(ws),
                               _stream(stream, codes)), "nvfp4_repack")


def nvfp4_dequant(wq, ws, tscale, rows, cols, out_f32=None, out_bf16=None, stream=None):
    _checked(*_planes(wq, ws, rows, cols), ("out_f32", out_f32, _F32, 4 * _prod(rows, cols), True),
             ("out_bf16", out_bf16, _BF16, 2 * _prod(rows, cols), True))
    _check(load().nvfp4_dequant(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(out_f32),
                                _ptr(out_bf16), _stream(stream, wq)), "nvfp4_dequant")


def nvfp4_gemv(wq, ws, tscale, rows, cols, X, n, Y, stream=None):
    _checked(*_planes(wq, ws, rows, cols), ("X", X, _BF16, 2 * _prod(n, cols), False),
             ("Y", Y, _F32, 4 * _prod(n, rows), False))
    _check(load().nvfp4_gemv(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(X), int(n), _ptr(Y),
                             _stream(stream, wq)), "nvfp4_gemv")


def nvfp4_gemv_argmax(wq, ws, tscale, rows, cols, X, n, logits, argmax, workspace, stream=None):
    _checked(*_planes(wq, ws, rows, cols), ("X", X, _BF16, 2 * _prod(n, cols), False),
             ("logits", logits, _F32, 4 * _prod(n, rows), True), ("argmax", argmax, _I32, 4 * int(n), False),
             ("workspace", workspace, _ANY, 0, False))
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().nvfp4_gemv_argmax(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(X), int(n),
                                    _ptr(logits), _ptr(argmax), _ptr(workspace), nbytes,
                                    _stream(stream, wq)), "nvfp4_gemv_argmax")


def nvfp4_gemv_argmax_noalloc(wq, ws, tscale, rows, cols, X, n, logits, argmax, stream=None):
    _checked(*_planes(wq, ws, rows, cols), ("X", X, _BF16, 2 * _prod(n, cols), False),
             ("logits", logits, _F32, 4 * _prod(n, rows), True), ("argmax", argmax, _I32, 4 * int(n), False))
    _check(load().nvfp4_gemv_argmax_noalloc(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(X), int(n),
                                            _ptr(logits), _ptr(argmax), _stream(stream, wq)),
           "nvfp4_gemv_argmax_noalloc")


def nvfp4_swiglu(gu, F, n, h, stream=None):
    _checked(("gu", gu, _F32, 8 * _prod(n, F), False), ("h", h, _BF16, 2 * _prod(n, F), False))
    _check(load().nvfp4_swiglu(_ptr(gu), int(F), int(n), _ptr(h), _stream(stream, gu)), "nvfp4_swiglu")


def nvfp4_gemv_swiglu(wq_gu, ws_gu, tscale, hidden, F, X, n, gu, h, stream=None):
    _checked(*_planes(wq_gu, ws_gu, 2 * int(F), hidden), ("X", X, _BF16, 2 * _prod(n, hidden), False),
             ("gu", gu, _F32, 8 * _prod(n, F), True), ("h", h, _BF16, 2 * _prod(n, F), False))
    _check(load().nvfp4_gemv_swiglu(_ptr(wq_gu), _ptr(ws_gu), float(tscale), int(hidden), int(F), _ptr(X),
                                    int(n), _ptr(gu), _ptr(h), _stream(stream, wq_gu)), "nvfp4_gemv_swiglu")


def _batch(products, cols, n, X=None, workspace=None):
    """Product descriptions (dicts with wq, ws, tscale, rows and optional y,
    argmax) -> (ctypes array of nvfp4_product, count), after the same tensor
    checks as the single-product calls."""
    products = list(products)
    specs = []
    for i, q in enumerate(products):
        rows = int(q["rows"])
        wq, ws = _planes(q["wq"], q["ws"], rows, cols)
        specs += [("products[%d].wq" % i,) + wq[1:], ("products[%d].ws" % i,) + ws[1:],
                  ("products[%d].y" % i, q.get("y"), _F32, 4 * _prod(n, rows), True),
                  ("products[%d].argmax" % i, q.get("argmax"), _I32, 4 * int(n), True)]
    if X is not None:
        specs.append(("X", X, _BF16, 2 * _prod(n, cols), False))
    specs.append(("workspace", workspace, _ANY, 0, True))
    _checked(*specs)
    arr = (_Product * max(1, len(products)))()
    for i, q in enumerate(products):
        arr[i] = _Product(_ptr(q["wq"]), _ptr(q["ws"]), float(q["tscale"]), int(q["rows"]), _ptr(q.get("y")),
                          _ptr(q.get("argmax")))
    return arr, len(products)


def nvfp4_gemv_batch_workspace_bytes(products, cols, n) -> int:
    arr, count = _batch(products, cols, n)
    return int(load().nvfp4_gemv_batch_workspace_bytes(arr, count, int(cols), int(n)))


def nvfp4_gemv_batch(products, cols, X, n, workspace=None, stream=None):
    """Several products of one X in one launch (nvfp4_gemv_batch); products:
    dicts with wq, ws, tscale, rows, and y and/or argmax tensors."""
    arr, count = _batch(products, cols, n, X, workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().nvfp4_gemv_batch(arr, count, int(cols), _ptr(X), int(n), _ptr(workspace), nbytes,
                                   _stream(stream, X)), "nvfp4_gemv_batch")


def alloc_repacked(rows: int, cols: int, device="cuda"):
    """Allocate (uninitialised) code and scale planes for nvfp4_repack."""
    nq, ns = nvfp4_repacked_code_bytes(rows, cols), nvfp4_repacked_scale_bytes(rows, cols)
    if nq == 0:
        raise NVFP4Error(-2, "alloc_repacked")
    return (torch.empty(nq, dtype=torch.uint8, device=device),
            torch.empty(ns, dtype=torch.uint8, device=device))


# ------------------------------------------------------------------- MXFP4 --

def mxfp4_repacked_code_bytes(rows: int, cols: int) -> int:
    return int(load().mxfp4_repacked_code_bytes(rows, cols))


def mxfp4_repacked_scale_bytes(rows: int, cols: int) -> int:
    return int(load().mxfp4_repacked_scale_bytes(rows, cols))


def mxfp4_quantize(W, rows, cols, tscale, codes, scales, stream=None):
    _checked(("W", W, _F32, 4 * _prod(rows, cols), False),
             ("codes", codes, _U8, _prod(rows, cols) // 2, False),
             ("scales", scales, _U8, _prod(rows, cols) // 32, False))
    _check(load().mxfp4_quantize(_ptr(W), rows, cols, float(tscale), _ptr(codes), _ptr(scales),
                                 _stream(stream, W)), "mxfp4_quantize")


def mxfp4_repack(codes, scales, rows, cols, wq, ws, stream=None):
    _checked(("codes", codes, _U8, _prod(rows, cols) // 2, False),
             ("scales", scales, _U8, _prod(rows, cols) // 32, False), *_planes(wq, ws, rows, cols, mx=True))
    _check(load().mxfp4_repack(_ptr(codes), _ptr(scales), rows, cols, _ptr(wq), _ptr(ws),
                               _stream(stream, codes)), "mxfp4_repack")


def mxfp4_dequant(wq, ws, tscale, rows, cols, out_f32=None, out_bf16=None, stream=None):
    _checked(*_planes(wq, ws, rows, cols, mx=True), ("out_f32", out_f32, _F32, 4 * _prod(rows, cols), True),
             ("out_bf16", out_bf16, _BF16, 2 * _prod(rows, cols), True))
    _check(load().mxfp4_dequant(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(out_f32),
                                _ptr(out_bf16), _stream(stream, wq)), "mxfp4_dequant")


def mxfp4_gemv(wq, ws, tscale, rows, cols, X, n, Y, stream=None):
    _checked(*_planes(wq, ws, rows, cols, mx=True), ("X", X, _BF16, 2 * _prod(n, cols), False),
             ("Y", Y, _F32, 4 * _prod(n, rows), False))
    _check(load().mxfp4_gemv(_ptr(wq), _ptr(ws), float(tscale), rows, cols, _ptr(X), int(n), _ptr(Y),
                             _stream(stream, wq)), "mxfp4_gemv")


def alloc_mx_repacked(rows: int, cols: int, device="cuda"):
    """Allocate (uninitialised) MXFP4 code and scale planes for mxfp4_repack."""
    nq, ns = mxfp4_repacked_code_bytes(rows, cols), mxfp4_repacked_scale_bytes(rows, cols)
    if nq == 0:
        raise NVFP4Error(-2, "alloc_mx_repacked")
    return (torch.empty(nq, dtype=torch.uint8, device=device),
            torch.empty(ns, dtype=torch.uint8, device=device))
