"""fp64 CPU oracle for the NVFP4 weight x bf16 activation matrix-vector path.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg import this package.  The product library
never does, and this package never imports the product library: the two share
no code, header, table or constant.  The arithmetic lives in plain C
(``nvfp4_oracle.c``, fp64, one sequential k-sum per output); this module only
marshals numpy arrays to it, plus three steps that are single numpy calls on
exact fp64 values (rounding to fp32, argmax, the tolerance bound).

Format (see ``nvfp4_oracle.c`` for the sources on the pages and the readings
taken where they are silent): E2M1 element codes, one E4M3 scale byte per 16
consecutive elements of a row, one fp32 tensor scale; canonical layout
``codes[R][K/2]`` (element k in the low nibble of byte k/2 when k is even) and
``scales[R][K/16]``.

A second block-scaled format, MXFP4 (E2M1 codes, one E8M0 power-of-two
scale per 32 elements; ``mx_*`` functions), shares the E2M1 decode.

Parity pins for every function here are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH) or (
            os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)
        ):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e2m1_encode_mag.restype = ctypes.c_int
        lib.oracle_e2m1_encode_mag.argtypes = [ctypes.c_double]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_quantize.restype = None
        lib.oracle_quantize.argtypes = [P, i64, i64, ctypes.c_float, P, P]
        lib.oracle_dequant.restype = None
        lib.oracle_dequant.argtypes = [P, P, ctypes.c_float, i64, i64, P]
        lib.oracle_gemv_rows.restype = None
        lib.oracle_gemv_rows.argtypes = [P, P, ctypes.c_float, i64, i64, P, i64,
                                         P, i64, P, P]
        lib.oracle_swiglu.restype = None
        lib.oracle_swiglu.argtypes = [P, i64, i64, P]
        lib.oracle_repack.restype = None
        lib.oracle_repack.argtypes = [P, P, i64, i64, P, P]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_int]
        lib.oracle_mx_quantize.restype = None
        lib.oracle_mx_quantize.argtypes = [P, i64, i64, ctypes.c_float, P, P]
        lib.oracle_mx_dequant.restype = None
        lib.oracle_mx_dequant.argtypes = [P, P, ctypes.c_float, i64, i64, P]
        lib.oracle_mx_gemv_rows.restype = None
        lib.oracle_mx_gemv_rows.argtypes = [P, P, ctypes.c_float, i64, i64, P, i64,
                                            P, i64, P, P]
        lib.oracle_mx_repack.restype = None
        lib.oracle_mx_repack.argtypes = [P, P, i64, i64, P, P]
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_shape(R: int, K: int):
    if R < 0 or K <= 0 or K % 16:
        raise ValueError("need R >= 0 and K a positive multiple of 16, got %d x %d" % (R, K))


# ------------------------------------------------------------------ scalars --

def num_threads() -> int:
    """Threads the oracle's row-parallel loops use (OpenMP)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's row-parallel loops (timing; results do not
    depend on it: every output is one sequential k-sum)."""
    _load().oracle_set_num_threads(int(n))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def e4m3_encode(q: float) -> int:
    """Nearest E4M3 byte to q >= 0 (ties to even, saturating at 448)."""
    return int(_load().oracle_e4m3_encode(float(q)))


def e2m1_encode_mag(v: float) -> int:
    """Nearest E2M1 magnitude code (0..7) to v >= 0 (ties to even, saturating at 6)."""
    return int(_load().oracle_e2m1_encode_mag(float(v)))


def bf16_rne(v: float) -> int:
    return int(_load().oracle_bf16_rne(float(v)))


# ------------------------------------------------------------------ tensors --

def quantize(W: np.ndarray, tscale: float = 1.0):
    """fp32 W[R][K] -> (codes uint8 [R][K/2], scales uint8 [R][K/16]), canonical layout."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    R, K = W.shape
    _check_shape(R, K)
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    _load().oracle_quantize(_ptr(W), R, K, float(tscale), _ptr(codes), _ptr(scales))
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray, tscale: float = 1.0) -> np.ndarray:
    """Exact fp64 w_hat[R][K] = e2m1 * e4m3 * tscale."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_shape(R, K)
    assert scales.shape == (R, K // 16)
    out = np.empty((R, K), np.float64)
    _load().oracle_dequant(_ptr(codes), _ptr(scales), float(tscale), R, K, _ptr(out))
    return out


def dequant_f32(codes, scales, tscale: float = 1.0) -> np.ndarray:
    """fp32 target of dequant: one round-to-nearest-even of the exact w_hat."""
    return dequant(codes, scales, tscale).astype(np.float32)


def dequant_bf16_bits(codes, scales) -> np.ndarray:
    """bf16 target of dequant: e2m1 * e4m3 without the tensor scale.  The
    product has at most 6 significant bits and magnitude in [2^-10, 2688], so
    it is a bf16 value exactly; returns its bit pattern (uint16)."""
    v = dequant(codes, scales, 1.0).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def gemv_rows(codes, scales, tscale: float, X_bits: np.ndarray, rows=None):
    """Y[n][i] = sum_k w_hat[rows[i]][k] * x_n[k] in fp64 (k ascending), and
    the magnitude sum S[n][i].  X_bits: bf16 bit patterns, uint16 [N][K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_shape(R, K)
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    if X_bits.ndim == 1:
        X_bits = X_bits[None, :]
    N = X_bits.shape[0]
    assert X_bits.shape[1] == K
    if rows is None:
        rows = np.arange(R, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < R)
    Y = np.zeros((N, rows.size), np.float64)
    S = np.zeros((N, rows.size), np.float64)
    _load().oracle_gemv_rows(_ptr(codes), _ptr(scales), float(tscale), R, K,
                             _ptr(X_bits), N, _ptr(rows), rows.size, _ptr(Y), _ptr(S))
    return Y, S


def gemv(codes, scales, tscale: float, X_bits: np.ndarray):
    return gemv_rows(codes, scales, tscale, X_bits, None)


def tolerance(S: np.ndarray) -> np.ndarray:
    """Parity bound on an fp32 output: |y - y_ref| <= 1e-5 * sum|w*x| + 1e-6."""
    return 1e-5 * S + 1e-6


def argmax_first(Y: np.ndarray) -> np.ndarray:
    """Per column n (rows of Y), the first index of the maximum: the lowest
    index wins ties.  numpy's argmax returns the first occurrence."""
    Y = np.asarray(Y, np.float64)
    if Y.ndim == 1:
        Y = Y[None, :]
    return np.argmax(Y, axis=1).astype(np.int64)


def swiglu(gu: np.ndarray) -> np.ndarray:
    """gu fp32 [N][2F] (gate then up) -> fp64 h[N][F] = g * u / (1 + exp(-g))."""
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    if gu.ndim == 1:
        gu = gu[None, :]
    N, F2 = gu.shape
    assert F2 % 2 == 0
    F = F2 // 2
    h = np.empty((N, F), np.float64)
    _load().oracle_swiglu(_ptr(gu), F, N, _ptr(h))
    return h


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    """Element-wise fp64 -> bf16 bit pattern (round to nearest, ties to even)."""
    lib = _load()
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    flat_in, flat_out = v.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_bf16_rne(float(flat_in[i]))
    return out


def repack(codes, scales):
    """Canonical (codes, scales) -> repacked (code plane, scale plane) bytes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_shape(R, K)
    ST = ((R + 15) // 16 + 3) // 4
    O = (K // 16 + 7) // 8
    wq = np.empty(ST * O * 4 * 64 * 16, np.uint8)
    ws = np.empty(ST * O * 4 * 16 * 8, np.uint8)
    _load().oracle_repack(_ptr(codes), _ptr(scales), R, K, _ptr(wq), _ptr(ws))
    return wq, ws


# -------------------------------------------------------------------- MXFP4 --
# The second block-scaled format (see the MXFP4 part of nvfp4_oracle.c): E2M1
# codes, one E8M0 scale byte (2^(b - 127)) per 32 elements of a row, an fp32
# tensor multiplier; canonical codes [R][K/2], scales [R][K/32].

def _check_mx_shape(R: int, K: int):
    if R < 0 or K <= 0 or K % 32:
        raise ValueError("need R >= 0 and K a positive multiple of 32, got %d x %d" % (R, K))


def e8m0_value(byte: int) -> float:
    return _load().oracle_e8m0_value(int(byte))


def mx_quantize(W: np.ndarray, tscale: float = 1.0):
    """fp32 W[R][K] -> (codes uint8 [R][K/2], scales uint8 [R][K/32])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    R, K = W.shape
    _check_mx_shape(R, K)
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 32), np.uint8)
    _load().oracle_mx_quantize(_ptr(W), R, K, float(tscale), _ptr(codes), _ptr(scales))
    return codes, scales


def mx_dequant(codes: np.ndarray, scales: np.ndarray, tscale: float = 1.0) -> np.ndarray:
    """Exact fp64 w_hat[R][K] = e2m1 * e8m0 * tscale."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_mx_shape(R, K)
    assert scales.shape == (R, K // 32)
    out = np.empty((R, K), np.float64)
    _load().oracle_mx_dequant(_ptr(codes), _ptr(scales), float(tscale), R, K, _ptr(out))
    return out


def mx_gemv_rows(codes, scales, tscale: float, X_bits: np.ndarray, rows=None):
    """As gemv_rows, for MXFP4 weights."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_mx_shape(R, K)
    assert scales.shape == (R, K // 32)
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    if X_bits.ndim == 1:
        X_bits = X_bits[None, :]
    N = X_bits.shape[0]
    assert X_bits.shape[1] == K
    if rows is None:
        rows = np.arange(R, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < R)
    Y = np.zeros((N, rows.size), np.float64)
    S = np.zeros((N, rows.size), np.float64)
    _load().oracle_mx_gemv_rows(_ptr(codes), _ptr(scales), float(tscale), R, K,
                                _ptr(X_bits), N, _ptr(rows), rows.size, _ptr(Y), _ptr(S))
    return Y, S


def mx_gemv(codes, scales, tscale: float, X_bits: np.ndarray):
    return mx_gemv_rows(codes, scales, tscale, X_bits, None)


def mx_repack(codes, scales):
    """Canonical MXFP4 (codes, scales) -> repacked (code plane, scale plane) bytes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    _check_mx_shape(R, K)
    ST = ((R + 15) // 16 + 3) // 4
    O = (K + 127) // 128
    wq = np.empty(ST * O * 4 * 64 * 16, np.uint8)
    ws = np.empty(ST * O * 4 * 16 * 4, np.uint8)
    _load().oracle_mx_repack(_ptr(codes), _ptr(scales), R, K, _ptr(wq), _ptr(ws))
    return wq, ws
