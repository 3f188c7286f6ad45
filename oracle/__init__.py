"""CPU oracle for the per-output-channel scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with ``fp8_gemm_channel_amd`` and never imports it.

The arithmetic lives in ``fp8_oracle.c`` (plain C, OpenMP over output rows);
this module only builds that file with gcc and marshals numpy arrays into it.
The definition it computes and the readings it takes are stated in the C
file's header:

    y[m,n] = bf16_rne( (sum_k dec(x[m,k]) * dec(w[n,k])) * scale[n] )

with the sum taken in fp64, where it is exact for K <= 171196; and, through the
general entry points (``gemm_epilogue``, ``gemm_epilogue_at``), for E4M3 or
E5M2 on either operand,

    y[m,n] = bf16_rne( act( acc[m,n] * scale[n] + bias[n] ) )

with the sum of products taken exactly (128-bit integers, IEEE rules for inf
and NaN) and act one of none / ReLU / SiLU / GELU (tanh form).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "fp8_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

#: Largest K for which the fp64 sum is exact (K * (448 * 2^9)^2 < 2^53).
EXACT_K_MAX = 171196

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``fp8_oracle.c`` into ``liboracle.so`` next to it (gcc, OpenMP)."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        build()
    lib = ctypes.CDLL(LIBRARY)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64 = ctypes.c_int64
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_double_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_fp8_gemm_acc.argtypes = [u8p, u8p, i64, i64, i64,
                                        ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.oracle_fp8_gemm_acc.restype = ctypes.c_int
    lib.oracle_fp8_gemm_scaled.argtypes = [u8p, u8p, ctypes.POINTER(ctypes.c_float),
                                           ctypes.POINTER(ctypes.c_uint16), i64, i64, i64,
                                           ctypes.c_int]
    lib.oracle_fp8_gemm_scaled.restype = ctypes.c_int
    lib.oracle_fp8_gemm_scaled_at.argtypes = [u8p, u8p, ctypes.POINTER(ctypes.c_float),
                                              i64, i64, i64,
                                              ctypes.POINTER(ctypes.c_int64),
                                              ctypes.POINTER(ctypes.c_int64), i64,
                                              ctypes.POINTER(ctypes.c_uint16), ctypes.c_int]
    lib.oracle_fp8_gemm_scaled_at.restype = ctypes.c_int
    lib.oracle_e4m3_decode_array.argtypes = [u8p, i64, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_e4m3_decode_array.restype = None
    lib.oracle_bf16_rne_array.argtypes = [ctypes.POINTER(ctypes.c_double), i64,
                                          ctypes.POINTER(ctypes.c_uint16)]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_e5m2_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e5m2_to_double.restype = ctypes.c_double
    lib.oracle_e5m2_decode_array.argtypes = [u8p, i64, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_e5m2_decode_array.restype = None
    lib.oracle_activation_array.argtypes = [ctypes.POINTER(ctypes.c_double), i64, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_double)]
    lib.oracle_activation_array.restype = None
    fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_fp8_gemm_epilogue.argtypes = [u8p, u8p, ctypes.c_int, ctypes.c_int, fp, fp, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_uint16), i64, i64, i64, ctypes.c_int]
    lib.oracle_fp8_gemm_epilogue.restype = ctypes.c_int
    lib.oracle_fp8_gemm_epilogue_at.argtypes = [u8p, u8p, ctypes.c_int, ctypes.c_int, fp, fp, ctypes.c_int,
                                                i64, i64, i64, ctypes.POINTER(ctypes.c_int64),
                                                ctypes.POINTER(ctypes.c_int64), i64,
                                                ctypes.POINTER(ctypes.c_uint16), ctypes.c_int]
    lib.oracle_fp8_gemm_epilogue_at.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _codes(a, name: str, ndim: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8 or a.ndim != ndim:
        raise TypeError(f"{name} must be a {ndim}-d uint8 array of FP8 codes")
    return a


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use by default."""
    return int(_load().oracle_max_threads())


def e4m3_to_double(codes) -> np.ndarray:
    """Decode E4M3 codes (any shape, uint8) to float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c, ctypes.c_uint8), c.size, _ptr(out, ctypes.c_double))
    return out


def bf16_rne(values) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_rne_array(_ptr(v, ctypes.c_double), v.size, _ptr(out, ctypes.c_uint16))
    return out


def gemm_acc(x, w, threads: int = 0) -> np.ndarray:
    """fp64 accumulator acc[M,N] = sum_k dec(x[m,k]) * dec(w[n,k]) (unscaled)."""
    x = _codes(x, "x", 2)
    w = _codes(w, "w", 2)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and w disagree on K")
    M, K = x.shape
    N = w.shape[0]
    acc = np.empty((M, N), np.float64)
    rc = _load().oracle_fp8_gemm_acc(_ptr(x, ctypes.c_uint8), _ptr(w, ctypes.c_uint8),
                                     M, N, K, _ptr(acc, ctypes.c_double), threads)
    if rc:
        raise ValueError("oracle_fp8_gemm_acc rejected its arguments")
    return acc


def gemm_scaled(x, w, scale, threads: int = 0) -> np.ndarray:
    """y[M,N] as uint16 bf16 bits: the full definition."""
    x = _codes(x, "x", 2)
    w = _codes(w, "w", 2)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    if x.shape[1] != w.shape[1] or s.shape != (w.shape[0],):
        raise ValueError("shape mismatch between x, w and scale")
    M, K = x.shape
    N = w.shape[0]
    y = np.empty((M, N), np.uint16)
    rc = _load().oracle_fp8_gemm_scaled(_ptr(x, ctypes.c_uint8), _ptr(w, ctypes.c_uint8),
                                        _ptr(s, ctypes.c_float), _ptr(y, ctypes.c_uint16),
                                        M, N, K, threads)
    if rc:
        raise ValueError("oracle_fp8_gemm_scaled rejected its arguments")
    return y


def gemm_scaled_at(x, w, scale, m_idx, n_idx, threads: int = 0) -> np.ndarray:
    """bf16 bits of y at the positions (m_idx[i], n_idx[i])."""
    x = _codes(x, "x", 2)
    w = _codes(w, "w", 2)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    if mi.shape != ni.shape or mi.ndim != 1:
        raise ValueError("m_idx and n_idx must be 1-d and of equal length")
    if x.shape[1] != w.shape[1] or s.shape != (w.shape[0],):
        raise ValueError("shape mismatch between x, w and scale")
    M, K = x.shape
    N = w.shape[0]
    out = np.empty(mi.shape, np.uint16)
    rc = _load().oracle_fp8_gemm_scaled_at(_ptr(x, ctypes.c_uint8), _ptr(w, ctypes.c_uint8),
                                           _ptr(s, ctypes.c_float), M, N, K,
                                           _ptr(mi, ctypes.c_int64), _ptr(ni, ctypes.c_int64),
                                           mi.size, _ptr(out, ctypes.c_uint16), threads)
    if rc:
        raise ValueError("oracle_fp8_gemm_scaled_at rejected its arguments")
    return out


# Operand formats and activations of the general entry points (the C file's
# header states the definitions).
FMT_E4M3, FMT_E5M2 = 0, 1
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3


def e5m2_to_double(codes) -> np.ndarray:
    """Decode E5M2 codes (any shape, uint8) to float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e5m2_decode_array(_ptr(c, ctypes.c_uint8), c.size, _ptr(out, ctypes.c_double))
    return out


def activation(z, act: int) -> np.ndarray:
    """The epilogue activation `act` applied to float64 values."""
    v = np.ascontiguousarray(z, dtype=np.float64)
    out = np.empty(v.shape, np.float64)
    _load().oracle_activation_array(_ptr(v, ctypes.c_double), v.size, int(act), _ptr(out, ctypes.c_double))
    return out


def _epilogue_args(x, w, scale, bias):
    x = _codes(x, "x", 2)
    w = _codes(w, "w", 2)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    if x.shape[1] != w.shape[1] or s.shape != (w.shape[0],):
        raise ValueError("shape mismatch between x, w and scale")
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.shape != s.shape:
            raise ValueError("bias must have one value per output channel")
    return x, w, s, b


def gemm_epilogue(x, w, scale, bias=None, act: int = ACT_NONE, x_format: int = FMT_E4M3,
                  w_format: int = FMT_E4M3, threads: int = 0) -> np.ndarray:
    """y[M,N] = bf16_rne(act(acc * scale + bias)) as uint16 bits, any formats."""
    x, w, s, b = _epilogue_args(x, w, scale, bias)
    M, K = x.shape
    N = w.shape[0]
    y = np.empty((M, N), np.uint16)
    bp = _ptr(b, ctypes.c_float) if b is not None else None
    rc = _load().oracle_fp8_gemm_epilogue(_ptr(x, ctypes.c_uint8), _ptr(w, ctypes.c_uint8), x_format,
                                          w_format, _ptr(s, ctypes.c_float), bp, act,
                                          _ptr(y, ctypes.c_uint16), M, N, K, threads)
    if rc:
        raise ValueError("oracle_fp8_gemm_epilogue rejected its arguments")
    return y


def gemm_epilogue_at(x, w, scale, m_idx, n_idx, bias=None, act: int = ACT_NONE,
                     x_format: int = FMT_E4M3, w_format: int = FMT_E4M3, threads: int = 0) -> np.ndarray:
    """bf16 bits of the general definition at the positions (m_idx[i], n_idx[i])."""
    x, w, s, b = _epilogue_args(x, w, scale, bias)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    if mi.shape != ni.shape or mi.ndim != 1:
        raise ValueError("m_idx and n_idx must be 1-d and of equal length")
    M, K = x.shape
    N = w.shape[0]
    out = np.empty(mi.shape, np.uint16)
    bp = _ptr(b, ctypes.c_float) if b is not None else None
    rc = _load().oracle_fp8_gemm_epilogue_at(_ptr(x, ctypes.c_uint8), _ptr(w, ctypes.c_uint8), x_format,
                                             w_format, _ptr(s, ctypes.c_float), bp, act, M, N, K,
                                             _ptr(mi, ctypes.c_int64), _ptr(ni, ctypes.c_int64), mi.size,
                                             _ptr(out, ctypes.c_uint16), threads)
    if rc:
        raise ValueError("oracle_fp8_gemm_epilogue_at rejected its arguments")
    return out


def bf16_bits_to_double(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
