"""Python binding of libfp8g.so, the MI355X (gfx950) scaled FP8 GEMM.

    y[m,n] = bf16_rne( (sum_k x[m,k] * w[n,k]) * scale[n] )

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/fp8g.h.  PyTorch supplies device memory and the current
stream.  If libfp8g.so is missing this module raises ImportError; there is no
fallback implementation.

Entry points (same names as the C ABI):
    fp8_gemm_scaled(x, w, scale, y, M, N, K, stream)        raw pointers
    fp8_gemm_scaled_ex(..., path, variant, split_k, stream)  forced plan
    fp8_gemm_scaled_act(x, w, scale, bias, y, M, N, K, x_format, w_format,
                        activation, stream)                   bias, activation, E5M2
    fp8_gemm_scaled_act_ex(..., path, variant, split_k, stream)
    fp8_gemm_scaled_act_timed(..., stream, start_event, stop_event)
                                                              events on the call's kernels
    fp8_gemm_scaled_noalloc(x, w, scale, y, M, N, K, path, variant, split_k, stream)
                                                              no allocation (library scratch)
    fp8_gemm_plan(M, N, K) / fp8_gemm_plan_ex(...)           host-only planner
    fp8_gemm_strerror(status), fp8_gemm_last_error()
and the tensor-level convenience wrapper
    fp8_gemm(x, w, scale, *, bias=None, act=ACT_NONE, out=None, path=0,
             variant=0, split_k=0, stream=None, events=None) -> y
(operand formats follow the tensors' dtypes: float8_e4m3fn or float8_e5m2).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# FP8G_LIBRARY selects another build of the same library (the LDS-poison debug
# build, libfp8g_lds_poison.so); the default is the product build.
LIBRARY = os.environ.get("FP8G_LIBRARY") or os.path.join(_PKG, "libfp8g.so")

FP8G_OK = 0
FP8G_ERR_INVALID_ARG = 1
FP8G_ERR_UNSUPPORTED = 2
FP8G_ERR_HIP = 3

PATH_NONE, PATH_ZERO, PATH_MAIN, PATH_SPLITK = 0, 1, 2, 3
PATH_NAMES = {PATH_NONE: "none", PATH_ZERO: "zero", PATH_MAIN: "main", PATH_SPLITK: "splitk"}

FMT_E4M3, FMT_E5M2 = 0, 1
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3

#: Every symbol include/fp8g.h declares.
EXPORTED_SYMBOLS = ("fp8_gemm_scaled", "fp8_gemm_scaled_ex", "fp8_gemm_scaled_act", "fp8_gemm_scaled_act_ex",
                    "fp8_gemm_scaled_act_timed", "fp8_gemm_scaled_noalloc", "fp8_gemm_plan", "fp8_gemm_plan_ex",
                    "fp8_gemm_strerror", "fp8_gemm_last_error")
#: Size of the device array the allocation-free entry point uses as workspace.
NOALLOC_SCRATCH_BYTES = 32 << 20


class Plan(ctypes.Structure):
    """Mirror of struct fp8g_plan."""

    _fields_ = [("path", ctypes.c_int32), ("variant", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("k_slice", ctypes.c_int64), ("group_m", ctypes.c_int32), ("k_tail", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("dp_tiles", ctypes.c_int32), ("sk_groups", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["path_name"] = PATH_NAMES.get(self.path, "?")
        return d


class Fp8gError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{fp8_gemm_strerror(status)}: {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7).
    # Importing torch first makes the loader bind libfp8g.so to that runtime
    # instead of loading a second HIP/HSA runtime, which would not see the GPU.
    import torch  # noqa: F401

    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is not built; run `python fp8_gemm_channel_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIBRARY)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.fp8_gemm_scaled.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_gemm_scaled.restype = ctypes.c_int
    lib.fp8_gemm_scaled_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.fp8_gemm_scaled_ex.restype = ctypes.c_int
    lib.fp8_gemm_scaled_act.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.fp8_gemm_scaled_act.restype = ctypes.c_int
    lib.fp8_gemm_scaled_act_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, vp]
    lib.fp8_gemm_scaled_act_ex.restype = ctypes.c_int
    lib.fp8_gemm_scaled_act_timed.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                              vp, vp, vp]
    lib.fp8_gemm_scaled_act_timed.restype = ctypes.c_int
    lib.fp8_gemm_scaled_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.fp8_gemm_scaled_noalloc.restype = ctypes.c_int
    lib.fp8_gemm_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    lib.fp8_gemm_plan.restype = ctypes.c_int
    lib.fp8_gemm_plan_ex.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.fp8_gemm_plan_ex.restype = ctypes.c_int
    lib.fp8_gemm_strerror.argtypes = [ctypes.c_int]
    lib.fp8_gemm_strerror.restype = ctypes.c_char_p
    lib.fp8_gemm_last_error.argtypes = []
    lib.fp8_gemm_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


# ------------------------------------------------------------ raw C-ABI calls --
def fp8_gemm_scaled(x: int, w: int, scale: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Direct call of the C entry point with device addresses; returns the status."""
    return _lib.fp8_gemm_scaled(x, w, scale, y, M, N, K, stream)


def fp8_gemm_scaled_ex(x: int, w: int, scale: int, y: int, M: int, N: int, K: int,
                       path: int = 0, variant: int = 0, split_k: int = 0, stream: int = 0) -> int:
    return _lib.fp8_gemm_scaled_ex(x, w, scale, y, M, N, K, path, variant, split_k, stream)


def fp8_gemm_scaled_act(x: int, w: int, scale: int, bias: int, y: int, M: int, N: int, K: int,
                        x_format: int = FMT_E4M3, w_format: int = FMT_E4M3, activation: int = ACT_NONE,
                        stream: int = 0) -> int:
    """C entry point with a bias (0 = none), an activation and operand formats."""
    return _lib.fp8_gemm_scaled_act(x, w, scale, bias or None, y, M, N, K, x_format, w_format, activation, stream)


def fp8_gemm_scaled_act_ex(x: int, w: int, scale: int, bias: int, y: int, M: int, N: int, K: int,
                           x_format: int = FMT_E4M3, w_format: int = FMT_E4M3, activation: int = ACT_NONE,
                           path: int = 0, variant: int = 0, split_k: int = 0, stream: int = 0) -> int:
    return _lib.fp8_gemm_scaled_act_ex(x, w, scale, bias or None, y, M, N, K, x_format, w_format, activation,
                                       path, variant, split_k, stream)


def fp8_gemm_scaled_act_timed(x: int, w: int, scale: int, bias: int, y: int, M: int, N: int, K: int,
                              x_format: int = FMT_E4M3, w_format: int = FMT_E4M3, activation: int = ACT_NONE,
                              path: int = 0, variant: int = 0, split_k: int = 0, stream: int = 0,
                              start_event: int = 0, stop_event: int = 0) -> int:
    """fp8_gemm_scaled_act_ex with hipEvent_t handles attached to the call's
    first and last kernels (0 = none)."""
    return _lib.fp8_gemm_scaled_act_timed(x, w, scale, bias or None, y, M, N, K, x_format, w_format, activation,
                                          path, variant, split_k, stream, start_event or None, stop_event or None)


def fp8_gemm_scaled_noalloc(x: int, w: int, scale: int, y: int, M: int, N: int, K: int,
                            path: int = 0, variant: int = 0, split_k: int = 0, stream: int = 0) -> int:
    """The allocation-free entry point (workspace from the library's device
    array, at most NOALLOC_SCRATCH_BYTES); device addresses; returns the status."""
    return _lib.fp8_gemm_scaled_noalloc(x, w, scale, y, M, N, K, path, variant, split_k, stream)


def fp8_gemm_plan(M: int, N: int, K: int) -> dict:
    return fp8_gemm_plan_ex(M, N, K)


def fp8_gemm_plan_ex(M: int, N: int, K: int, path: int = 0, variant: int = 0, split_k: int = 0) -> dict:
    p = Plan()
    st = _lib.fp8_gemm_plan_ex(M, N, K, path, variant, split_k, ctypes.byref(p))
    if st != FP8G_OK:
        raise Fp8gError(st, fp8_gemm_last_error())
    return p.as_dict()


def fp8_gemm_strerror(status: int) -> str:
    return _lib.fp8_gemm_strerror(status).decode()


def fp8_gemm_last_error() -> str:
    return _lib.fp8_gemm_last_error().decode()


# ------------------------------------------------------------- tensor wrapper --
def fp8_gemm(x, w, scale, *, bias=None, act: int = ACT_NONE, x_format=None, w_format=None, out=None,
             path: int = 0, variant: int = 0, split_k: int = 0, stream=None, events=None):
    """y = bf16(act((x @ w^T) * scale + bias)) on the GPU; returns a new [M, N]
    bfloat16 tensor (or writes `out`).  x: [M,K], w: [N,K] float8_e4m3fn or
    float8_e5m2 (or uint8 codes, E4M3 unless x_format / w_format say E5M2);
    scale, bias: [N] float32; all contiguous on the same CUDA/HIP device.
    `events` = (start, stop) torch.cuda.Event(enable_timing=True) pair: start
    is recorded when the call's first kernel begins, stop when its last kernel
    ends (start.elapsed_time(stop) is the GPU time of the call)."""
    import torch

    def codes(t, name, fmt):
        if t.dtype == torch.float8_e5m2:
            dfmt = FMT_E5M2
        elif t.dtype in (torch.float8_e4m3fn, torch.uint8):
            dfmt = FMT_E4M3
        else:
            raise TypeError(f"{name} must be float8_e4m3fn, float8_e5m2 or uint8 codes, got {t.dtype}")
        if fmt is None:
            fmt = dfmt
        elif t.dtype != torch.uint8 and fmt != dfmt:
            raise TypeError(f"{name}: format {fmt} does not match dtype {t.dtype}")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-d tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        return t, fmt

    x, x_format = codes(x, "x", x_format)
    w, w_format = codes(w, "w", w_format)
    if scale.dtype != torch.float32 or scale.dim() != 1 or not scale.is_contiguous() or not scale.is_cuda:
        raise TypeError("scale must be a contiguous 1-d float32 GPU tensor")
    M, K = x.shape
    N, K2 = w.shape
    if K2 != K or scale.numel() != N:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w {tuple(w.shape)}, scale {tuple(scale.shape)}")
    if not (x.device == w.device == scale.device):
        raise ValueError("x, w and scale must be on the same device")
    if bias is not None:
        if bias.dtype != torch.float32 or bias.shape != scale.shape or not bias.is_contiguous() \
                or bias.device != scale.device:
            raise TypeError("bias must be a contiguous [N] float32 tensor on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bfloat16 tensor")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        args = (x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr() if bias is not None else None,
                out.data_ptr(), M, N, K, x_format, w_format, act, path, variant, split_k, stream.cuda_stream)
        if events is None:
            st = _lib.fp8_gemm_scaled_act_ex(*args)
        else:
            for e in events:
                if e.cuda_event == 0:  # torch creates the HIP event at its first record
                    e.record(stream)
            st = _lib.fp8_gemm_scaled_act_timed(*args, events[0].cuda_event, events[1].cuda_event)
    if st != FP8G_OK:
        raise Fp8gError(st, fp8_gemm_last_error())
    return out
