"""Seeded synthetic inputs for the scaled FP8 GEMM.

This module is shared by the oracle's tests, the GPU parity tests and bench.py.
It holds no GEMM arithmetic: it only draws seeded random numbers and quantises
them to FP8 E4M3 codes with torch's own fp32 -> float8_e4m3fn cast.

Recipe (the pages describe no value distributions beyond a "numeric stress"
mode, so these are readings; each is stated in the design doc):
  * x[M,K] and w[N,K]: N(0, sigma^2) fp32 draws from one CPU
    ``torch.Generator`` seeded with ``seed`` (x first, then w), clamped to
    +-448 (the largest finite E4M3 value), then cast to ``float8_e4m3fn``,
    which rounds to nearest, ties to even.  Clamping first makes the cast
    saturating.  sigma = 1 is the default workload.
  * scale[N]: U[0.005, 0.02] fp32 drawn after w from the same generator.
  * E5M2 operands (``fp8_inputs_fmt``): the same draws clamped to +-57344 and
    cast to ``float8_e5m2`` (round to nearest, ties to even).
  * bias[N] (``bias_values``): U[-0.5, 0.5] fp32 from its own generator, about
    the spread of the scaled sums at K = 4096, so activations see both signs.
The same host bytes feed the oracle and, copied to device memory, the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: x + w (1 B each) + scale (4 B) + y (2 B)."""
        return self.M * self.K + self.N * self.K + 4 * self.N + 2 * self.M * self.N


#: The five benchmark shapes, in the order they are reported.
WORKLOADS = (
    Workload("square-256", 256, 256, 256),
    Workload("square-4096", 4096, 4096, 4096),
    Workload("decode-m32", 32, 12288, 4096),
    Workload("odd-k-4127", 4096, 4096, 4127),
    Workload("square-8192", 8192, 8192, 8192),
)

WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}


def quantize_e4m3(values: torch.Tensor) -> np.ndarray:
    """Saturating round-to-nearest-even fp32 -> E4M3 codes (uint8 numpy array)."""
    v = values.to(torch.float32).clamp(-E4M3_MAX, E4M3_MAX)
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def fp8_inputs(M: int, N: int, K: int, seed: int = 42, sigma: float = 1.0,
               scale_lo: float = 0.005, scale_hi: float = 0.02):
    """Return (x[M,K] uint8, w[N,K] uint8, scale[N] float32) for one seed."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = quantize_e4m3(torch.randn(M, K, generator=g) * sigma)
    w = quantize_e4m3(torch.randn(N, K, generator=g) * sigma)
    scale = (scale_lo + (scale_hi - scale_lo) * torch.rand(N, generator=g)).numpy().astype(np.float32)
    return x, w, scale


E5M2_MAX = 57344.0
FMT_E4M3, FMT_E5M2 = 0, 1


def quantize_e5m2(values: torch.Tensor) -> np.ndarray:
    """Saturating round-to-nearest-even fp32 -> E5M2 codes (uint8 numpy array)."""
    v = values.to(torch.float32).clamp(-E5M2_MAX, E5M2_MAX)
    return v.to(torch.float8_e5m2).view(torch.uint8).numpy().copy()


def fp8_inputs_fmt(M: int, N: int, K: int, x_format: int, w_format: int, seed: int = 42, sigma: float = 1.0,
                   scale_lo: float = 0.005, scale_hi: float = 0.02):
    """As fp8_inputs, with each operand quantised to its format (FMT_E4M3 / FMT_E5M2)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = {FMT_E4M3: quantize_e4m3, FMT_E5M2: quantize_e5m2}
    x = q[x_format](torch.randn(M, K, generator=g) * sigma)
    w = q[w_format](torch.randn(N, K, generator=g) * sigma)
    scale = (scale_lo + (scale_hi - scale_lo) * torch.rand(N, generator=g)).numpy().astype(np.float32)
    return x, w, scale


def bias_values(N: int, seed: int, lo: float = -0.5, hi: float = 0.5) -> np.ndarray:
    """Seeded per-column bias, U[lo, hi] fp32."""
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    return (lo + (hi - lo) * torch.rand(N, generator=g)).numpy().astype(np.float32)


def random_codes(shape, seed: int, allow_nan: bool = False) -> np.ndarray:
    """Uniformly random E4M3 codes over all 256 (or the 254 finite) patterns."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    if not allow_nan:
        nan = (c & 0x7F) == 0x7F
        c[nan] = c[nan] & 0xF8  # replace NaN codes by the same-sign 256.0 code
    return c


def sample_positions(M: int, N: int, count: int, seed: int):
    """Seeded output positions that always include the four corners."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, M, size=count, dtype=np.int64)
    n = rng.integers(0, N, size=count, dtype=np.int64)
    corners_m = np.array([0, 0, M - 1, M - 1], np.int64)
    corners_n = np.array([0, N - 1, 0, N - 1], np.int64)
    return np.concatenate([corners_m, m]), np.concatenate([corners_n, n])
