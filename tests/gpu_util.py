"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare its bf16 output with the oracle's, element by element.

Tolerance (per element, both sides widened to double):
    |y_gpu - y_ref| <= 1e-2 + 1e-2 * |y_ref|,  NaN matches NaN only.
For stress inputs whose dot products cancel heavily (outside the five seeded
benchmark shapes) a tolerance relative to |y| cannot be met by any fp32
accumulation, in any order, so those tests add the conditioning term
    gamma * scale[n] * sum_k |x[m,k] * w[n,k]|.
Two roundings make up the error: the gfx950 fp8 MFMA does not add the products
of one instruction in exact fp32 (measured: errors up to about 2^-15 .. 2^-13
of the largest product in the instruction's K block, which is at most that
block's sum |x w|), and fp32 accumulation across blocks adds about
2^-24 * sqrt(K/64) relative.  Measured on MI355X, the error beyond the base
bound as a fraction of scale[n] * sum_k |x w|: inputs drawn N(0, sigma^2), then
quantised, up to 2^-18.8 (sigma = 100, K = 129; 2^-20 .. 2^-21 at K = 4096 and
4127), so those tests take gamma = COND_GAMMA_GAUSS = 2^-16; uniformly random
codes (2^-9 .. 448), whose large products sit beside tiny ones in one MFMA
block, up to 2^-15.0, so they take gamma = COND_GAMMA_CODES = 2^-12.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp8_gemm_channel_amd as fg
import oracle

ATOL = 1e-2
RTOL = 1e-2
COND_GAMMA_GAUSS = 2.0 ** -16  # 7x the measured worst case of N(0, sigma^2) draws
COND_GAMMA_CODES = 2.0 ** -12  # 8x the measured worst case of uniformly random codes


def conditioning(x: np.ndarray, w: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """scale[n] * sum_k |x[m,k] * w[n,k]| (exact sum via the oracle on the
    sign-cleared codes)."""
    return oracle.gemm_acc(x & 0x7F, w & 0x7F) * np.abs(scale.astype(np.float64))[None, :]


def say(msg: str) -> None:
    """Name the GPU step about to run (so a fault can be traced to its case)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(x: np.ndarray, w: np.ndarray, scale: np.ndarray, *, path=0, variant=0, split_k=0,
        sentinel: bool = True) -> np.ndarray:
    """y bits (uint16 [M,N]) from the GPU for host inputs; the output buffer is
    pre-filled with 0xFFFF (a NaN) so an unwritten element cannot pass."""
    M, K = x.shape
    N = w.shape[0]
    xd, wd, sd = to_dev(x), to_dev(w), to_dev(scale.astype(np.float32))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if sentinel and out.numel():
        out.view(torch.int16).fill_(-1)
    fg.fp8_gemm(xd, wd, sd, out=out, path=path, variant=variant, split_k=split_k)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def compare(got: np.ndarray, ref: np.ndarray, what: str = "", cond: np.ndarray | None = None,
            gamma: float = COND_GAMMA_GAUSS) -> dict:
    """Assert the tolerance on every element; return diagnostics.  `cond`
    (same shape) adds gamma * cond to the bound (stress inputs only)."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    g = oracle.bf16_bits_to_double(got)
    r = oracle.bf16_bits_to_double(ref)
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int((gn != rn).sum())} elements)"
    ok = ~rn
    err = np.abs(g[ok] - r[ok])
    bound = ATOL + RTOL * np.abs(r[ok])
    if cond is not None:
        bound = bound + gamma * cond[ok]
    bad = err > bound
    if bad.any():
        idx = np.argmax(err - bound)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements outside tolerance; worst "
                             f"got {g[ok][idx]!r} ref {r[ok][idx]!r}")
    # diagnostics: exact matches and bf16 ulp distance (same-sign finite values)
    gi = got[ok].astype(np.int32)
    ri = ref[ok].astype(np.int32)
    exact = float(np.mean(gi == ri)) if gi.size else 1.0
    same_sign = (gi >> 15) == (ri >> 15)
    ulp = int(np.max(np.abs(gi - ri)[same_sign])) if same_sign.any() else 0
    out = {"exact": exact, "max_ulp": ulp, "max_err": float(err.max()) if err.size else 0.0}
    if cond is not None and err.size:
        # the error beyond the base bound as a fraction of the conditioning term
        # (log2): what gamma has to cover, for the record
        c = cond[ok]
        excess = err - (ATOL + RTOL * np.abs(r[ok]))
        sel = (excess > 0) & (c > 0)
        ratio = float(np.max(excess[sel] / c[sel])) if sel.any() else 0.0
        out["log2_excess_over_cond"] = float(np.log2(ratio)) if ratio > 0 else float("-inf")
        say(f"{what}: error beyond the base bound / (scale sum|x w|) = 2^{out['log2_excess_over_cond']:.1f} "
            f"({int(sel.sum())} elements beyond the base bound)")
    return out
