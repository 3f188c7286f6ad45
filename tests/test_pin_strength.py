"""The oracle's pins can see plausible mistakes (no GPU).

Each mutant below is a small numpy re-implementation of the oracle's steps
with ONE planted mistake of the kind a hand-written oracle could contain: a
wrong exponent bias, flushed subnormals, a wrong rounding rule, a dropped or
misplaced term, a transposed operand, a wrong scale index, a low-precision
sum, a sign error.  The mistakes live only here, on the CPU; the unmutated
numpy version must pass every pin, and each mutant must fail at least one.
"""
import numpy as np
import pytest

from tests import oracle_pins as pins


def _decode_ok(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _bf16_rne_ok(v):
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    for i, x in np.ndenumerate(v):
        out[i] = pins.exact_bf16_bits(float(x))
    return out


class NumpyOracle:
    """Unmutated reference shape for the mutants (must pass all pins)."""

    def decode(self, codes):
        return _decode_ok(codes)

    def bf16(self, v):
        return _bf16_rne_ok(v)

    def acc(self, x, w):
        return self.decode(x) @ self.decode(w).T

    def scaled(self, x, w, scale):
        a = self.acc(x, w)
        return self.bf16(a * np.asarray(scale, np.float64)[None, :])


class Bias8(NumpyOracle):
    def decode(self, codes):
        return _decode_ok(codes) / 2.0


class FlushSubnormals(NumpyOracle):
    def decode(self, codes):
        d = _decode_ok(codes)
        c = np.asarray(codes, np.uint8)
        return np.where(((c >> 3) & 15) == 0, 0.0 * np.sign(d), d)


class NanAsFinite(NumpyOracle):
    def decode(self, codes):
        c = np.asarray(codes, np.uint8)
        d = _decode_ok(codes)
        return np.where((c & 0x7F) == 0x7F, np.where(c >> 7, -480.0, 480.0), d)


class Bf16Truncate(NumpyOracle):
    def bf16(self, v):
        v = np.asarray(v, np.float64)
        f = v.astype(np.float32)
        b = (f.view(np.uint32) >> 16).astype(np.uint16)
        return np.where(np.isnan(v), np.uint16(0x7FC0), b)


class Bf16TiesAway(NumpyOracle):
    def bf16(self, v):
        v = np.asarray(v, np.float64)
        out = _bf16_rne_ok(v)
        a = np.abs(v)
        for i, x in np.ndenumerate(a):
            b = int(out[i]) & 0x7FFF
            if b >= 0x7F80 or not np.isfinite(x) or x == 0:
                continue
            lo = pins.exact_bf16_bits(float(x))
            # tie? check the exact midpoint to the next value up
            nxt = np.frombuffer(np.array([(b + 1) << 16], np.uint32).tobytes(), np.float32)[0]
            cur = np.frombuffer(np.array([b << 16], np.uint32).tobytes(), np.float32)[0]
            if x == (float(cur) + float(nxt)) / 2 and lo == b:
                out[i] = (out[i] & 0x8000) | (b + 1)
        return out


class Bf16ViaFloat32(NumpyOracle):
    """Double rounding: fp64 -> fp32 (RNE) -> bf16 (RNE)."""

    def bf16(self, v):
        f = np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
        return _bf16_rne_ok(f)


class Bf16SaturateNoInf(NumpyOracle):
    def bf16(self, v):
        out = _bf16_rne_ok(v)
        big = (out & 0x7FFF) == 0x7F80
        return np.where(big, (out & 0x8000) | 0x7F7F, out).astype(np.uint16)


class DropLastK(NumpyOracle):
    def acc(self, x, w):
        if x.shape[1] == 0:
            return super().acc(x, w)
        return self.decode(x[:, :-1]) @ self.decode(w[:, :-1]).T


class ShiftedK(NumpyOracle):
    """Pairs x[m,k] with w[n,k+1] (an off-by-one in the second operand)."""

    def acc(self, x, w):
        if x.shape[1] <= 1:
            return super().acc(x, w)
        wr = np.roll(w, -1, axis=1)
        return self.decode(x) @ self.decode(wr).T


class TransposedWeight(NumpyOracle):
    """Reads w as column-major [K,N] storage."""

    def acc(self, x, w):
        N, K = w.shape
        wt = np.ascontiguousarray(w).reshape(K, N).T
        return self.decode(x) @ self.decode(wt).T


class ScaleByRow(NumpyOracle):
    def scaled(self, x, w, scale):
        a = self.acc(x, w)
        s = np.asarray(scale, np.float64)
        idx = np.arange(a.shape[0]) % max(1, s.size)
        return self.bf16(a * s[idx][:, None]) if s.size else self.bf16(a)


class Float32Sum(NumpyOracle):
    def acc(self, x, w):
        dx = self.decode(x).astype(np.float32)
        dw = self.decode(w).astype(np.float32)
        out = np.zeros((dx.shape[0], dw.shape[0]), np.float32)
        for k in range(dx.shape[1]):
            out = (out + np.outer(dx[:, k], dw[:, k]).astype(np.float32)).astype(np.float32)
        return out.astype(np.float64)


class SignFlip(NumpyOracle):
    def acc(self, x, w):
        return -super().acc(x, w)


MUTANTS = [Bias8, FlushSubnormals, NanAsFinite, Bf16Truncate, Bf16TiesAway, Bf16ViaFloat32,
           Bf16SaturateNoInf, DropLastK, ShiftedK, TransposedWeight, ScaleByRow, Float32Sum,
           SignFlip]

# pins cheap enough to run on the slow numpy mutants
FAST = [c for c in pins.ALL_CHECKS if c.__name__ not in ("check_bf16_vs_torch_on_float32",)]


def _failing_pins(impl):
    failed = []
    for check in FAST:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
    return failed


def test_unmutated_numpy_oracle_passes_all_pins():
    assert _failing_pins(NumpyOracle()) == []


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_each_planted_mistake_is_caught(mutant):
    failed = _failing_pins(mutant())
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"



# ------------------------------------------------ general formats and epilogue
def _decode5_ok(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s, e, m = c >> 7, (c >> 2) & 31, c & 3
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -16),
                   np.ldexp((4 + m).astype(np.float64), (e - 17).astype(np.int64)))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def _act_ok(z, act):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        if act == pins.ACT_RELU:
            out = np.where(z > 0, z, 0.0)
        elif act == pins.ACT_SILU:
            out = z / (1.0 + np.exp(-z))
        elif act == pins.ACT_GELU_TANH:
            out = 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))
        else:
            out = z.copy()
    lim = np.where(z > 0, z, -0.0 if act in (pins.ACT_SILU, pins.ACT_GELU_TANH) else 0.0)
    out = np.where(np.isinf(z) & (act != pins.ACT_NONE), lim, out)
    return np.where(np.isnan(z), z, out)


class NumpyEpilogue:
    """Unmutated reference shape for the epilogue mutants (must pass all pins)."""

    def decode5(self, codes):
        return _decode5_ok(codes)

    def act(self, z, act):
        return _act_ok(z, act)

    def decode_fmt(self, codes, fmt):
        return _decode_ok(codes) if fmt == pins.FMT_E4M3 else self.decode5(codes)

    def dot(self, a, b):
        """Exact sum of products with IEEE special-value rules (Fractions)."""
        from fractions import Fraction
        tot, nan, pinf, ninf = Fraction(0), False, False, False
        for p, q in zip(a, b):
            p, q = float(p), float(q)
            if np.isnan(p) or np.isnan(q):
                nan = True
            elif np.isinf(p) or np.isinf(q):
                if p == 0 or q == 0:
                    nan = True
                elif (p < 0) != (q < 0):
                    ninf = True
                else:
                    pinf = True
            else:
                tot += Fraction(p) * Fraction(q)
        if nan or (pinf and ninf):
            return float("nan")
        if pinf or ninf:
            return float("inf") if pinf else float("-inf")
        return float(tot)

    def z(self, acc, scale, bias, n):
        return acc * float(scale[n]) + (float(bias[n]) if bias is not None else 0.0)

    def epi(self, x, w, scale, bias, act, xf, wf):
        dx, dw = self.decode_fmt(x, xf), self.decode_fmt(w, wf)
        M, N = dx.shape[0], dw.shape[0]
        z = np.array([[self.z(self.dot(dx[m], dw[n]), scale, bias, n) for n in range(N)] for m in range(M)],
                     np.float64).reshape(M, N)
        return _bf16_rne_ok(self.act(z, act))


class E5m2Bias16(NumpyEpilogue):
    def decode5(self, codes):
        return _decode5_ok(codes) / 2.0


class E5m2InfIsFinite(NumpyEpilogue):
    def decode5(self, codes):
        d = _decode5_ok(codes)
        return np.where(np.isinf(d), np.sign(d) * 65536.0, d)


class NaiveFp64Sum(NumpyEpilogue):
    def dot(self, a, b):
        s = 0.0
        for p, q in zip(a, b):
            s += float(p) * float(q)
        return s


class InfTimesZeroIsZero(NumpyEpilogue):
    def dot(self, a, b):
        a = np.where(np.isinf(a) & (np.asarray(b) == 0), 0.0, a)
        b = np.where(np.isinf(b) & (np.asarray(a) == 0), 0.0, b)
        return super().dot(a, b)


class BiasBeforeScale(NumpyEpilogue):
    def z(self, acc, scale, bias, n):
        return (acc + (float(bias[n]) if bias is not None else 0.0)) * float(scale[n])


class BiasByRow(NumpyEpilogue):
    def epi(self, x, w, scale, bias, act, xf, wf):
        if bias is None:
            return super().epi(x, w, scale, bias, act, xf, wf)
        M = np.asarray(x).shape[0]
        rows = np.array([float(bias[m % len(bias)]) for m in range(M)], np.float32)
        out = np.empty((M, np.asarray(w).shape[0]), np.uint16)
        for m in range(M):
            out[m] = super().epi(x[m:m + 1], w, scale, np.full(len(bias), rows[m], np.float32), act, xf, wf)[0]
        return out


class ActBeforeScale(NumpyEpilogue):
    def epi(self, x, w, scale, bias, act, xf, wf):
        dx, dw = self.decode_fmt(x, xf), self.decode_fmt(w, wf)
        M, N = dx.shape[0], dw.shape[0]
        acc = np.array([[self.dot(dx[m], dw[n]) for n in range(N)] for m in range(M)], np.float64).reshape(M, N)
        a = self.act(acc, act) * np.asarray(scale, np.float64)[None, :]
        if bias is not None:
            a = a + np.asarray(bias, np.float64)[None, :]
        return _bf16_rne_ok(a)


class SiluIsSigmoid(NumpyEpilogue):
    def act(self, z, act):
        if act == pins.ACT_SILU:
            z = np.asarray(z, np.float64)
            with np.errstate(over="ignore"):
                return np.where(np.isnan(z), z, 1.0 / (1.0 + np.exp(-z)))
        return super().act(z, act)


class GeluErf(NumpyEpilogue):
    def act(self, z, act):
        if act == pins.ACT_GELU_TANH:
            from math import erf, sqrt
            z = np.asarray(z, np.float64)
            return np.array([v if not np.isfinite(v) else 0.5 * v * (1 + erf(v / sqrt(2))) for v in z.ravel()]
                            ).reshape(z.shape)
        return super().act(z, act)


class ReluKeepsNegative(NumpyEpilogue):
    def act(self, z, act):
        if act == pins.ACT_RELU:
            return np.asarray(z, np.float64).copy()
        return super().act(z, act)


EPI_MUTANTS = [E5m2Bias16, E5m2InfIsFinite, NaiveFp64Sum, InfTimesZeroIsZero, BiasBeforeScale, BiasByRow,
               ActBeforeScale, SiluIsSigmoid, GeluErf, ReluKeepsNegative]


def _failing_epi_pins(impl):
    failed = []
    for check in pins.EPI_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
    return failed


def test_unmutated_numpy_epilogue_passes_all_pins():
    assert _failing_epi_pins(NumpyEpilogue()) == []


@pytest.mark.parametrize("mutant", EPI_MUTANTS, ids=lambda m: m.__name__)
def test_each_planted_epilogue_mistake_is_caught(mutant):
    failed = _failing_epi_pins(mutant())
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"
