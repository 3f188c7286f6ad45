"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each check takes an implementation object with four methods

    decode(codes uint8[...])            -> float64[...]   E4M3 code -> value
    bf16(values float64[...])           -> uint16[...]    round to bf16 bits
    acc(x uint8[M,K], w uint8[N,K])     -> float64[M,N]   unscaled sum
    scaled(x, w, scale float32[N])      -> uint16[M,N]    y as bf16 bits

and raises AssertionError when the implementation disagrees with what the
format definitions, exact arithmetic, a library routine or a closed form fix.
``test_oracle.py`` runs every check on the C oracle (all must pass);
``test_pin_strength.py`` runs them on oracles with planted mistakes (each
mutant must fail at least one), which shows the pins can see such mistakes.

Nothing here computes y the way the oracle does: expected values come from
exact rational arithmetic (fractions.Fraction) with a brute-force search over
all bf16 / E4M3 values, from integer (int64) sums, from torch's float8 and
bfloat16 conversions, or from hand derivations stored under tests/golden/.
"""
from __future__ import annotations

import bisect
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- references --
def torch_decode(codes) -> np.ndarray:
    """Library decode: torch's float8_e4m3fn -> float64 conversion."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_table():
    """All non-negative finite bf16 values as Fractions, ascending, plus 2^128.

    Built by widening every bit pattern 0x0000..0x7F7F through torch (library
    bfloat16 -> float64, exact), not from any formula of the oracle's.  The
    virtual entry 2^128 with bits 0x7F80 (inf) makes IEEE overflow fall out of
    the nearest/ties-to-even search: values at or past the midpoint between the
    largest finite value (odd significand) and 2^128 (even) round to inf.
    """
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    fr = [Fraction(float(v)) for v in vals]
    fr.append(Fraction(2) ** 128)
    return fr


_BF16 = None


def exact_bf16_bits(value) -> int:
    """Round an exact value (Fraction/float) to bf16 bits by brute-force search."""
    global _BF16
    if _BF16 is None:
        _BF16 = _bf16_table()
    if isinstance(value, float):
        if value != value:
            return 0x7FC0
        if value in (float("inf"), float("-inf")):
            return 0x7F80 | (0x8000 if value < 0 else 0)
        neg = np.signbit(value)
        value = Fraction(value)
    else:
        neg = value < 0
    a = abs(value)
    i = bisect.bisect_left(_BF16, a)
    if i >= len(_BF16):
        b = 0x7F80
    elif _BF16[i] == a:
        b = i
    else:
        lo, hi = i - 1, i
        dlo, dhi = a - _BF16[lo], _BF16[hi] - a
        if dlo < dhi:
            b = lo
        elif dhi < dlo:
            b = hi
        else:
            b = lo if lo % 2 == 0 else hi
    if b >= 0x7F80:
        b = 0x7F80
    return b | (0x8000 if neg else 0)


def load_spot_values():
    out = []
    with open(os.path.join(GOLDEN, "e4m3fn_spot_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                out.append((int(code, 16), float(val)))
    return out


def load_bf16_cases():
    out = []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            v = float(parts[0]) if parts[0] in ("nan", "inf") else float.fromhex(parts[0])
            out.append((v, int(parts[1], 16), " ".join(parts[2:])))
    return out


def load_closed_forms():
    out = []
    with open(os.path.join(GOLDEN, "closed_forms.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            out.append(dict(name=p[0], M=int(p[1]), N=int(p[2]), K=int(p[3]), x=p[4], w=p[5],
                            scale=float.fromhex(p[6]), expected=int(p[7], 16)))
    return out


def _closed_form_operands(case):
    M, N, K = case["M"], case["N"], case["K"]

    def build(spec, rows):
        a = np.zeros((rows, K), np.uint8)
        if K == 0:
            return a
        if spec.endswith("_if_k>=4096_else_0x00"):
            a[:, 4096:] = int(spec.split("_")[0], 16)
        elif "," in spec:
            a[:, :] = np.array([int(s, 16) for s in spec.split(",")], np.uint8)[None, :]
        else:
            a[:, :] = int(spec, 16)
        return a

    return build(case["x"], M), build(case["w"], N), np.full(N, case["scale"], np.float32)


def e4m3_ints(codes) -> np.ndarray:
    """Integer n with value = n * 2^-9 (library decode, exact)."""
    v = torch_decode(codes) * 512.0
    assert np.all(v == np.round(v))
    return v.astype(np.int64)


def finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = 0x38
    return c


# -------------------------------------------------------------------- checks --
def check_decode_spot_values(impl):
    for code, val in load_spot_values():
        got = float(impl.decode(np.array([code], np.uint8))[0])
        if val != val:
            assert got != got, f"code {code:#04x}: expected NaN, got {got}"
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (
                f"code {code:#04x}: expected {val}, got {got}")


def check_decode_all_codes_vs_torch(impl):
    codes = np.arange(256, dtype=np.uint8)
    got = impl.decode(codes)
    ref = torch_decode(codes)
    both_nan = np.isnan(got) & np.isnan(ref)
    same = (got == ref) & (np.signbit(got) == np.signbit(ref))
    bad = ~(both_nan | same)
    assert not bad.any(), f"decode differs from torch on codes {np.nonzero(bad)[0][:8]}"


def check_bf16_golden(impl):
    cases = load_bf16_cases()
    got = impl.bf16(np.array([c[0] for c in cases], np.float64))
    for (v, exp, note), g in zip(cases, got):
        assert int(g) == exp, f"bf16({v!r}) = {int(g):#06x}, expected {exp:#06x} ({note})"


def check_bf16_bruteforce(impl, n=4000, seed=7):
    rng = np.random.default_rng(seed)
    # log-uniform magnitudes across subnormal, normal and overflow ranges
    mags = np.ldexp(rng.random(n) + 0.5, rng.integers(-140, 130, size=n))
    # exact midpoints between neighbouring bf16 values, and their neighbours
    b = rng.integers(0, 0x7F7F, size=n // 4).astype(np.int16)
    lo = torch.from_numpy(b).view(torch.bfloat16).double().numpy()
    hi = torch.from_numpy(b + 1).view(torch.bfloat16).double().numpy()
    mids = (lo + hi) / 2
    vals = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    vals = vals * np.where(rng.random(vals.size) < 0.5, -1.0, 1.0)
    got = impl.bf16(vals)
    for v, g in zip(vals, got):
        e = exact_bf16_bits(float(v))
        assert int(g) == e, f"bf16({float(v).hex()}) = {int(g):#06x}, expected {e:#06x}"


def check_bf16_vs_torch_on_float32(impl, n=200000, seed=8):
    """For fp32-representable inputs, torch's float32 -> bfloat16 cast is RNE."""
    rng = np.random.default_rng(seed)
    f32 = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = impl.bf16(f32.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on fp32 inputs"


def check_acc_int64_exact(impl, seed=11):
    rng = np.random.default_rng(seed)
    for (M, N, K) in [(3, 5, 1), (7, 9, 129), (13, 6, 4127), (4, 4, 2000)]:
        x = finite_codes(rng, (M, K))
        w = finite_codes(rng, (N, K))
        ref = (e4m3_ints(x) @ e4m3_ints(w).T).astype(np.float64) * 2.0 ** -18
        got = impl.acc(x, w)
        assert np.array_equal(got, ref), f"accumulator not exact at {(M, N, K)}"


def check_acc_vs_torch_matmul(impl, seed=12):
    rng = np.random.default_rng(seed)
    M, N, K = 9, 11, 4127
    x = finite_codes(rng, (M, K))
    w = finite_codes(rng, (N, K))
    ref = (torch.from_numpy(torch_decode(x)) @ torch.from_numpy(torch_decode(w)).T).numpy()
    assert np.array_equal(impl.acc(x, w), ref), "accumulator differs from torch float64 matmul"


def check_tiny_bruteforce(impl, seed=13):
    """y for M,N,K <= 4 from exact Fraction sums, exact product with the fp32
    scale, and a brute-force bf16 search."""
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1), (2, 3, 4), (4, 4, 4), (3, 2, 1), (4, 1, 3), (2, 2, 0)]
    for (M, N, K) in shapes:
        for rep in range(4):
            x = finite_codes(rng, (M, K))
            w = finite_codes(rng, (N, K))
            scale = rng.uniform(0.005, 0.02, size=N).astype(np.float32)
            if rep == 1:
                scale = (2.0 ** rng.integers(-20, 20, size=N)).astype(np.float32)
            dx, dw = torch_decode(x), torch_decode(w)
            got = impl.scaled(x, w, scale)
            for m in range(M):
                for n in range(N):
                    s = sum((Fraction(float(dx[m, k])) * Fraction(float(dw[n, k])) for k in range(K)),
                            Fraction(0))
                    e = exact_bf16_bits(s * Fraction(float(scale[n])))
                    assert int(got[m, n]) == e, (
                        f"y[{m},{n}] at {(M, N, K)} = {int(got[m, n]):#06x}, expected {e:#06x}")


def check_closed_forms(impl):
    for case in load_closed_forms():
        x, w, scale = _closed_form_operands(case)
        y = impl.scaled(x, w, scale)
        assert y.shape == (case["M"], case["N"])
        assert np.all(y == case["expected"]), (
            f"{case['name']}: got {np.unique(y)}, expected {case['expected']:#06x}")


def check_pm_one_closed_form(impl, seed=14):
    """x, w in {+1, -1}, scale 2^-6: y = (integer dot) / 64 exactly while
    |dot| <= 256 (8 significant bits fit bf16)."""
    rng = np.random.default_rng(seed)
    M, N, K = 6, 10, 4127
    sx = rng.choice([-1, 1], size=(M, K))
    sw = rng.choice([-1, 1], size=(N, K))
    x = np.where(sx > 0, 0x38, 0xB8).astype(np.uint8)
    w = np.where(sw > 0, 0x38, 0xB8).astype(np.uint8)
    dot = sx.astype(np.int64) @ sw.astype(np.int64).T
    assert np.abs(dot).max() <= 256
    exp = torch.from_numpy(dot.astype(np.float32) / 64).to(torch.bfloat16)
    # dot/64 is exactly representable in bf16, so the cast does not round
    exp = exp.view(torch.int16).numpy().view(np.uint16)
    y = impl.scaled(x, w, np.full(N, 2.0 ** -6, np.float32))
    assert np.array_equal(y, exp), "+-1 closed form differs"


def check_tail_position(impl):
    """Only k in [4096, 4127) of w is non-zero: every y must be 31 * scale, and
    moving one 1 out of the tail changes the result (catches dropped or
    duplicated tail bytes)."""
    M, N, K = 3, 4, 4127
    x = np.full((M, K), 0x38, np.uint8)
    w = np.zeros((N, K), np.uint8)
    w[:, 4096:] = 0x38
    w[1, 4126] = 0x40          # last byte of row 1 is 2.0 instead of 1.0
    scale = np.full(N, 2.0 ** -6, np.float32)
    y = impl.scaled(x, w, scale)
    vals = torch.from_numpy(y.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.all(vals[:, [0, 2, 3]] == 31 / 64)
    assert np.all(vals[:, 1] == 32 / 64)


def check_identity_weight(impl, seed=15):
    rng = np.random.default_rng(seed)
    M, K = 5, 64
    x = finite_codes(rng, (M, K))
    w = np.zeros((K, K), np.uint8)
    np.fill_diagonal(w, 0x38)
    scale = rng.uniform(0.005, 0.02, size=K).astype(np.float32)
    y = impl.scaled(x, w, scale)
    dx = torch_decode(x)
    for m in range(M):
        for n in range(K):
            e = exact_bf16_bits(Fraction(float(dx[m, n])) * Fraction(float(scale[n])))
            assert int(y[m, n]) == e, f"identity weight y[{m},{n}]"


def check_zero_pad_invariance(impl, seed=16):
    rng = np.random.default_rng(seed)
    M, N, K = 7, 9, 100
    x = finite_codes(rng, (M, K))
    w = finite_codes(rng, (N, K))
    scale = rng.uniform(0.005, 0.02, size=N).astype(np.float32)
    y = impl.scaled(x, w, scale)
    for r in (1, 28, 157):
        xp = np.concatenate([x, np.zeros((M, r), np.uint8)], axis=1)
        wp = np.concatenate([w, np.zeros((N, r), np.uint8)], axis=1)
        assert np.array_equal(impl.scaled(xp, wp, scale), y), f"zero padding by {r} changed y"


def check_scale_linearity(impl, seed=17):
    rng = np.random.default_rng(seed)
    M, N, K = 6, 8, 300
    x = finite_codes(rng, (M, K))
    w = finite_codes(rng, (N, K))
    scale = rng.uniform(0.005, 0.02, size=N).astype(np.float32)
    y = impl.scaled(x, w, scale)
    yv = torch.from_numpy(y.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for j in (-3, 4):
        y2 = impl.scaled(x, w, (scale * np.float32(2.0 ** j)).astype(np.float32))
        y2v = torch.from_numpy(y2.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
        assert np.array_equal(y2v, yv * 2.0 ** j), f"scale * 2^{j} did not scale y exactly"


def check_nan_propagates(impl):
    M, N, K = 3, 4, 5
    x = np.full((M, K), 0x38, np.uint8)
    w = np.full((N, K), 0x38, np.uint8)
    x[1, 2] = 0x7F
    y = impl.scaled(x, w, np.ones(N, np.float32))
    assert np.all(y[1] == 0x7FC0) and np.all(y[[0, 2]] == exact_bf16_bits(5.0))


ALL_CHECKS = [
    check_decode_spot_values,
    check_decode_all_codes_vs_torch,
    check_bf16_golden,
    check_bf16_bruteforce,
    check_bf16_vs_torch_on_float32,
    check_acc_int64_exact,
    check_acc_vs_torch_matmul,
    check_tiny_bruteforce,
    check_closed_forms,
    check_pm_one_closed_form,
    check_tail_position,
    check_identity_weight,
    check_zero_pad_invariance,
    check_scale_linearity,
    check_nan_propagates,
]


# ======================================================================
# General formats and the bias / activation epilogue.
#
# These checks take an implementation with three more methods
#
#     decode5(codes uint8[...])                       -> float64  E5M2 -> value
#     act(z float64[...], act int)                    -> float64  activation
#     epi(x, w, scale, bias|None, act, x_fmt, w_fmt)  -> uint16   y as bf16 bits
#
# Expected values come from torch's float8_e5m2 / float8_e4m3fn conversions,
# numpy's float16 (an E5M2 code is the top byte of an fp16), exact Fraction
# sums with IEEE rules for the special values written out here, torch's
# float64 activation functions, and closed forms.
FMT_E4M3, FMT_E5M2 = 0, 1
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3


def torch_decode5(codes) -> np.ndarray:
    """Library decode: torch's float8_e5m2 -> float64 conversion."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e5m2).to(torch.float64).numpy()


def _decode_fmt(codes, fmt):
    return torch_decode(codes) if fmt == FMT_E4M3 else torch_decode5(codes)


def torch_act(z, act):
    t = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float64))
    if act == ACT_RELU:
        t = torch.nn.functional.relu(t)
    elif act == ACT_SILU:
        t = torch.nn.functional.silu(t)
    elif act == ACT_GELU_TANH:
        t = torch.nn.functional.gelu(t, approximate="tanh")
    return t.numpy()


def exact_epilogue(x, w, scale, bias, act, xf, wf):
    """y bits from exact Fraction sums of library-decoded values (finite z only
    goes through torch's activation; the special-value rules are IEEE's)."""
    dx, dw = _decode_fmt(x, xf), _decode_fmt(w, wf)
    M, K = dx.shape
    N = dw.shape[0]
    out = np.empty((M, N), np.uint16)
    for m in range(M):
        for n in range(N):
            tot, nan, pinf, ninf = Fraction(0), False, False, False
            for k in range(K):
                a, b = float(dx[m, k]), float(dw[n, k])
                if np.isnan(a) or np.isnan(b):
                    nan = True
                elif np.isinf(a) or np.isinf(b):
                    if a == 0.0 or b == 0.0:
                        nan = True
                    elif (a < 0) != (b < 0):
                        ninf = True
                    else:
                        pinf = True
                else:
                    tot += Fraction(a) * Fraction(b)
            if nan or (pinf and ninf):
                acc = float("nan")
            elif pinf or ninf:
                acc = float("inf") if pinf else float("-inf")
            else:
                acc = float(tot)  # correctly rounded
            z = acc * float(scale[n]) + (float(bias[n]) if bias is not None else 0.0)
            if np.isfinite(z):
                v = float(torch_act(np.array([z]), act)[0])
            else:
                v = z
                if np.isinf(z) and act != ACT_NONE and z < 0:
                    v = 0.0 if act == ACT_RELU else -0.0
            out[m, n] = 0x7FC0 if np.isnan(v) else exact_bf16_bits(v)
    return out


def check_e5m2_decode_vs_fp16_and_torch(impl):
    codes = np.arange(256, dtype=np.uint8)
    got = impl.decode5(codes)
    half = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    lib = torch_decode5(codes)
    for ref in (half, lib):
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok])
        assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def check_e5m2_spot_values(impl):
    # OCP E5M2: bias 15, 2 mantissa bits, exponent 31 = inf / NaN
    cases = {0x3C: 1.0, 0x7B: 57344.0, 0x01: 2.0 ** -16, 0x04: 2.0 ** -14, 0x03: 0.75 * 2.0 ** -14,
             0x3D: 1.25, 0xC0: -2.0, 0x7C: float("inf"), 0xFC: float("-inf"), 0x00: 0.0}
    got = impl.decode5(np.array(list(cases), np.uint8))
    assert np.array_equal(got, np.array(list(cases.values())))
    nan = impl.decode5(np.array([0x7D, 0x7E, 0x7F, 0xFD, 0xFF], np.uint8))
    assert np.all(np.isnan(nan))
    assert np.signbit(impl.decode5(np.array([0x80], np.uint8))[0])


def check_epi_e4m3_plain_is_the_scaled_definition(impl, seed=21):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 256, (5, 37), dtype=np.uint8)
    w = rng.integers(0, 256, (6, 37), dtype=np.uint8)
    s = rng.uniform(0.001, 3.0, 6).astype(np.float32)
    got = impl.epi(x, w, s, None, ACT_NONE, FMT_E4M3, FMT_E4M3)
    assert np.array_equal(got, exact_epilogue(x, w, s, None, ACT_NONE, FMT_E4M3, FMT_E4M3))


def check_epi_vs_exact_all_formats_and_acts(impl, seed=22):
    rng = np.random.default_rng(seed)
    for xf in (FMT_E4M3, FMT_E5M2):
        for wf in (FMT_E4M3, FMT_E5M2):
            for act in (ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH):
                M, N, K = 3, 4, int(rng.integers(1, 12))
                x = rng.integers(0, 256, (M, K), dtype=np.uint8)
                w = rng.integers(0, 256, (N, K), dtype=np.uint8)
                s = rng.uniform(-2.0, 2.0, N).astype(np.float32)
                b = rng.uniform(-4.0, 4.0, N).astype(np.float32)
                got = impl.epi(x, w, s, b, act, xf, wf)
                ref = exact_epilogue(x, w, s, b, act, xf, wf)
                assert np.array_equal(got, ref), (xf, wf, act)


def check_epi_small_values_through_every_act(impl, seed=23):
    """Sums near the activations' interesting range (|z| < 8), all formats."""
    rng = np.random.default_rng(seed)
    small4 = np.array([c for c in range(256) if abs(float(torch_decode(np.array([c], np.uint8))[0])) <= 1.0],
                      np.uint8)
    small5 = np.array([c for c in range(256)
                       if abs(float(torch_decode5(np.array([c], np.uint8))[0])) <= 1.0], np.uint8)
    for act in (ACT_RELU, ACT_SILU, ACT_GELU_TANH):
        for xf, wf in ((FMT_E4M3, FMT_E5M2), (FMT_E5M2, FMT_E5M2)):
            px = small4 if xf == FMT_E4M3 else small5
            pw = small4 if wf == FMT_E4M3 else small5
            x = rng.choice(px, (4, 9))
            w = rng.choice(pw, (5, 9))
            s = rng.uniform(0.5, 1.5, 5).astype(np.float32)
            b = rng.uniform(-2.0, 2.0, 5).astype(np.float32)
            assert np.array_equal(impl.epi(x, w, s, b, act, xf, wf), exact_epilogue(x, w, s, b, act, xf, wf))


def check_epi_exact_cancellation_e5m2(impl):
    # 57344^2 + 2^-32 - 57344^2 = 2^-32 exactly; scaled by 2^32 it is 1.0.  A
    # plain fp64 running sum loses the middle term (0x0000 instead of 0x3F80).
    x = np.array([[0x7B, 0x01, 0xFB]], np.uint8)
    w = np.array([[0x7B, 0x01, 0x7B]], np.uint8)
    got = impl.epi(x, w, np.array([2.0 ** 32], np.float32), None, ACT_NONE, FMT_E5M2, FMT_E5M2)
    assert int(got[0, 0]) == 0x3F80


def check_epi_special_values(impl):
    one5, two5, zero, inf5, ninf5, nan5 = 0x3C, 0x40, 0x00, 0x7C, 0xFC, 0x7E
    s1 = np.ones(1, np.float32)

    def y(xs, ws, act=ACT_NONE, xf=FMT_E5M2, wf=FMT_E5M2, bias=None):
        return int(impl.epi(np.array([xs], np.uint8), np.array([ws], np.uint8), s1, bias, act, xf, wf)[0, 0])

    assert y([inf5], [zero]) == 0x7FC0                      # inf * 0
    assert y([inf5, ninf5], [one5, one5]) == 0x7FC0         # inf - inf
    assert y([inf5, one5], [two5, one5]) == 0x7F80          # inf * 2 + 1
    assert y([ninf5], [two5]) == 0xFF80
    assert y([nan5], [zero]) == 0x7FC0
    assert y([ninf5], [one5], ACT_RELU) == 0x0000           # relu(-inf) = 0
    assert y([ninf5], [one5], ACT_SILU) == 0x8000           # limit -0
    assert y([ninf5], [one5], ACT_GELU_TANH) == 0x8000
    assert y([inf5], [one5], ACT_GELU_TANH) == 0x7F80
    assert y([inf5], [one5], ACT_SILU) == 0x7F80
    # an E4M3 NaN operand against an E5M2 zero
    assert y([0x7F], [zero], xf=FMT_E4M3) == 0x7FC0


def check_epi_order_of_scale_bias_act(impl):
    x = np.array([[0x40]], np.uint8)    # E4M3 2.0
    w = np.array([[0x3C]], np.uint8)    # E4M3 1.5  -> acc = 3
    # scale before bias: 3 * 2 + 1 = 7 (bias first would give 8)
    got = impl.epi(x, w, np.array([2.0], np.float32), np.array([1.0], np.float32), ACT_NONE, FMT_E4M3, FMT_E4M3)
    assert int(got[0, 0]) == exact_bf16_bits(7.0)
    # activation last: relu(-3 * 1 + 5) = 2 (relu first would give 5)
    xn = np.array([[0xC0]], np.uint8)   # E4M3 -2.0 -> acc = -3
    got = impl.epi(xn, w, np.array([1.0], np.float32), np.array([5.0], np.float32), ACT_RELU, FMT_E4M3, FMT_E4M3)
    assert int(got[0, 0]) == exact_bf16_bits(2.0)


def check_epi_bias_per_column(impl):
    x = np.zeros((3, 4), np.uint8)
    w = np.zeros((5, 4), np.uint8)
    b = np.array([1.0, -2.0, 3.5, 0.25, -0.125], np.float32)
    got = impl.epi(x, w, np.ones(5, np.float32), b, ACT_NONE, FMT_E5M2, FMT_E4M3)
    ref = np.array([[exact_bf16_bits(float(v)) for v in b]] * 3, np.uint16)
    assert np.array_equal(got, ref)


def check_act_closed_forms(impl):
    import math
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 1.0, -1.0, 40.0, -40.0])
    silu = impl.act(z, ACT_SILU)
    # sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4
    ref = [0.0, 0.75 * math.log(3.0), -0.25 * math.log(3.0), 1 / (1 + math.exp(-1)),
           -1 / (1 + math.exp(1)), 40.0, -40.0 * math.exp(-40.0)]
    assert np.allclose(silu, ref, rtol=1e-14, atol=0)
    relu = impl.act(z, ACT_RELU)
    assert np.array_equal(relu, np.maximum(z, 0.0))
    gelu = impl.act(np.array([0.0, 1.0, 40.0]), ACT_GELU_TANH)
    c = math.sqrt(2.0 / math.pi)
    assert np.allclose(gelu, [0.0, 0.5 * (1 + math.tanh(c * 1.044715)), 40.0], rtol=1e-14, atol=0)
    assert np.array_equal(impl.act(z, ACT_NONE), z)


EPI_CHECKS = [
    check_e5m2_decode_vs_fp16_and_torch,
    check_e5m2_spot_values,
    check_epi_e4m3_plain_is_the_scaled_definition,
    check_epi_vs_exact_all_formats_and_acts,
    check_epi_small_values_through_every_act,
    check_epi_exact_cancellation_e5m2,
    check_epi_special_values,
    check_epi_order_of_scale_bias_act,
    check_epi_bias_per_column,
    check_act_closed_forms,
]
