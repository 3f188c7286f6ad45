"""The CPU oracle against its pins (no GPU).

The oracle (oracle/fp8_oracle.c) is checked against facts that do not come
from it: the E4M3 and bf16 format definitions (hand-derived fixtures under
tests/golden/), torch's float8/bfloat16 conversions and float64 matmul,
exact integer and rational arithmetic, closed forms and invariants.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import oracle_pins as pins


class COracle:
    """The C oracle behind the interface the pin checks expect."""

    decode = staticmethod(oracle.e4m3_to_double)
    bf16 = staticmethod(oracle.bf16_rne)
    acc = staticmethod(oracle.gemm_acc)
    scaled = staticmethod(oracle.gemm_scaled)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(COracle())


class COracleEpilogue:
    """The C oracle's general-format and epilogue entry points."""

    decode5 = staticmethod(oracle.e5m2_to_double)
    act = staticmethod(oracle.activation)

    @staticmethod
    def epi(x, w, scale, bias, act, xf, wf):
        return oracle.gemm_epilogue(x, w, scale, bias, act, xf, wf)


@pytest.mark.parametrize("check", pins.EPI_CHECKS, ids=lambda c: c.__name__)
def test_oracle_epilogue_pin(check):
    check(COracleEpilogue())


def test_epilogue_sampled_positions_match_full():
    rng = np.random.default_rng(9)
    x = rng.integers(0, 256, (29, 300), dtype=np.uint8)
    w = rng.integers(0, 256, (31, 300), dtype=np.uint8)
    s = rng.uniform(0.01, 1.0, 31).astype(np.float32)
    b = rng.uniform(-1, 1, 31).astype(np.float32)
    y = oracle.gemm_epilogue(x, w, s, b, oracle.ACT_SILU, oracle.FMT_E5M2, oracle.FMT_E4M3)
    mi, ni = synth.sample_positions(29, 31, 300, seed=10)
    at = oracle.gemm_epilogue_at(x, w, s, mi, ni, b, oracle.ACT_SILU, oracle.FMT_E5M2, oracle.FMT_E4M3)
    assert np.array_equal(at, y[mi, ni])


def test_sampled_positions_match_full():
    x, w, s = synth.fp8_inputs(37, 53, 300, seed=3)
    y = oracle.gemm_scaled(x, w, s)
    mi, ni = synth.sample_positions(37, 53, 500, seed=4)
    assert np.array_equal(oracle.gemm_scaled_at(x, w, s, mi, ni), y[mi, ni])


def test_thread_count_does_not_change_result():
    x, w, s = synth.fp8_inputs(64, 40, 1000, seed=5)
    assert np.array_equal(oracle.gemm_scaled(x, w, s, threads=1), oracle.gemm_scaled(x, w, s, threads=3))


def test_oracle_rejects_bad_arguments():
    x = np.zeros((2, 3), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_scaled(x, np.zeros((4, 5), np.uint8), np.ones(4, np.float32))
    with pytest.raises(ValueError):
        oracle.gemm_scaled_at(x, np.zeros((4, 3), np.uint8), np.ones(4, np.float32), [2], [0])
    with pytest.raises(TypeError):
        oracle.gemm_scaled(x.astype(np.int16), np.zeros((4, 3), np.uint8), np.ones(4, np.float32))


def test_empty_extents():
    assert oracle.gemm_scaled(np.zeros((0, 4), np.uint8), np.zeros((3, 4), np.uint8),
                              np.ones(3, np.float32)).shape == (0, 3)
    y = oracle.gemm_scaled(np.zeros((2, 0), np.uint8), np.zeros((3, 0), np.uint8), np.ones(3, np.float32))
    assert np.all(y == 0)


# ------------------------------------------------------------ input generator --
def _nearest_e4m3_bruteforce(v: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code to each fp32 value, ties to even mantissa,
    saturating at +-448, by exhaustive search over the 127 non-negative finite
    codes (decoded by torch)."""
    codes = np.arange(0x7F, dtype=np.uint8)                # 0x00 .. 0x7E
    vals = pins.torch_decode(codes)                        # ascending
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest codes pick the even one on a tie
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out = codes[pick]
    return np.where(np.signbit(v), out | 0x80, out).astype(np.uint8)


@pytest.mark.parametrize("sigma", [1.0, 100.0, 0.01])
def test_quantizer_is_saturating_rne(sigma):
    g = torch.Generator().manual_seed(21)
    v = torch.randn(100000, generator=g) * sigma
    # add exact midpoints between neighbouring codes, both parities
    vals = pins.torch_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = torch.cat([v, torch.from_numpy(mids), -torch.from_numpy(mids),
                   torch.tensor([448.0, 449.0, 464.0, 465.0, 1e6, -1e6, 0.0])])
    got = synth.quantize_e4m3(v)
    exp = _nearest_e4m3_bruteforce(v.numpy())
    z = (exp & 0x7F) == 0
    assert np.array_equal(got[~z], exp[~z])
    assert np.all((got[z] & 0x7F) == 0)


def test_generator_is_seeded_and_in_range():
    a = synth.fp8_inputs(16, 24, 64, seed=42)
    b = synth.fp8_inputs(16, 24, 64, seed=42)
    c = synth.fp8_inputs(16, 24, 64, seed=43)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(a[0], c[0])
    x, w, s = a
    assert x.dtype == np.uint8 and w.dtype == np.uint8 and s.dtype == np.float32
    assert not np.any((x & 0x7F) == 0x7F) and not np.any((w & 0x7F) == 0x7F)
    assert s.min() >= 0.005 and s.max() <= 0.02
