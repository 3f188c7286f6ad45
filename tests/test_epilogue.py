"""GPU parity of the epilogue variants and operand formats: per-column bias,
elementwise activation (ReLU, SiLU, tanh-form GELU) and E5M2 operands, through
the C ABI entry fp8_gemm_scaled_act(_ex), against the oracle's general
definition  y = bf16(act(acc * scale + bias))  on the same seeded inputs.

Sources on the pages: the per-output-channel scale is applied by a per-column
linear-combination + per-column bias + elementwise-activation epilogue
("DeepSeek V4 Flash (0731)", CUTLASS 3.x SM90 fp8 GEMM cell); the f8f6f4
matrix-core kind takes either FP8 format ("Claude Fable 5", tcgen05 cell).
"""
import numpy as np
import pytest
import torch

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import compare, say, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [(0, 0), (1, 1), (0, 1), (1, 0)]  # (x format, w format); 0 = E4M3, 1 = E5M2
ACTS = [fg.ACT_NONE, fg.ACT_RELU, fg.ACT_SILU, fg.ACT_GELU_TANH]


def run_epi(x, w, s, b, act, xf, wf, *, path=0, variant=0, split_k=0):
    """y bits from the GPU (output pre-filled with NaN so unwritten elements fail)."""
    M, K = x.shape
    N = w.shape[0]
    xd, wd, sd = to_dev(x), to_dev(w), to_dev(s.astype(np.float32))
    bd = to_dev(b.astype(np.float32)) if b is not None else None
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if out.numel():
        out.view(torch.int16).fill_(-1)
    fg.fp8_gemm(xd, wd, sd, bias=bd, act=act, x_format=xf, w_format=wf, out=out, path=path, variant=variant,
                split_k=split_k)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(M, N, K, act, xf, wf, with_bias=True, seed=31, **kw):
    x, w, s = synth.fp8_inputs_fmt(M, N, K, xf, wf, seed=seed)
    b = synth.bias_values(N, seed) if with_bias else None
    say(f"epilogue M={M} N={N} K={K} act={act} fmt=({xf},{wf}) bias={with_bias} {kw}")
    got = run_epi(x, w, s, b, act, xf, wf, **kw)
    ref = oracle.gemm_epilogue(x, w, s, b, act, xf, wf)
    compare(got, ref, f"M={M} N={N} K={K} act={act} fmt=({xf},{wf}) {kw}")


# default plans: main tiles (v18, v10 with a K tail), split-K with 1 and several slices
@pytest.mark.parametrize("shape", [(300, 520, 1000), (520, 300, 4127), (32, 1000, 4127), (17, 777, 3000)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
@pytest.mark.parametrize("act", ACTS)
def test_default_plan(shape, fmts, act):
    _case(*shape, act, *fmts)


@pytest.mark.parametrize("act", ACTS)
def test_no_bias(act):
    _case(300, 264, 777, act, 1, 0, with_bias=False)
    _case(40, 500, 777, act, 0, 1, with_bias=False)


# every variant built for all formats, with a ragged tile edge and a K tail
@pytest.mark.parametrize("variant", [3, 10, 17, 18])
@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
def test_main_variants_all_formats(variant, fmts):
    _case(300, 520, 257, fg.ACT_GELU_TANH, *fmts, path=fg.PATH_MAIN, variant=variant)
    _case(129, 70, 1000, fg.ACT_SILU, *fmts, path=fg.PATH_MAIN, variant=variant)


# the whole-line-row kernel (variant 20, K tail), every format and activation
@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
def test_main_cache_line_rows_all_formats(fmts):
    _case(272, 528, 257, fg.ACT_GELU_TANH, *fmts, path=fg.PATH_MAIN, variant=20)
    _case(256, 80, 1001, fg.ACT_SILU, *fmts, path=fg.PATH_MAIN, variant=20)
    _case(256, 256, 4127, fg.ACT_RELU, *fmts, path=fg.PATH_MAIN, variant=20)


# the register-tile kernel (K % 16 == 0), every format and activation, with and
# without a bias, ragged edges and partial row pieces
@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
def test_main_register_tiles_all_formats(fmts):
    _case(300, 520, 256, fg.ACT_GELU_TANH, *fmts, path=fg.PATH_MAIN, variant=27)
    _case(129, 70, 1040, fg.ACT_SILU, *fmts, path=fg.PATH_MAIN, variant=27)
    _case(33, 301, 48, fg.ACT_RELU, *fmts, path=fg.PATH_MAIN, variant=27)
    _case(64, 64, 128, fg.ACT_RELU, *fmts, path=fg.PATH_MAIN, variant=27, with_bias=False)


# the one-wave-per-SIMD kernel (K % 128 == 0), every format and activation
@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
def test_main_one_wave_per_simd_all_formats(fmts):
    _case(300, 520, 256, fg.ACT_GELU_TANH, *fmts, path=fg.PATH_MAIN, variant=19)
    _case(129, 70, 1024, fg.ACT_SILU, *fmts, path=fg.PATH_MAIN, variant=19)
    _case(257, 300, 384, fg.ACT_RELU, *fmts, path=fg.PATH_MAIN, variant=19)
    _case(260, 264, 128, fg.ACT_NONE, *fmts, path=fg.PATH_MAIN, variant=19)


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 21, 22, 23, 24])
@pytest.mark.parametrize("fmts", FORMATS[1:], ids=lambda f: f"x{f[0]}w{f[1]}")
def test_splitk_ring_variants_all_formats(variant, fmts):
    for M in (1, 16, 40, 64):
        try:
            fg.fp8_gemm_plan_ex(M, 777, 3000, path=fg.PATH_SPLITK, variant=variant)
        except fg.Fp8gError:
            continue  # more w rows than this M allows
        _case(M, 777, 3000, fg.ACT_RELU, *fmts, path=fg.PATH_SPLITK, variant=variant, split_k=3)
        _case(M, 264, 600, fg.ACT_SILU, *fmts, path=fg.PATH_SPLITK, variant=variant, split_k=1)


# bias and activation on the E4M3-only variant (stream-K)
def test_stream_k_epilogue():
    _case(300, 520, 1000, fg.ACT_GELU_TANH, 0, 0, path=fg.PATH_MAIN, variant=16)


def test_e4m3_only_variants_reject_e5m2():
    x = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(fg.Fp8gError):
        fg.fp8_gemm(x, w, s, x_format=fg.FMT_E5M2, path=fg.PATH_MAIN, variant=16)


def test_empty_k_with_bias_and_activation():
    M, N = 33, 70
    x = np.zeros((M, 0), np.uint8)
    w = np.zeros((N, 0), np.uint8)
    s = synth.bias_values(N, 3, 0.5, 2.0)
    b = synth.bias_values(N, 4, -3.0, 3.0)
    for act in ACTS:
        for bias in (b, None):
            say(f"K=0 act={act} bias={bias is not None}")
            got = run_epi(x, w, s, bias, act, 1, 0)
            compare(got, oracle.gemm_epilogue(x, w, s, bias, act, 1, 0), f"K=0 act={act}")


def test_e5m2_special_codes():
    """Every E5M2 code, including +-inf and NaN, against IEEE rules for the sum."""
    rng = np.random.default_rng(12)
    M, N, K = 70, 90, 300
    x = rng.integers(0, 256, (M, K), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K), dtype=np.uint8)
    # keep most rows finite so that finite results are compared too
    fin = lambda c: np.where((c & 0x7C) == 0x7C, c & 0xF3, c).astype(np.uint8)
    x[: M // 2] = fin(x[: M // 2])
    w[: N // 2] = fin(w[: N // 2])
    s = np.ones(N, np.float32)
    say("e5m2 special codes")
    got = run_epi(x, w, s, None, fg.ACT_NONE, 1, 1)
    ref = oracle.gemm_epilogue(x, w, s, None, fg.ACT_NONE, 1, 1)
    # magnitudes span 2^-32 .. 2^32: fp32 accumulation error is relative to
    # the sum of |products| (conditioning term as in the other stress tests)
    cond = oracle.bf16_bits_to_double(oracle.gemm_epilogue(x & 0x7F, w & 0x7F, s, None, 0, 1, 1))
    g, r = oracle.bf16_bits_to_double(got), oracle.bf16_bits_to_double(ref)
    assert np.array_equal(np.isnan(g), np.isnan(r)), "NaN positions differ"
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), "infinities differ"
    ok = np.isfinite(r) & np.isfinite(cond)
    err = np.abs(g[ok] - r[ok])
    bound = 1e-2 + 1e-2 * np.abs(r[ok]) + 2.0 ** -12 * cond[ok]
    assert np.all(err <= bound), f"{int((err > bound).sum())} finite elements outside tolerance"


@pytest.mark.parametrize("name,fmts,act", [("decode-m32", (1, 1), fg.ACT_SILU),
                                           ("square-4096", (0, 1), fg.ACT_GELU_TANH),
                                           ("odd-k-4127", (1, 0), fg.ACT_RELU)])
def test_benchmark_shapes_sampled(name, fmts, act):
    wl = synth.WORKLOAD_BY_NAME[name]
    x, w, s = synth.fp8_inputs_fmt(wl.M, wl.N, wl.K, *fmts, seed=42)
    b = synth.bias_values(wl.N, 42)
    say(f"{name} fmts={fmts} act={act}")
    got = run_epi(x, w, s, b, act, *fmts)
    mi, ni = synth.sample_positions(wl.M, wl.N, 4000, seed=3)
    ref = oracle.gemm_epilogue_at(x, w, s, mi, ni, b, act, *fmts)
    compare(got[mi, ni], ref, f"{name} sampled")


@pytest.mark.parametrize("fmts", FORMATS, ids=lambda f: f"x{f[0]}w{f[1]}")
@pytest.mark.parametrize("act", ACTS)
def test_odd_k_epilogue_full(fmts, act):
    """Odd K on 256 x 256 tiles (rows at any byte, K tail masked in the
    kernel), every format and activation, every element."""
    M, N, K = 520, 600, 3001
    assert fg.fp8_gemm_plan(M, N, K)["k_tail"] == 1
    x, w, s = synth.fp8_inputs_fmt(M, N, K, *fmts, seed=13)
    b = synth.bias_values(N, 13)
    say(f"odd-K epilogue fmts={fmts} act={act}")
    got = run_epi(x, w, s, b, act, *fmts, path=fg.PATH_MAIN, variant=10)
    compare(got, oracle.gemm_epilogue(x, w, s, b, act, *fmts), "odd-K epilogue")
