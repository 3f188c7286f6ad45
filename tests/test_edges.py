"""GPU edge cases, numeric stress, recompute-on-live-data and determinism,
each checked against the oracle on the same inputs.

The recompute cases follow the pages' audits: every call must read the live
operands (an in-place overwrite of the same buffer must change the output and
match the reference; "Kimi K3 (256k)", SM90 WGMMA cell), including a change
confined to a row and to the K-tail bytes that a sampled cache key would miss
("Qwen 3.8 Max", stale odd-K pad-cache cell), and in-place rescaling of the
weight and of the scale ("GLM-5.2", B200 TMA Triton cell).
"""
import numpy as np
import pytest
import torch

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import COND_GAMMA_CODES, compare, conditioning, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 4127])
@pytest.mark.parametrize("M", [1, 31, 33, 65, 200])
def test_edge_k_and_m(M, K):
    N = 72 if M <= 64 else 136
    x, w, s = synth.fp8_inputs(M, N, K, seed=M * 1000 + K)
    say(f"edge M={M} N={N} K={K}")
    compare(run(x, w, s), oracle.gemm_scaled(x, w, s), f"M={M} K={K}")


@pytest.mark.parametrize("N", [1, 3, 5, 31, 33, 255, 257])
def test_edge_n_not_multiple(N):
    for M in (17, 100):
        x, w, s = synth.fp8_inputs(M, N, 300, seed=N)
        say(f"edge N={N} M={M}")
        compare(run(x, w, s), oracle.gemm_scaled(x, w, s), f"N={N} M={M}")


def test_k_zero_gives_zeros_and_empty_extents_are_no_ops():
    say("K=0")
    y = run(np.zeros((5, 0), np.uint8), np.zeros((7, 0), np.uint8), np.ones(7, np.float32))
    assert np.all(y == 0)
    for (M, N) in [(0, 7), (5, 0)]:
        y = run(np.zeros((M, 3), np.uint8), np.zeros((N, 3), np.uint8), np.ones(N, np.float32))
        assert y.shape == (M, N)


@pytest.mark.parametrize("sigma", [100.0, 0.01])
@pytest.mark.parametrize("shape", [(300, 264, 4127), (32, 1000, 4096), (64, 520, 129)])
def test_numeric_stress_distributions(sigma, shape):
    """sigma=100 saturates codes at +-448 and cancels heavily (conditioning
    term in the bound); sigma=0.01 is mostly subnormal E4M3 and zeros."""
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=5, sigma=sigma)
    say(f"stress sigma={sigma} {shape}")
    compare(run(x, w, s), oracle.gemm_scaled(x, w, s), f"sigma={sigma}", cond=conditioning(x, w, s))


@pytest.mark.parametrize("scale_kind", ["tiny", "one", "pow2"])
def test_numeric_stress_scales(scale_kind):
    M, N, K = 96, 264, 1000
    x, w, _ = synth.fp8_inputs(M, N, K, seed=6)
    rng = np.random.default_rng(6)
    s = {"tiny": np.full(N, 1e-4, np.float32), "one": np.ones(N, np.float32),
         "pow2": (2.0 ** rng.integers(-12, 6, size=N)).astype(np.float32)}[scale_kind]
    say(f"scale {scale_kind}")
    # a large scale amplifies the fp32 rounding of cancelling sums: conditioning term
    compare(run(x, w, s), oracle.gemm_scaled(x, w, s), scale_kind, cond=conditioning(x, w, s))


def test_all_codes_random_including_nan():
    """Uniform random codes over all 256 patterns (NaN included): NaN positions
    must match the oracle's exactly, everything else within tolerance (with the
    conditioning term: codes span 2^-9 .. 448, so sums cancel heavily)."""
    M, N, K = 70, 90, 200
    x = synth.random_codes((M, K), seed=1, allow_nan=False)
    w = synth.random_codes((N, K), seed=2, allow_nan=False)
    x[3, 17] = 0x7F
    w[5, 100] = 0xFF
    s = np.full(N, 0.01, np.float32)
    say("nan propagation")
    cond = conditioning(x, w, s)
    compare(run(x, w, s), oracle.gemm_scaled(x, w, s), "nan", cond=np.nan_to_num(cond), gamma=COND_GAMMA_CODES)


def _call_live(xd, wd, sd, out):
    fg.fp8_gemm(xd, wd, sd, out=out)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("shape", [(4096, 4096, 4127), (32, 12288, 4096), (300, 520, 4127)])
def test_recompute_on_in_place_changes(shape):
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=9)
    xd, wd, sd = to_dev(x), to_dev(w), to_dev(s)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mi, ni = synth.sample_positions(M, N, 3000, seed=10)
    mi = np.concatenate([mi, np.zeros(N, np.int64)])      # all of row 0
    ni = np.concatenate([ni, np.arange(N)])

    def check(tag):
        say(f"recompute {shape} {tag}")
        got = _call_live(xd, wd, sd, out)
        compare(got[mi, ni], oracle.gemm_scaled_at(x, w, s, mi, ni), tag)
        return got

    y0 = check("initial")
    # 1. overwrite row 0 of x in place, only its K-tail bytes (past the last multiple of 128)
    tail0 = (K // 128) * 128
    x[0, tail0:] = synth.quantize_e4m3(torch.full((K - tail0,), 3.0))
    xd[0].copy_(torch.from_numpy(x[0]))
    y1 = check("x row 0 tail")
    if K % 128:
        assert not np.array_equal(y0[0], y1[0]), "row 0 did not change after its tail bytes did"
    assert np.array_equal(y0[1:], y1[1:])
    # 2. rescale the weight in place (all rows), same pointer
    w[:] = synth.quantize_e4m3(torch.from_numpy(oracle.e4m3_to_double(w) * 0.5))
    wd.copy_(torch.from_numpy(w))
    check("w halved")
    # 3. change the scale in place
    s[:] = s[::-1].copy()
    sd.copy_(torch.from_numpy(s))
    check("scale reversed")


def test_alternating_k_shapes_share_nothing():
    a = synth.fp8_inputs(256, 384, 4127, seed=11)
    b = synth.fp8_inputs(256, 384, 4096, seed=12)
    ra, rb = oracle.gemm_scaled(*a), oracle.gemm_scaled(*b)
    for i in range(3):
        say(f"alternate K {i}")
        compare(run(*a), ra, "K=4127")
        compare(run(*b), rb, "K=4096")


def test_splitk_back_to_back_calls_without_sync():
    """Split-K calls queued on one stream with no synchronisation between them:
    each call's last-arriving workgroups must add exactly that call's partials
    (stream-ordered workspaces may reuse the same memory and its old tickets)."""
    cases = [((32, 1000, 4127), 4), ((17, 777, 3000), 3), ((32, 1000, 4127), 7), ((64, 264, 600), 2)]
    data = [synth.fp8_inputs(M, N, K, seed=20 + i) for i, ((M, N, K), _) in enumerate(cases)]
    dev = [tuple(to_dev(a.astype(np.float32) if a.dtype != np.uint8 else a) for a in d) for d in data]
    refs = [oracle.gemm_scaled(*d) for d in data]
    outs = []
    say("split-K back to back, 5 rounds of 4 shapes")
    for _ in range(5):
        for ((M, N, K), S), (xd, wd, sd) in zip(cases, dev):
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            out.view(torch.int16).fill_(-1)
            fg.fp8_gemm(xd, wd, sd, out=out, path=fg.PATH_SPLITK, split_k=S)
            outs.append(out)
    torch.cuda.synchronize()
    first = [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs[:len(cases)]]
    for i, (f, r) in enumerate(zip(first, refs)):
        compare(f, r, f"case {i}")
    for j, o in enumerate(outs[len(cases):]):
        got = o.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, first[j % len(cases)]), f"call {j + len(cases)} differs"


def test_workspace_calls_on_two_streams():
    """Workspace-using calls (split-K partials and tickets, stream-K partials)
    queued on two streams that run concurrently: each call's
    workspace is its own, so every output matches the oracle and the repeats
    match bit for bit."""
    cases = [((32, 1000, 4127), dict(path=fg.PATH_SPLITK, split_k=4)),
             ((300, 520, 4127), dict(path=fg.PATH_MAIN, variant=16, split_k=3)),
             ((64, 264, 600), dict(path=fg.PATH_SPLITK, split_k=3)),
             ((512, 768, 1000), dict(path=fg.PATH_MAIN, variant=16, split_k=7))]
    data = [synth.fp8_inputs(M, N, K, seed=40 + i) for i, ((M, N, K), _) in enumerate(cases)]
    dev = [(to_dev(x), to_dev(w), to_dev(s)) for (x, w, s) in data]
    refs = [oracle.gemm_scaled(*d) for d in data]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    say("workspace calls on two streams, 4 rounds")
    for r in range(4):
        for i, (((M, N, K), kw), (xd, wd, sd)) in enumerate(zip(cases, dev)):
            st = streams[(i + r) % 2]
            with torch.cuda.stream(st):
                out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                out.view(torch.int16).fill_(-1)
                fg.fp8_gemm(xd, wd, sd, out=out, stream=st, **kw)
            outs.append((i, out))
    torch.cuda.synchronize()
    first = {}
    for i, out in outs:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        if i not in first:
            compare(got, refs[i], f"two streams, case {i}")
            first[i] = got
        else:
            assert np.array_equal(got, first[i]), f"case {i}: a repeat differs"


@pytest.mark.parametrize("shape,kw", [
    ((4096, 4096, 4127), {}), ((32, 12288, 4096), {}),
    ((32, 12288, 4096), dict(path=fg.PATH_SPLITK, split_k=4)), ((256, 256, 256), {}),
])
def test_deterministic(shape, kw):
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=13)
    say(f"determinism {shape} {kw}")
    ys = [run(x, w, s, **kw) for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_unaligned_operands_and_output():
    """x and w start at odd byte addresses, y at a 2-byte (not 8-byte) boundary."""
    M, N, K = 100, 130, 333
    x, w, s = synth.fp8_inputs(M, N, K, seed=14)
    xb = torch.zeros(M * K + 1, dtype=torch.uint8, device="cuda")
    wb = torch.zeros(N * K + 3, dtype=torch.uint8, device="cuda")
    xb[1:].copy_(torch.from_numpy(x.reshape(-1)))
    wb[3:].copy_(torch.from_numpy(w.reshape(-1)))
    sd = to_dev(s)
    yb = torch.full((M * N + 1,), -1, dtype=torch.int16, device="cuda")
    say("unaligned pointers")
    st = fg.fp8_gemm_scaled(xb.data_ptr() + 1, wb.data_ptr() + 3, sd.data_ptr(), yb.data_ptr() + 2,
                            M, N, K, torch.cuda.current_stream().cuda_stream)
    assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
    torch.cuda.synchronize()
    got = yb[1:].cpu().numpy().view(np.uint16).reshape(M, N)
    compare(got, oracle.gemm_scaled(x, w, s), "unaligned")
    assert int(yb[0].item()) == -1, "wrote before y"


def test_status_codes_on_gpu():
    x = torch.zeros((4, 8), dtype=torch.uint8, device="cuda")
    w = torch.zeros((4, 8), dtype=torch.uint8, device="cuda")
    s = torch.ones(4, dtype=torch.float32, device="cuda")
    with pytest.raises(fg.Fp8gError):
        fg.fp8_gemm(x, w, s, path=fg.PATH_SPLITK, variant=42)
    with pytest.raises(ValueError):
        fg.fp8_gemm(x, w[:, :4].contiguous(), s)
    with pytest.raises(TypeError):
        fg.fp8_gemm(x.to(torch.int16), w, s)


@pytest.mark.parametrize("shape,kw", [
    ((130, 136, 1_000_003), {}),                               # main path, long odd rows
    ((300, 264, 1_000_003), dict(path=fg.PATH_MAIN, variant=10)),  # 256 x 256 tiles, in place
    ((3, 200, 2_000_001), {}),                                 # split-K path
    ((40, 300, 1_048_576 + 17), dict(path=fg.PATH_SPLITK, split_k=7)),
])
def test_long_k(shape, kw):
    """K up to 2^21: 32-bit buffer offsets, many K steps and slices."""
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=17, scale_lo=1e-4, scale_hi=2e-4)
    say(f"long K {shape} {kw}")
    got = run(x, w, s, **kw)
    mi, ni = synth.sample_positions(M, N, 600, seed=18)
    compare(got[mi, ni], oracle.gemm_scaled_at(x, w, s, mi, ni), f"long K {shape}")
