"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, within 1e-2 + 1e-2 * |ref|.

Sizes the oracle finishes in seconds are compared in full; they span several
tiles and ragged tails on every path and configuration.  The five benchmark
shapes run with the default plan (the launch configuration bench.py times);
the large ones are compared on sampled outputs that the oracle computes one
by one, always including full rows and columns at the tile edges.
"""
import numpy as np
import pytest

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import compare, run, say

pytestmark = pytest.mark.gpu


def _full_case(M, N, K, seed=42, **kw):
    x, w, s = synth.fp8_inputs(M, N, K, seed=seed)
    say(f"full M={M} N={N} K={K} seed={seed} {kw}")
    got = run(x, w, s, **kw)
    ref = oracle.gemm_scaled(x, w, s)
    return compare(got, ref, f"M={M} N={N} K={K} {kw}")


# ------------------------------------------------- main path, every variant --
MAIN_SHAPES = [(300, 520, 4127), (257, 129, 200), (128, 128, 128), (65, 70, 33), (520, 264, 1000),
               # K below one 16-byte chunk, one chunk + 1, one step + 1 byte, exactly three steps
               (70, 300, 1), (40, 33, 17), (256, 256, 257), (300, 300, 384)]


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7, 9, 10, 16, 17, 18])
@pytest.mark.parametrize("shape", MAIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_variants_full(variant, shape):
    _full_case(*shape, path=fg.PATH_MAIN, variant=variant)


# ------------------------- main path, one wave per SIMD (variant 19, K % 128 == 0) --
# One to five 128-byte K steps (the guarded last three steps alone, then with
# the branch-free body before them), rows past M and N, a long K, and an odd K
# through the row realignment.
V19_SHAPES = [(256, 256, 128), (257, 129, 256), (300, 300, 384), (300, 520, 512), (256, 256, 640),
              (513, 777, 4096), (40, 700, 1024)]


@pytest.mark.parametrize("shape", V19_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_one_wave_per_simd(shape):
    _full_case(*shape, path=fg.PATH_MAIN, variant=19)


def test_main_one_wave_per_simd_matches_eight_wave():
    """Variants 19 and 10 add the same products in the same order: bit for bit
    the same output, also with realigned rows (odd K)."""
    for (M, N, K, sk) in [(300, 520, 1024, 0), (513, 264, 4127, 2)]:
        x, w, s = synth.fp8_inputs(M, N, K, seed=13)
        say(f"v19 vs v10 {M}x{N}x{K}")
        a = run(x, w, s, path=fg.PATH_MAIN, variant=19, split_k=sk)
        b = run(x, w, s, path=fg.PATH_MAIN, variant=10, split_k=sk)
        assert np.array_equal(a, b)
        compare(a, oracle.gemm_scaled(x, w, s), f"{M}x{N}x{K} v19")


# ------------------------------------------- main path, stream-K (variant 16) --
# Forced stream-K workgroup counts on small grids: ranges that end inside a
# tile, ranges that cover several tiles, tiles with one to many contributors,
# a K tail that falls into a partial segment, one workgroup per unit.
@pytest.mark.parametrize("shape,groups", [
    ((300, 300, 384), [1, 2, 3, 5, 7, 12]),      # 4 tiles x 3 steps
    ((256, 256, 257), [1, 2, 3]),                # 1 tile: 2 steps + the tail
    ((513, 520, 1000), [5, 16, 40, 72]),         # 9 tiles x 8 steps (last one a tail)
    ((70, 300, 1), [1, 2]),                      # K below one chunk: one step per tile
    ((600, 700, 2050), [3, 11, 50, 100]),        # 9 tiles x 17 steps, 2-byte tail
])
def test_stream_k_forced_groups(shape, groups):
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=5)
    ref = oracle.gemm_scaled(x, w, s)
    for g in groups:
        plan = fg.fp8_gemm_plan_ex(M, N, K, path=fg.PATH_MAIN, variant=16, split_k=g)
        assert plan["sk_groups"] == g and plan["dp_tiles"] == 0
        say(f"stream-K {shape} groups={g}")
        compare(run(x, w, s, path=fg.PATH_MAIN, variant=16, split_k=g), ref, f"{shape} groups={g}")


def test_stream_k_whole_waves_and_remainder():
    """528 tiles: the first full wave is computed one tile per workgroup, the
    last full wave and the 16 remaining tiles by 256 stream-K workgroups."""
    M, N, K = 4096, 8448, 384
    plan = fg.fp8_gemm_plan_ex(M, N, K, path=fg.PATH_MAIN, variant=16)
    assert plan["dp_tiles"] == 256 and plan["sk_groups"] == 256 and plan["grid"] == 512
    x, w, s = synth.fp8_inputs(M, N, K, seed=6)
    say(f"stream-K {M}x{N}x{K} plan {plan}")
    compare(run(x, w, s, path=fg.PATH_MAIN, variant=16), oracle.gemm_scaled(x, w, s), "dp + stream-K")


def test_stream_k_deterministic():
    """Partial sums are added in K order whichever workgroup finishes a tile."""
    M, N, K = 513, 520, 4000
    x, w, s = synth.fp8_inputs(M, N, K, seed=8)
    say("stream-K determinism")
    ys = [run(x, w, s, path=fg.PATH_MAIN, variant=16, split_k=100) for _ in range(4)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


# ------------------------------------------- split-K path, forced splits ------
@pytest.mark.parametrize("split_k", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("M", [1, 31, 32, 33, 64])
def test_splitk_full(M, split_k):
    _full_case(M, 1000, 4127, path=fg.PATH_SPLITK, split_k=split_k)


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5])
def test_splitk_variants(variant):
    """Every rows-per-workgroup configuration of the LDS-ring kernel (16 *
    variant rows), with and without split-K, for each x-row staging width the
    variant supports."""
    if variant <= 2:
        _full_case(40, 777, 3000, path=fg.PATH_SPLITK, variant=variant, split_k=3)
    if variant <= 4:
        _full_case(32, 1024, 4096, path=fg.PATH_SPLITK, variant=variant, split_k=1)
    _full_case(16, 1000, 4127, path=fg.PATH_SPLITK, variant=variant, split_k=2)


@pytest.mark.parametrize("variant", [21, 22, 23, 24])
def test_splitk_eight_wave_variants(variant):
    """The LDS-ring kernel with 8 waves (16 * (variant - 20) rows per
    workgroup), every x-row staging width it supports, with and without
    split-K, with a K tail and chunk counts that are not multiples of 8."""
    for M in (1, 16, 32, 40, 64):
        try:
            fg.fp8_gemm_plan_ex(M, 777, 3000, path=fg.PATH_SPLITK, variant=variant)
        except fg.Fp8gError:
            continue  # more w rows than this M allows
        _full_case(M, 777, 3000, path=fg.PATH_SPLITK, variant=variant, split_k=3)
        _full_case(M, 1000, 4127, path=fg.PATH_SPLITK, variant=variant, split_k=1)
        _full_case(M, 264, 600, path=fg.PATH_SPLITK, variant=variant, split_k=1)


@pytest.mark.parametrize("M", [65, 100, 128])
def test_splitk_up_to_128_x_rows(M):
    """The 4-wave ring kernel with 128 staged x rows (two chunks deep), forced
    onto the split-K path: both row counts, with and without split-K and a
    K tail, plus the planner's own pick."""
    for variant in (1, 2):
        _full_case(M, 777, 3000, path=fg.PATH_SPLITK, variant=variant, split_k=3)
        _full_case(M, 1000, 4127, path=fg.PATH_SPLITK, variant=variant, split_k=1)
    _full_case(M, 264, 600, path=fg.PATH_SPLITK)


@pytest.mark.parametrize("variant", [11, 12, 13, 14, 15])
@pytest.mark.parametrize("M", [1, 16, 17, 32, 40, 64])
def test_splitk_direct_variants(variant, M):
    """The direct-to-register kernel (16 * (variant - 10) rows per workgroup)
    for every x-row block count, with ragged N, a K tail whose last chunk has
    pieces with 0, 1..15 and 16 valid bytes, and 1..3 K slices."""
    _full_case(M, 777, 3000, path=fg.PATH_SPLITK, variant=variant, split_k=3)
    _full_case(M, 1024, 4096, path=fg.PATH_SPLITK, variant=variant, split_k=1)
    _full_case(M, 1000, 4127, path=fg.PATH_SPLITK, variant=variant, split_k=2)
    _full_case(M, 264, 600, path=fg.PATH_SPLITK, variant=variant, split_k=1)


# ---------------------------------------------------- the benchmark shapes ----
def _sampled(x, w, s, got, seed, count=6000, edges=()):
    M, N = got.shape
    mi, ni = synth.sample_positions(M, N, count, seed)
    rows = [r for r in edges if r < M]
    cols = [c for c in edges if c < N]
    for r in rows:                           # full rows
        mi = np.concatenate([mi, np.full(N, r)])
        ni = np.concatenate([ni, np.arange(N)])
    for c in cols:                           # full columns
        mi = np.concatenate([mi, np.arange(M)])
        ni = np.concatenate([ni, np.full(M, c)])
    ref = oracle.gemm_scaled_at(x, w, s, mi, ni)
    return compare(got[mi, ni], ref, f"sampled {M}x{N}")


@pytest.mark.parametrize("wl", synth.WORKLOADS, ids=lambda w: w.name)
def test_benchmark_shape(wl):
    x, w, s = synth.fp8_inputs(wl.M, wl.N, wl.K, seed=42)
    plan = fg.fp8_gemm_plan(wl.M, wl.N, wl.K)
    say(f"{wl.name} default plan {plan}")
    got = run(x, w, s)
    if wl.M * wl.N * wl.K <= 10**11:
        compare(got, oracle.gemm_scaled(x, w, s), wl.name)
    else:
        # first/last rows and columns of tiles, plus random positions
        t = 256
        edges = (0, t - 1, t, wl.M - 1, wl.N - 1)
        _sampled(x, w, s, got, seed=7, edges=edges)


@pytest.mark.parametrize("seed", [123, 456])
@pytest.mark.parametrize("name", ["square-256", "decode-m32", "odd-k-4127"])
def test_benchmark_shape_other_seeds(name, seed):
    wl = synth.WORKLOAD_BY_NAME[name]
    x, w, s = synth.fp8_inputs(wl.M, wl.N, wl.K, seed=seed)
    say(f"{name} seed={seed}")
    got = run(x, w, s)
    if wl.M * wl.N * wl.K <= 10**11:
        compare(got, oracle.gemm_scaled(x, w, s), name)
    else:
        _sampled(x, w, s, got, seed=seed, edges=(0, 255, 256, wl.M - 1))


# ------------------------------------- odd K: operand rows realigned first ----
@pytest.mark.parametrize("variant", [2, 3, 10, 17, 18])
@pytest.mark.parametrize("shape", [(300, 520, 4127), (70, 300, 1), (40, 33, 17), (256, 256, 257), (129, 300, 1003)],
                         ids=lambda s: "x".join(map(str, s)))
def test_row_realignment_matches_in_place(variant, shape):
    """split_k = 2 copies x and w into zero-padded 128-byte rows before the
    kernel; the sums are the same as reading the rows in place (split_k = 1),
    bit for bit, and both match the oracle."""
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=9)
    say(f"realign {shape} variant {variant}")
    padded = run(x, w, s, path=fg.PATH_MAIN, variant=variant, split_k=2)
    in_place = run(x, w, s, path=fg.PATH_MAIN, variant=variant, split_k=1)
    compare(padded, oracle.gemm_scaled(x, w, s), f"{shape} v{variant} padded")
    assert np.array_equal(padded, in_place), "padded rows changed the sums"


def test_row_realignment_unaligned_pointers():
    """Operand pointers at odd byte addresses with an odd K, default plan (pads)."""
    import torch
    M, N, K = 2304, 2560, 3001
    x, w, s = synth.fp8_inputs(M, N, K, seed=10)
    assert fg.fp8_gemm_plan(M, N, K)["pad_k"] == 3072
    xb = torch.zeros(M * K + 3, dtype=torch.uint8, device="cuda")
    wb = torch.zeros(N * K + 5, dtype=torch.uint8, device="cuda")
    xb[3:].copy_(torch.from_numpy(x.reshape(-1)))
    wb[5:].copy_(torch.from_numpy(w.reshape(-1)))
    sd = torch.from_numpy(s).cuda()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("realign with unaligned operand pointers")
    st = fg.fp8_gemm_scaled(xb.data_ptr() + 3, wb.data_ptr() + 5, sd.data_ptr(), y.data_ptr(), M, N, K,
                            torch.cuda.current_stream().cuda_stream)
    assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    mi, ni = synth.sample_positions(M, N, 4000, seed=11)
    compare(got[mi, ni], oracle.gemm_scaled_at(x, w, s, mi, ni), "unaligned + realigned")
