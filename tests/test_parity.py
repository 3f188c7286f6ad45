"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, within 1e-2 + 1e-2 * |ref|.

Every comparison covers every element.  Small shapes span several tiles and
ragged tails on every path and configuration; the five benchmark shapes run
at their full sizes with the default plan (the launch configuration bench.py
times), the oracle computing all of their outputs (about 17 s for 8192^3 on
16 host threads).
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


@pytest.mark.parametrize("variant", [3, 10, 16, 17, 18])
@pytest.mark.parametrize("shape", MAIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_variants_full(variant, shape):
    _full_case(*shape, path=fg.PATH_MAIN, variant=variant)


# ------------------------------- main path, register tiles (variant 27, K % 16 == 0) --
# One wave per 16 x 16 block, operands loaded straight into the MFMA registers:
# one K piece (16), a part step, one to many steps (more than the eight kept in
# flight: 2048 is sixteen), ragged M and N (partial 8-byte row pieces, N odd),
# single rows and columns.
V27_SHAPES = [(256, 256, 256), (1, 1, 16), (17, 33, 48), (16, 16, 128), (300, 520, 1024), (65, 70, 2048),
              (255, 257, 144), (64, 1000, 1040), (33, 7, 4096), (128, 130, 272)]


@pytest.mark.parametrize("shape", V27_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_register_tiles(shape):
    """Variant 27 against the oracle, every element, and bit for bit against
    variant 3 (both add the same 128-byte K steps with the same instruction in
    the same order)."""
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=27)
    say(f"v27 {shape}")
    a = run(x, w, s, path=fg.PATH_MAIN, variant=27)
    compare(a, oracle.gemm_scaled(x, w, s), f"{shape} v27")
    b = run(x, w, s, path=fg.PATH_MAIN, variant=3)
    assert np.array_equal(a, b), "variant 27 differs from variant 3"


# ------------------------- main path, one wave per SIMD (variant 19, K % 128 == 0) --
# One to five 128-byte K steps (the guarded last three steps alone, then with
# the branch-free body before them), rows past M and N, a long K.
V19_SHAPES = [(256, 256, 128), (257, 129, 256), (300, 300, 384), (300, 520, 512), (256, 256, 640),
              (513, 777, 4096), (40, 700, 1024)]


@pytest.mark.parametrize("shape", V19_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_one_wave_per_simd(shape):
    _full_case(*shape, path=fg.PATH_MAIN, variant=19)


def test_main_one_wave_per_simd_matches_eight_wave():
    """Variants 19 and 10 add the same products in the same order: bit for bit
    the same output."""
    for (M, N, K) in [(300, 520, 1024), (513, 264, 4224)]:
        x, w, s = synth.fp8_inputs(M, N, K, seed=13)
        say(f"v19 vs v10 {M}x{N}x{K}")
        a = run(x, w, s, path=fg.PATH_MAIN, variant=19)
        b = run(x, w, s, path=fg.PATH_MAIN, variant=10)
        assert np.array_equal(a, b)
        compare(a, oracle.gemm_scaled(x, w, s), f"{M}x{N}x{K} v19")


# ------------- main path, rows fetched as whole cache lines (variant 20, odd K) --
# K from two steps (129, the smallest K the variant takes) to many, with every
# kind of tail (1, 3, 17, 127 bytes past the last whole step, ...); M, N
# multiples of 16 (the variant needs M K and N K multiples of 16) with rows past
# M and N in the edge tiles.
V20_SHAPES = [(256, 256, 4127), (272, 400, 4127), (512, 768, 1001), (256, 512, 131), (304, 256, 145),
              (256, 256, 129), (528, 272, 257), (256, 256, 383), (256, 256, 4113), (256, 256, 4225),
              (256, 256, 4095), (48, 560, 3001), (768, 256, 8191), (272, 288, 641), (16, 16, 259)]


@pytest.mark.parametrize("shape", V20_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_main_cache_line_rows(shape):
    """Variant 20 against the oracle, every element, and bit for bit against
    variant 10 (both add the same 128-byte K steps in the same order)."""
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=21)
    say(f"v20 {shape}")
    a = run(x, w, s, path=fg.PATH_MAIN, variant=20)
    compare(a, oracle.gemm_scaled(x, w, s), f"{shape} v20")
    b = run(x, w, s, path=fg.PATH_MAIN, variant=10)
    assert np.array_equal(a, b), "variant 20 differs from variant 10"


# ---------------------- launches with more tiles than compute units (write-back y) --
# More tiles than the GPU's 256 compute units switch the 16-byte y stores from
# non-temporal to write-back: whole tiles, ragged edge tiles (M or N past the
# last whole tile), the column-pair stores of variant 20 and the 128-row tiles.
MULTIWAVE_CASES = [((4100, 4352, 512), 19), ((4352, 4352, 1001), 20), ((4100, 4352, 1001), 10),
                   ((4352, 4104, 300), 18)]


@pytest.mark.parametrize("shape,variant", MULTIWAVE_CASES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else f"v{v}")
def test_multiwave_write_back_stores(shape, variant):
    M, N, K = shape
    p = fg.fp8_gemm_plan_ex(M, N, K, path=fg.PATH_MAIN, variant=variant)
    assert p["variant"] == variant
    assert -(-M // p["tile_m"]) * -(-N // p["tile_n"]) > 256, "the case must have more tiles than compute units"
    _full_case(M, N, K, seed=5, path=fg.PATH_MAIN, variant=variant)


def test_odd_k_operands_inside_larger_buffers():
    """K = 4127 (every row start offset mod 128 over 128 rows) with the operands
    starting 0, 16 and 80 rows into larger buffers (128-byte aligned, then 112
    and 48 bytes into a line), on the default plan and on the whole-line
    variant 20, which falls back to variant 10 for operands that are not
    128-byte aligned when it was not forced.  Every element, every time."""
    import torch
    M, N, K = 512, 528, 4127
    x, w, s = synth.fp8_inputs(M, N, K, seed=22)
    ref = oracle.gemm_scaled(x, w, s)
    for skip in (0, 16, 80):  # whole rows before the operands: 128-aligned starts only when skip*K % 128 == 0
        xb = torch.zeros((skip + M) * K, dtype=torch.uint8, device="cuda")
        wb = torch.zeros((skip + N) * K, dtype=torch.uint8, device="cuda")
        xb[skip * K:].copy_(torch.from_numpy(x.reshape(-1)))
        wb[skip * K:].copy_(torch.from_numpy(w.reshape(-1)))
        sd = torch.from_numpy(s).cuda()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        say(f"v20 offsets skip={skip}")
        st = fg.fp8_gemm_scaled(xb.data_ptr() + skip * K, wb.data_ptr() + skip * K, sd.data_ptr(), y.data_ptr(),
                                M, N, K, torch.cuda.current_stream().cuda_stream)
        assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
        torch.cuda.synchronize()
        compare(y.view(torch.int16).cpu().numpy().view(np.uint16), ref, f"skip={skip}")
        aligned = skip * K % 128 == 0
        st = fg.fp8_gemm_scaled_ex(xb.data_ptr() + skip * K, wb.data_ptr() + skip * K, sd.data_ptr(), y.data_ptr(),
                                   M, N, K, fg.PATH_MAIN, 20, 0, torch.cuda.current_stream().cuda_stream)
        if aligned:
            assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
            torch.cuda.synchronize()
            compare(y.view(torch.int16).cpu().numpy().view(np.uint16), ref, f"skip={skip} v20")
        else:  # forced whole-line rows need 128-byte-aligned operands
            assert st == fg.FP8G_ERR_INVALID_ARG and "128-byte" in fg.fp8_gemm_last_error()


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


# ---------------------------------------------------- the benchmark shapes ----
@pytest.mark.parametrize("wl", synth.WORKLOADS, ids=lambda w: w.name)
def test_benchmark_shape(wl):
    """Full size, default plan, every element against the oracle."""
    x, w, s = synth.fp8_inputs(wl.M, wl.N, wl.K, seed=42)
    plan = fg.fp8_gemm_plan(wl.M, wl.N, wl.K)
    say(f"{wl.name} default plan {plan}")
    got = run(x, w, s)
    diag = compare(got, oracle.gemm_scaled(x, w, s), wl.name)
    say(f"{wl.name}: {diag}")


@pytest.mark.parametrize("seed", [123, 456])
@pytest.mark.parametrize("name", ["square-256", "decode-m32", "odd-k-4127"])
def test_benchmark_shape_other_seeds(name, seed):
    wl = synth.WORKLOAD_BY_NAME[name]
    x, w, s = synth.fp8_inputs(wl.M, wl.N, wl.K, seed=seed)
    say(f"{name} seed={seed}")
    compare(run(x, w, s), oracle.gemm_scaled(x, w, s), f"{name} seed={seed}")


# ------------------------------------------------- odd K, rows read in place ----
def test_odd_k_no_workspace_plan():
    """The odd-K benchmark shape runs one kernel on the operand rows as they
    lie: no workspace, nothing copied."""
    p = fg.fp8_gemm_plan(4096, 4096, 4127)
    assert p["path_name"] == "main" and p["workspace_bytes"] == 0 and p["k_tail"] == 1


def test_odd_k_unaligned_pointers():
    """Operand pointers at odd byte addresses with an odd K on 256 x 256 tiles,
    every element."""
    import torch
    M, N, K = 2304, 2560, 3001
    x, w, s = synth.fp8_inputs(M, N, K, seed=10)
    xb = torch.zeros(M * K + 3, dtype=torch.uint8, device="cuda")
    wb = torch.zeros(N * K + 5, dtype=torch.uint8, device="cuda")
    xb[3:].copy_(torch.from_numpy(x.reshape(-1)))
    wb[5:].copy_(torch.from_numpy(w.reshape(-1)))
    sd = torch.from_numpy(s).cuda()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("odd K with unaligned operand pointers")
    st = fg.fp8_gemm_scaled(xb.data_ptr() + 3, wb.data_ptr() + 5, sd.data_ptr(), y.data_ptr(), M, N, K,
                            torch.cuda.current_stream().cuda_stream)
    assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    compare(got, oracle.gemm_scaled(x, w, s), "unaligned odd K")
