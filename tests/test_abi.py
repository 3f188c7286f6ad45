"""The C-ABI library: it loads, exports what include/fp8g.h declares, plans the
five benchmark shapes as intended and rejects bad arguments before any HIP
call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import fp8_gemm_channel_amd as fg
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fp8g.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_gemm_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fg.LIBRARY)
    names = declared_functions()
    assert names, "no declarations found"
    assert set(names) == set(fg.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/fp8g.h but not exported"


def test_strerror_is_static_and_total():
    assert fg.fp8_gemm_strerror(0) == "success"
    assert fg.fp8_gemm_strerror(1) == "invalid argument"
    assert fg.fp8_gemm_strerror(3) == "HIP runtime error"
    assert fg.fp8_gemm_strerror(12345) == "unknown status"


def _splitk_workspace(p, M, N):
    # one 128-byte ticket line per column tile, padded to 256 bytes, then fp32
    # partials [column tile][split_k][M][tile_n]
    tiles = -(-N // p["tile_n"])
    return -(-tiles * 128 // 256) * 256 + tiles * p["split_k"] * M * p["tile_n"] * 4


@pytest.mark.parametrize("wl", synth.WORKLOADS, ids=lambda w: w.name)
def test_plan_of_benchmark_shapes(wl):
    p = fg.fp8_gemm_plan(wl.M, wl.N, wl.K)
    if wl.M <= 128:
        assert p["path_name"] == "splitk"
        assert p["split_k"] >= 1 and p["k_slice"] * p["split_k"] >= wl.K
        assert (p["split_k"] - 1) * p["k_slice"] < wl.K, "no empty slice"
        assert p["k_slice"] % 128 == 0
        assert p["workspace_bytes"] == (_splitk_workspace(p, wl.M, wl.N) if p["split_k"] > 1 else 0)
    else:
        assert p["path_name"] == "main"
        assert p["grid"] == -(-wl.M // p["tile_m"]) * -(-wl.N // p["tile_n"])
        assert p["k_tail"] == (wl.K % p["tile_k"] != 0)
        assert p["workspace_bytes"] == 0, "the main path copies nothing"
    if wl.M >= 4096:
        assert (p["tile_m"], p["tile_n"]) == (256, 256) and p["grid"] >= 256
    if wl.name == "odd-k-4127":
        assert p["k_tail"] == 1


def test_plan_special_extents():
    assert fg.fp8_gemm_plan(0, 5, 7)["path_name"] == "none"
    assert fg.fp8_gemm_plan(5, 0, 7)["path_name"] == "none"
    assert fg.fp8_gemm_plan(5, 6, 0)["path_name"] == "zero"
    p = fg.fp8_gemm_plan(1, 1, 1)
    assert p["path_name"] == "splitk" and p["split_k"] == 1 and p["k_tail"] == 1
    p = fg.fp8_gemm_plan(129, 1, 1)
    assert p["path_name"] == "main" and p["k_tail"] == 1
    assert fg.fp8_gemm_plan(128, 1, 1)["path_name"] == "splitk"


def test_plan_overrides():
    p = fg.fp8_gemm_plan_ex(32, 12288, 4096, fg.PATH_SPLITK, 1, 4)
    assert p["split_k"] == 4 and p["k_slice"] == 1024
    assert p["workspace_bytes"] == _splitk_workspace(p, 32, 12288)
    p = fg.fp8_gemm_plan_ex(32, 4096, 4096, fg.PATH_MAIN, 18, 0)
    assert p["path_name"] == "main" and p["tile_m"] == 128
    # split_k larger than the number of 128-byte chunks collapses to non-empty slices
    p = fg.fp8_gemm_plan_ex(8, 100, 300, fg.PATH_SPLITK, 0, 8)
    assert p["split_k"] == 3 and p["k_slice"] == 128
    # 8-wave LDS-ring variants: 16 * (variant - 20) w rows, fewer rows for wider x
    p = fg.fp8_gemm_plan_ex(32, 12288, 4096, fg.PATH_SPLITK, 23, 1)
    assert p["variant"] == 23 and p["tile_n"] == 48 and p["grid"] == 256 and p["workspace_bytes"] == 0
    assert fg.fp8_gemm_plan_ex(16, 1000, 4096, fg.PATH_SPLITK, 24, 0)["tile_n"] == 64
    assert fg.fp8_gemm_plan_ex(64, 1000, 4096, fg.PATH_SPLITK, 21, 0)["tile_m"] == 64


# Split-K picks of the planner on shapes measured on MI355X (cold, events attached to
# the kernel); each is the best or within 9% of the best of every (variant, S) tried.
@pytest.mark.parametrize("shape,pick", [
    ((32, 12288, 4096), (23, 1)),   # decode: 48 rows, 8 waves, 256 workgroups
    ((1, 12288, 4096), (24, 1)),    # 64 rows when x is at most 16 rows
    ((32, 1536, 4096), (21, 1)),    # few columns and short K: no K split (96 workgroups)
    ((8, 1024, 28672), (21, 4)),    # few columns, long K: 4 slices of 7 KiB
    ((16, 4096, 16384), (24, 4)),
    ((32, 8192, 8192), (23, 1)),
    ((64, 12288, 4096), (2, 1)),    # 64 x rows: 4-wave kernel, 32 w rows
    ((64, 1536, 4096), (1, 2)),
    ((64, 1024, 28672), (1, 4)),
    ((64, 7168, 2048), (2, 1)),     # 32 rows reach 160 workgroups: 16 rows would re-read x twice as often
])
def test_plan_splitk_rule(shape, pick):
    p = fg.fp8_gemm_plan(*shape)
    assert p["path_name"] == "splitk" and (p["variant"], p["split_k"]) == pick


@pytest.mark.parametrize("M", [1, 16, 17, 32, 33, 64, 65, 128])
@pytest.mark.parametrize("N", [1, 100, 4096, 65536])
@pytest.mark.parametrize("K", [1, 4127, 100000])
def test_plan_splitk_invariants(M, N, K):
    """Every automatic split-K plan: a kernel that exists for this M, slices of
    whole 128-byte chunks covering K with none empty, and a grid of column tiles
    times slices."""
    p = fg.fp8_gemm_plan(M, N, K)
    v, S = p["variant"], p["split_k"]
    assert (v in (21, 22, 23, 24)) if M <= 32 else (v in (1, 2))
    assert p["tile_n"] == 16 * (v - 20 if v > 20 else v)
    assert p["k_slice"] % 128 == 0 and (S - 1) * p["k_slice"] < K <= S * p["k_slice"]
    assert p["grid"] == -(-N // p["tile_n"]) * S
    assert p["workspace_bytes"] == (_splitk_workspace(p, M, N) if S > 1 else 0)


@pytest.mark.parametrize("args", [
    (-1, 4, 4), (4, -1, 4), (4, 4, -1), (4, 4, (1 << 24)), (2**31, 4, 4), (4, 2**30, 4), (2**30, 4, 4),
])
def test_plan_rejects_bad_dims(args):
    with pytest.raises(fg.Fp8gError) as e:
        fg.fp8_gemm_plan(*args)
    assert e.value.status == fg.FP8G_ERR_INVALID_ARG


def test_plan_limits():
    """The largest M and N are accepted where the launch fits the grid limit;
    a launch of 2^32 work-items or more is refused as unsupported."""
    big = 2**30 - 1
    p = fg.fp8_gemm_plan(big, 256, 128)
    assert p["path_name"] == "main" and p["grid"] * 512 < 2**32
    with pytest.raises(fg.Fp8gError) as e:
        fg.fp8_gemm_plan(1, big, 128)          # 2^26 split-K workgroups of 256+ threads
    assert e.value.status == fg.FP8G_ERR_UNSUPPORTED
    with pytest.raises(fg.Fp8gError) as e:
        fg.fp8_gemm_plan(big, big, 128)        # too many tiles
    assert e.value.status == fg.FP8G_ERR_UNSUPPORTED


def test_plan_odd_k_reads_rows_in_place():
    """K % 128 != 0: no copy and no workspace on any path; the last K step is
    masked in the kernel."""
    for shape in [(4096, 4096, 4127), (4096, 4096, 4112), (256, 256, 257), (2048, 2048, 2049),
                  (32, 12288, 4127), (8192, 8192, 8191)]:
        p = fg.fp8_gemm_plan(*shape)
        assert p["workspace_bytes"] == 0 and p["k_tail"] == 1, (shape, p)
    assert fg.fp8_gemm_plan(4096, 4096, 4096)["k_tail"] == 0
    # the main path takes no split_k outside stream-K
    for sk in (1, 2):
        with pytest.raises(fg.Fp8gError):
            fg.fp8_gemm_plan_ex(4096, 4096, 4127, fg.PATH_MAIN, 0, sk)


def test_plan_main_kernel_choice():
    """256 x 256 tiles without a K tail run on the one-wave-per-SIMD kernel
    (variant 19); odd K on its whole-line form (variant 20) where M K and N K
    are multiples of 16; other K tails on the eight-wave kernel (variant 10)."""
    assert fg.fp8_gemm_plan(8192, 8192, 8192)["variant"] == 19
    assert fg.fp8_gemm_plan(4096, 4096, 4096)["variant"] == 19      # 256 tiles
    odd = fg.fp8_gemm_plan(4096, 4096, 4127)                           # rows read in place
    assert odd["variant"] == 20 and odd["k_tail"] == 1 and odd["workspace_bytes"] == 0
    assert fg.fp8_gemm_plan(4104, 4096, 4127)["variant"] == 10         # M K not a multiple of 16
    assert fg.fp8_gemm_plan(4096, 4096, 4128)["variant"] == 10         # even K
    # the whole-line variant (opt-in) needs odd K and M K, N K multiples of 16
    assert fg.fp8_gemm_plan_ex(4096, 4096, 4127, fg.PATH_MAIN, 20, 0)["variant"] == 20
    assert fg.fp8_gemm_plan_ex(48, 560, 3001, fg.PATH_MAIN, 20, 0)["variant"] == 20
    for shape in [(4097, 4096, 4127), (4096, 4104, 4127), (4096, 4104, 4128), (256, 256, 1000), (256, 256, 4096),
                  (256, 256, 127), (256, 512, 17), (16, 16, 1)]:
        with pytest.raises(fg.Fp8gError):
            fg.fp8_gemm_plan_ex(*shape, fg.PATH_MAIN, 20, 0)
    # one K step (odd K up to 127) runs on the eight-wave kernel
    assert fg.fp8_gemm_plan(4096, 4096, 127)["variant"] == 10
    assert fg.fp8_gemm_plan(4096, 4096, 129)["variant"] == 20
    assert fg.fp8_gemm_plan(3072, 3072, 3072)["variant"] == 19      # 144 tiles
    # tiny problems (at most 256 blocks of 16 x 16, K <= 256, K % 16 == 0): register tiles
    tiny = fg.fp8_gemm_plan(256, 256, 256)
    assert tiny["variant"] == 27 and (tiny["tile_m"], tiny["tile_n"], tiny["grid"]) == (16, 16, 256)
    assert fg.fp8_gemm_plan(240, 240, 256)["variant"] == 27
    for shape in [(256, 256, 384), (320, 320, 256), (256, 256, 255)]:
        assert fg.fp8_gemm_plan(*shape)["variant"] == 3, shape
    with pytest.raises(fg.Fp8gError):
        fg.fp8_gemm_plan_ex(256, 256, 255, fg.PATH_MAIN, 27, 0)     # K % 16 != 0
    forced = fg.fp8_gemm_plan_ex(300, 300, 384, fg.PATH_MAIN, 19, 0)
    assert forced["variant"] == 19 and forced["grid"] == 4 and forced["tile_k"] == 128
    assert fg.fp8_gemm_plan_ex(4096, 4096, 4096, fg.PATH_MAIN, 10, 0)["variant"] == 10
    # variant 19 has no K tail
    with pytest.raises(fg.Fp8gError):
        fg.fp8_gemm_plan_ex(256, 256, 257, fg.PATH_MAIN, 19, 0)


@pytest.mark.parametrize("kw", [
    dict(path=7), dict(variant=99), dict(split_k=65),
    dict(split_k=-1), dict(path=fg.PATH_MAIN, split_k=1), dict(path=fg.PATH_SPLITK, variant=9),
    dict(path=fg.PATH_MAIN, variant=1), dict(path=fg.PATH_MAIN, variant=6), dict(path=fg.PATH_MAIN, variant=9),
    dict(path=fg.PATH_SPLITK, variant=18), dict(path=fg.PATH_SPLITK, variant=25),
    dict(path=fg.PATH_SPLITK, variant=24), dict(path=fg.PATH_SPLITK, variant=22, M=40),
    dict(path=fg.PATH_SPLITK, M=129), dict(path=fg.PATH_SPLITK, variant=3, M=65),
    dict(path=fg.PATH_SPLITK, variant=21, M=65), dict(path=fg.PATH_SPLITK, variant=11, M=65),
])
def test_plan_rejects_bad_overrides(kw):
    M = kw.pop("M", 32)
    with pytest.raises(fg.Fp8gError) as e:
        fg.fp8_gemm_plan_ex(M, 256, 256, kw.get("path", 0), kw.get("variant", 0), kw.get("split_k", 0))
    assert e.value.status == fg.FP8G_ERR_INVALID_ARG


# Argument checks happen before any HIP call, so these use host addresses that
# are never dereferenced.
FAKE = 1 << 20


@pytest.mark.parametrize("case,detail", [
    (dict(y=0), "y is null"),
    (dict(scale=0), "scale is null"),
    (dict(x=0), "x or w is null"),
    (dict(w=0), "x or w is null"),
    (dict(scale=FAKE * 40 + 2), "4-byte"),
    (dict(y=FAKE * 40 + 1), "2-byte"),
    (dict(y=FAKE * 2), "overlaps"),
    (dict(M=-3), "negative"),
])
def test_scaled_rejects_bad_arguments_without_hip(case, detail):
    a = dict(x=FAKE * 2, w=FAKE * 4, scale=FAKE * 6, y=FAKE * 8, M=16, N=16, K=64)
    a.update(case)
    st = fg.fp8_gemm_scaled(a["x"], a["w"], a["scale"], a["y"], a["M"], a["N"], a["K"], 0)
    assert st == fg.FP8G_ERR_INVALID_ARG
    assert detail in fg.fp8_gemm_last_error()


def test_timed_entry_checks_arguments_like_the_others():
    st = fg.fp8_gemm_scaled_act_timed(FAKE * 2, FAKE * 4, FAKE * 6, 0, 0, 16, 16, 64, stream=0,
                                      start_event=FAKE * 10, stop_event=FAKE * 12)
    assert st == fg.FP8G_ERR_INVALID_ARG and "y is null" in fg.fp8_gemm_last_error()
    st = fg.fp8_gemm_scaled_act_timed(FAKE * 2, FAKE * 4, FAKE * 6, 0, FAKE * 8, 16, 16, 64, activation=9)
    assert st == fg.FP8G_ERR_INVALID_ARG and "activation" in fg.fp8_gemm_last_error()


def test_noalloc_refuses_oversized_workspace_without_hip():
    """The allocation-free entry point checks the plan's workspace against its
    device array before any HIP call."""
    M, N, K, plan = 128, 65536, 4096, (fg.PATH_SPLITK, 0, 8)
    assert fg.fp8_gemm_plan_ex(M, N, K, *plan)["workspace_bytes"] > fg.NOALLOC_SCRATCH_BYTES
    st = fg.fp8_gemm_scaled_noalloc(FAKE * 2, FAKE * 4, FAKE * 6, FAKE * 40, M, N, K, *plan, 0)
    assert st == fg.FP8G_ERR_UNSUPPORTED and "allocation-free" in fg.fp8_gemm_last_error()
    # argument checks come first, as for the other entry points
    st = fg.fp8_gemm_scaled_noalloc(FAKE * 2, FAKE * 4, FAKE * 6, 0, 16, 16, 64, 0, 0, 0, 0)
    assert st == fg.FP8G_ERR_INVALID_ARG


def test_empty_extent_is_a_no_op_even_with_null_pointers():
    assert fg.fp8_gemm_scaled(0, 0, 0, 0, 0, 16, 16, 0) == fg.FP8G_OK
    assert fg.fp8_gemm_scaled(0, 0, 0, 0, 16, 0, 16, 0) == fg.FP8G_OK


def test_no_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this checks the GPU-less error path")
    st = fg.fp8_gemm_scaled(FAKE * 2, FAKE * 4, FAKE * 6, FAKE * 8, 16, 16, 64, 0)
    assert st == fg.FP8G_ERR_HIP
    assert "hipGetDevice" in fg.fp8_gemm_last_error()
