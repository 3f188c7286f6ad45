"""The allocation-free entry point, fp8_gemm_scaled_noalloc, called through
the C ABI: the same plans as fp8_gemm_scaled_ex, with the workspace (split-K
partials and tickets, stream-K partial tiles and tickets) in the library's
per-GPU device array instead of its memory pool.  Each case makes two calls in
a row on one stream, the second on a smaller input, and checks both against
the existing entry point (bit for bit: same kernels, same sums) and against
the oracle (1e-2 + 1e-2 |ref| per element)."""
import numpy as np
import pytest
import torch

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import compare, say, to_dev

pytestmark = pytest.mark.gpu

# (first shape, second smaller shape, forced plan (path, variant, split_k))
CASES = [
    ("splitk-forced", (32, 1000, 4127), (16, 500, 3000), (fg.PATH_SPLITK, 0, 4)),
    ("splitk-default", (8, 1024, 28672), (8, 512, 8192), (0, 0, 0)),
    ("splitk-many-slices", (64, 1536, 4096), (40, 264, 2000), (fg.PATH_SPLITK, 1, 7)),
    ("stream-k", (513, 520, 1000), (300, 300, 384), (fg.PATH_MAIN, 16, 40)),
    ("no-workspace", (256, 256, 256), (64, 72, 100), (0, 0, 0)),
    # the whole-line odd-K kernel: no workspace, two spilled registers in scratch
    ("odd-k-lines", (528, 304, 3001), (272, 288, 641), (fg.PATH_MAIN, 20, 0)),
]


def _inputs(shape, seed):
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=seed)
    return (x, w, s), (to_dev(x), to_dev(w), to_dev(s))


def _launch(entry, dev, shape, plan, stream):
    M, N, K = shape
    xd, wd, sd = dev
    y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")  # 0xFFFF: a NaN, so unwritten elements fail
    st = entry(xd.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), M, N, K, *plan, stream)
    assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
    return y


@pytest.mark.parametrize("name,first,second,plan", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_allocating_entry(name, first, second, plan):
    stream = torch.cuda.current_stream().cuda_stream
    host1, dev1 = _inputs(first, 61)
    host2, dev2 = _inputs(second, 62)
    for shape in (first, second):
        need = fg.fp8_gemm_plan_ex(*shape, *plan)["workspace_bytes"]
        assert need <= fg.NOALLOC_SCRATCH_BYTES, (shape, need)
    say(f"noalloc {name}: {first} then {second}, plan {plan}")
    # two calls in a row on one stream, the second smaller, then the reference calls
    a1 = _launch(fg.fp8_gemm_scaled_noalloc, dev1, first, plan, stream)
    a2 = _launch(fg.fp8_gemm_scaled_noalloc, dev2, second, plan, stream)
    b1 = _launch(fg.fp8_gemm_scaled_ex, dev1, first, plan, stream)
    b2 = _launch(fg.fp8_gemm_scaled_ex, dev2, second, plan, stream)
    torch.cuda.synchronize()
    for got, ref, host, shape in ((a1, b1, host1, first), (a2, b2, host2, second)):
        g = got.cpu().numpy().view(np.uint16)
        r = ref.cpu().numpy().view(np.uint16)
        assert np.array_equal(g, r), f"{name} {shape}: differs from fp8_gemm_scaled_ex"
        compare(g, oracle.gemm_scaled(*host), f"{name} {shape}")


def test_noalloc_allocates_no_device_memory():
    """After a first call (which loads the library's code and its device array
    on this GPU), further calls with a 20 MB workspace leave the device's free
    memory unchanged; the pool-backed entry point would reserve the workspace."""
    stream = torch.cuda.current_stream().cuda_stream
    shape, plan = (513, 520, 1000), (fg.PATH_MAIN, 16, 40)
    assert fg.fp8_gemm_plan_ex(*shape, *plan)["workspace_bytes"] > 20 << 20
    _, dev = _inputs(shape, 63)
    y = torch.empty(shape[:2], dtype=torch.int16, device="cuda")
    def call():
        st = fg.fp8_gemm_scaled_noalloc(dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(), y.data_ptr(),
                                        *shape, *plan, stream)
        assert st == fg.FP8G_OK, fg.fp8_gemm_last_error()
    call()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    say("noalloc: five more calls, free memory watched")
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)


def test_noalloc_refuses_oversized_workspace():
    """A plan whose workspace exceeds the device array is refused before
    anything is enqueued (FP8G_ERR_UNSUPPORTED)."""
    M, N, K, plan = 128, 65536, 4096, (fg.PATH_SPLITK, 0, 8)
    assert fg.fp8_gemm_plan_ex(M, N, K, *plan)["workspace_bytes"] > fg.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    w = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    s = torch.ones(N, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    st = fg.fp8_gemm_scaled_noalloc(x.data_ptr(), w.data_ptr(), s.data_ptr(), y.data_ptr(), M, N, K, *plan,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == fg.FP8G_ERR_UNSUPPORTED
    assert "allocation-free" in fg.fp8_gemm_last_error()
