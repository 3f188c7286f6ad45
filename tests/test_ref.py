"""libfp8g_ref.so, the reference kernels bench.py times beside the GEMM:
host-side argument checks (no GPU); on the GPU, that every HBM stream reads
every word of the weight exactly once (XOR checksum) and that the MFMA loop
runs its rounds (its sums scale with the round count)."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "fp8_gemm_channel_amd", "libfp8g_ref.so")
MODES = (0, 1, 2)


def load():
    if not os.path.exists(PATH):
        pytest.fail(f"{PATH} is missing: python fp8_gemm_channel_amd/build.py --ref")
    lib = ctypes.CDLL(PATH)
    lib.fp8g_stream_out_words.restype = ctypes.c_longlong
    lib.fp8g_stream_out_words.argtypes = [ctypes.c_int] * 3
    lib.fp8g_stream_launch.restype = ctypes.c_int
    lib.fp8g_stream_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    lib.fp8g_mfma_ref_launch.restype = ctypes.c_int
    lib.fp8g_mfma_ref_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint] + [ctypes.c_void_p] * 3
    return lib


def test_output_sizes_and_rejected_shapes():
    lib = load()
    assert lib.fp8g_stream_out_words(0, 12288, 4096) == 256 * 512
    assert lib.fp8g_stream_out_words(1, 480, 1024) == 20 * 512
    assert lib.fp8g_stream_out_words(2, 480, 1024) == 1024 * 256
    assert lib.fp8g_stream_out_words(7, 480, 1024) == -2
    # shapes the streams do not take are refused before any HIP call
    for n, k in ((0, 1024), (47, 1024), (480, 1000), (480, 0), (48 * 1024, 1 << 21)):
        for m in MODES:
            assert lib.fp8g_stream_launch(m, None, n, k, None, None, None, None) == -1, (m, n, k)
    for grid, iters in ((0, 10), (65537, 10), (16, 0), (16, 1000001)):
        assert lib.fp8g_mfma_ref_launch(None, grid, iters, 1, None, None, None) == -1, (grid, iters)


@pytest.mark.gpu
@pytest.mark.parametrize("n,k", [(480, 1024), (12288, 4096), (96, 128)])
def test_streams_read_every_word_once(n, k):
    import torch

    lib = load()
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(n * 7 + k)
    w = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    want = int(np.bitwise_xor.reduce(w.view(np.uint32), axis=None))
    wd = torch.from_numpy(w).to(dev)
    stream = torch.cuda.current_stream(dev)
    for m in MODES:
        out = torch.full((int(lib.fp8g_stream_out_words(m, n, k)),), -1, dtype=torch.int32, device=dev)
        print(f"stream mode {m} on {n} x {k}", flush=True)
        assert lib.fp8g_stream_launch(m, wd.data_ptr(), n, k, out.data_ptr(), stream.cuda_stream, None, None) == 0
        torch.cuda.synchronize()
        got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32), axis=None))
        assert got == want, (m, hex(got), hex(want))


@pytest.mark.gpu
def test_mfma_loop_sums_scale_with_rounds():
    """Every accumulator gets the same products each round, so the per-thread
    sums after 2r rounds are twice those after r rounds (to fp32 rounding)."""
    import torch

    lib = load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    sums = []
    for iters in (3, 6):
        out = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device=dev)
        print(f"mfma loop, 8 workgroups, {iters} rounds", flush=True)
        assert lib.fp8g_mfma_ref_launch(out.data_ptr(), 8, iters, 7, stream.cuda_stream, None, None) == 0
        torch.cuda.synchronize()
        sums.append(out.cpu().numpy().astype(np.float64))
    a, b = sums
    assert np.isfinite(a).all() and np.isfinite(b).all()
    assert np.abs(a).max() > 0
    np.testing.assert_allclose(b, 2 * a, rtol=1e-4, atol=1e-3 * np.abs(a).max())
