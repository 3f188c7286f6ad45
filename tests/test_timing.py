"""Events attached to the call's own kernels (fp8_gemm_scaled_act_timed): the
output is the same bits as the untimed call, and the attached window (first
kernel's start to last kernel's end) lies inside a hipEventRecord pair placed
around the same call."""
import numpy as np
import pytest
import torch

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import compare, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ((256, 256, 256), {}),                           # main path, one kernel
    ((32, 1536, 4096), {}),                          # split-K path with in-launch reduction
    ((300, 264, 4127), {}),                          # main path, K tail in place
    ((64, 72, 0), {}),                               # K = 0: the zero kernel
    ((0, 72, 64), {}),                               # no kernel at all
]


def _events():
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:  # create the HIP events before the timed call
        e.record()
    torch.cuda.synchronize()
    return evs


@pytest.mark.parametrize("shape,kw", CASES, ids=lambda c: str(c))
def test_timed_call_matches_untimed_and_nests_in_markers(shape, kw):
    M, N, K = shape
    x, w, s = synth.fp8_inputs(M, N, K, seed=31)
    xd, wd, sd = to_dev(x), to_dev(w), to_dev(s)
    say(f"timed {shape} {kw}")
    ref = fg.fp8_gemm(xd, wd, sd, **kw)
    m0, m1, a0, a1 = _events()
    stream = torch.cuda.current_stream()
    for _ in range(3):
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        m0.record(stream)
        fg.fp8_gemm(xd, wd, sd, out=out, events=(a0, a1), **kw)
        m1.record(stream)
        m1.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        attached, marker = a0.elapsed_time(a1), m0.elapsed_time(m1)
        assert 0.0 <= attached <= marker, (attached, marker)
        if M and N:
            assert attached > 0.0
    if M and N and K:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        compare(got, oracle.gemm_scaled(x, w, s), f"timed {shape}")
