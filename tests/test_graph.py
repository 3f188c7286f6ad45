"""HIP graph capture of the entry points (GPU).

Callers that replay work through graphs capture a call once and replay it.
Every path that uses a workspace is captured here: split-K with several
slices (partials and call-id tickets: the ticket words must not need zeroing
between replays) and stream-K, plus main-path calls with a K tail (one on the
whole-line odd-K kernel, which uses scratch memory for two spilled registers).  Each graph is replayed several times with the program's own eager
work (a different GEMM, a synchronisation) in between, and every replay is
compared with the eager result bit for bit, after the inputs were rewritten in
place, so that a replay that reused stale data would show.
"""
import numpy as np
import pytest
import torch

import fp8_gemm_channel_amd as fg
import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

CASES = [
    ("splitk-S4", (32, 1000, 4127), dict(path=fg.PATH_SPLITK, split_k=4)),
    ("splitk-S8-bias-silu", (17, 777, 3000), dict(path=fg.PATH_SPLITK, split_k=8)),
    ("main-odd-k", (700, 520, 3001), dict(path=fg.PATH_MAIN, variant=10)),
    # the default odd-K kernel (rows as whole cache lines; it keeps two spilled
    # registers in scratch memory), edge tiles in both dimensions
    ("main-odd-k-lines", (528, 304, 3001), dict(path=fg.PATH_MAIN, variant=20)),
    ("stream-k", (513, 520, 1000), dict(path=fg.PATH_MAIN, variant=16, split_k=40)),
    ("main-v18-gelu", (300, 520, 1000), dict(path=fg.PATH_MAIN, variant=18)),
]


@pytest.mark.parametrize("name,shape,kw", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, shape, kw):
    M, N, K = shape
    act = fg.ACT_SILU if "silu" in name else fg.ACT_GELU_TANH if "gelu" in name else fg.ACT_NONE
    x, w, s = synth.fp8_inputs(M, N, K, seed=77)
    xd, wd, sd = (torch.from_numpy(a).cuda() for a in (x, w, s))
    bd = torch.from_numpy(synth.bias_values(N, 77)).cuda() if act != fg.ACT_NONE else None
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    other = synth.fp8_inputs(64, 96, 333, seed=78)
    od = [torch.from_numpy(a).cuda() for a in other]

    def call():
        fg.fp8_gemm(xd, wd, sd, bias=bd, act=act, out=out, **kw)

    say(f"graph {name}: eager")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    eager = out.clone()

    say(f"graph {name}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        # rewrite the inputs in place (same values: the expected output stays the
        # eager one) and clear the output, then do unrelated eager work
        xd.copy_(torch.from_numpy(x))
        wd.copy_(torch.from_numpy(w))
        out.view(torch.int16).fill_(-1)
        fg.fp8_gemm(*od)
        torch.cuda.synchronize()
        say(f"graph {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs from eager"

    # a changed input must change the replayed output (the graph reads live data)
    wd.copy_(torch.from_numpy(np.ascontiguousarray(w[::-1])))
    g.replay()
    torch.cuda.synchronize()
    assert not torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay ignored the new weights"
    del g
