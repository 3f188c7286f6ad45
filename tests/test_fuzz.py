"""Seeded random shapes and forced plans, each checked against the oracle
element by element: every path, every kernel variant the planner accepts for
the shape, random K splits and stream-K group counts, ragged tile edges and K
tails.  The draw is fixed (seed 2024), so a failure names a reproducible case."""
import numpy as np
import pytest

import fp8_gemm_channel_amd as fg
import oracle
import synth
from tests.gpu_util import compare, run, say

pytestmark = pytest.mark.gpu

MAIN_VARIANTS = [0, 3, 10, 16, 17, 18, 19, 20, 27]
SPLITK_VARIANTS = [0, 1, 2, 3, 4, 5, 21, 22, 23, 24]


def _draw_plan(rng, M, N, K):
    """A valid forced plan for the shape (path, variant, split_k), drawn until
    the planner accepts it; split-K for M <= 128 in 60% of the draws."""
    splitk = M <= 128 and rng.random() < 0.6
    for _ in range(200):
        if splitk:
            path, variant = fg.PATH_SPLITK, int(rng.choice(SPLITK_VARIANTS))
            split_k = int(rng.choice([0, 1, 2, 3, 5, 8]))
        else:
            path, variant = fg.PATH_MAIN, int(rng.choice(MAIN_VARIANTS))
            split_k = int(rng.integers(1, 40)) if variant == 16 and rng.random() < 0.7 else 0
        try:
            fg.fp8_gemm_plan_ex(M, N, K, path, variant, split_k)
            return path, variant, split_k
        except fg.Fp8gError:
            continue
    return 0, 0, 0


def _cases(count=300, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.integers(1, 129)) if rng.random() < 0.45 else int(rng.integers(129, 700))
        N = int(rng.integers(1, 700))
        K = int(rng.choice([rng.integers(1, 300), rng.integers(300, 5000)]))
        out.append((M, N, K, *_draw_plan(rng, M, N, K), int(rng.integers(0, 2**31))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M{}N{}K{}p{}v{}s{}".format(*c[:6]))
def test_fuzz_forced_plans(case):
    M, N, K, path, variant, split_k, seed = case
    x, w, s = synth.fp8_inputs(M, N, K, seed=seed)
    plan = fg.fp8_gemm_plan_ex(M, N, K, path, variant, split_k)
    say(f"fuzz M={M} N={N} K={K} path={path} variant={variant} split_k={split_k} -> {plan}")
    compare(run(x, w, s, path=path, variant=variant, split_k=split_k), oracle.gemm_scaled(x, w, s),
            f"fuzz {case}")
