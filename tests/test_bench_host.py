"""bench.py's host logic, on the CPU: the roofline of each benchmark shape, the
rule that committed profile summaries count only for the kernel sources they
were taken on, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("wl", synth.WORKLOADS, ids=lambda w: w.name)
def test_roofline_of_benchmark_shapes(wl):
    """t_roof = max(FLOPs / 5.0 PFLOP/s, bytes / 8.0 TB/s), the bound the larger term."""
    flops = 2.0 * wl.M * wl.N * wl.K
    nbytes = wl.M * wl.K + wl.N * wl.K + 4 * wl.N + 2 * wl.M * wl.N
    assert wl.flops == flops and wl.bytes == nbytes
    t_mfma, t_hbm = flops / 5.0e15, nbytes / 8.0e12
    assert bench.roof_seconds(wl) == pytest.approx(max(t_mfma, t_hbm), rel=1e-12)
    assert bench.bound_of(wl) == ("mfma" if t_mfma >= t_hbm else "hbm")


def test_bounds_of_the_five_shapes():
    bounds = {w.name: bench.bound_of(w) for w in synth.WORKLOADS}
    assert bounds == {"square-256": "hbm", "square-4096": "mfma", "decode-m32": "hbm",
                      "odd-k-4127": "mfma", "square-8192": "mfma"}
    # 8192^3 at 5.0 PFLOP/s: 219.9 us
    assert bench.roof_seconds(synth.WORKLOAD_BY_NAME["square-8192"]) == pytest.approx(219.902e-6, rel=1e-4)


def test_profile_summaries_count_only_for_their_sources(monkeypatch, tmp_path):
    trace = tmp_path / "trace.md"
    traffic = tmp_path / "traffic.md"
    trace.write_text("- kernel_source_sha256: `abc`\n- avg_us_square-8192: `351.41`\n")
    traffic.write_text("- workload: `square-8192`\n- kernel_source_sha256: `abc`\n"
                       "- hbm_bytes_per_launch: `940716552`\n")
    monkeypatch.setattr(bench, "TRACE_SUMMARY", str(trace))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(traffic))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.traced_launch_us("square-8192") == pytest.approx(351.41)
    assert bench.measured_traffic("square-8192") == 940716552
    assert bench.measured_traffic("square-4096") is None        # another workload
    assert bench.traced_launch_us("odd-k-4127") is None          # not in the summary
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def")
    assert bench.traced_launch_us("square-8192") is None         # other sources
    assert bench.measured_traffic("square-8192") is None
    monkeypatch.setattr(bench, "TRACE_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.traced_launch_us("square-8192") is None


def test_kernel_source_hash_covers_the_dominant_kernel():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and int(h, 16) >= 0
    names = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    assert names == {"fp8g_kernels.hpp", "fp8g_launch_main4w.hip"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
