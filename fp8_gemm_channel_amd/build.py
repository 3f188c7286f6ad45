"""Build libfp8g.so (the HIP library behind include/fp8g.h) in-tree for gfx950.

    python fp8_gemm_channel_amd/build.py [--verbose] [--lds-poison]

--lds-poison builds the debug library libfp8g_lds_poison.so instead: every
LDS-DMA is preceded by a NaN fill of its destination (FP8G_LDS_POISON), so a
read that runs ahead of its DMA shows up as NaN outputs.  Load it by setting
FP8G_LIBRARY to its path before importing the package.

--ref builds libfp8g_ref.so instead: the reference kernels (HBM streams and
an MFMA loop) that bench.py times beside the GEMM (csrc/fp8g_ref.hip; no part
of the GEMM interface).

(run as a file: importing the package loads the library this builds)

hipcc cross-compiles the device code for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libfp8g.so")
POISON_LIBRARY = os.path.join(PKG, "libfp8g_lds_poison.so")
REF_LIBRARY = os.path.join(PKG, "libfp8g_ref.so")
REF_SOURCE = os.path.join(CSRC, "fp8g_ref.hip")
SOURCES = [os.path.join(CSRC, f) for f in ("fp8g_api.cpp", "fp8g_kernels.hip", "fp8g_noalloc.hip")] + sorted(
    os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.startswith("fp8g_launch_") and f.endswith(".hip"))

# Packed-fp32 VALU instructions are kept out of every device build.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Known-harmless diagnostics: the host pass does not know the packed-fp32
# feature, and m0 is clobbered on purpose by the LDS-DMA asm.
_NOISE = ("packed-fp32-ops", "clobber list contains reserved registers: m0",
          "Reserved registers on the clobber list", "warnings generated", "asm volatile(",
          "^", "| ", "In file included from")


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines()
                     if not any(n in l for n in _NOISE) and not l.strip().startswith(("9", "|")))


def build(verbose: bool = False, jobs: int = 0, lds_poison: bool = False) -> str:
    """Compile every translation unit (in parallel) and link libfp8g.so in-tree
    (or, with lds_poison, the debug library libfp8g_lds_poison.so)."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    target = POISON_LIBRARY if lds_poison else LIBRARY
    tag = ".tmp%d%s" % (os.getpid(), "p" if lds_poison else "")
    objs = [os.path.join(CSRC, os.path.basename(src) + tag + ".o") for src in SOURCES]
    defines = ["-DFP8G_LDS_POISON"] if lds_poison else []

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc, *HIPCC_FLAGS, *defines, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True)

    jobs = jobs or min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0") or 0) or os.cpu_count() or 1)
    tmp = target + tag
    try:
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(compile_one, zip(SOURCES, objs)))
        for src, res in zip(SOURCES, results):
            out = _filter(res.stdout + res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + out)
            if verbose and out.strip():
                print(out)
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + _filter(res.stdout + res.stderr))
        os.replace(tmp, target)
    finally:
        for f in objs + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return target


def build_ref(verbose: bool = False) -> str:
    """Compile and link libfp8g_ref.so (the reference kernels) in-tree."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = REF_LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, REF_SOURCE]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = _filter(res.stdout + res.stderr)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on fp8g_ref.hip:\n" + out)
        if verbose and out.strip():
            print(out)
        os.replace(tmp, REF_LIBRARY)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return REF_LIBRARY


if __name__ == "__main__":
    if "--ref" in sys.argv:
        print(build_ref(verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv, lds_poison="--lds-poison" in sys.argv))
