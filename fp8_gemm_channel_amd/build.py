"""Build libfp8g.so (the HIP library behind include/fp8g.h) in-tree for gfx950.

    python -m fp8_gemm_channel_amd.build [--verbose]

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
SOURCES = [os.path.join(CSRC, "fp8g_api.cpp"), os.path.join(CSRC, "fp8g_kernels.hip")]

# Packed-fp32 VALU instructions are kept out of every device build.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # Known-harmless diagnostics: the host pass does not know the packed-fp32
    # feature, and m0 is clobbered on purpose by the LDS-DMA asm.
    noise = ("packed-fp32-ops", "clobber list contains reserved registers: m0",
             "Reserved registers on the clobber list", "warnings generated", "asm volatile(",
             "^", "| ")
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if not any(n in l for n in noise) and not l.strip().startswith(("9", "|")))
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
