"""Build libgdn.so (the HIP library behind include/gdn.h) for gfx950 in-tree.

    python -m chunked_gated_delta_05_amd.build [-v]

hipcc compiles the kernels and the host API into one shared library next to
this file. Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_host.cpp"),
           os.path.join(CSRC, "gdn_noalloc.hip"), os.path.join(CSRC, "gdn_bwd.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


BUILD = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    warn = ["-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
    kobj = os.path.join(BUILD, "gdn_kernels.o")
    hobj = os.path.join(BUILD, "gdn_host.o")
    nobj = os.path.join(BUILD, "gdn_noalloc.o")
    bobj = os.path.join(BUILD, "gdn_bwd.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in ordinary VGPRs: the state update scales them
          # with VALU ops every chunk, which AGPR accumulators turn into copies
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          *warn, *inc, "-c", SOURCES[0], "-o", kobj], verbose)
    _run([HIPCC, "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", *warn, *inc, "-I", "/opt/rocm/include",
          "-x", "c++", "-c", SOURCES[1], "-o", hobj], verbose)
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          *warn, *inc, "-c", SOURCES[2], "-o", nobj], verbose)
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          *warn, *inc, "-c", SOURCES[3], "-o", bobj], verbose)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", kobj, hobj, nobj, bobj, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
