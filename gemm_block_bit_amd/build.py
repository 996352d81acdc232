"""Build libgbb.so in-tree: HIP kernels with hipcc for gfx950, host C++ with g++.

Usage: python -m gemm_block_bit_amd.build   (or gemm_block_bit_amd.build.build())
The shared library lands next to this file; objects go to <repo>/_build/.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgbb.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

COMMON = ["-std=c++17", "-fPIC", "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]
# Packed-fp32 instructions are switched off for the device code; the host pass
# of hipcc reports that it does not know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + COMMON
CXX_FLAGS = ["-O2", "-Wall", "-Wextra", "-fno-fast-math"] + COMMON

# graph.cpp is host code on the HIP runtime (stream capture), so hipcc builds it too
HIP_SOURCES = ["decode.hip", "decode64.hip", "prefill.hip", "w48.hip", "debug.hip", "noalloc.hip", "graph.cpp"]
# per-source extra flags: the decode kernel reads its MFMA results with VALU
# code right away, so it keeps them in VGPRs rather than accumulation
# registers; its single-token kernel takes its arguments preloaded into
# scalar registers
HIP_EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
             "decode64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
             # the W4.4A8 kernels scale their int32 MFMA results with VALU code
             # right away too, so they also keep them in VGPRs
             "w48.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CXX_SOURCES = ["pack.cpp", "api.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libgbb.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, s + ".o")
        jobs.append([HIPCC] + HIP_FLAGS + HIP_EXTRA.get(s, []) + ["-c", os.path.join(CSRC, s), "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, s + ".o")
        jobs.append([CXX] + CXX_FLAGS + ["-c", os.path.join(CSRC, s), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
