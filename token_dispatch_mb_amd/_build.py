"""Compile libmoebal.so in place with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoebal.so")
# reference kernels bounding the dispatch (a measurement library of its own)
CEILING_LIB = os.path.join(HERE, "libmoebal_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments arrive preloaded in SGPRs (gfx940+), saving each
    # latency-bound plan kernel its first scalar-memory round trip
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build_library(verbose: bool = False, extra: list[str] | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=ROOT)
    os.replace(tmp, LIB)
    return LIB


def build_ceiling(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = CEILING_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "ceiling", "ceiling.hip"), "-o", tmp]
    if verbose:
        print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=ROOT)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    build_library(verbose=True)
    build_ceiling(verbose=True)
