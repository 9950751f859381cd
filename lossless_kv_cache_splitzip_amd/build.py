"""Build libsplitzip.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "splitzip.hip"), os.path.join(HERE, "csrc", "pipeline.hip"),
        os.path.join(HERE, "csrc", "calibrate.hip")]
LIB = os.path.join(HERE, "libsplitzip.so")
# the benchmark's copy / read ceiling kernels, a library of their own
CEILING_SRC = os.path.join(HERE, "csrc", "copy_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libszceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(srcs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(SRCS, LIB, verbose)
    _compile([CEILING_SRC], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
