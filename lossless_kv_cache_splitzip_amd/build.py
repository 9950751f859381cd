"""Build libsplitzip.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "splitzip.hip"), os.path.join(HERE, "csrc", "pipeline.hip"),
        os.path.join(HERE, "csrc", "calibrate.hip")]
LIB = os.path.join(HERE, "libsplitzip.so")
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


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
