"""Resource guard for the streaming kernels (CPU only: hipcc cross-compiles
for gfx950).  The encode and decode kernels are bound by their HBM streams
and measured fastest with eight 256-thread workgroups per CU; fewer
workgroups per CU, or register spills to scratch memory, cost them 1-10%.
This test compiles the library's kernels the way the build does and fails
if a streaming kernel needs scratch memory or falls below 8 waves per SIMD,
or if any other kernel of the library spills to scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lossless_kv_cache_splitzip_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

STREAMING = [
    "encode_dense_bf16_kernel", "encode_dense_e5m2_kernel",
    "decode_bf16_kernel", "decode_e5m2_kernel",
    "calib_hist_kernel",
]


def _resources(source: str):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-c", "-o", os.devnull,
           os.path.join(SRC, source), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600).stderr
    res, name = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            res[name] = {}
            continue
        m = re.search(r"(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\d+)",
                      line)
        if m and name:
            res[name][m.group(1).split()[0]] = int(m.group(2))
    return res


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_streaming_kernels_keep_full_occupancy_and_no_scratch():
    res = {}
    for source in ("splitzip.hip", "calibrate.hip"):
        res.update(_resources(source))
    assert res, "no kernel resource report from hipcc"
    for kernel in STREAMING:
        hits = [v for k, v in res.items() if kernel in k]
        assert hits, f"{kernel}: not found in the resource report"
        r = hits[0]
        print(kernel, r, flush=True)
        assert r.get("ScratchSize", 0) == 0, f"{kernel} spills to scratch: {r}"
        assert r.get("Occupancy") == 8, f"{kernel} runs below 8 waves per SIMD: {r}"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_kernel_spills_to_scratch():
    res = {}
    for source in ("splitzip.hip", "calibrate.hip", "pipeline.hip", "copy_ceiling.hip"):
        res.update(_resources(source))
    assert len(res) >= 20, sorted(res)
    assert any("encode_single_bf16_kernel" in k for k in res) and any("encode_single_e5m2_kernel" in k for k in res)
    for kernel, r in res.items():
        assert r.get("ScratchSize", 0) == 0, f"{kernel} spills to scratch: {r}"
