"""The CPU oracle and the host code of libsplitzip built with AddressSanitizer
and UndefinedBehaviorSanitizer (no recovery: the first report ends the
process), and the CPU tests that exercise them run against those builds in a
child process:

* the oracle (gcc) under the oracle's pins and the ablation variants' pins;
* libsplitzip's host code (hipcc, instrumentation on the host pass only:
  -Xarch_host before each sanitizer flag) under the host-side ABI tests
  (calibration, size queries, argument errors returned before any GPU work).

Every parity verdict rests on the oracle, and the ABI's argument checks guard
the GPU, so both must be free of memory errors and undefined behaviour.
Builds go to _build/sanitize (not part of the product)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run_child(preload: str, code: str, args):
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:], flush=True)
    assert "ERROR: AddressSanitizer" not in out, "AddressSanitizer report"
    assert "runtime error:" not in out and "UndefinedBehaviorSanitizer" not in out, "UndefinedBehaviorSanitizer report"
    assert r.returncode == 0, f"child exited with {r.returncode}"
    return out


def test_oracle_pins_under_asan_and_ubsan():
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(gcc_asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    os.makedirs(BUILD, exist_ok=True)
    lib = os.path.join(BUILD, "libsplitzip_oracle.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-shared", "-fPIC", "-o", lib,
                           os.path.join(ROOT, "oracle", "splitzip_oracle.c")])
    code = ("import sys, pytest, oracle\n"
            "oracle.use_library(sys.argv[1])\n"
            "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
            "                      'tests/test_oracle_pins.py', 'tests/test_oracle_variants.py']))\n")
    out = _run_child(gcc_asan, code, [lib])
    assert " passed" in out


def test_host_abi_under_asan_and_ubsan():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    os.makedirs(BUILD, exist_ok=True)
    lib = os.path.join(BUILD, "libsplitzip.so")
    src = os.path.join(ROOT, "lossless_kv_cache_splitzip_amd", "csrc")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                           "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                           "-Xarch_host", "-shared-libsan", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-o", lib,
                           os.path.join(src, "splitzip.hip"), os.path.join(src, "pipeline.hip"),
                           os.path.join(src, "calibrate.hip")])
    code = ("import sys, pytest\n"
            "import lossless_kv_cache_splitzip_amd._native as N\n"
            "N.LIB_PATH = sys.argv[1]\n"
            "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi_cpu.py']))\n")
    out = _run_child(rt[-1], code, [lib])
    assert " passed" in out
