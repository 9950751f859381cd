"""The C ABI used from plain C (tests/c_abi/roundtrip.c, built by
__graft_entry__.build()): hipMalloc'd buffers, the default stream, no Python
or PyTorch in the process. BF16 and E5M2 round trips, the closed-form stream
size, the corrupt-stream status and host-detectable errors, the stream of
splitzip_compress_static (the entry point that allocates nothing) against
splitzip_compress's; then the device calibration against the host one, both
ablation variants, and the chunk-pipelined transfer through pinned host
memory on four streams."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "roundtrip")


def test_plain_c_round_trip():
    assert os.path.exists(EXE), "tests/c_abi/roundtrip is missing: run __graft_entry__.build()"
    print("case plain-C round trip", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stdout.splitlines() if l.startswith("c-abi ok:")]
    assert len(lines) == 5
