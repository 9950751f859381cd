"""The decoder's acceptance test equals the oracle's: streams damaged at
random in the chunk-offset table, the escape records and the E / S header
fields, or handed over with fewer bytes than they hold, are rejected by the
GPU (d_status = E_CORRUPT) exactly when the oracle's validation rejects them;
a damaged stream that is still valid (an escape moved to another free
position, an exponent replaced by another in range) decodes to the oracle's
result bit for bit.  Short chunks (the decoder loads all of a chunk's records
in every tile) and long chunks (it searches for the tile's records) are both
covered, for BF16 and E5M2.
"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O
from paritylib import u64

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
DEV = "cuda"


def _gpu_status_and_output(stream: np.ndarray, n: int, dtype: int, in_bytes: int):
    dev = torch.from_numpy(stream).to(DEV)
    y, st = sz.decompress(dev, n, dtype, in_bytes=in_bytes)
    torch.cuda.synchronize()
    return int(st.item()), kvsynth.to_numpy_bits(y)


def _mutations(good: np.ndarray, dtype: int, n: int, rng, count: int):
    """(stream, in_bytes, label) cases, each damaged in one way."""
    sec = O.sections(dtype, n, 1)
    E = u64(good, 16)
    S = good.size
    off0, off1 = sec["offsets"], sec["offsets"] + 8 * (sec["chunks"] + 1)
    esc = sec["esc"]
    for i in range(count):
        t = good.copy()
        kind = i % 6
        if kind == 0:  # a byte of the chunk-offset table
            t[rng.integers(off0, off1)] = rng.integers(0, 256)
            yield t, S, "offset byte"
        elif kind == 1 and E:  # a byte of an escape record
            t[esc + rng.integers(0, 3 * E)] = rng.integers(0, 256)
            yield t, S, "record byte"
        elif kind == 2 and E:  # the low position byte of a record, nudged by one
            r = int(rng.integers(0, E))
            t[esc + 3 * r] = (int(t[esc + 3 * r]) + int(rng.choice([-1, 1]))) & 0xFF
            yield t, S, "position nudge"
        elif kind == 3 and E > 1:  # two neighbouring records swapped
            r = int(rng.integers(0, E - 1))
            a, b = esc + 3 * r, esc + 3 * r + 3
            t[a:a + 3], t[b:b + 3] = good[b:b + 3], good[a:a + 3]
            yield t, S, "records swapped"
        elif kind == 4:  # E or S in the header off by a little
            field = 16 if rng.integers(0, 2) else 24
            v = u64(good, field) + int(rng.choice([-3, -1, 1, 3]))
            t[field:field + 8] = np.frombuffer(np.uint64(v).tobytes(), np.uint8)
            yield t, S, "header E/S"
        else:  # fewer bytes than the stream holds
            yield t, S - int(rng.integers(1, 16)), "truncated"


CASES = [
    # (dtype, n, data sigma, calibration sample): short chunks, then long ones
    (O.BF16, 4 * 65536 + 123, 1.0, 4000),
    (O.BF16, 3 * 65536 + 5001, 2.5, 300),
    (O.E5M2, 4 * 65536 + 77, 1.0, 4000),
    (O.E5M2, 2 * 65536 + 999, 3.0, 300),
]


@pytest.mark.parametrize("dtype,n,sigma,calib", CASES,
                         ids=["bf16-short", "bf16-long", "e5m2-short", "e5m2-long"])
def test_gpu_rejects_exactly_what_the_oracle_rejects(dtype, n, sigma, calib):
    xh = kvsynth.to_numpy_bits(kvsynth.random_bits(n, dtype, seed=int(n) % 1000, sigma=sigma))
    cb = O.calibrate(dtype, xh[:calib])
    good = O.compress(dtype, xh, cb)
    E = u64(good, 16)
    per_chunk = E / max(1, (n + 65535) // 65536)
    print(f"case fuzz dtype={dtype} n={n} escapes={E} ({per_chunk:.0f} per chunk)", flush=True)
    if sigma > 2:
        assert per_chunk > 1024  # the decoder's long-chunk path
    else:
        assert 0 < per_chunk <= 1024
    rng = np.random.default_rng(n)
    rejected = accepted = 0
    for t, in_bytes, label in _mutations(good, dtype, n, rng, 120):
        want = O.validate(t[:in_bytes], dtype, n)
        got, y = _gpu_status_and_output(t, n, dtype, in_bytes)
        assert got == want, f"{label}: GPU status {got}, oracle {want}"
        if want == O.OK:
            accepted += 1
            assert np.array_equal(y, O.decompress(t[:in_bytes], dtype, n)), f"{label}: output differs"
        else:
            rejected += 1
    print(f"  rejected {rejected}, still valid {accepted}", flush=True)
    assert rejected > 0
