"""The decoders' acceptance test equals the oracle's: streams damaged at
random in the chunk-offset table, the codes, the escape section and the E / S
header fields, or handed over with fewer bytes than they hold, are rejected by
the GPU (d_status = E_CORRUPT) exactly when the oracle's validation rejects
them; a damaged stream that is still valid (another code, an escape moved to
another free position, an exponent replaced by another in range) decodes to
the oracle's result bit for bit.  Short chunks (the decoder loads all of a
chunk's records in every tile: one group of four records per thread up to
1024 records, two up to 2048) and long chunks (it searches for the tile's
records) are all covered, for BF16 and E5M2, and so are the two ablation
variants' decoders.
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


def _a256(x):
    return (x + 255) // 256 * 256


def _layout(good: np.ndarray, n: int, code_bytes: int, rec: int):
    """Offsets table, code section and escape section of a one-codebook stream."""
    C = (n + 65535) // 65536
    off0 = 64 + 16
    code0 = _a256(off0 + 8 * (C + 1))
    E = u64(good, 16)
    esc = u64(good, 24) - rec * E
    return (off0, off0 + 8 * (C + 1)), (code0, code0 + code_bytes), esc, E


def _mutations(good: np.ndarray, n: int, code_bytes: int, rec: int, rng, count: int):
    """(stream, in_bytes, label) cases, each damaged in one way: a byte of the
    offset table, of the codes or of the escape section; a record position
    nudged by one or two records swapped (position records only); E or S in
    the header off by a little; fewer bytes than the stream holds; a codebook
    entry repeated or replaced."""
    (off0, off1), (code0, code1), esc, E = _layout(good, n, code_bytes, rec)
    S = good.size
    kinds = 8
    for i in range(count):
        t = good.copy()
        kind = i % kinds
        if kind == 7:
            # a codebook entry: a copy of another entry (a repeat) or any byte
            # (out of range for E5M2 when >= 32, else still a valid codebook)
            j = int(rng.integers(0, 16))
            t[64 + j] = good[64 + (j + int(rng.integers(1, 16))) % 16] if rng.integers(0, 2) else rng.integers(0, 256)
            yield t, S, "codebook byte"
        elif kind == 0:
            t[rng.integers(off0, off1)] = rng.integers(0, 256)
            yield t, S, "offset byte"
        elif kind == 1:
            t[rng.integers(code0, code1)] = rng.integers(0, 256)
            yield t, S, "code byte"
        elif kind == 2 and E:
            t[esc + rng.integers(0, rec * E)] = rng.integers(0, 256)
            yield t, S, "escape byte"
        elif kind == 3:
            field = 16 if rng.integers(0, 2) else 24
            v = u64(good, field) + int(rng.choice([-3, -1, 1, 3]))
            t[field:field + 8] = np.frombuffer(np.uint64(v).tobytes(), np.uint8)
            yield t, S, "header E/S"
        elif kind == 4:
            yield t, S - int(rng.integers(1, 16)), "truncated"
        elif kind == 5 and E and rec == 3:
            r = int(rng.integers(0, E))
            t[esc + 3 * r] = (int(t[esc + 3 * r]) + int(rng.choice([-1, 1]))) & 0xFF
            yield t, S, "position nudge"
        elif kind == 6 and E > 1 and rec == 3:
            r = int(rng.integers(0, E - 1))
            a, b = esc + 3 * r, esc + 3 * r + 3
            t[a:a + 3], t[b:b + 3] = good[b:b + 3], good[a:a + 3]
            yield t, S, "records swapped"


def _check(cases, gpu_decode, oracle_status, oracle_decode):
    rejected = accepted = 0
    for t, in_bytes, label in cases:
        want = oracle_status(t[:in_bytes])
        dev = torch.from_numpy(t).to(DEV)
        y, st = gpu_decode(dev, in_bytes)
        torch.cuda.synchronize()
        got = int(st.item())
        assert got == want, f"{label}: GPU status {got}, oracle {want}"
        if want == O.OK:
            accepted += 1
            assert np.array_equal(kvsynth.to_numpy_bits(y), oracle_decode(t[:in_bytes])), f"{label}: output differs"
        else:
            rejected += 1
    print(f"  rejected {rejected}, still valid {accepted}", flush=True)
    assert rejected > 0 and accepted > 0


CASES = [
    # (dtype, n, data sigma, calibration sample, most records in a chunk: (lo, hi]):
    # short chunks of one and two record groups per thread, then long ones
    (O.BF16, 4 * 65536 + 123, 1.0, 4000, (0, 1024)),
    (O.BF16, 3 * 65536 + 777, 2.0, 300, (1024, 2048)),
    (O.BF16, 3 * 65536 + 5001, 2.5, 300, (2048, 65536)),
    (O.E5M2, 4 * 65536 + 77, 1.0, 4000, (0, 1024)),
    (O.E5M2, 3 * 65536 + 555, 1.8, 300, (1024, 2048)),
    (O.E5M2, 2 * 65536 + 999, 3.0, 300, (2048, 65536)),
]


def _data(dtype, n, sigma, calib):
    xh = kvsynth.to_numpy_bits(kvsynth.random_bits(n, dtype, seed=int(n) % 1000, sigma=sigma))
    return xh, O.calibrate(dtype, xh[:calib])


@pytest.mark.parametrize("dtype,n,sigma,calib,most", CASES,
                         ids=["bf16-short", "bf16-short2", "bf16-long", "e5m2-short", "e5m2-short2", "e5m2-long"])
def test_gpu_rejects_exactly_what_the_oracle_rejects(dtype, n, sigma, calib, most):
    xh, cb = _data(dtype, n, sigma, calib)
    good = O.compress(dtype, xh, cb)
    E = u64(good, 16)
    C = (n + 65535) // 65536
    per_chunk = [u64(good, 80 + 8 * (c + 1)) - u64(good, 80 + 8 * c) for c in range(C)]
    print(f"case fuzz dtype={dtype} n={n} escapes={E} per chunk {per_chunk}", flush=True)
    assert most[0] < max(per_chunk) <= most[1]  # the decoder path the case is for
    code_bytes = (n + 1) // 2
    _check(_mutations(good, n, code_bytes, 3, np.random.default_rng(n), 140),
           lambda dev, ib: sz.decompress(dev, n, dtype, in_bytes=ib),
           lambda t: O.validate(t, dtype, n),
           lambda t: O.decompress(t, dtype, n))


@pytest.mark.parametrize("variant", [O.SENTINEL, O.TOP8], ids=["sentinel", "top8"])
@pytest.mark.parametrize("sigma", [0.3, 1.0, 2.5], ids=["narrow", "few", "many"])  # top-8 chunks: ~1700, ~4300, ~20700 records
def test_variant_decoders_reject_exactly_what_the_oracle_rejects(variant, sigma):
    n = 3 * 65536 + 4321
    xh, cb = _data(O.BF16, n, sigma, 4000 if sigma < 2 else 300)
    good = O.variant_compress(variant, xh, cb)
    print(f"case fuzz variant={variant} sigma={sigma} escapes={u64(good, 16)}", flush=True)
    code_bytes = 3 * ((n + 7) // 8) if variant == O.TOP8 else (n + 1) // 2
    rec = 1 if variant == O.SENTINEL else 3
    _check(_mutations(good, n, code_bytes, rec, np.random.default_rng(variant * 100 + int(sigma)), 100),
           lambda dev, ib: sz.variant_decompress(variant, dev, n, in_bytes=ib),
           lambda t: O.variant_decompress_rc(variant, t, n)[0],
           lambda t: O.variant_decompress(variant, t, n))


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2], ids=["bf16", "e5m2"])
@pytest.mark.parametrize("n,k", [(3 * 65536 + 777, 5), (65536 + 5, 100), (0, 3)],
                         ids=["unused-codebook", "more-codebooks-than-workgroups", "empty"])
def test_every_codebook_is_validated(dtype, n, k):
    """A stream is rejected when any of its K codebooks, used by a chunk or
    not, repeats an entry or (E5M2) holds one of 32 or more, as the oracle's
    validation rejects it; a codebook changed into another valid one still
    decodes as the oracle decodes it.  With 100 codebooks and 9 tiles the
    checks are spread over the workgroups several codebooks apiece."""
    rng = np.random.default_rng(1000 * k + dtype)
    xh = kvsynth.to_numpy_bits(kvsynth.random_bits(max(n, 1), dtype, seed=7, sigma=1.0))[:n]
    vals = 256 if dtype == O.BF16 else 32
    cbs = np.stack([rng.permutation(vals)[:16] for _ in range(k)]).astype(np.uint8)
    good = O.compress(dtype, xh, cbs, 65536)
    print(f"case codebooks dtype={dtype} n={n} K={k} S={good.size}", flush=True)
    cases = []
    for c in range(k):
        for how in ("repeat", "out_of_range", "other_valid"):
            if how == "out_of_range" and dtype == O.BF16:
                continue
            t = good.copy()
            j = int(rng.integers(0, 16))
            at = 64 + 16 * c + j
            if how == "repeat":
                t[at] = good[64 + 16 * c + (j + 1) % 16]
            elif how == "out_of_range":
                t[at] = int(rng.integers(32, 256))
            else:
                free = sorted(set(range(vals)) - set(int(v) for v in good[64 + 16 * c:64 + 16 * c + 16]))
                t[at] = free[int(rng.integers(0, len(free)))]
            cases.append((t, t.size, f"codebook {c} {how}"))
    _check_codebook_cases(cases, dtype, n)


def _check_codebook_cases(cases, dtype, n):
    rejected = accepted = 0
    for t, in_bytes, label in cases:
        want = O.validate(t, dtype, n)
        y, st = sz.decompress(torch.from_numpy(t).to(DEV), n, dtype, in_bytes=in_bytes)
        torch.cuda.synchronize()
        assert int(st.item()) == want, f"{label}: GPU status {int(st.item())}, oracle {want}"
        if want == O.OK:
            accepted += 1
            assert np.array_equal(kvsynth.to_numpy_bits(y), O.decompress(t, dtype, n)), f"{label}: output differs"
        else:
            rejected += 1
    print(f"  rejected {rejected}, still valid {accepted}", flush=True)
    assert rejected > 0 and accepted > 0


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2], ids=["bf16", "e5m2"])
@pytest.mark.parametrize("last", [10, 65536], ids=["short-last-chunk", "full-last-chunk"])
def test_chunk_with_more_records_than_elements(dtype, last):
    """Chunk offsets that give the last chunk more records than it has
    elements (its start moved down into the previous chunk's records, E and S
    unchanged) are rejected, as the oracle rejects them.  A chunk holds at
    most one record per element; the decoder checks that bound before it
    keeps a chunk's record count in 32 bits."""
    n = 65536 + last
    xh = kvsynth.to_numpy_bits(kvsynth.random_bits(n, dtype, seed=9, kind="uniform_bits"))
    cb = O.calibrate(dtype, xh[:2000])
    good = O.compress(dtype, xh, cb)
    off1 = u64(good, 80 + 8)
    cases = []
    for k in (1, last + 1, 5000):
        k = min(k, off1)
        t = good.copy()
        t[88:96] = np.frombuffer(np.uint64(off1 - k).tobytes(), np.uint8)
        got_last = u64(t, 80 + 16) - u64(t, 88)
        print(f"case more-records dtype={dtype} n={n} last chunk {last} elements, {got_last} records", flush=True)
        cases.append((t, t.size, f"last chunk {got_last} records for {last} elements"))
    assert any(u64(t, 80 + 16) - u64(t, 88) > last for t, _, _ in cases)
    for t, in_bytes, label in cases:
        want = O.validate(t, dtype, n)
        assert want == O.E_CORRUPT, label
        y, st = sz.decompress(torch.from_numpy(t).to(DEV), n, dtype, in_bytes=in_bytes)
        torch.cuda.synchronize()
        assert int(st.item()) == sz.E_CORRUPT, f"{label}: GPU status {int(st.item())}"
