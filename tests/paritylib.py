"""Helpers of the GPU parity tests (imported by tests only).

``compare_with_oracle`` checks a GPU stream byte for byte against the CPU
oracle.  Small inputs are compressed by the oracle in one call.  Large inputs
are cut into pieces of whole 65536-element chunks that share one codebook;
the oracle compresses each piece as a stream of its own (in a thread pool:
ctypes releases the GIL), and every section of the GPU stream is compared with
the matching piece: nibbles, sign|mantissa bytes, escape records, chunk
offsets (shifted by the escapes of earlier pieces), header and padding.  All
section offsets come from the oracle's own layout function.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle as O

CHUNK = 65536


def u64(buf: np.ndarray, off: int) -> int:
    return int(np.frombuffer(buf[off:off + 8].tobytes(), dtype="<u8")[0])


def sm_bytes(dtype: int, n: int) -> int:
    return n if dtype == O.BF16 else 3 * ((n + 7) // 8)


def piece_bounds(n: int, n_codebooks: int, segment_elems: int, max_piece: int):
    """Pieces [a, b) of whole chunks, each inside one codebook segment."""
    seg = segment_elems if n_codebooks > 1 else n
    step = max(CHUNK, (min(seg, max_piece) // CHUNK) * CHUNK)
    out = []
    a = 0
    while a < n:
        seg_end = min(n, (a // seg + 1) * seg) if n_codebooks > 1 else n
        b = min(seg_end, a + step)
        out.append((a, b))
        a = b
    return out


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def compare_with_oracle(gpu: np.ndarray, dtype: int, x: np.ndarray, cbs: np.ndarray, segment_elems: int,
                        max_piece: int = 1 << 24) -> int:
    """Assert that ``gpu`` (the stream bytes, exactly S long) equals the
    oracle's stream of ``x``.  Returns the escape count."""
    cbs = np.ascontiguousarray(cbs, dtype=np.uint8).reshape(-1, 16)
    K = cbs.shape[0]
    n = x.size
    if n <= max_piece:
        want = O.compress(dtype, x, cbs, segment_elems)
        assert gpu.size == want.size, (gpu.size, want.size)
        bad = np.nonzero(gpu != want)[0]
        assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
        return u64(want, 16)

    sec = O.sections(dtype, n, K)
    pieces = piece_bounds(n, K, segment_elems, max_piece)

    def run(ab):
        a, b = ab
        k = 0 if K == 1 else a // segment_elems
        return O.compress(dtype, x[a:b], cbs[k])

    with cf.ThreadPoolExecutor(_threads()) as ex:
        streams = list(ex.map(run, pieces))

    E = sum(u64(s, 16) for s in streams)
    assert u64(gpu, 16) == E, (u64(gpu, 16), E)
    S = O.stream_size(dtype, n, K, E)
    assert gpu.size == S and u64(gpu, 24) == S
    # header: fields that do not depend on the split equal the first piece's
    first = streams[0]
    assert np.array_equal(gpu[0:8], first[0:8])                 # magic, version, dtype, log2
    assert u64(gpu, 8) == n
    assert int(np.frombuffer(gpu[32:36].tobytes(), "<u4")[0]) == sec["chunks"]
    assert int(np.frombuffer(gpu[36:40].tobytes(), "<u4")[0]) == K
    assert u64(gpu, 40) == (n if K == 1 else segment_elems)
    assert not gpu[48:64].any()
    assert np.array_equal(gpu[64:64 + 16 * K], cbs.reshape(-1))
    offs = np.frombuffer(gpu[sec["offsets"]:sec["offsets"] + 8 * (sec["chunks"] + 1)].tobytes(), "<u8")
    before = 0
    for (a, b), s in zip(pieces, streams):
        ps = O.sections(dtype, b - a, 1)
        e_k = u64(s, 16)
        # nibbles
        g = gpu[sec["nib"] + a // 2: sec["nib"] + (b + 1) // 2]
        w = s[ps["nib"]: ps["nib"] + (b - a + 1) // 2]
        assert np.array_equal(g, w), f"nibbles differ in [{a}, {b})"
        # sign|mantissa
        sa = sm_bytes(dtype, a)
        g = gpu[sec["sm"] + sa: sec["sm"] + sa + sm_bytes(dtype, b - a)]
        w = s[ps["sm"]: ps["sm"] + sm_bytes(dtype, b - a)]
        assert np.array_equal(g, w), f"sign|mantissa differ in [{a}, {b})"
        # escape records
        g = gpu[sec["esc"] + 3 * before: sec["esc"] + 3 * (before + e_k)]
        w = s[ps["esc"]: ps["esc"] + 3 * e_k]
        assert np.array_equal(g, w), f"escape records differ in [{a}, {b})"
        # chunk offsets
        c0 = a // CHUNK
        pc = ps["chunks"]
        po = np.frombuffer(s[ps["offsets"]:ps["offsets"] + 8 * (pc + 1)].tobytes(), "<u8")
        assert np.array_equal(offs[c0:c0 + pc + 1], po + np.uint64(before)), f"offsets differ in [{a}, {b})"
        before += e_k
    # padding between sections
    ends = [(sec["offsets"] + 8 * (sec["chunks"] + 1), sec["nib"]),
            (sec["nib"] + (n + 1) // 2, sec["sm"]),
            (sec["sm"] + sm_bytes(dtype, n), sec["esc"])]
    for lo, hi in ends:
        assert not gpu[lo:hi].any(), f"padding [{lo}, {hi}) not zero"
    return E
