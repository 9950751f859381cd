"""CPU oracle of the SplitZip exponent codec (plain scalar C, loaded via ctypes).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
(``lossless_kv_cache_splitzip_amd``) never imports it and shares no code with it.

The C source (``splitzip_oracle.c``) states what each step computes and which
passage of the SplitZip pages ("SplitZip: Ultra Fast Lossless KV Compression
for Disaggregated LLM Serving", arXiv 2605.01708v2) it follows.

Pinned by ``tests/test_oracle_pins.py``: exhaustive BF16/E5M2 round trips,
the closed-form stream size, brute-force top-16 calibration, escape sets
against an independent numpy count, a hand-worked stream, the explainer's
"position 50" escape example, and the pages' 16/12 and 8/7 ratio limits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "splitzip_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsplitzip_oracle.so")

BF16 = 1
E5M2 = 2
OK = 0
E_INVALID = -1
E_CAPACITY = -2
E_CODEBOOK = -3
E_CORRUPT = -4

_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain -O2, no vector intrinsics)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC]
    )
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path: str | None):
    """Point this module at another build of the oracle source (the mutation
    tests load deliberately broken copies); ``None`` restores the default."""
    global _lib
    _lib = None if path is None else _bind(ctypes.CDLL(path))


def _bind(lib):
    u64, u32, i32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p
    lib.szo_stream_size.argtypes = [i32, u64, u32, u64]
    lib.szo_stream_size.restype = u64
    lib.szo_max_size.argtypes = [i32, u64, u32]
    lib.szo_max_size.restype = u64
    lib.szo_calibrate.argtypes = [i32, vp, u64, vp]
    lib.szo_calibrate.restype = i32
    lib.szo_compress.argtypes = [i32, vp, u64, vp, u32, u64, vp, u64, ctypes.POINTER(u64)]
    lib.szo_compress.restype = i32
    lib.szo_validate.argtypes = [vp, u64, i32, u64]
    lib.szo_validate.restype = i32
    lib.szo_decompress.argtypes = [vp, u64, i32, u64, vp]
    lib.szo_decompress.restype = i32
    lib.szo_count_escapes.argtypes = [i32, vp, u64, vp, u32, u64]
    lib.szo_count_escapes.restype = u64
    lib.szo_sections.argtypes = [i32, u64, u32, vp]
    lib.szo_sections.restype = i32
    lib.szo_variant_stream_size.argtypes = [i32, u64, u32, u64]
    lib.szo_variant_stream_size.restype = u64
    lib.szo_variant_max_size.argtypes = [i32, u64, u32]
    lib.szo_variant_max_size.restype = u64
    lib.szo_variant_compress.argtypes = [i32, vp, u64, vp, u32, u64, vp, u64, ctypes.POINTER(u64)]
    lib.szo_variant_compress.restype = i32
    lib.szo_variant_decompress.argtypes = [i32, vp, u64, u64, vp]
    lib.szo_variant_decompress.restype = i32
    return lib


def _elem_dtype(dtype: int):
    if dtype == BF16:
        return np.uint16
    return np.uint8  # E5M2; any other code is passed through for the C side to reject


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _as_elems(x, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(x)
    want = _elem_dtype(dtype)
    if a.dtype != want:
        a = a.view(want) if a.dtype.itemsize == np.dtype(want).itemsize else a.astype(want)
    return a.reshape(-1)


def _as_codebooks(codebooks) -> np.ndarray:
    cbs = np.ascontiguousarray(np.asarray(codebooks, dtype=np.uint8)).reshape(-1, 16)
    return cbs


def stream_size(dtype: int, n: int, n_codebooks: int, n_escapes: int) -> int:
    return int(_load().szo_stream_size(dtype, n, n_codebooks, n_escapes))


def sections(dtype: int, n: int, n_codebooks: int) -> dict:
    """Section offsets of a stream (chunks, offsets table, nibbles, sign|mantissa, escapes)."""
    out = np.zeros(5, dtype=np.uint64)
    rc = _load().szo_sections(dtype, n, n_codebooks, _ptr(out))
    if rc != OK:
        raise ValueError(f"szo_sections failed: {rc}")
    c, off, nib, sm, esc = (int(v) for v in out)
    return {"chunks": c, "offsets": off, "nib": nib, "sm": sm, "esc": esc}


def max_size(dtype: int, n: int, n_codebooks: int) -> int:
    return int(_load().szo_max_size(dtype, n, n_codebooks))


def calibrate(dtype: int, samples) -> np.ndarray:
    a = _as_elems(samples, dtype)
    cb = np.zeros(16, dtype=np.uint8)
    rc = _load().szo_calibrate(dtype, _ptr(a), a.size, _ptr(cb))
    if rc != OK:
        raise ValueError(f"szo_calibrate failed: {rc}")
    return cb


def compress_rc(dtype: int, x, codebooks, segment_elems: int = 0, capacity: int | None = None):
    """Returns (status, stream bytes or None)."""
    a = _as_elems(x, dtype)
    cbs = _as_codebooks(codebooks)
    K = cbs.shape[0]
    cap = max_size(dtype, a.size, max(K, 1)) if capacity is None else capacity
    out = np.zeros(max(cap, 1), dtype=np.uint8)
    nbytes = ctypes.c_uint64(0)
    rc = _load().szo_compress(
        dtype, _ptr(a), a.size, _ptr(cbs) if cbs.size else None, K, segment_elems, _ptr(out), cap,
        ctypes.byref(nbytes),
    )
    if rc != OK:
        return rc, None
    return rc, out[: nbytes.value].copy()


def compress(dtype: int, x, codebooks, segment_elems: int = 0) -> np.ndarray:
    rc, s = compress_rc(dtype, x, codebooks, segment_elems)
    if rc != OK:
        raise ValueError(f"szo_compress failed: {rc}")
    return s


def validate(stream, dtype: int, n: int) -> int:
    s = np.ascontiguousarray(np.asarray(stream, dtype=np.uint8))
    return int(_load().szo_validate(_ptr(s), s.size, dtype, n))


def decompress_rc(stream, dtype: int, n: int):
    s = np.ascontiguousarray(np.asarray(stream, dtype=np.uint8))
    out = np.zeros(n, dtype=_elem_dtype(dtype))
    rc = _load().szo_decompress(_ptr(s), s.size, dtype, n, _ptr(out))
    return rc, (out if rc == OK else None)


def decompress(stream, dtype: int, n: int) -> np.ndarray:
    rc, out = decompress_rc(stream, dtype, n)
    if rc != OK:
        raise ValueError(f"szo_decompress failed: {rc}")
    return out


def count_escapes(dtype: int, x, codebooks, segment_elems: int = 0) -> int:
    a = _as_elems(x, dtype)
    cbs = _as_codebooks(codebooks)
    return int(_load().szo_count_escapes(dtype, _ptr(a), a.size, _ptr(cbs), cbs.shape[0], segment_elems))


# ---- ablation variants (BF16): 1 = top-15 + sentinel, 2 = top-8 (3-bit codes)
SENTINEL = 1
TOP8 = 2


def variant_stream_size(variant: int, n: int, K: int, E: int) -> int:
    return int(_load().szo_variant_stream_size(variant, n, K, E))


def variant_max_size(variant: int, n: int, K: int) -> int:
    return int(_load().szo_variant_max_size(variant, n, K))


def variant_compress(variant: int, x, codebooks, segment_elems: int = 0) -> np.ndarray:
    a = _as_elems(x, BF16)
    cbs = _as_codebooks(codebooks)
    K = cbs.shape[0]
    cap = max(variant_max_size(variant, a.size, max(K, 1)), 1)
    out = np.zeros(cap, dtype=np.uint8)
    nbytes = ctypes.c_uint64(0)
    rc = _load().szo_variant_compress(variant, _ptr(a), a.size, _ptr(cbs) if cbs.size else None, K, segment_elems,
                                      _ptr(out), cap, ctypes.byref(nbytes))
    if rc != OK:
        raise ValueError(f"szo_variant_compress failed: {rc}")
    return out[:nbytes.value].copy()


def variant_decompress_rc(variant: int, stream, n: int):
    s = np.ascontiguousarray(np.asarray(stream, dtype=np.uint8))
    out = np.zeros(max(n, 1), dtype=np.uint16)
    rc = int(_load().szo_variant_decompress(variant, _ptr(s), s.size, n, _ptr(out)))
    return rc, (out[:n] if rc == OK else None)


def variant_decompress(variant: int, stream, n: int) -> np.ndarray:
    rc, y = variant_decompress_rc(variant, stream, n)
    if rc != OK:
        raise ValueError(f"szo_variant_decompress failed: {rc}")
    return y
