"""ctypes binding of libsplitzip (include/splitzip.h): argument marshalling only.

Every step of the codec runs in the HIP library; this module converts torch
tensors and numpy arrays into pointers, sizes and streams.  It raises if the
library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsplitzip.so")

BF16 = 1
FP8_E5M2 = 2
OK = 0
E_INVALID = -1
E_CAPACITY = -2
E_CODEBOOK = -3
E_CORRUPT = -4
E_HIP = -5

EXPORTS = (
    "splitzip_calibrate",
    "splitzip_max_compressed_size",
    "splitzip_compress",
    "splitzip_decompress",
    "splitzip_status_string",
)

_lib = None


class SplitZipError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def load():
    """Load libsplitzip.so (built by ``lossless_kv_cache_splitzip_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libsplitzip.so not found at {LIB_PATH}; build it with "
            "`python -m lossless_kv_cache_splitzip_amd.build` (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    i32, u32, sz, vp = ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
    lib.splitzip_calibrate.argtypes = [i32, vp, sz, vp]
    lib.splitzip_calibrate.restype = i32
    lib.splitzip_max_compressed_size.argtypes = [i32, sz, u32]
    lib.splitzip_max_compressed_size.restype = sz
    lib.splitzip_compress.argtypes = [i32, vp, sz, vp, u32, sz, vp, sz, vp, vp]
    lib.splitzip_compress.restype = i32
    lib.splitzip_decompress.argtypes = [vp, sz, i32, sz, vp, vp, vp]
    lib.splitzip_decompress.restype = i32
    lib.splitzip_status_string.argtypes = [i32]
    lib.splitzip_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().splitzip_status_string(int(status)).decode()


# ------------------------------------------------------------ raw C-ABI calls
def splitzip_calibrate(dtype: int, host_samples) -> np.ndarray:
    """Top-16 exponent codebook of host samples (numpy or CPU tensor bits)."""
    a = _host_bits(host_samples, dtype)
    cb = np.zeros(16, dtype=np.uint8)
    rc = load().splitzip_calibrate(dtype, a.ctypes.data if a.size else None, a.size, cb.ctypes.data)
    if rc != OK:
        raise SplitZipError(rc, "splitzip_calibrate")
    return cb


def splitzip_max_compressed_size(dtype: int, n_elems: int, n_codebooks: int) -> int:
    return int(load().splitzip_max_compressed_size(dtype, n_elems, n_codebooks))


def splitzip_compress(dtype: int, d_in: int, n_elems: int, h_codebooks: np.ndarray, n_codebooks: int,
                      segment_elems: int, d_out: int, out_capacity: int, d_out_bytes: int | None,
                      stream: int | None) -> int:
    cbs = np.ascontiguousarray(h_codebooks, dtype=np.uint8)
    return int(load().splitzip_compress(dtype, d_in or None, n_elems, cbs.ctypes.data, n_codebooks,
                                        segment_elems, d_out or None, out_capacity, d_out_bytes or None,
                                        stream or None))


def splitzip_decompress(d_in: int, in_bytes: int, dtype: int, n_elems: int, d_out: int,
                        d_status: int | None, stream: int | None) -> int:
    return int(load().splitzip_decompress(d_in or None, in_bytes, dtype, n_elems, d_out or None,
                                          d_status or None, stream or None))


# -------------------------------------------------------- torch conveniences
def _host_bits(x, dtype: int) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    a = np.ascontiguousarray(x).reshape(-1)
    want = np.uint16 if dtype == BF16 else np.uint8
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise ValueError(f"samples of itemsize {a.dtype.itemsize} do not match dtype {dtype}")
        a = a.view(want)
    return a


def _dtype_of(t) -> int:
    import torch
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype in (torch.float8_e5m2, torch.uint8):
        return FP8_E5M2
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def compress(x, codebooks, segment_elems: int = 0, out=None, out_bytes=None, stream=None):
    """Compress a contiguous device tensor of BF16 (bfloat16/int16 bits) or
    E5M2 (float8_e5m2/uint8 bits) values.

    Returns ``(out, out_bytes)``: the uint8 device buffer holding the stream at
    its start, and a one-element int64 device tensor with the stream size.
    Nothing is synchronized."""
    import torch
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    dtype = _dtype_of(x)
    cbs = np.ascontiguousarray(np.asarray(codebooks, dtype=np.uint8)).reshape(-1, 16)
    k = cbs.shape[0]
    n = x.numel()
    cap = splitzip_max_compressed_size(dtype, n, k)
    if cap == 0:
        raise SplitZipError(E_INVALID, "splitzip_max_compressed_size")
    if out is None:
        out = torch.empty(cap, dtype=torch.uint8, device=x.device)
    if out_bytes is None:
        out_bytes = torch.zeros(1, dtype=torch.int64, device=x.device)
    rc = splitzip_compress(dtype, x.data_ptr(), n, cbs, k, segment_elems, out.data_ptr(), out.numel(),
                           out_bytes.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_compress")
    return out, out_bytes


def decompress(stream_buf, n_elems: int, dtype: int, out=None, status=None, in_bytes: int | None = None,
               stream=None):
    """Decompress a stream held in a uint8 device tensor.  Returns ``(out,
    status)`` where ``status`` is a one-element int32 device tensor: 0, or
    E_CORRUPT once a corrupt stream was seen (a passed-in ``status`` is not
    cleared first).  Nothing is synchronized."""
    import torch
    if not stream_buf.is_cuda or not stream_buf.is_contiguous():
        raise ValueError("stream must be a contiguous device tensor")
    if out is None:
        out = torch.empty(n_elems, dtype=torch.int16 if dtype == BF16 else torch.uint8, device=stream_buf.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=stream_buf.device)
    nbytes = stream_buf.numel() * stream_buf.element_size() if in_bytes is None else in_bytes
    rc = splitzip_decompress(stream_buf.data_ptr(), nbytes, dtype, n_elems, out.data_ptr(), status.data_ptr(),
                             _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_decompress")
    return out, status
