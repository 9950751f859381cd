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
E_TOO_LARGE = -6
VARIANT_TOP15_SENTINEL = 1
VARIANT_TOP8 = 2

EXPORTS = (
    "splitzip_calibrate",
    "splitzip_max_compressed_size",
    "splitzip_compress",
    "splitzip_decompress",
    "splitzip_status_string",
    "splitzip_variant_max_compressed_size",
    "splitzip_variant_compress",
    "splitzip_variant_decompress",
    "splitzip_calibrate_device_work_bytes",
    "splitzip_calibrate_device",
    "splitzip_pipeline_sizes",
    "splitzip_pipeline_transfer",
    "splitzip_compress_static",
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
    lib.splitzip_variant_max_compressed_size.argtypes = [i32, sz, u32]
    lib.splitzip_variant_max_compressed_size.restype = sz
    lib.splitzip_variant_compress.argtypes = [i32, vp, sz, vp, u32, sz, vp, sz, vp, vp]
    lib.splitzip_variant_compress.restype = i32
    lib.splitzip_variant_decompress.argtypes = [i32, vp, sz, sz, vp, vp, vp]
    lib.splitzip_variant_decompress.restype = i32
    lib.splitzip_calibrate_device_work_bytes.argtypes = [i32, u32]
    lib.splitzip_calibrate_device_work_bytes.restype = sz
    lib.splitzip_calibrate_device.argtypes = [i32, vp, sz, sz, u32, vp, vp, sz, vp]
    lib.splitzip_calibrate_device.restype = i32
    lib.splitzip_pipeline_sizes.argtypes = [i32, sz, u32, sz, sz, u32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.splitzip_pipeline_sizes.restype = i32
    lib.splitzip_pipeline_transfer.argtypes = [i32, vp, sz, vp, u32, sz, sz, u32, i32, vp, sz, vp, sz, vp, vp, vp, vp]
    lib.splitzip_pipeline_transfer.restype = i32
    lib.splitzip_compress_static.argtypes = [i32, vp, sz, vp, u32, sz, vp, sz, vp, vp]
    lib.splitzip_compress_static.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().splitzip_status_string(int(status)).decode()


# ------------------------------------------------------------ raw C-ABI calls
def _host_codebooks(h_codebooks, n_codebooks: int) -> np.ndarray:
    """The codebooks as contiguous bytes, at least 16 per codebook (the
    library reads n_codebooks x 16 bytes through the pointer)."""
    cbs = np.ascontiguousarray(h_codebooks, dtype=np.uint8)
    if cbs.size < 16 * n_codebooks:
        raise ValueError(f"h_codebooks holds {cbs.size} bytes, {16 * n_codebooks} needed for {n_codebooks} codebooks")
    return cbs


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
    cbs = _host_codebooks(h_codebooks, n_codebooks)
    return int(load().splitzip_compress(dtype, d_in or None, n_elems, cbs.ctypes.data, n_codebooks,
                                        segment_elems, d_out or None, out_capacity, d_out_bytes or None,
                                        stream or None))


def splitzip_compress_static(dtype: int, d_in: int, n_elems: int, h_codebooks: np.ndarray, n_codebooks: int,
                             segment_elems: int, d_out: int, out_capacity: int, d_out_bytes: int | None,
                             stream: int | None) -> int:
    cbs = _host_codebooks(h_codebooks, n_codebooks)
    return int(load().splitzip_compress_static(dtype, d_in or None, n_elems, cbs.ctypes.data, n_codebooks,
                                               segment_elems, d_out or None, out_capacity, d_out_bytes or None,
                                               stream or None))


def splitzip_decompress(d_in: int, in_bytes: int, dtype: int, n_elems: int, d_out: int,
                        d_status: int | None, stream: int | None) -> int:
    return int(load().splitzip_decompress(d_in or None, in_bytes, dtype, n_elems, d_out or None,
                                          d_status or None, stream or None))


def splitzip_variant_max_compressed_size(variant: int, n_elems: int, n_codebooks: int) -> int:
    return int(load().splitzip_variant_max_compressed_size(variant, n_elems, n_codebooks))


def variant_compress(variant: int, x, codebooks, segment_elems: int = 0, out=None, out_bytes=None, stream=None):
    """Compress a contiguous BF16 device tensor into an ablation-variant
    stream; returns (out, out_bytes) as ``compress``."""
    import torch
    if not x.is_cuda or not x.is_contiguous() or _dtype_of(x) != BF16:
        raise ValueError("x must be a contiguous BF16 device tensor")
    cbs, k = _codebook_bytes(codebooks)
    if out is None:
        cap = splitzip_variant_max_compressed_size(variant, x.numel(), k)
        if cap == 0:
            raise SplitZipError(E_INVALID, "splitzip_variant_max_compressed_size")
        out = torch.empty(cap, dtype=torch.uint8, device=x.device)
    if out_bytes is None:
        out_bytes = torch.zeros(1, dtype=torch.int64, device=x.device)
    _device_buffer(out, "out", 0)  # its true size goes to the library, which checks the capacity
    _out_bytes_word(out_bytes)
    rc = load().splitzip_variant_compress(variant, x.data_ptr() or None, x.numel(), cbs, k, segment_elems,
                                          out.data_ptr(), _nbytes(out), out_bytes.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_variant_compress")
    return out, out_bytes


def variant_decompress(variant: int, stream_buf, n_elems: int, out=None, status=None, in_bytes: int | None = None,
                       stream=None):
    """Decode an ablation-variant stream held in a uint8 device tensor;
    returns (out, status) as ``decompress``."""
    import torch
    _device_buffer(stream_buf, "stream", 0)
    if out is None:
        out = torch.empty(n_elems, dtype=torch.int16, device=stream_buf.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=stream_buf.device)
    _device_buffer(out, "out", 2 * n_elems)
    _status_word(status)
    nbytes = _nbytes(stream_buf) if in_bytes is None else int(in_bytes)
    if nbytes > _nbytes(stream_buf):
        raise ValueError(f"in_bytes {nbytes} exceeds the stream buffer ({_nbytes(stream_buf)} bytes)")
    rc = load().splitzip_variant_decompress(variant, stream_buf.data_ptr(), nbytes, n_elems, out.data_ptr(),
                                            status.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_variant_decompress")
    return out, status


def splitzip_calibrate_device_work_bytes(dtype: int, n_codebooks: int) -> int:
    return int(load().splitzip_calibrate_device_work_bytes(dtype, n_codebooks))


def splitzip_calibrate_device(dtype: int, d_samples: int, n_elems: int, segment_elems: int, n_codebooks: int,
                              d_codebooks_out: int, d_work: int, work_bytes: int, stream: int | None) -> int:
    return int(load().splitzip_calibrate_device(dtype, d_samples or None, n_elems, segment_elems, n_codebooks,
                                                d_codebooks_out or None, d_work or None, work_bytes,
                                                stream or None))


def calibrate_device(x, n_codebooks: int = 1, segment_elems: int = 0, out=None, work=None, stream=None):
    """Codebooks of a contiguous device tensor (one per segment) computed on
    the GPU; returns a (n_codebooks, 16) uint8 device tensor.  Nothing is
    synchronized."""
    import torch
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    dtype = _dtype_of(x)
    need = splitzip_calibrate_device_work_bytes(dtype, n_codebooks)
    if need == 0:
        raise SplitZipError(E_INVALID, "splitzip_calibrate_device_work_bytes")
    if out is None:
        out = torch.empty((n_codebooks, 16), dtype=torch.uint8, device=x.device)
    if work is None:
        work = torch.empty(need, dtype=torch.uint8, device=x.device)
    _device_buffer(out, "out", 16 * n_codebooks)
    _device_buffer(work, "work", need)
    rc = splitzip_calibrate_device(dtype, x.data_ptr(), x.numel(), segment_elems, n_codebooks, out.data_ptr(),
                                   work.data_ptr(), _nbytes(work), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_calibrate_device")
    return out


def splitzip_pipeline_sizes(dtype: int, n_elems: int, n_codebooks: int, segment_elems: int, group_elems: int,
                            depth: int) -> tuple[int, int]:
    """(device work bytes, pinned host link bytes) of a pipelined transfer."""
    d, h = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = load().splitzip_pipeline_sizes(dtype, n_elems, n_codebooks, segment_elems, group_elems, depth,
                                        ctypes.byref(d), ctypes.byref(h))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_pipeline_sizes")
    return int(d.value), int(h.value)


def splitzip_pipeline_transfer(dtype: int, d_in: int, n_elems: int, h_codebooks: np.ndarray, n_codebooks: int,
                               segment_elems: int, group_elems: int, depth: int, compress: bool, d_work: int,
                               work_bytes: int, h_link: int, link_bytes: int, d_out: int, d_status: int | None,
                               h_group_bytes: np.ndarray | None, streams) -> int:
    cbs = _host_codebooks(h_codebooks, n_codebooks)
    arr = (ctypes.c_void_p * 4)(*[int(s) for s in streams])
    gb = None
    if h_group_bytes is not None:  # the library writes one u64 per group through it
        groups = -(-n_elems // group_elems) if group_elems > 0 else 0
        if (not isinstance(h_group_bytes, np.ndarray) or h_group_bytes.dtype != np.uint64
                or not h_group_bytes.flags.c_contiguous or h_group_bytes.size < groups):
            raise ValueError(f"h_group_bytes must be a contiguous uint64 array of at least {groups} entries")
        gb = h_group_bytes.ctypes.data
    return int(load().splitzip_pipeline_transfer(dtype, d_in or None, n_elems, cbs.ctypes.data, n_codebooks,
                                                 segment_elems, group_elems, depth, int(bool(compress)),
                                                 d_work or None, work_bytes, h_link or None, link_bytes,
                                                 d_out or None, d_status or None, gb, arr))


# -------------------------------------------------------- torch conveniences
def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _device_buffer(t, name: str, min_bytes: int):
    """A contiguous device tensor of at least min_bytes bytes, else ValueError
    (the library writes through its pointer for that many bytes)."""
    if not hasattr(t, "is_cuda") or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(t) < min_bytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, {min_bytes} needed")
    return t


def _word(t, name: str, dtypes, allow_host: bool):
    """A one-or-more-element tensor of one of `dtypes` that the GPU may write:
    device memory, or (allow_host) pinned host memory."""
    if not hasattr(t, "dtype") or t.dtype not in dtypes:
        raise ValueError(f"{name} must be a tensor of {' or '.join(str(d) for d in dtypes)}")
    if t.numel() < 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with at least one element")
    if not t.is_cuda and not (allow_host and t.is_pinned()):
        raise ValueError(f"{name} must be device memory" + (" or pinned host memory" if allow_host else ""))
    return t


def _out_bytes_word(t):
    import torch
    return _word(t, "out_bytes", (torch.int64, torch.uint64), allow_host=True)


def _status_word(t):
    import torch
    return _word(t, "status", (torch.int32,), allow_host=False)


def _elem_bytes(dtype: int) -> int:
    return 2 if dtype == BF16 else 1


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
    """The HIP stream of `stream`, or torch's current stream on the current
    device (through torch's raw-stream accessor when it has one: building a
    Stream object costs more than the launch it is for)."""
    import torch
    if stream is not None:
        return int(stream.cuda_stream)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(torch.cuda.current_device()))
    return int(torch.cuda.current_stream().cuda_stream)


def _codebook_bytes(codebooks):
    """(bytes, K) of K x 16 codebook entries.  The library reads them during
    the call only, so a bytes copy is passed as the host pointer (cheaper than
    a ctypes view of the array)."""
    a = codebooks if type(codebooks) is np.ndarray and codebooks.dtype == np.uint8 else \
        np.asarray(codebooks, dtype=np.uint8)
    if a.size == 0 or a.size % 16:
        raise ValueError(f"codebooks must hold K x 16 entries, got {a.size}")
    return a.tobytes(), a.size // 16


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
    cbs, k = _codebook_bytes(codebooks)
    n = x.numel()
    if out is None:
        cap = splitzip_max_compressed_size(dtype, n, k)
        if cap == 0:
            raise SplitZipError(E_INVALID, "splitzip_max_compressed_size")
        out = torch.empty(cap, dtype=torch.uint8, device=x.device)
    if out_bytes is None:
        out_bytes = torch.zeros(1, dtype=torch.int64, device=x.device)
    _device_buffer(out, "out", 0)  # its true size goes to the library, which checks the capacity
    _out_bytes_word(out_bytes)
    rc = load().splitzip_compress(dtype, x.data_ptr() or None, n, cbs, k, segment_elems, out.data_ptr(),
                                  _nbytes(out), out_bytes.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_compress")
    return out, out_bytes


def compress_static(x, codebooks, segment_elems: int = 0, out=None, out_bytes=None, stream=None):
    """``compress`` through splitzip_compress_static: the encoder's
    workspace in the library's own device memory, for inputs of at most
    2048 tiles (32 MiB); up to 512 tiles (8 MiB) in one launch.  Calls that
    overlap on one GPU race."""
    import torch
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    dtype = _dtype_of(x)
    cbs, k = _codebook_bytes(codebooks)
    if out is None:  # room for the largest stream (and more: the workspace splitzip_compress needs)
        out = torch.empty(splitzip_max_compressed_size(dtype, x.numel(), k), dtype=torch.uint8, device=x.device)
    if out_bytes is None:
        out_bytes = torch.zeros(1, dtype=torch.int64, device=x.device)
    _device_buffer(out, "out", 0)  # the library checks the capacity
    _out_bytes_word(out_bytes)
    rc = load().splitzip_compress_static(dtype, x.data_ptr() or None, x.numel(), cbs, k, segment_elems,
                                         out.data_ptr(), _nbytes(out), out_bytes.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_compress_static")
    return out, out_bytes


def decompress(stream_buf, n_elems: int, dtype: int, out=None, status=None, in_bytes: int | None = None,
               stream=None):
    """Decompress a stream held in a uint8 device tensor.  Returns ``(out,
    status)`` where ``status`` is a one-element int32 device tensor: 0, or
    E_CORRUPT once a corrupt stream was seen (a passed-in ``status`` is not
    cleared first).  Nothing is synchronized."""
    import torch
    if dtype not in (BF16, FP8_E5M2):
        raise ValueError(f"unknown dtype {dtype}")
    _device_buffer(stream_buf, "stream", 0)
    if out is None:
        out = torch.empty(n_elems, dtype=torch.int16 if dtype == BF16 else torch.uint8, device=stream_buf.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=stream_buf.device)
    _device_buffer(out, "out", n_elems * _elem_bytes(dtype))
    _status_word(status)
    nbytes = _nbytes(stream_buf) if in_bytes is None else int(in_bytes)
    if nbytes > _nbytes(stream_buf):
        raise ValueError(f"in_bytes {nbytes} exceeds the stream buffer ({_nbytes(stream_buf)} bytes)")
    rc = load().splitzip_decompress(stream_buf.data_ptr() or None, nbytes, dtype, n_elems, out.data_ptr() or None,
                                    status.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise SplitZipError(rc, "splitzip_decompress")
    return out, status


_hip = None


def _hip_runtime():
    """The HIP runtime, for the coherent pinned host buffer of the link."""
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the runtime torch was built with)
        for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("libamdhip64 not found")
        _hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        _hip.hipHostMalloc.restype = ctypes.c_int
        _hip.hipHostFree.argtypes = [ctypes.c_void_p]
        _hip.hipHostFree.restype = ctypes.c_int
    return _hip


HIP_HOST_MALLOC_COHERENT = 0x40000000


class Pipeline:
    """Buffers and streams of a chunk-pipelined transfer (device work area,
    coherent pinned host link buffer, four streams), reusable across calls of
    the same shape.  ``transfer(x, out)`` moves ``x`` into ``out`` through
    the link, compressed or raw, and returns the bytes each group sent.

    The pinned link buffer is released by ``close()`` (or at the end of a
    ``with`` block), after the four streams have drained; a finalizer makes
    no HIP call, so a pipeline never closed keeps its buffer until the
    process ends."""

    DRAIN_S = 60.0  # longest wait for the streams before close() gives up

    def __init__(self, dtype: int, n_elems: int, codebooks, segment_elems: int, group_elems: int, depth: int,
                 device=None, host_flags: int = HIP_HOST_MALLOC_COHERENT):
        import torch
        self._link = ctypes.c_void_p(0)
        self.dtype, self.n, self.seg, self.group, self.depth = dtype, n_elems, segment_elems, group_elems, depth
        self.cbs = np.ascontiguousarray(np.asarray(codebooks, dtype=np.uint8)).reshape(-1, 16)
        self.work_bytes, self.link_bytes = splitzip_pipeline_sizes(dtype, n_elems, self.cbs.shape[0], segment_elems,
                                                                   group_elems, depth)
        self.groups = -(-n_elems // group_elems)
        self.slot = (self.link_bytes - (-(-8 * self.groups // 256) * 256)) // depth
        self.work = torch.empty(self.work_bytes, dtype=torch.uint8, device=device)
        rc = _hip_runtime().hipHostMalloc(ctypes.byref(self._link), self.link_bytes, host_flags)
        if rc != 0 or not self._link.value:
            self._link = ctypes.c_void_p(0)
            raise RuntimeError(f"hipHostMalloc failed ({rc})")
        self.streams = [torch.cuda.Stream(device=device) for _ in range(4)]
        if self.work.data_ptr() % 256 or self._link.value % 256:
            self.close()
            raise RuntimeError("pipeline buffers are not 256-byte aligned")
        self.link = np.ctypeslib.as_array((ctypes.c_uint8 * self.link_bytes).from_address(self._link.value))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def _drain(self) -> bool:
        """Wait (at most DRAIN_S seconds) until the four streams are idle."""
        import time
        t_end = time.monotonic() + self.DRAIN_S
        while not all(s.query() for s in self.streams):
            if time.monotonic() > t_end:
                return False
            time.sleep(1e-4)
        return True

    def close(self):
        """Release the pinned link buffer once no queued copy can still use it.
        If the streams do not drain in time the buffer is left allocated
        (freeing memory a copy engine may still write would be worse)."""
        if not self._link.value:
            return
        if self._drain():
            _hip_runtime().hipHostFree(self._link)
        self._link = ctypes.c_void_p(0)
        self.link = None

    def __del__(self):
        if getattr(self, "_link", None) is not None and self._link.value:
            import warnings
            warnings.warn("Pipeline was not closed; its pinned link buffer stays allocated until exit",
                          ResourceWarning, stacklevel=2)

    def transfer(self, x, out, compress: bool = True, status=None):
        if not self._link.value:
            raise RuntimeError("pipeline is closed")
        nb = self.n * _elem_bytes(self.dtype)
        _device_buffer(x, "x", nb)
        _device_buffer(out, "out", nb)
        if x.numel() * x.element_size() != nb or out.numel() * out.element_size() != nb:
            raise ValueError("x and out must hold exactly the planned elements")
        if status is not None:
            _status_word(status)
        sizes = np.zeros(self.groups, dtype=np.uint64)
        rc = splitzip_pipeline_transfer(self.dtype, x.data_ptr(), self.n, self.cbs, self.cbs.shape[0], self.seg,
                                        self.group, self.depth, compress, self.work.data_ptr(), self.work_bytes,
                                        self._link.value, self.link_bytes, out.data_ptr(),
                                        None if status is None else status.data_ptr(), sizes,
                                        [s.cuda_stream for s in self.streams])
        if rc != OK:
            # work the call queued before it failed may still be running on
            # the four streams: let it finish before the caller reuses x, out
            # or this pipeline's buffers
            self._drain()
            raise SplitZipError(rc, "splitzip_pipeline_transfer")
        return sizes

    def slot_stream(self, g: int, nbytes: int) -> np.ndarray:
        """Bytes of group g's stream as they sit in the host link buffer
        (valid after a transfer while g is among the last ``depth`` groups)."""
        off = (g % self.depth) * self.slot
        return self.link[off:off + nbytes].copy()
