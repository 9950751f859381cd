"""Host-side checks of libsplitzip that need no GPU: the library loads, it
exports every function include/splitzip.h declares, host calibration agrees
with the oracle, size queries, and argument errors that return before any
GPU work is enqueued."""
import os
import re

import numpy as np
import pytest

import kvsynth
import oracle as O

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(splitzip_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_function():
    lib = sz.load()
    declared = _declared_functions()
    assert {"splitzip_calibrate", "splitzip_max_compressed_size", "splitzip_compress",
            "splitzip_decompress"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(sz.EXPORTS) == declared


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
def test_host_calibration_matches_oracle(dtype):
    for seed in range(6):
        x = kvsynth.to_numpy_bits(kvsynth.random_bits(50000, dtype, seed=seed, sigma=0.5 + seed / 2))
        assert np.array_equal(sz.splitzip_calibrate(dtype, x), O.calibrate(dtype, x))
    # ties and unseen values
    x = np.array([5 << 7, 9 << 7, 9 << 7, 5 << 7, 200 << 7], dtype=np.uint16)
    assert np.array_equal(sz.splitzip_calibrate(O.BF16, x), O.calibrate(O.BF16, x))
    assert np.array_equal(sz.splitzip_calibrate(O.BF16, np.zeros(0, np.uint16)), np.arange(16))


def test_max_compressed_size():
    for dtype in (O.BF16, O.E5M2):
        for n, k in [(0, 1), (1, 1), (65537, 2), (536870912, 32)]:
            cap = sz.splitzip_max_compressed_size(dtype, n, k)
            assert cap >= O.max_size(dtype, n, k) + 2052 * (-(-n // 8192))
            assert cap % 8 == 0
    assert sz.splitzip_max_compressed_size(3, 10, 1) == 0
    assert sz.splitzip_max_compressed_size(O.BF16, 10, 0) == 0
    assert sz.splitzip_max_compressed_size(O.BF16, (1 << 36) + 1, 1) == 0
    assert sz.splitzip_max_compressed_size(O.BF16, 1 << 36, 1) > 0


def test_argument_errors_return_before_any_gpu_work():
    cb = np.arange(16, dtype=np.uint8)
    fake = 1 << 20  # aligned, never dereferenced: every call below fails validation first
    assert sz.splitzip_compress(3, fake, 10, cb, 1, 0, fake, 1 << 30, None, None) == sz.E_INVALID
    assert sz.splitzip_compress(O.BF16, fake + 2, 10, cb, 1, 0, fake, 1 << 30, None, None) == sz.E_INVALID
    assert sz.splitzip_compress(O.BF16, fake, 10, cb, 1, 0, 0, 1 << 30, None, None) == sz.E_INVALID
    dup = cb.copy(); dup[3] = dup[4]
    assert sz.splitzip_compress(O.BF16, fake, 10, dup, 1, 0, fake, 1 << 30, None, None) == sz.E_CODEBOOK
    assert sz.splitzip_compress(O.E5M2, fake, 10, cb + 20, 1, 0, fake, 1 << 30, None, None) == sz.E_CODEBOOK
    assert sz.splitzip_compress(O.BF16, fake, 10, cb, 1, 0, fake, 100, None, None) == sz.E_CAPACITY
    two = np.stack([cb, cb])
    assert sz.splitzip_compress(O.BF16, fake, 200000, two, 2, 65536, fake, 1 << 30, None, None) == sz.E_INVALID
    assert sz.splitzip_compress(O.BF16, fake, 100, two, 2, 1000, fake, 1 << 30, None, None) == sz.E_INVALID
    assert sz.splitzip_decompress(fake, 63, O.BF16, 10, fake, None, None) == sz.E_INVALID
    # the static-scratch encoder refuses a bad dtype and inputs beyond its limit first
    assert sz.splitzip_compress_static(3, fake, 10, cb, 1, 0, fake, 1 << 30, None, None) == sz.E_INVALID
    assert sz.splitzip_compress_static(O.BF16, fake, 2048 * 8192 + 1, cb, 1, 0, fake, 1 << 40, None,
                                       None) == sz.E_TOO_LARGE
    assert sz.splitzip_compress_static(O.E5M2, fake, 2048 * 16384 + 1, cb, 1, 0, fake, 1 << 40, None,
                                       None) == sz.E_TOO_LARGE
    assert sz.splitzip_decompress(fake, 1000, 7, 10, fake, None, None) == sz.E_INVALID
    assert sz.splitzip_decompress(fake, 1000, O.BF16, 10, fake + 8, None, None) == sz.E_INVALID
    assert sz.status_string(sz.E_CORRUPT) == "corrupt stream"


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "lossless_kv_cache_splitzip_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.replace("oracle`", ""), fn


def test_pipeline_sizes_and_argument_errors():
    # sizes: two device slots and one host slot per depth step, each slot at
    # least the group's worst-case stream with workspace
    G = 4 * 65536
    d, h = sz.splitzip_pipeline_sizes(O.BF16, 10 * G + 12345, 1, 0, G, 3)
    slot = -(-max(sz.splitzip_max_compressed_size(O.BF16, G, 1), 2 * G) // 256) * 256
    assert d == 2 * 3 * slot and h == 3 * slot + 256  # 11 groups: 88 bytes of sizes
    # per-layer codebooks: groups of whole segments carry several codebooks
    seg = 2 * 65536
    d2, _ = sz.splitzip_pipeline_sizes(O.BF16, 8 * seg, 8, seg, 2 * seg, 2)
    assert d2 >= 4 * sz.splitzip_max_compressed_size(O.BF16, 2 * seg, 2)
    bad = [
        (O.BF16, 1 << 20, 1, 0, 65536, 1),        # depth 1
        (O.BF16, 1 << 20, 1, 0, 65536, 33),       # depth > 32
        (O.BF16, 1 << 20, 1, 0, 65536 + 8, 2),    # group not whole chunks
        (O.BF16, 1 << 20, 1, 0, 0, 2),            # empty group
        (7, 1 << 20, 1, 0, 65536, 2),             # dtype
        (O.BF16, 1 << 20, 0, 0, 65536, 2),        # no codebook
        (O.BF16, 1 << 20, 4, 3 * 65536, 2 * 65536, 2),   # group neither divides nor is divided by segment
        (O.BF16, 1 << 20, 2, 65536, 65536, 2),    # codebooks do not cover n
    ]
    for args in bad:
        with pytest.raises(sz.SplitZipError) as e:
            sz.splitzip_pipeline_sizes(*args)
        assert e.value.status == sz.E_INVALID, args


def test_calibrate_device_work_bytes_and_argument_errors():
    assert sz.splitzip_calibrate_device_work_bytes(O.BF16, 1) == 256 * 8
    assert sz.splitzip_calibrate_device_work_bytes(O.E5M2, 80) == 80 * 32 * 8
    assert sz.splitzip_calibrate_device_work_bytes(O.BF16, 0) == 0
    assert sz.splitzip_calibrate_device_work_bytes(9, 1) == 0
    # rejected on the host before any GPU work: fake (never dereferenced)
    # 16-aligned addresses
    p, w = 1 << 20, 1 << 21
    cases = [
        ((O.BF16, 0, 100, 0, 1, p, w, 4096, None), sz.E_INVALID),       # null samples
        ((O.BF16, p + 2, 100, 0, 1, p, w, 4096, None), sz.E_INVALID),   # misaligned samples
        ((O.BF16, p, 100, 0, 1, 0, w, 4096, None), sz.E_INVALID),       # null output
        ((O.BF16, p, 100, 0, 1, p, 0, 4096, None), sz.E_INVALID),       # null work
        ((O.BF16, p, 100, 0, 1, p, w, 100, None), sz.E_CAPACITY),       # work too small
        ((O.BF16, p, 100, 10, 4, p, w, 1 << 16, None), sz.E_INVALID),   # segments do not cover n
        ((O.BF16, p, 100, 0, 4, p, w, 1 << 16, None), sz.E_INVALID),    # K > 1 needs a segment length
        ((7, p, 100, 0, 1, p, w, 4096, None), sz.E_INVALID),            # dtype
    ]
    for args, want in cases:
        assert sz.splitzip_calibrate_device(*args) == want, args


def test_variant_max_size_and_argument_errors():
    for v in (sz.VARIANT_TOP15_SENTINEL, sz.VARIANT_TOP8):
        for n, k in [(0, 1), (1, 1), (8191, 1), (1 << 20, 4)]:
            cap = sz.splitzip_variant_max_compressed_size(v, n, k)
            assert cap >= O.variant_max_size(v, n, k) and cap % 256 == 0
            # the workspace stages up to 512 escape records per 8192-element tile, 1024 for top-8
            slot = 1024 if v == sz.VARIANT_TOP8 else 512
            assert cap >= O.variant_max_size(v, n, k) + (4 * slot + 4) * (-(-n // 8192))
    assert sz.splitzip_variant_max_compressed_size(0, 100, 1) == 0
    assert sz.splitzip_variant_max_compressed_size(3, 100, 1) == 0
    lib = sz.load()
    cb = np.arange(16, dtype=np.uint8)
    p = 1 << 20
    assert lib.splitzip_variant_compress(3, p, 100, cb.ctypes.data, 1, 0, p, 1 << 20, None, None) == sz.E_INVALID
    assert lib.splitzip_variant_compress(1, p, 100, cb.ctypes.data, 1, 0, p, 100, None, None) == sz.E_CAPACITY
    dup = cb.copy()
    dup[3] = dup[4]
    assert lib.splitzip_variant_compress(2, p, 100, dup.ctypes.data, 1, 0, p, 1 << 20, None, None) == sz.E_CODEBOOK
    assert lib.splitzip_variant_decompress(0, p, 4096, 100, p, None, None) == sz.E_INVALID
    assert lib.splitzip_variant_decompress(1, p, 32, 100, p, None, None) == sz.E_INVALID   # shorter than a header


def test_raw_wrappers_refuse_short_host_arrays():
    # the library would read 16 x n_codebooks bytes, or write one u64 per
    # group, through these pointers: the wrappers refuse arrays that are too short
    fake = 1 << 20
    cb = np.arange(16, dtype=np.uint8)
    with pytest.raises(ValueError):
        sz.splitzip_compress(O.BF16, fake, 10, cb, 2, 65536, fake, 1 << 30, None, None)
    with pytest.raises(ValueError):
        sz.splitzip_compress_static(O.BF16, fake, 10, cb[:8], 1, 0, fake, 1 << 30, None, None)
    with pytest.raises(ValueError):
        sz._native.splitzip_pipeline_transfer(O.BF16, fake, 3 * 65536, cb, 1, 0, 65536, 2, True, fake, 1 << 20,
                                              fake, 1 << 20, fake, None, np.zeros(2, np.uint64), [0, 0, 0, 0])
    with pytest.raises(ValueError):
        sz._native.splitzip_pipeline_transfer(O.BF16, fake, 3 * 65536, cb, 1, 0, 65536, 2, True, fake, 1 << 20,
                                              fake, 1 << 20, fake, None, np.zeros(3, np.int64), [0, 0, 0, 0])
