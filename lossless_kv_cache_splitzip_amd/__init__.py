"""libsplitzip: the SplitZip lossless exponent codec for BF16 / FP8 E5M2 KV
caches on AMD Instinct MI355X (gfx950), hand-written HIP behind a C ABI.

The C ABI is declared in ``include/splitzip.h``; ``_native`` binds it with
ctypes (marshalling only).  Build the library with
``python -m lossless_kv_cache_splitzip_amd.build``.
"""
from ._native import (  # noqa: F401
    BF16,
    E_CAPACITY,
    E_CODEBOOK,
    E_CORRUPT,
    E_HIP,
    E_INVALID,
    E_TOO_LARGE,
    EXPORTS,
    FP8_E5M2,
    LIB_PATH,
    OK,
    VARIANT_TOP15_SENTINEL,
    VARIANT_TOP8,
    Pipeline,
    SplitZipError,
    calibrate_device,
    compress,
    compress_static,
    decompress,
    load,
    splitzip_calibrate,
    splitzip_calibrate_device,
    splitzip_calibrate_device_work_bytes,
    splitzip_compress,
    splitzip_compress_static,
    splitzip_decompress,
    splitzip_max_compressed_size,
    splitzip_pipeline_sizes,
    splitzip_pipeline_transfer,
    status_string,
    splitzip_variant_max_compressed_size,
    variant_compress,
    variant_decompress,
)
