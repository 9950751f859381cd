"""Benchmark of the SplitZip exponent codec on one MI355X.

One step = compress + decompress of the whole workload (every step of the
hot path: split, code map, nibble/sign|mantissa packing, escape compaction and
device-wide offset scan, header; then LUT decode, recombine, escape overwrite).
Inputs are resident in HBM before the timed region.  Prints one JSON line.

Default workload: Llama-3-8B-shaped prefill KV cache, BF16
[32 layers, 2, 8192 tokens, 8 kv heads, 128] = 1 GiB, per-layer codebooks.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "lossless_kv_cache_splitzip_amd", "csrc", "splitzip.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def ceiling_lib():
    """The copy / read ceiling kernels (libszceiling.so, built beside
    libsplitzip.so)."""
    import ctypes
    path = os.path.join(ROOT, "lossless_kv_cache_splitzip_amd", "libszceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} missing: build with `python -m lossless_kv_cache_splitzip_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz_t = ctypes.c_void_p, ctypes.c_size_t
    lib.szceiling_copy.argtypes = [vp, vp, sz_t, vp]
    lib.szceiling_copy.restype = ctypes.c_int
    lib.szceiling_read.argtypes = [vp, sz_t, vp, ctypes.c_uint32, vp]
    lib.szceiling_read.restype = ctypes.c_int
    return lib


def ceiling_leg(src, stream, reps: int = 20):
    """Measured ceilings on `src` (a device tensor, the timed workload):
    the hand-written copy kernel (16 bytes per lane, non-temporal; read +
    write bytes / time), the read-only kernel (bytes / time) and torch's
    device-to-device copy (hipMemcpy path), each the median of `reps`
    event-timed launches after 3 warm-ups."""
    import numpy as np
    import torch

    lib = ceiling_lib()
    b = src.view(torch.uint8)
    nbytes = b.numel() - b.numel() % 16
    dst = torch.empty_like(b)
    hits = torch.zeros(1, dtype=torch.int32, device=b.device)
    sh = stream.cuda_stream

    def timed(f, moved):
        for _ in range(3):
            f()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            f()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([moved / (e0.elapsed_time(e1) / 1e3) / 1e9 for e0, e1 in ev]))

    def copy():
        assert lib.szceiling_copy(b.data_ptr(), dst.data_ptr(), nbytes, sh) == 0

    def read():
        assert lib.szceiling_read(b.data_ptr(), nbytes, hits.data_ptr(), 0x9E3779B9, sh) == 0

    res = {"copy_kernel_GBps": timed(copy, 2 * nbytes), "read_kernel_GBps": timed(read, nbytes),
           "memcpy_d2d_GBps": timed(lambda: dst.copy_(b), 2 * b.numel()), "bytes": int(b.numel())}
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], b[:nbytes])
    del dst
    return res


def lscpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # noqa: BLE001 - fall back to /proc/cpuinfo
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def counter_traffic(kernels, workload: str):
    """HBM bytes per call (summed over the given kernels) from the committed
    rocprofv3 counter summary of this workload, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(PROFILES, f"{workload}_trace_and_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != source_digest():
        return None
    total = 0.0
    for k in kernels:
        t = re.search(r"hbm_bytes_per_launch\[" + re.escape(k) + r"\]:\s*([0-9.eE+]+)", text)
        if not t:
            return None
        total += float(t.group(1))
    return total


def cpu_baseline(wl, cbs, budget_s: float, threads: int):
    """The oracle as it stands (single-threaded C), timed on whole layers of
    the timed GPU tensor itself (copied to the host) with the codebooks the
    GPU used, one layer after another, until about budget_s seconds of CPU
    work (at least one layer): compress, then decompress.  The same layers
    are then run again, one layer per thread on `threads` host threads (the
    oracle's C calls release the GIL), as the chunk-parallel CPU figure."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import kvsynth
    import oracle

    spec = wl.spec
    dtype = spec.dtype
    per_layer = cbs.shape[0] > 1
    layer_n = spec.layer_elems if per_layer else wl.n
    n_layers = spec.layers if per_layer else 1
    done = raw = 0
    t_enc = t_dec = 0.0
    layers = []
    while done < n_layers and (t_enc + t_dec) < budget_s:
        x = kvsynth.to_numpy_bits(wl.data[done * layer_n:(done + 1) * layer_n])
        cb = cbs[done if per_layer else 0]
        t0 = time.perf_counter()
        s = oracle.compress(dtype, x, cb)
        t1 = time.perf_counter()
        y = oracle.decompress(s, dtype, x.size)
        t2 = time.perf_counter()
        assert np.array_equal(y, x)
        t_enc += t1 - t0
        t_dec += t2 - t1
        raw += x.nbytes
        done += 1
        layers.append((x, cb))
    model = lscpu_model()
    serial = {
        "value": raw / (t_enc + t_dec) / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {n_layers} layers ({raw / 2**20:.0f} MiB raw) of the timed workload: the same bytes "
                  f"as the GPU run (copied from the device tensor) and the same per-layer codebooks, "
                  f"compress + decompress, one thread",
        "cpu_model": model,
        "encode_GBps": raw / t_enc / 1e9,
        "decode_GBps": raw / t_dec / 1e9,
    }

    def one(item):
        x, cb = item
        s = oracle.compress(dtype, x, cb)
        return np.array_equal(oracle.decompress(s, dtype, x.size), x)

    threads = max(1, min(threads, len(layers)))
    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        ok = all(pool.map(one, layers))
        t1 = time.perf_counter()
    assert ok
    parallel = {
        "value": raw / (t1 - t0) / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the same {done} layers, compress + decompress, one layer per thread on {threads} threads",
        "cpu_model": model,
    }
    return serial, parallel


def link_leg(wl, cbs, seg, dtype, reps: int = 5):
    """The pages' transfer setting on one GPU: the workload moves through
    pinned host memory over PCIe in groups of 32 MiB of raw data (one layer
    of the 1 GiB cache; 4 to 128 MiB and depths 3 to 8 measured, 32 MiB at
    depth 4 fastest), up to 4 groups in flight, raw and compressed (compress
    -> copy to host -> copy back -> decompress, copies by the copy engines).
    Wall time of the blocking pipelined call, after one warm-up of each:
    `reps` raw and compressed transfers alternate, so a spell of slower host
    copies (the host's PCIe and memory are shared with other work) falls on
    both; the best of each and the median of the pairs' ratios are reported.
    As context, the copy engines moving the whole tensor to host and back at
    once."""
    import numpy as np
    import torch

    import lossless_kv_cache_splitzip_amd as sz

    elem = wl.data.element_size()
    group = (32 << 20) // elem
    if seg and seg % group and group % seg:
        group = seg
    out = torch.empty_like(wl.data)
    status = torch.zeros(1, dtype=torch.int32, device=wl.data.device)
    res = {}
    times = {"raw": [], "compressed": []}
    with sz.Pipeline(dtype, wl.n, cbs, seg, group, 4, device=wl.data.device) as p:
        best = {m: (float("inf"), 0, 0.0) for m in times}
        for r in range(reps + 1):
            for mode in times:
                torch.cuda.synchronize()
                t0, c0 = time.perf_counter(), time.process_time()
                sizes = p.transfer(wl.data, out, compress=(mode == "compressed"), status=status)
                t1, c1 = time.perf_counter(), time.process_time()
                assert int(status.item()) == 0 and torch.equal(out.view(torch.uint8), wl.data.view(torch.uint8))
                if r:  # the first pair warms up
                    times[mode].append((t1 - t0) * 1e3)
                    if t1 - t0 < best[mode][0]:
                        best[mode] = (t1 - t0, int(sizes.sum()), (c1 - c0) / (t1 - t0))
        for mode, (t, sent, cpu_frac) in best.items():
            res[mode] = (t * 1e3, sent, cpu_frac)
    # copy engines: the whole tensor to pinned host memory, and a second
    # pinned buffer to the device, concurrently (both link directions)
    src = wl.data.view(torch.uint8)
    h1 = torch.empty(src.numel(), dtype=torch.uint8, pin_memory=True)
    h2 = torch.empty(src.numel(), dtype=torch.uint8, pin_memory=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    dma = float("inf")
    for r in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            h1.copy_(src, non_blocking=True)
        with torch.cuda.stream(s2):
            out.view(torch.uint8).copy_(h2, non_blocking=True)
        torch.cuda.synchronize()
        if r:
            dma = min(dma, time.perf_counter() - t0)
    del h1, h2, out
    raw_ms, raw_sent, raw_cpu = res["raw"]
    c_ms, c_sent, c_cpu = res["compressed"]
    return {
        "link": "pinned host memory over PCIe, copy engines both ways",
        "group_elems": group, "depth": 4,
        "raw_ms": raw_ms, "compressed_ms": c_ms, "speedup": raw_ms / c_ms,
        "speedup_paired_median": float(np.median([a / b for a, b in zip(times["raw"], times["compressed"])])),
        "raw_ms_all": times["raw"], "compressed_ms_all": times["compressed"],
        "raw_bytes": raw_sent, "compressed_bytes": c_sent,
        "raw_GBps": wl.raw_bytes / (raw_ms / 1e3) / 1e9,
        "compressed_GBps": wl.raw_bytes / (c_ms / 1e3) / 1e9,
        "copy_engines_both_ways_ms": dma * 1e3,
        # host CPU time of the process during the best transfer, per second of it
        "host_cpu_per_wall_raw": raw_cpu, "host_cpu_per_wall_compressed": c_cpu,
    }


def calibrate_leg(wl, seg, cbs, stream, reps: int = 10):
    """On-device calibration of the workload's codebooks (one per layer, one
    call), the step the pages keep offline: event-timed mean of `reps` calls
    after two warm-ups; the codebooks are checked against the host ones."""
    import numpy as np
    import torch

    import lossless_kv_cache_splitzip_amd as sz

    k = cbs.shape[0]
    seg_k = seg if k > 1 else 0
    out = torch.empty((k, 16), dtype=torch.uint8, device=wl.data.device)
    work = torch.empty(sz.splitzip_calibrate_device_work_bytes(wl.spec.dtype, k), dtype=torch.uint8,
                       device=wl.data.device)
    for _ in range(2):
        sz.calibrate_device(wl.data, k, seg_k, out=out, work=work, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        sz.calibrate_device(wl.data, k, seg_k, out=out, work=work, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the bench's codebooks come from separate calibration draws; the device
    # codebooks of the data itself are checked against the host routine on
    # the first layer
    xh = kvsynth_bits(wl.data[:seg if k > 1 else wl.n])
    assert np.array_equal(out[0].cpu().numpy(), sz.splitzip_calibrate(wl.spec.dtype, xh))
    return {"codebooks": k, "ms": ms, "GBps": wl.raw_bytes / (ms / 1e3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": wl.raw_bytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": wl.raw_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS}}


def ablation_leg(wl, cbs, seg, stream, main_enc_ms, main_dec_ms, reps: int = 10):
    """The pages' two rejected designs on the same workload (BF16 only):
    top-15 + sentinel and top-8 3-bit codes.  Event-timed mean of `reps`
    compress and decompress calls after a checked warm-up round trip."""
    import numpy as np
    import torch

    import lossless_kv_cache_splitzip_amd as sz

    res = {}
    for name, v in (("top15_sentinel", sz.VARIANT_TOP15_SENTINEL), ("top8", sz.VARIANT_TOP8)):
        out, nb = sz.variant_compress(v, wl.data, cbs, seg, stream=stream)
        dec = torch.empty_like(wl.data)
        status = torch.zeros(1, dtype=torch.int32, device=wl.data.device)
        sz.variant_decompress(v, out, wl.n, out=dec, status=status, stream=stream)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and torch.equal(dec.view(torch.uint8), wl.data.view(torch.uint8))
        n_bytes = int(nb.item())
        n_esc = int(np.frombuffer(out[16:24].cpu().numpy().tobytes(), "<u8")[0])
        times = {}
        for what in ("enc", "dec"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                if what == "enc":
                    sz.variant_compress(v, wl.data, cbs, seg, out=out, out_bytes=nb, stream=stream)
                else:
                    sz.variant_decompress(v, out, wl.n, out=dec, status=status, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times[what] = e0.elapsed_time(e1) / reps
        res[name] = {"compression_ratio": wl.raw_bytes / n_bytes, "escape_rate": n_esc / wl.n,
                     "encode_ms": times["enc"], "decode_ms": times["dec"],
                     "decode_GBps": wl.raw_bytes / (times["dec"] / 1e3) / 1e9,
                     "decode_slowdown_vs_top16": times["dec"] / main_dec_ms,
                     "encode_slowdown_vs_top16": times["enc"] / main_enc_ms}
        del out, dec
    return res


def per_layer_graph_leg(reps: int = 50):
    """One-layer calls as a serving stack makes them, layer by layer: the
    4 MiB one-layer BF16 workload (kv_layer_bf16), per-call time of `reps`
    back-to-back eager calls against one replay of a HIP graph holding `reps`
    captured calls (event-timed).  The replayed stream must equal the eager
    one and the round trip must be exact."""
    import numpy as np
    import torch

    import kvsynth
    import lossless_kv_cache_splitzip_amd as sz

    wl = kvsynth.make("kv_layer_bf16", device="cuda")
    d = wl.spec.dtype
    cbs = np.stack([sz.splitzip_calibrate(d, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    cap = sz.splitzip_max_compressed_size(d, wl.n, cbs.shape[0])
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    y = torch.empty_like(wl.data)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            sz.compress(wl.data, cbs, out=out, out_bytes=nb)
            sz.decompress(out, wl.n, d, out=y, status=st, in_bytes=cap)
    torch.cuda.synchronize()
    eager_stream = out[:int(nb.item())].clone()

    def enc():
        for _ in range(reps):
            sz.compress(wl.data, cbs, out=out, out_bytes=nb)

    def dec():
        for _ in range(reps):
            sz.decompress(out, wl.n, d, out=y, status=st, in_bytes=cap)

    out_s = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb_s = torch.zeros(1, dtype=torch.int64, device="cuda")

    def enc_static():
        for _ in range(reps):
            sz.compress_static(wl.data, cbs, out=out_s, out_bytes=nb_s)

    with torch.cuda.stream(side):
        enc_static()
    torch.cuda.synchronize()
    assert torch.equal(out_s[:int(nb_s.item())], eager_stream)
    graphs = {}
    for name, f in (("enc", enc), ("dec", dec), ("enc_static", enc_static)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs[name] = g
    torch.cuda.synchronize()

    def per_call_us(f):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f()
        torch.cuda.synchronize()
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    def host_us(f, calls: int = 200):
        """Host time per call, nothing synchronized inside the loop."""
        import time as _t
        f()
        torch.cuda.synchronize()
        t0 = _t.perf_counter()
        for _ in range(calls):
            f()
        t1 = _t.perf_counter()
        torch.cuda.synchronize()
        return (t1 - t0) / calls * 1e6

    lib = sz.load()
    s0 = torch.cuda.current_stream().cuda_stream
    cb_bytes = np.ascontiguousarray(cbs, dtype=np.uint8).tobytes()
    S = int(nb.item())
    host = {
        "python_compress": host_us(lambda: sz.compress(wl.data, cbs, out=out, out_bytes=nb)),
        "python_compress_static": host_us(lambda: sz.compress_static(wl.data, cbs, out=out_s, out_bytes=nb_s)),
        "python_decompress": host_us(lambda: sz.decompress(out, wl.n, d, out=y, status=st, in_bytes=cap)),
        "c_compress": host_us(lambda: lib.splitzip_compress(d, wl.data.data_ptr(), wl.n, cb_bytes, 1, 0,
                                                            out.data_ptr(), cap, nb.data_ptr(), s0)),
        "c_compress_static": host_us(lambda: lib.splitzip_compress_static(d, wl.data.data_ptr(), wl.n, cb_bytes, 1, 0,
                                                                          out_s.data_ptr(), cap, nb_s.data_ptr(), s0)),
        "c_decompress": host_us(lambda: lib.splitzip_decompress(out.data_ptr(), S, d, wl.n, y.data_ptr(),
                                                                st.data_ptr(), s0)),
    }

    res = {"workload": "kv_layer_bf16", "raw_bytes": wl.raw_bytes, "calls": reps,
           # host time per call without synchronization: eager calls through the
           # Python binding are partly host-bound
           "host_us_per_call": host,
           "eager_encode_us": per_call_us(enc), "eager_decode_us": per_call_us(dec),
           "graph_encode_us": per_call_us(graphs["enc"].replay), "graph_decode_us": per_call_us(graphs["dec"].replay),
           # splitzip_compress_static: one launch, workspace in the library's own memory
           "eager_encode_static_us": per_call_us(enc_static),
           "graph_encode_static_us": per_call_us(graphs["enc_static"].replay)}
    y.zero_()
    out_s.zero_()
    graphs["enc"].replay()
    graphs["dec"].replay()
    graphs["enc_static"].replay()
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and torch.equal(out[:int(nb.item())], eager_stream)
    assert torch.equal(out_s[:int(nb_s.item())], eager_stream)
    assert torch.equal(y.view(torch.uint8), wl.data.view(torch.uint8))
    return res


WORKLOADS = ["kv_layer_bf16", "llama3_8b_kv_bf16", "long_ctx_heavy_tail_bf16", "edge_const_exponent",
             "edge_uniform_bits", "edge_special_values", "llama3_70b_kv_e5m2"]


def algorithmic_bytes(dtype: int, n: int, n_esc: int) -> int:
    """Bytes a compress (or decompress) call must move: the raw values, the
    codes, the sign|mantissa section and 3 bytes per escape."""
    import kvsynth
    raw = n * (2 if dtype == kvsynth.BF16 else 1)
    dense = (n + 1) // 2 + (n if dtype == kvsynth.BF16 else 3 * ((n + 7) // 8))
    return raw + dense + 3 * n_esc


def make_evict(dev, stream):
    """Before a cold call: 512 MiB written, then a separate 768 MiB read (the
    memory-side cache holds 256 MB), so the timed call finds neither its own
    data cached nor dirty lines of the eviction left to write back."""
    import torch
    lib = ceiling_lib()
    w = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    r = torch.zeros(768 << 20, dtype=torch.uint8, device=dev)
    hits = torch.zeros(1, dtype=torch.int32, device=dev)

    def evict(i: int):
        w.fill_(i & 0xFF)
        assert lib.szceiling_read(r.data_ptr(), r.numel(), hits.data_ptr(), 0x9E3779B9, stream.cuda_stream) == 0

    return evict


def warm_up(fs, min_s: float = 0.2):
    """Runs the calls in `fs` in turn for at least min_s seconds (and three
    rounds): the GPU's clocks ramp up under load after an idle spell."""
    import time as _t
    import torch
    t0 = _t.perf_counter()
    r = 0
    while r < 3 or _t.perf_counter() - t0 < min_s:
        for f in fs:
            f()
        torch.cuda.synchronize()
        r += 1


def timed_calls_ms(f, stream, reps: int, evict=None):
    """Mean event time (ms) of `reps` calls of f on `stream`; with `evict`,
    the caches are flushed of f's data before each call, outside the timed
    interval."""
    import numpy as np
    import torch
    ev = []
    for i in range(reps):
        if evict is not None:
            evict(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def workload_leg(name, dev, stream, evict, reps: int = 10, prebuilt=None):
    """One workload at full size: warm (back-to-back calls) and cold (the
    memory-side cache evicted before each call) event-timed compress and
    decompress, the copy-kernel ceiling on its input, ratio, escape rate,
    algorithmic bytes and roofline fractions.  The round trip is checked."""
    import numpy as np
    import torch

    import kvsynth
    import lossless_kv_cache_splitzip_amd as sz

    if prebuilt is None:
        wl = kvsynth.make(name, device=dev)
        cbs = np.stack([sz.splitzip_calibrate(wl.spec.dtype, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    else:
        wl, cbs = prebuilt
    d = wl.spec.dtype
    seg = wl.segment_elems if cbs.shape[0] > 1 else 0
    cap = sz.splitzip_max_compressed_size(d, wl.n, cbs.shape[0])
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.int64, device=dev)
    y = torch.empty_like(wl.data)
    st = torch.zeros(1, dtype=torch.int32, device=dev)

    def enc():
        sz.compress(wl.data, cbs, seg, out=out, out_bytes=nb, stream=stream)

    def dec():
        sz.decompress(out, wl.n, d, out=y, status=st, in_bytes=cap, stream=stream)

    enc()
    dec()
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and torch.equal(y.view(torch.uint8), wl.data.view(torch.uint8)), name
    S = int(nb.item())
    E = int(np.frombuffer(out[16:24].cpu().numpy().tobytes(), "<u8")[0])
    warm_up([enc, dec])
    t = {"encode_ms": timed_calls_ms(enc, stream, reps), "decode_ms": timed_calls_ms(dec, stream, reps),
         "encode_cold_ms": timed_calls_ms(enc, stream, reps, evict),
         "decode_cold_ms": timed_calls_ms(dec, stream, reps, evict)}
    ceil = ceiling_leg(wl.data, stream, reps=10)
    alg = algorithmic_bytes(d, wl.n, E)
    raw = wl.raw_bytes
    res = {"element_type": "bf16" if d == kvsynth.BF16 else "fp8_e5m2", "elements": wl.n, "raw_bytes": raw,
           "codebooks": int(cbs.shape[0]), "compression_ratio": raw / S, "escape_rate": E / wl.n,
           "algorithmic_bytes": alg, "copy_kernel_GBps": ceil["copy_kernel_GBps"]}
    for k, ms in t.items():
        what = k.replace("_ms", "")
        res[k] = ms
        res[what + "_GBps"] = raw / (ms / 1e3) / 1e9                     # raw bytes per second
        res[what + "_frac_of_8TBps"] = alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS  # algorithmic bytes
        res[what + "_frac_of_copy_kernel"] = alg / (ms / 1e3) / 1e9 / ceil["copy_kernel_GBps"]
    del out, y, nb, st
    if prebuilt is None:
        del wl
    torch.cuda.empty_cache()
    return res


def kvsynth_bits(t):
    import kvsynth
    return kvsynth.to_numpy_bits(t)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_kv_bf16")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1),
                    help="host threads of the parallel oracle run (at most 16 by default)")
    ap.add_argument("--no-link", action="store_true", help="skip the pipelined host-link transfer leg")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the one-layer graph leg (its calls launch the same kernels on a 4 MiB input)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload map")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the timed steps and the copy ceiling (for rocprofv3 runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this codec benchmark runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.profile_run:
        args.no_link = args.no_layer = args.no_workloads = True
        args.cpu_budget = 0

    import numpy as np
    import torch

    import kvsynth
    import lossless_kv_cache_splitzip_amd as sz

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {args.workload} on {torch.cuda.get_device_name(dev)}")
    wl = kvsynth.make(args.workload, device=dev)
    dtype = wl.spec.dtype
    cbs = np.stack([sz.splitzip_calibrate(dtype, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    seg = wl.segment_elems if cbs.shape[0] > 1 else 0
    n = wl.n
    raw = wl.raw_bytes
    cap = sz.splitzip_max_compressed_size(dtype, n, cbs.shape[0])
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    out_bytes = torch.zeros(1, dtype=torch.int64, device=dev)
    dec = torch.empty_like(wl.data)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        sz.compress(wl.data, cbs, seg, out=out, out_bytes=out_bytes, stream=stream)
        e_mid.record(stream)
        sz.decompress(out, n, dtype, out=dec, status=status, in_bytes=cap, stream=stream)

    # correctness of the timed configuration
    e_mid = torch.cuda.Event(enable_timing=True)
    step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(dec.view(torch.uint8), wl.data.view(torch.uint8)), \
        "round trip failed"
    stream_bytes = int(out_bytes.item())
    n_esc = int(np.frombuffer(out[16:24].cpu().numpy().tobytes(), "<u8")[0])
    log(f"[bench] n={n} codebooks={cbs.shape[0]} stream={stream_bytes} escapes={n_esc} "
        f"ratio={raw / stream_bytes:.4f}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b, c in ev:
        a.record(stream)
        e_mid = b
        step()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    dec_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, encode {enc_ms:.3f} ms, decode {dec_ms:.3f} ms")

    # measured ceilings on the same input: hand-written copy and read kernels,
    # and torch's device-to-device copy
    ceil = ceiling_leg(wl.data, stream)
    copy_gbps = ceil["copy_kernel_GBps"]
    log(f"[bench] copy kernel {copy_gbps:.0f} GB/s, read kernel {ceil['read_kernel_GBps']:.0f} GB/s, "
        f"torch copy {ceil['memcpy_d2d_GBps']:.0f} GB/s")

    alg = algorithmic_bytes(dtype, n, n_esc)   # same for encode (read raw, write stream) and decode
    enc_gbps = alg / (enc_ms / 1e3) / 1e9
    dec_gbps = alg / (dec_ms / 1e3) / 1e9
    sfx = "bf16" if dtype == kvsynth.BF16 else "e5m2"
    # the launches of one compress call: a prep launch only for more than 128
    # codebooks (else the header work rides in another launch), the block
    # sums only for more than 64 blocks of 64 tiles
    tiles = -(-n // (8192 if dtype == kvsynth.BF16 else 16384))
    enc_kernels = (["prep_kernel"] if cbs.shape[0] > 128 else []) + [f"encode_dense_{sfx}_kernel"] + \
        (["encode_sums_kernel"] if -(-tiles // 64) > 64 else []) + [f"encode_place_{sfx}_kernel"]
    dname = f"decode_{sfx}_kernel"

    # the host-link leg first: host copies measured slower after the legs below
    link = None if args.no_link else link_leg(wl, cbs, seg, dtype)
    if link:
        log(f"[bench] link: raw {link['raw_ms']:.2f} ms, compressed {link['compressed_ms']:.2f} ms, "
            f"speedup {link['speedup']:.3f} (paired median {link['speedup_paired_median']:.3f}), host CPU {link['host_cpu_per_wall_compressed']:.2f} s per s")
    workloads = None
    if not args.no_workloads:
        evict = make_evict(dev, stream)
        workloads = {}
        for name in WORKLOADS:
            log(f"[bench] workload {name}")
            workloads[name] = workload_leg(name, dev, stream, evict,
                                           prebuilt=(wl, cbs) if name == args.workload else None)
            r = workloads[name]
            log(f"[bench]   ratio {r['compression_ratio']:.4f} escapes {100 * r['escape_rate']:.2f}% "
                f"encode {r['encode_GBps']:.0f} GB/s ({r['encode_frac_of_8TBps']:.3f}; cold "
                f"{r['encode_cold_frac_of_8TBps']:.3f}) decode {r['decode_GBps']:.0f} GB/s "
                f"({r['decode_frac_of_8TBps']:.3f}; cold {r['decode_cold_frac_of_8TBps']:.3f})")
        del evict
        torch.cuda.empty_cache()
    abl = calib = layer = None
    if not args.profile_run:
        abl = ablation_leg(wl, cbs, seg, stream, enc_ms, dec_ms) if dtype == kvsynth.BF16 else None
        if abl:
            for k, r in abl.items():
                log(f"[bench] {k}: ratio {r['compression_ratio']:.4f}, escapes {100 * r['escape_rate']:.2f}%, "
                    f"decode {r['decode_ms']:.3f} ms ({r['decode_slowdown_vs_top16']:.2f}x top-16)")
        calib = calibrate_leg(wl, seg, cbs, stream)
        log(f"[bench] device calibration of {calib['codebooks']} codebooks: {calib['ms']:.3f} ms "
            f"({calib['GBps']:.0f} GB/s)")
    if not args.no_layer:
        layer = per_layer_graph_leg()
        log(f"[bench] one-layer calls: eager {layer['eager_encode_us']:.1f} / {layer['eager_decode_us']:.1f} us, "
            f"graph-replayed {layer['graph_encode_us']:.1f} / {layer['graph_decode_us']:.1f} us (encode / decode); "
            f"one-launch encode eager {layer['eager_encode_static_us']:.1f} us, "
            f"graph-replayed {layer['graph_encode_static_us']:.1f} us")
    cpu, cpu_par = cpu_baseline(wl, cbs, args.cpu_budget, args.cpu_threads) if args.cpu_budget > 0 else (None, None)

    line = {
        "metric": "encode & decode GB/s of raw BF16 KV, compression ratio, % of HBM roofline",
        "value": raw / (ms_per_step / 1e3) / 1e9,
        "unit": "GB/s (raw bytes per compress+decompress round trip)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16" if dtype == kvsynth.BF16 else "u8",
        "data": "synthetic",
        "config": {"workload": args.workload, "elements": n, "raw_bytes": raw,
                   "shape": [wl.spec.layers, 2, wl.spec.tokens, wl.spec.heads, wl.spec.head_dim],
                   "element_type": "bf16" if dtype == kvsynth.BF16 else "fp8_e5m2",
                   "codebooks": int(cbs.shape[0])},
        "encode_GBps": raw / (enc_ms / 1e3) / 1e9,
        "decode_GBps": raw / (dec_ms / 1e3) / 1e9,
        "encode_ms": enc_ms,
        "decode_ms": dec_ms,
        "compression_ratio": raw / stream_bytes,
        "escape_rate": n_esc / n,
        "copy_kernel_GBps": copy_gbps,
        "read_kernel_GBps": ceil["read_kernel_GBps"],
        "memcpy_d2d_GBps": ceil["memcpy_d2d_GBps"],
        # the longest single kernel of a step; a decompress call is exactly one
        # launch of it, so the event interval is its duration
        "roofline": {"bound": "hbm", "kernel": dname, "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dec_gbps / HBM_PEAK_GBPS, "frac_of_copy_kernel": dec_gbps / copy_gbps,
                     "frac_of_memcpy": dec_gbps / ceil["memcpy_d2d_GBps"],
                     "traffic": counter_traffic([dname], args.workload), "algorithmic_bytes": alg},
        # a compress call: the launches listed in "kernel"
        "roofline_encode": {"bound": "hbm", "kernel": "+".join(enc_kernels), "achieved": enc_gbps,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": enc_gbps / HBM_PEAK_GBPS,
                            "frac_of_copy_kernel": enc_gbps / copy_gbps,
                            "frac_of_memcpy": enc_gbps / ceil["memcpy_d2d_GBps"],
                            "traffic": counter_traffic(enc_kernels, args.workload), "algorithmic_bytes": alg},
        "cpu_baseline": cpu,
        "workloads": workloads,
        "link_transfer": link,
        "calibrate_device": calib,
        "ablations": abl,
        "per_layer_graph": layer,
        "cpu_baseline_parallel": cpu_par,
        "pages_context": {"encode_GBps": 613.3, "decode_GBps": 2181.8, "hardware": "not stated in the pages"},
        "kernel_source_sha256_16": source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
