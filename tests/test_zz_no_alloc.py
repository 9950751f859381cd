"""splitzip_compress_static, the compress entry point that allocates nothing
(its workspace is the library's own device array): called through the C ABI,
its stream equals splitzip_compress's byte for byte, on two calls in a row
(the second with a smaller input), at the size limit, with escape-heavy tiles
(placed by re-encoding), several and many codebooks, the exact minimum
capacity, an empty input, and replayed from a HIP graph.  Sizes beyond its
limit are refused before any GPU work.

Inputs of at most 512 tiles take one launch whose workgroups exchange escape
counts through the static array (each count carries an epoch taken from a
counter every workgroup advances, which keeps earlier calls' counts out):
covered at the 512/513-tile boundary, over a run of calls whose sizes rise
and fall (interleaved with the two-launch path), over enough calls for the
epoch to wrap, with codebooks that do not fit the kernel arguments, and with
the counts computed from the input (SPLITZIP_STATIC_WAIT_POLLS=0, so no
workgroup waits for another)."""
import os

import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
DEV = "cuda"


def _min_capacity(dtype, n, k):
    """Bytes of the largest stream, rounded up to 256 (the oracle's layout)."""
    return (O.max_size(dtype, n, k) + 255) // 256 * 256


def _reference(x, cbs, seg):
    """splitzip_compress's stream of x (the existing entry point)."""
    out, nb = sz.compress(x, cbs, seg)
    torch.cuda.synchronize()
    return out[:int(nb.item())].clone()


def _static(x, cbs, seg, cap=None, fill=0xA5):
    """splitzip_compress_static into a buffer of cap bytes (pre-filled, so
    bytes the call fails to write show up)."""
    dtype = sz._native._dtype_of(x)
    k = np.asarray(cbs).reshape(-1, 16).shape[0]
    cap = cap or _min_capacity(dtype, x.numel(), k)
    out = torch.full((cap,), fill, dtype=torch.uint8, device=DEV)
    nb = torch.zeros(1, dtype=torch.int64, device=DEV)
    rc = sz.splitzip_compress_static(dtype, x.data_ptr(), x.numel(), np.ascontiguousarray(cbs, dtype=np.uint8), k, seg,
                                     out.data_ptr(), cap, nb.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, out, int(nb.item())


def _check(x, cbs, seg, label):
    print(f"case static {label} n={x.numel()} k={np.asarray(cbs).reshape(-1, 16).shape[0]}", flush=True)
    want = _reference(x, cbs, seg)
    rc, out, nb = _static(x, cbs, seg)
    assert rc == sz.OK, sz.status_string(rc)
    assert nb == want.numel(), (nb, want.numel())
    assert torch.equal(out[:nb], want), f"{label}: stream differs from splitzip_compress's"
    dtype = sz._native._dtype_of(x)
    y, st = sz.decompress(out[:nb], x.numel(), dtype)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and torch.equal(y.view(torch.uint8), x.view(torch.uint8))
    return out[:nb]


def _layer(name, **kw):
    wl = kvsynth.make(name, device=DEV, **kw)
    cbs = np.stack([sz.splitzip_calibrate(wl.spec.dtype, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    return wl, cbs


def test_two_calls_in_a_row_second_smaller_bf16():
    wl, cbs = _layer("kv_layer_bf16")  # 2,097,152 values: 256 tiles
    got = _check(wl.data, cbs[:1], 0, "one layer")
    xh = kvsynth.to_numpy_bits(wl.data)
    assert np.array_equal(got.cpu().numpy(), O.compress(O.BF16, xh, cbs[:1]))
    small = wl.data[:300_001].contiguous()  # 37 tiles, ragged tail
    _check(small, cbs[:1], 0, "smaller, ragged")


def test_two_calls_in_a_row_second_smaller_e5m2():
    wl, cbs = _layer("llama3_70b_kv_e5m2", layers=3, tokens=1024)  # 3 layers of 2,097,152 values
    seg = wl.segment_elems
    _check(wl.data, cbs, seg, "3 layers, 3 codebooks")
    _check(wl.data[:2 * seg + 77].contiguous(), cbs, seg, "smaller, ragged")


def test_size_limit():
    x = kvsynth.random_bits(2048 * 8192, kvsynth.BF16, seed=3, device=DEV)  # exactly 2048 tiles
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(x[:100_000]))
    _check(x, cb, 0, "2048 tiles")
    y = kvsynth.random_bits(2048 * 16384, kvsynth.E5M2, seed=6, device=DEV)  # E5M2: 2048 tiles of 16384
    _check(y, O.calibrate(O.E5M2, kvsynth.to_numpy_bits(y[:100_000])), 0, "2048 E5M2 tiles")
    big = kvsynth.random_bits(2048 * 8192 + 1, kvsynth.BF16, seed=4, device=DEV)
    rc, _, _ = _static(big, cb, 0, cap=_min_capacity(O.BF16, big.numel(), 1))
    assert rc == sz.E_TOO_LARGE


def test_escape_heavy_tiles_and_capacity():
    # uniform bit patterns: every tile holds far more escapes than its
    # staging slot, so the placement pass encodes them again
    x = kvsynth.random_bits(600_001, kvsynth.BF16, seed=5, device=DEV, kind="uniform_bits")
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(x[:5000]))
    _check(x, cb, 0, "uniform bits")
    cap = _min_capacity(O.BF16, x.numel(), 1)
    rc, _, _ = _static(x, cb, 0, cap=cap - 1)
    assert rc == sz.E_CAPACITY
    rc, _, _ = _static(x, cb, 0, cap=cap)
    assert rc == sz.OK


def test_many_codebooks():
    # more codebooks than fit the kernel arguments: the header launches of their own
    x = kvsynth.random_bits(200 * 65536 + 3, kvsynth.BF16, seed=8, device=DEV, sigma=2.0)
    rng = np.random.default_rng(8)
    cbs = np.stack([rng.permutation(256)[:16] for _ in range(201)]).astype(np.uint8)
    _check(x, cbs, 65536, "201 codebooks")


def test_empty_input():
    x = torch.empty(0, dtype=torch.int16, device=DEV)
    cb = np.arange(16, dtype=np.uint8)
    rc, out, nb = _static(x, cb, 0)
    assert rc == sz.OK
    assert np.array_equal(out[:nb].cpu().numpy(), O.compress(O.BF16, np.zeros(0, np.uint16), cb))


def test_graph_replays_match_eager_calls():
    wl, cbs = _layer("kv_layer_bf16", tokens=512)
    x = wl.data.clone()
    cap = _min_capacity(O.BF16, x.numel(), 1)
    out = torch.empty(cap, dtype=torch.uint8, device=DEV)
    nb = torch.zeros(1, dtype=torch.int64, device=DEV)
    cb = np.ascontiguousarray(cbs[:1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up on the capture stream
        assert sz.compress_static(x, cb, out=out, out_bytes=nb)[0] is out
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sz.compress_static(x, cb, out=out, out_bytes=nb)
    torch.cuda.synchronize()
    for r in range(4):
        x.copy_(kvsynth.random_bits(x.numel(), kvsynth.BF16, seed=100 + r, device=DEV))
        torch.cuda.synchronize()
        want = _reference(x, cb, 0)
        g.replay()
        torch.cuda.synchronize()
        assert int(nb.item()) == want.numel() and torch.equal(out[:want.numel()], want), f"replay {r}"


def test_one_launch_boundary():
    for dtype, tile, seed in ((kvsynth.BF16, 8192, 11), (kvsynth.E5M2, 16384, 12)):
        x = kvsynth.random_bits(513 * tile, dtype, seed=seed, device=DEV, sigma=1.5)
        cb = O.calibrate(dtype, kvsynth.to_numpy_bits(x[:100_000]))
        _check(x[:512 * tile].contiguous(), cb, 0, f"512 tiles (one launch) dtype={dtype}")
        _check(x, cb, 0, f"513 tiles (two launches) dtype={dtype}")
        _check(x[:512 * tile - 5].contiguous(), cb, 0, f"512 tiles, ragged dtype={dtype}")


def test_one_launch_sizes_rise_and_fall():
    # count words of a larger earlier call must never pass for this call's
    x = kvsynth.random_bits(1000 * 8192, kvsynth.BF16, seed=13, device=DEV, sigma=2.0)
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(x[:100_000]))
    for tiles in (500, 3, 500, 1, 512, 1000, 200, 37, 512, 2):
        n = tiles * 8192 - (tiles % 3)
        _check(x[:n].contiguous(), cb, 0, f"{tiles} tiles in a run of calls")


def test_one_launch_codebooks_beyond_kernel_arguments():
    # 201 codebooks for 10 chunks: the header launch of its own, then the one launch
    x = kvsynth.random_bits(10 * 65536 - 9, kvsynth.BF16, seed=14, device=DEV, sigma=2.0)
    rng = np.random.default_rng(14)
    cbs = np.stack([rng.permutation(256)[:16] for _ in range(201)]).astype(np.uint8)
    _check(x, cbs, 65536, "201 codebooks, 10 chunks")


def test_one_launch_epoch_wraps():
    # the epoch is the arrival counter modulo 2^15: about 45,000 tiles over
    # 200 calls of cycling sizes cross the wrap at least once
    x = kvsynth.random_bits(512 * 8192, kvsynth.BF16, seed=16, device=DEV, sigma=2.0)
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(x[:100_000]))
    sizes = [512, 1, 300, 17, 512, 64, 2, 400, 511, 33]
    refs = {}
    for tiles in sizes:
        n = tiles * 8192 - (tiles % 5)
        refs[tiles] = (x[:n].contiguous(), _reference(x[:n].contiguous(), cb, 0))
    total = 0
    for call in range(200):
        tiles = sizes[call % len(sizes)]
        xi, want = refs[tiles]
        rc, out, nb = _static(xi, cb, 0)
        assert rc == sz.OK and nb == want.numel() and torch.equal(out[:nb], want), f"call {call}: {tiles} tiles"
        total += tiles
    assert total > 2 ** 15


@pytest.mark.parametrize("case", ["bf16 per-layer", "bf16 escape-heavy", "e5m2 per-layer"])
def test_one_launch_counts_computed_when_not_awaited(case):
    old = os.environ.get("SPLITZIP_STATIC_WAIT_POLLS")
    os.environ["SPLITZIP_STATIC_WAIT_POLLS"] = "0"
    try:
        if case == "bf16 per-layer":
            wl, cbs = _layer("llama3_8b_kv_bf16", layers=4, tokens=128)  # 4 layers of 262,144: 128 tiles
            _check(wl.data, cbs, wl.segment_elems, case)
        elif case == "bf16 escape-heavy":
            x = kvsynth.random_bits(40 * 8192 + 17, kvsynth.BF16, seed=15, device=DEV, kind="uniform_bits")
            _check(x, O.calibrate(O.BF16, kvsynth.to_numpy_bits(x[:5000])), 0, case)
        else:
            wl, cbs = _layer("llama3_70b_kv_e5m2", layers=2, tokens=256)  # 2 layers of 524,288: 64 tiles
            _check(wl.data, cbs, wl.segment_elems, case)
    finally:
        if old is None:
            del os.environ["SPLITZIP_STATIC_WAIT_POLLS"]
        else:
            os.environ["SPLITZIP_STATIC_WAIT_POLLS"] = old
