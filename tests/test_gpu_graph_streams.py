"""Stream-ordered use of the C ABI: compress + decompress captured in a HIP
graph and replayed with eager work between the replays, calls on two
streams in flight at once, and calls from two host threads at once.  Every
stream equals the oracle's byte for byte and every round trip is bit-exact.

The entry points only launch kernels on the caller's stream (no allocation,
no memset, no synchronization), which is what makes them capturable.
"""
import threading

import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")


def _stream_bytes(out, nb):
    return out[:int(nb.item())].cpu().numpy()


def _check(dtype, x, cbs, seg, out, nb, y, st):
    xh = kvsynth.to_numpy_bits(x)
    assert np.array_equal(_stream_bytes(out, nb), O.compress(dtype, xh, cbs, seg))
    assert int(st.item()) == 0
    assert np.array_equal(kvsynth.to_numpy_bits(y), xh)


@pytest.mark.parametrize("name", ["llama3_8b_kv_bf16", "llama3_70b_kv_e5m2"])
def test_graph_replays_match_the_oracle(name):
    wl = kvsynth.make(name, device="cuda", layers=3, tokens=96)
    dtype = wl.spec.dtype
    cbs = np.stack([sz.splitzip_calibrate(dtype, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    seg = wl.segment_elems
    n = wl.n
    x = wl.data.clone()
    cap = sz.splitzip_max_compressed_size(dtype, n, cbs.shape[0])
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    y = torch.empty_like(x)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"case graph {name} n={n} codebooks={cbs.shape[0]}", flush=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up on the capture stream's kind of stream
        sz.compress(x, cbs, seg, out=out, out_bytes=nb)
        sz.decompress(out, n, dtype, out=y, status=st, in_bytes=cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _check(dtype, x, cbs, seg, out, nb, y, st)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sz.compress(x, cbs, seg, out=out, out_bytes=nb)
        sz.decompress(out, n, dtype, out=y, status=st, in_bytes=cap)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(7)
    for r in range(4):
        # eager work between replays: new input contents (a permutation of
        # the workload, so escapes move between tiles and chunks) and a
        # cleared output
        perm = torch.randperm(n, generator=gen).cuda()
        x.copy_(wl.data[perm])
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(dtype, x, cbs, seg, out, nb, y, st)
        # the same call made eagerly gives the same stream
        out2, nb2 = sz.compress(x, cbs, seg)
        torch.cuda.synchronize()
        assert int(nb2.item()) == int(nb.item())
        assert torch.equal(out2[:int(nb.item())], out[:int(nb.item())])


def _inputs():
    a = kvsynth.random_bits(3 * 65536 + 1001, O.BF16, seed=21, device="cuda", sigma=1.5)
    b = kvsynth.random_bits(5 * 65536 + 77, O.E5M2, seed=22, device="cuda", sigma=1.5)
    return [(O.BF16, a), (O.E5M2, b)]


def test_two_streams_in_flight():
    cases = _inputs()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cbs = [O.calibrate(d, kvsynth.to_numpy_bits(x)[:20000]) for d, x in cases]
    results = [[], []]
    for rep in range(3):
        for i, ((dtype, x), s) in enumerate(zip(cases, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                out, nb = sz.compress(x, cbs[i])
                y, st = sz.decompress(out, x.numel(), dtype, in_bytes=out.numel())
            results[i].append((out, nb, y, st))
    torch.cuda.synchronize()
    for i, (dtype, x) in enumerate(cases):
        for out, nb, y, st in results[i]:
            _check(dtype, x, cbs[i], 0, out, nb, y, st)


def test_two_host_threads():
    cases = _inputs()
    cbs = [O.calibrate(d, kvsynth.to_numpy_bits(x)[:20000]) for d, x in cases]
    results = [[], []]
    errors = []

    def work(i):
        try:
            dtype, x = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    out, nb = sz.compress(x, cbs[i])
                    y, st = sz.decompress(out, x.numel(), dtype, in_bytes=out.numel())
                    results[i].append((out, nb, y, st))
            s.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (dtype, x) in enumerate(cases):
        assert len(results[i]) == 5
        for out, nb, y, st in results[i]:
            _check(dtype, x, cbs[i], 0, out, nb, y, st)
