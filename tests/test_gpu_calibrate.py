"""On-device calibration: every codebook equals the oracle's calibration of
the same samples (16 most frequent exponents, ties to the lower exponent,
unseen exponents filling up ascending), for one segment and for many,
including ragged and unaligned segments, empty ones, ties and all-equal
data, and for the per-layer codebooks of the full-size workloads."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")


def _check(x, dtype, k, seg):
    print(f"case calibrate dtype={dtype} n={x.numel()} K={k} seg={seg}", flush=True)
    got = sz.calibrate_device(x, k, seg)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    xh = kvsynth.to_numpy_bits(x)
    size = seg if k > 1 else max(xh.size, 1)
    for j in range(k):
        want = O.calibrate(dtype, xh[j * size:(j + 1) * size])
        assert np.array_equal(got[j], want), (j, got[j], want)


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
def test_one_segment_random_distributions(dtype):
    for seed, sigma in [(1, 0.3), (2, 1.0), (3, 3.0), (4, 8.0)]:
        x = kvsynth.random_bits(1_000_003, dtype, seed=seed, device="cuda", sigma=sigma)
        _check(x, dtype, 1, 0)


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
def test_many_segments_ragged_and_unaligned(dtype):
    x = kvsynth.random_bits(300_001, dtype, seed=7, device="cuda", sigma=2.0)
    _check(x, dtype, 31, 10_000)      # segment starts not 16-byte aligned, ragged last
    _check(x, dtype, 5, 65_536 + 3)
    _check(x, dtype, 40, 10_000)      # 9 trailing segments hold no element


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
def test_tiny_and_empty(dtype):
    for n in (0, 1, 7, 15, 17):
        x = kvsynth.random_bits(max(n, 1), dtype, seed=n, device="cuda", sigma=1.0)[:n]
        x = x.contiguous()
        got = sz.calibrate_device(x, 1, 0)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy()[0], O.calibrate(dtype, kvsynth.to_numpy_bits(x))), n


def test_ties_go_to_the_lower_exponent():
    # exponents 9 and 5 twice each, 200 once, 3 twice: order 3, 5, 9, 200, then unseen ascending
    vals = np.array([9, 5, 9, 5, 200, 3, 3], dtype=np.uint16) << 7
    x = torch.from_numpy(vals.view(np.int16)).cuda()
    got = sz.calibrate_device(x, 1, 0)
    torch.cuda.synchronize()
    want = O.calibrate(O.BF16, vals)
    assert list(want[:4]) == [3, 5, 9, 200]
    assert np.array_equal(got.cpu().numpy()[0], want)


def test_single_exponent_fills_ascending():
    x = torch.full((123_457,), (77 << 7) | 0x35, dtype=torch.int16, device="cuda")
    got = sz.calibrate_device(x, 1, 0)
    torch.cuda.synchronize()
    assert list(got.cpu().numpy()[0]) == [77] + list(range(15))


@pytest.mark.parametrize("name", ["llama3_8b_kv_bf16", "llama3_70b_kv_e5m2"])
def test_full_size_per_layer_codebooks(name):
    # one codebook per layer of the whole tensor, in one call
    wl = kvsynth.make(name, device="cuda")
    _check(wl.data, wl.spec.dtype, wl.spec.layers, wl.spec.layer_elems)
