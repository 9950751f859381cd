"""A seeded sweep of 120 random configurations through the GPU codec, each
compared with the oracle: the stream byte for byte, the round trip bit for
bit, the on-device calibration of its segments against the host one, and
(inputs within its limit) splitzip_compress_static's stream against
splitzip_compress's.  The configurations mix the two element types; sizes
from empty to 9M elements, many of them a few elements either side of a
tile, chunk or one-launch boundary; one codebook or several segments of whole
chunks (some segments longer than needed, some codebooks unused; a second
sweep takes 129 to 259 codebooks, more than one launch's arguments hold, so
the codebooks are written by launches of their own); and data
from narrow exponent distributions (few escapes) to uniformly random bit
patterns (nearly every element escapes).  The codebooks are either calibrated
on a sample of each segment or random valid ones.  Every case prints its
parameters first, so a failure names it."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
DEV = "cuda"
CASES = 120


def _size(rng, dtype):
    tile = 8192 if dtype == O.BF16 else 16384
    pick = rng.integers(0, 6)
    if pick == 0:
        return int(rng.integers(0, 70_000))
    if pick == 1:
        return int(rng.integers(70_000, 3_000_000))
    base = [tile, 65536, 512 * tile][pick - 2] if pick < 5 else 2048 * tile // 16
    return max(0, int(base * rng.integers(1, 4) + rng.integers(-3, 4)))


def _case(i):
    rng = np.random.default_rng(10_000 + i)
    dtype = O.BF16 if rng.integers(0, 3) else O.E5M2
    n = min(_size(rng, dtype), 9_000_000)
    chunks = max(1, -(-n // 65536))
    if rng.integers(0, 3) == 0 or chunks == 1:
        k, seg = 1, 0
    else:
        seg_chunks = int(rng.integers(1, chunks + 1))
        seg = 65536 * seg_chunks
        k = -(-max(n, 1) // seg) + int(rng.integers(0, 3))  # sometimes unused codebooks at the end
    kind = "uniform_bits" if rng.integers(0, 8) == 0 else "gaussian"
    sigma = float(rng.choice([0.3, 1.0, 2.0, 3.0]))
    random_cb = bool(rng.integers(0, 4) == 0)
    return rng, dtype, n, k, seg, kind, sigma, random_cb


@pytest.mark.parametrize("chunk", range(4))
def test_random_configurations_match_the_oracle(chunk):
    for i in range(chunk * CASES // 4, (chunk + 1) * CASES // 4):
        rng, dtype, n, k, seg, kind, sigma, random_cb = _case(i)
        print(f"case sweep {i}: dtype={dtype} n={n} K={k} segment={seg} kind={kind} sigma={sigma} "
              f"random_codebooks={random_cb}", flush=True)
        x = kvsynth.random_bits(n, dtype, seed=i, device=DEV, kind=kind, sigma=sigma)
        xh = kvsynth.to_numpy_bits(x)
        vals = 256 if dtype == O.BF16 else 32
        if random_cb:
            cbs = np.stack([rng.permutation(vals)[:16] for _ in range(k)]).astype(np.uint8)
        else:
            span = seg if k > 1 else max(n, 1)
            cbs = np.stack([O.calibrate(dtype, xh[c * span:c * span + 4096]) for c in range(k)])
        want = O.compress(dtype, xh, cbs, seg)
        out, nb = sz.compress(x, cbs, seg)
        torch.cuda.synchronize()
        S = int(nb.item())
        assert S == want.size, f"case {i}: stream size {S}, oracle {want.size}"
        assert np.array_equal(out[:S].cpu().numpy(), want), f"case {i}: stream differs from the oracle's"
        y, st = sz.decompress(out[:S], n, dtype)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, f"case {i}: status {int(st.item())}"
        assert np.array_equal(kvsynth.to_numpy_bits(y), xh), f"case {i}: round trip differs"
        # the on-device calibration of the same segments equals the host one
        span = seg if k > 1 else max(n, 1)
        dev_cbs = sz.calibrate_device(x, k, seg).cpu().numpy()
        host_cbs = np.stack([O.calibrate(dtype, xh[c * span:(c + 1) * span]) for c in range(k)])
        assert np.array_equal(dev_cbs, host_cbs), f"case {i}: device calibration differs"
        tile = 8192 if dtype == O.BF16 else 16384
        if n <= 2048 * tile:
            s_out, s_nb = sz.compress_static(x, cbs, seg)
            torch.cuda.synchronize()
            assert int(s_nb.item()) == S and torch.equal(s_out[:S], out[:S]), f"case {i}: static stream differs"


@pytest.mark.parametrize("variant", [O.SENTINEL, O.TOP8], ids=["sentinel", "top8"])
def test_random_configurations_of_the_ablation_variants(variant):
    """The same sweep's BF16 configurations (40 of them) through the two
    ablation variants: stream byte for byte against the oracle's variant,
    round trip bit for bit."""
    done = 0
    for i in range(CASES):
        rng, dtype, n, k, seg, kind, sigma, random_cb = _case(i)
        if dtype != O.BF16:
            continue
        print(f"case sweep variant={variant} {i}: n={n} K={k} segment={seg} kind={kind} sigma={sigma}", flush=True)
        x = kvsynth.random_bits(n, O.BF16, seed=i, device=DEV, kind=kind, sigma=sigma)
        xh = kvsynth.to_numpy_bits(x)
        span = seg if k > 1 else max(n, 1)
        cbs = np.stack([O.calibrate(O.BF16, xh[c * span:c * span + 4096]) for c in range(k)])
        want = O.variant_compress(variant, xh, cbs, seg)
        out, nb = sz.variant_compress(variant, x, cbs, seg)
        torch.cuda.synchronize()
        S = int(nb.item())
        assert S == want.size and np.array_equal(out[:S].cpu().numpy(), want), f"case {i}: variant stream differs"
        y, st = sz.variant_decompress(variant, out[:S], n)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and np.array_equal(kvsynth.to_numpy_bits(y), xh), f"case {i}: round trip"
        done += 1
        if done == 40:
            break
    assert done == 40


MANY = 16


def _many_case(i):
    """129 to 259 codebooks over segments of one chunk (BF16) or one or two
    (E5M2), the last used one partly covered and up to 3 after it unused;
    every input within splitzip_compress_static's 2048 tiles."""
    rng = np.random.default_rng(20_000 + i)
    dtype = O.BF16 if i % 2 == 0 else O.E5M2
    seg = 65536 * (1 if dtype == O.BF16 else int(rng.integers(1, 3)))
    k_used = int(rng.integers(129, 257))
    n = (k_used - 1) * seg + int(rng.integers(1, seg + 1))
    k = k_used + int(rng.integers(0, 4))
    kind = "uniform_bits" if i % 5 == 4 else "gaussian"
    return rng, dtype, n, k, k_used, seg, kind


@pytest.mark.parametrize("half", range(2))
def test_random_configurations_with_many_codebooks(half):
    """Stream, round trip, on-device calibration and the static entry point
    against the oracle with more codebooks than the launch arguments hold;
    the BF16 cases also through both ablation variants."""
    for i in range(half * MANY // 2, (half + 1) * MANY // 2):
        rng, dtype, n, k, k_used, seg, kind = _many_case(i)
        print(f"case many-codebooks {i}: dtype={dtype} n={n} K={k} (used {k_used}) segment={seg} kind={kind}",
              flush=True)
        x = kvsynth.random_bits(n, dtype, seed=500 + i, device=DEV, kind=kind, sigma=2.0)
        xh = kvsynth.to_numpy_bits(x)
        vals = 256 if dtype == O.BF16 else 32
        cbs = np.stack([O.calibrate(dtype, xh[c * seg:c * seg + 2048]) if c < k_used else
                        rng.permutation(vals)[:16].astype(np.uint8) for c in range(k)])
        want = O.compress(dtype, xh, cbs, seg)
        out, nb = sz.compress(x, cbs, seg)
        torch.cuda.synchronize()
        S = int(nb.item())
        assert S == want.size and np.array_equal(out[:S].cpu().numpy(), want), f"case {i}: stream differs"
        y, st = sz.decompress(out[:S], n, dtype)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and np.array_equal(kvsynth.to_numpy_bits(y), xh), f"case {i}: round trip"
        dev_cbs = sz.calibrate_device(x, k, seg).cpu().numpy()
        host_cbs = np.stack([O.calibrate(dtype, xh[c * seg:(c + 1) * seg]) for c in range(k)])
        assert np.array_equal(dev_cbs, host_cbs), f"case {i}: device calibration differs"
        tile = 8192 if dtype == O.BF16 else 16384
        if n <= 2048 * tile:
            s_out, s_nb = sz.compress_static(x, cbs, seg)
            torch.cuda.synchronize()
            assert int(s_nb.item()) == S and torch.equal(s_out[:S], out[:S]), f"case {i}: static stream differs"
        if dtype == O.BF16:
            for variant in (O.SENTINEL, O.TOP8):
                want_v = O.variant_compress(variant, xh, cbs, seg)
                out_v, nb_v = sz.variant_compress(variant, x, cbs, seg)
                torch.cuda.synchronize()
                S_v = int(nb_v.item())
                assert S_v == want_v.size and np.array_equal(out_v[:S_v].cpu().numpy(), want_v), \
                    f"case {i}: variant {variant} stream differs"
                y_v, st_v = sz.variant_decompress(variant, out_v[:S_v], n)
                torch.cuda.synchronize()
                assert int(st_v.item()) == 0 and np.array_equal(kvsynth.to_numpy_bits(y_v), xh), \
                    f"case {i}: variant {variant} round trip"
