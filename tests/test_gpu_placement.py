"""GPU parity of the escape placement: sizes that give each range width of
the placement pass (8, 16, 32 and 64 tiles per workgroup: the width is the
power of two from 8 to 64 that gives about 2048 workgroups), with tiles whose
escapes overflow their 512-record staging slot at range, block (64 tiles) and
super-block (4096 tiles) boundaries and at random places, among tiles with few
escapes; tiles with exactly 512 and 513 escapes sit on the staging limit.

Streams are compared byte for byte with the CPU oracle and decoded back on
the GPU bit-exactly (integer work: tolerance 0).
"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O
from paritylib import compare_with_oracle

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
DEV = "cuda"
SLOT = 512  # staged records per tile


def _say(*a):
    print(*a, flush=True)


def _tile_elems(dtype):
    return 8192 if dtype == O.BF16 else 16384


def _escape_value(dtype, cb):
    """A bit pattern whose exponent is outside codebook cb."""
    if dtype == O.BF16:
        e = next(v for v in range(254, 0, -1) if v not in set(cb.tolist()))
        return e << 7
    e = next(v for v in range(30, 0, -1) if v not in set(cb.tolist()))
    return e << 2


# (dtype, tiles, ragged elements cut from the end, codebook segments of this many chunks or 0)
CASES = [
    (O.BF16, 1000, 77, 0),            # 8 tiles per workgroup
    (O.BF16, 16384 + 5, 1234, 32),    # 16
    (O.BF16, 32768 + 3, 0, 0),        # 32
    (O.BF16, 65536 + 9, 4097, 64),    # 64
    (O.E5M2, 16384 + 5, 999, 16),     # 16 (E5M2 tiles hold 16384 elements)
]


@pytest.mark.parametrize("dtype,tiles,ragged,seg_chunks", CASES,
                         ids=[f"{'bf16' if c[0] == O.BF16 else 'e5m2'}-{c[1]}" for c in CASES])
def test_placement_ranges_with_overflowing_tiles(dtype, tiles, ragged, seg_chunks):
    te = _tile_elems(dtype)
    n = tiles * te - ragged
    _say(f"case placement dtype={dtype} tiles={tiles} n={n} seg_chunks={seg_chunks}")
    x = kvsynth.random_bits(n, dtype, seed=7000 + tiles, device=DEV)
    sample = kvsynth.to_numpy_bits(x[: 1 << 20])
    cb0 = sz.splitzip_calibrate(dtype, sample)
    if seg_chunks:
        seg = seg_chunks * 65536
        K = (n + seg - 1) // seg
        rng = np.random.default_rng(tiles)
        # the same 16 exponents in another order per segment: other codes, same escapes
        cbs = np.stack([rng.permutation(cb0) for _ in range(K)]).astype(np.uint8)
    else:
        seg, K = 0, 1
        cbs = cb0[None, :]

    # tiles made of uniformly random bits (thousands of escapes each)
    rng = np.random.default_rng(100 + tiles)
    heavy = {0, 1, 7, 8, 15, 16, 31, 32, 63, 64, 65, 127, 128, 4095, 4096, 4097, tiles - 1}
    heavy |= set(rng.integers(0, tiles, size=24).tolist())
    heavy = sorted(t for t in heavy if t < tiles)
    for t in heavy:
        a, b = t * te, min(n, (t + 1) * te)
        x[a:b] = kvsynth.random_bits(b - a, dtype, seed=t, device=DEV, kind="uniform_bits")
    # tiles with exactly SLOT and SLOT + 1 escapes on top of their own
    esc = _escape_value(dtype, cb0)
    limit = [t for t in (2, 3, 66, 4098, tiles - 2) if 0 <= t < tiles and t not in heavy]
    for i, t in enumerate(limit):
        a, b = t * te, min(n, (t + 1) * te)
        tile = kvsynth.to_numpy_bits(x[a:b]).astype(np.int64)
        if dtype == O.BF16:
            exps = (tile >> 7) & 0xFF
        else:
            exps = (tile >> 2) & 0x1F
        own = int((~np.isin(exps, cb0)).sum())
        want = SLOT + (i % 2)
        free = np.nonzero(np.isin(exps, cb0))[0]
        add = max(0, want - own)
        pos = np.random.default_rng(t).choice(free, size=add, replace=False)
        sign = tile[pos] & (0x8000 if dtype == O.BF16 else 0x80)
        low = tile[pos] & (0x7F if dtype == O.BF16 else 0x03)
        vals = sign | esc | low
        idx = torch.from_numpy(pos + a).to(DEV)
        v = torch.from_numpy(vals.astype(np.int64)).to(DEV)
        if dtype == O.BF16:
            x[idx] = (v - 65536 * (v >= 32768).to(torch.int64)).to(torch.int16)
        else:
            x[idx] = v.to(torch.uint8)
    xh = kvsynth.to_numpy_bits(x)
    for i, t in enumerate(limit):  # the planted counts are what the case claims
        tile = xh[t * te:min(n, (t + 1) * te)].astype(np.int64)
        exps = (tile >> 7) & 0xFF if dtype == O.BF16 else (tile >> 2) & 0x1F
        assert int((~np.isin(exps, cb0)).sum()) == SLOT + (i % 2)

    out, nb = sz.compress(x, cbs, seg)
    torch.cuda.synchronize()
    n_bytes = int(nb.item())
    gpu = out[:n_bytes].cpu().numpy()
    E = compare_with_oracle(gpu, dtype, xh, cbs, seg)
    _say(f"  escapes={E} heavy tiles={len(heavy)} limit tiles={limit}")
    y, st = sz.decompress(out[:n_bytes], n, dtype)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y.view(torch.uint8), x.view(torch.uint8))
