"""Ablation variants on the GPU (top-15 + sentinel, top-8 with 3-bit codes):
the GPU streams equal the oracle's byte for byte, and the GPU decoders
reproduce the input bit for bit, on ragged and edge sizes, all BF16 bit
patterns, several codebook segments, and reject corrupted streams."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
V = [sz.VARIANT_TOP15_SENTINEL, sz.VARIANT_TOP8]
ORACLE_V = {sz.VARIANT_TOP15_SENTINEL: O.SENTINEL, sz.VARIANT_TOP8: O.TOP8}


def _roundtrip(v, x, cbs, seg=0):
    print(f"case variant {v} n={x.numel()} K={np.asarray(cbs).reshape(-1, 16).shape[0]} seg={seg}", flush=True)
    out, nb = sz.variant_compress(v, x, cbs, seg)
    torch.cuda.synchronize()
    n_bytes = int(nb.item())
    got = out[:n_bytes].cpu().numpy()
    xh = kvsynth.to_numpy_bits(x)
    want = O.variant_compress(ORACLE_V[v], xh, cbs, seg)
    assert got.size == want.size and np.array_equal(got, want)
    y, st = sz.variant_decompress(v, out[:n_bytes], x.numel())
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(kvsynth.to_numpy_bits(y), xh)
    return got


@pytest.mark.parametrize("v", V)
def test_small_workloads(v):
    for tokens, trim in [(1024, 0), (1000, 3)]:
        wl = kvsynth.make("kv_layer_bf16", device="cuda", tokens=tokens)
        cb = sz.splitzip_calibrate(O.BF16, kvsynth.to_numpy_bits(wl.calib[0]))
        _roundtrip(v, wl.data[:wl.n - trim].contiguous(), cb)


@pytest.mark.parametrize("v", V)
def test_edge_sizes(v):
    base = kvsynth.random_bits(200_003, O.BF16, seed=11, device="cuda", sigma=2.0)
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(base))
    for n in (0, 1, 2, 7, 8, 9, 8191, 8192, 8193, 65535, 65536, 65537, 131073, 200_003):
        _roundtrip(v, base[:n].contiguous(), cb)


@pytest.mark.parametrize("v", V)
def test_all_bit_patterns(v):
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).cuda()
    x = torch.cat([x, x.flip(0)[:30001]]).contiguous()
    for cb in (np.arange(16, dtype=np.uint8), np.array([127, 126, 128, 125, 129, 124, 130, 123, 131, 122, 132, 121, 133, 120, 134, 119], np.uint8)):
        _roundtrip(v, x, cb)


@pytest.mark.parametrize("v", V)
def test_segment_codebooks(v):
    wl = kvsynth.make("llama3_8b_kv_bf16", device="cuda", layers=5, tokens=256)
    cbs = np.stack([sz.splitzip_calibrate(O.BF16, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    _roundtrip(v, wl.data, cbs, wl.segment_elems)


@pytest.mark.parametrize("v", V)
def test_escape_heavy(v):
    wl = kvsynth.make("edge_uniform_bits", device="cuda", tokens=200)
    cb = sz.splitzip_calibrate(O.BF16, kvsynth.to_numpy_bits(wl.calib[0]))
    _roundtrip(v, wl.data, cb)


@pytest.mark.parametrize("v", V)
def test_corrupt_streams_are_reported(v):
    x = kvsynth.random_bits(100_000, O.BF16, seed=3, device="cuda", sigma=2.0)
    cb = O.calibrate(O.BF16, kvsynth.to_numpy_bits(x))
    good = _roundtrip(v, x, cb)
    other = sz.VARIANT_TOP8 if v == sz.VARIANT_TOP15_SENTINEL else sz.VARIANT_TOP15_SENTINEL
    cases = []
    s = good.copy(); s[48] = other; cases.append((v, s))                  # variant byte
    cases.append((other, good.copy()))                                    # decoded as the other variant
    s = good.copy(); s[24] ^= 1; cases.append((v, s))                     # total size
    if v == sz.VARIANT_TOP15_SENTINEL:
        s = good.copy()
        nib0 = 256  # code section of a 1-codebook, 2-chunk stream
        s[nib0:nib0 + 64] = 0xFF; cases.append((v, s))                    # more sentinels than values
    for dv, s in cases:
        buf = torch.from_numpy(s).cuda()
        _, st = sz.variant_decompress(dv, buf, x.numel())
        torch.cuda.synchronize()
        assert int(st.item()) == sz.E_CORRUPT
    # the main decoder rejects variant streams
    _, st = sz.decompress(torch.from_numpy(good).cuda(), x.numel(), sz.BF16)
    torch.cuda.synchronize()
    assert int(st.item()) == sz.E_CORRUPT


@pytest.mark.parametrize("v", V)
def test_quarter_gib_against_oracle(v):
    # 8 layers of the Llama-3-8B-shaped cache (256 MiB), per-layer codebooks
    wl = kvsynth.make("llama3_8b_kv_bf16", device="cuda", layers=8)
    cbs = np.stack([sz.splitzip_calibrate(O.BF16, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    _roundtrip(v, wl.data, cbs, wl.segment_elems)
