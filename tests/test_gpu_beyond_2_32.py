"""More than 2^32 elements: a BF16 tensor of 2^32 + 12,345 values (8 GiB) and
an FP8 E5M2 tensor of 2^32 + 777 values (4 GiB), each in three codebook
segments, so that element, tile, chunk and escape indices all pass 32 bits.
The GPU stream is compared with the oracle's byte for byte (piecewise, per
segment) and decoded back bit-exactly."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O
from paritylib import compare_with_oracle

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
DEV = "cuda"


@pytest.mark.parametrize("dtype,ragged", [(O.BF16, 12345), (O.E5M2, 777)], ids=["bf16", "e5m2"])
def test_more_than_2_32_elements(dtype, ragged):
    n = (1 << 32) + ragged
    seg = 65536 * 22000  # 1.44e9 elements per codebook: three segments
    K = -(-n // seg)
    print(f"case dtype={dtype} n={n} K={K} segment={seg}", flush=True)
    x = torch.empty(n, dtype=torch.int16 if dtype == O.BF16 else torch.uint8, device=DEV)
    step = 1 << 28
    for i, a in enumerate(range(0, n, step)):
        b = min(n, a + step)
        x[a:b] = kvsynth.random_bits(b - a, dtype, seed=900 + i, device=DEV, sigma=1.0 + 0.25 * (i % 3))
    cbs = np.stack([sz.splitzip_calibrate(dtype, kvsynth.to_numpy_bits(x[k * seg:k * seg + (1 << 20)]))
                    for k in range(K)])
    out, nb = sz.compress(x, cbs, seg)
    torch.cuda.synchronize()
    n_bytes = int(nb.item())
    print(f"  stream {n_bytes} bytes, ratio {x.element_size() * n / n_bytes:.4f}", flush=True)
    gpu = out[:n_bytes].cpu().numpy()
    xh = kvsynth.to_numpy_bits(x)
    E = compare_with_oracle(gpu, dtype, xh, cbs, seg)
    print(f"  escapes {E}: stream equals the oracle's", flush=True)
    assert E > (1 << 20)
    del gpu, xh
    y, st = sz.decompress(out[:n_bytes], n, dtype)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y, x)
    print("  round trip exact", flush=True)
