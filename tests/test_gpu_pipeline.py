"""Chunk-pipelined transfer through pinned host memory (compress -> copy to
host -> copy back -> decompress, several groups in flight): the received
tensor equals the sent one bit for bit, every group's stream equals the
oracle's stream of the same elements and codebooks, and the raw mode moves
the same bytes."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle as O

pytestmark = pytest.mark.gpu

sz = pytest.importorskip("lossless_kv_cache_splitzip_amd")
CHUNK = 65536


def _group_codebooks(cbs, seg, g, group, n):
    """Codebooks and segment length of group g's own stream."""
    if cbs.shape[0] == 1:
        return cbs[:1], 0
    first = g * group
    ng = min(group, n - first)
    if group % seg == 0:
        k = -(-ng // seg)
        return cbs[first // seg:first // seg + k], (seg if k > 1 else 0)
    return cbs[first // seg:first // seg + 1], 0


def _run(name, group, depth, layers=None, tokens=None, trim=0, check_streams=True):
    print(f"case pipeline {name} group={group} depth={depth} trim={trim}", flush=True)
    kw = {}
    if layers:
        kw["layers"] = layers
    if tokens:
        kw["tokens"] = tokens
    wl = kvsynth.make(name, device="cuda", **kw)
    dtype = wl.spec.dtype
    cbs = np.stack([sz.splitzip_calibrate(dtype, kvsynth.to_numpy_bits(c)) for c in wl.calib])
    seg = wl.segment_elems if cbs.shape[0] > 1 else 0
    x = wl.data[:wl.n - trim].contiguous() if trim else wl.data
    n = x.numel()
    p = sz.Pipeline(dtype, n, cbs, seg, group, depth, device="cuda")
    try:
        return _transfer_and_check(p, x, n, dtype, cbs, seg, group, depth, name, check_streams)
    finally:
        p.close()


def _transfer_and_check(p, x, n, dtype, cbs, seg, group, depth, name, check_streams):
    out = torch.empty_like(x)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sizes = p.transfer(x, out, compress=True, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out.view(torch.uint8), x.view(torch.uint8))
    xh = kvsynth.to_numpy_bits(x)
    if check_streams:
        # the last `depth` groups' streams are still in the host ring
        for g in range(max(0, p.groups - depth), p.groups):
            gcb, gseg = _group_codebooks(cbs, seg, g, group, n)
            want = O.compress(dtype, xh[g * group:(g + 1) * group], gcb, gseg)
            assert int(sizes[g]) == want.size
            assert np.array_equal(p.slot_stream(g, int(sizes[g])), want), g
    # raw mode: same pipeline, uncompressed groups
    out2 = torch.empty_like(x)
    raw = p.transfer(x, out2, compress=False)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.uint8), x.view(torch.uint8))
    assert int(raw.sum()) == n * x.element_size()
    assert int(sizes.sum()) < int(raw.sum()) or "uniform" in name
    return sizes


def test_pipeline_one_codebook_all_groups_checked():
    # 2,097,152 elements in 8 groups of 4 chunks, all 8 streams kept (depth 8)
    _run("kv_layer_bf16", 4 * CHUNK, 8)


def test_pipeline_ragged_tail_and_shallow_ring():
    # last group partial (odd element count), ring of 2
    _run("kv_layer_bf16", 3 * CHUNK, 2, trim=12345)


def test_pipeline_single_chunk_groups():
    # many tiny groups: the host polls 32 sizes, ring of 2
    _run("kv_layer_bf16", CHUNK, 2, trim=3)


def test_pipeline_groups_inside_segments():
    # per-layer codebooks, a segment (layer) = 8 chunks, groups of 2 chunks
    _run("llama3_8b_kv_bf16", 2 * CHUNK, 4, layers=4, tokens=256)


def test_pipeline_groups_of_whole_segments():
    # groups of 2 segments carry 2 codebooks each; last group holds one
    _run("llama3_8b_kv_bf16", 16 * CHUNK, 3, layers=5, tokens=256)


def test_pipeline_e5m2():
    _run("llama3_70b_kv_e5m2", 4 * CHUNK, 3, layers=3, tokens=512, trim=7)


def test_pipeline_escape_heavy_group():
    # uniform bit patterns expand (ratio < 1): slots hold the worst case
    _run("edge_uniform_bits", 8 * CHUNK, 2, tokens=1024)


def test_pipeline_full_size_launch_configuration():
    # the 1 GiB workload in the configuration the benchmark times: groups of
    # 32 MiB (one layer, 256 chunks), four in flight
    _run("llama3_8b_kv_bf16", 256 * CHUNK, 4)
