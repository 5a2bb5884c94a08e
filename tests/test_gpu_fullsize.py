"""Full-size parity in the benchmark's own launch configuration.

The packed caches are built exactly as bench.py builds them (bench.CacheWorkload: one
quantize call per appended chunk covering every layer's K and V, one dequantize call for
the whole cache).  The oracle then recomputes sampled scale groups from the same bf16
inputs: the group amax over the whole group, and codes, scale bytes and bf16 output for
sampled rows (first, last and random rows of each sampled group).  Every group's amax is
also checked against a max over its input.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_group(w, chunk, layer, kv, rule, rng, n_rows=1024, check_out=True):
    cfg = w.cfg
    src = w.sources[chunk]
    gi = layer * 2 + kv                       # group index inside the chunk's slab
    r0 = gi * cfg.rows_per_group
    x = _u16(src[r0:r0 + cfg.rows_per_group])  # whole group, host copy of the exact input
    A = oracle.group_amax(x)
    g = chunk * cfg.groups_per_chunk + gi
    assert w.amax[g].item() == A, (chunk, layer, kv)
    rows = np.unique(np.concatenate([[0, 1, cfg.rows_per_group - 1],
                                     rng.integers(0, cfg.rows_per_group, n_rows)]))
    oc, os_ = oracle.quantize_rows(x[rows], A, rule)
    base = chunk * w.slab_rows + r0
    idx = torch.from_numpy(base + rows).to(DEV)
    gc = w.codes.index_select(0, idx).cpu().numpy()
    gs = w.scales.index_select(0, idx).cpu().numpy()
    assert np.array_equal(gc, oc), (chunk, layer, kv, "codes")
    assert np.array_equal(gs, os_), (chunk, layer, kv, "scales")
    if check_out:
        oy = oracle.dequantize_rows(oc, os_, A)
        gy = _u16(w.out.index_select(0, idx))
        assert np.array_equal(gy, oy), (chunk, layer, kv, "dequant")


def _all_group_amax(w):
    cfg = w.cfg
    want = []
    for c in range(cfg.chunks):
        s = w.sources[c].view(cfg.groups_per_chunk, -1)
        want.append(s.abs().amax(dim=1).float())
    return torch.cat(want)


def test_full_cache_read_30_layers():
    """30 layers x K,V x 32760 tokens x 12 heads x 128, mse-quantized in 7 chunks of 4680."""
    cfg = synth.C3
    w = bench.CacheWorkload(cfg, "mse", DEV, keep_sources=True)
    w.append()
    w.dequantize_all()
    torch.cuda.synchronize()
    assert torch.equal(w.amax, _all_group_amax(w))
    rng = np.random.default_rng(3)
    picks = [(0, 0, 0), (6, 29, 1), (3, 17, 0), (6, 0, 1)] + [
        (int(rng.integers(cfg.chunks)), int(rng.integers(cfg.layers)), int(rng.integers(2)))
        for _ in range(4)]
    for c, l, kv in picks:
        _check_group(w, c, l, kv, "mse", rng)


def test_rollout_step_5b_every_rule():
    """30 layers, 24 heads, 36960-token cache (14 chunks of 2640): append under each rule,
    then the whole-cache dequantize of the static_6 cache."""
    cfg = synth.C4
    w = bench.CacheWorkload(cfg, "static_6", DEV, keep_sources=True)
    rng = np.random.default_rng(4)
    last = cfg.chunks - 1
    for rule in ("static_6", "static_4", "mse"):
        w.rule = rule
        w.append()
        torch.cuda.synchronize()
        for l, kv in [(0, 0), (29, 1), (int(rng.integers(30)), int(rng.integers(2)))]:
            _check_group(w, last, l, kv, rule, rng, check_out=False)
    w.rule = "static_6"
    w.append()
    w.dequantize_all()
    torch.cuda.synchronize()
    assert torch.equal(w.amax, _all_group_amax(w))
    for c, l, kv in [(0, 0, 0), (last, 29, 1), (7, 13, 0), (int(rng.integers(14)), 5, 1)]:
        _check_group(w, c, l, kv, "static_6", rng)
