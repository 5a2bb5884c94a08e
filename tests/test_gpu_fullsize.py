"""Full-size parity in the benchmark's own launch configuration, over every scale group.

The packed caches are built exactly as bench.py builds them (bench.CacheWorkload: one
quantize call per appended chunk covering every layer's K and V, one dequantize call for
the whole cache).  The oracle then recomputes every scale group from the same bf16 inputs
-- group amax, every code byte, every scale byte -- and dequantizes its own packed bytes,
which must equal the GPU's bf16 output of the whole cache bit for bit.  The groups are
spread over the host's threads (the oracle's C calls release the GIL).  Every group's amax
is also checked against a max over its input taken on the device.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bench
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
THREADS = max(1, min(16, os.cpu_count() or 1))


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _host_cache(w, with_out=True):
    h = {"codes": w.codes.cpu().numpy(), "scales": w.scales.cpu().numpy(),
         "amax": w.amax.cpu().numpy()}
    if with_out:
        h["out"] = _u16(w.out)
    return h


def _check_group(h, src_h, w, chunk, gi, rule, check_out):
    """Oracle vs GPU for group gi of chunk `chunk`: amax, codes, scales (and the bf16 output
    of the whole-cache dequantize).  Returns a list of mismatch descriptions."""
    rpg = w.cfg.rows_per_group
    x = src_h[gi * rpg:(gi + 1) * rpg]
    oc, os_, oa = oracle.quantize(x, rpg, rule)
    r0 = chunk * w.slab_rows + gi * rpg
    g = chunk * w.cfg.groups_per_chunk + gi
    bad = []
    if h["amax"][g].view(np.uint32) != oa[0].view(np.uint32):
        bad.append((chunk, gi, "amax"))
    if not np.array_equal(h["codes"][r0:r0 + rpg], oc):
        bad.append((chunk, gi, "codes"))
    if not np.array_equal(h["scales"][r0:r0 + rpg], os_):
        bad.append((chunk, gi, "scales"))
    if check_out and not np.array_equal(h["out"][r0:r0 + rpg], oracle.dequantize(oc, os_, oa, rpg)):
        bad.append((chunk, gi, "bf16 output"))
    return bad


def _check_chunks(w, h, chunks, rule, check_out):
    bad = []
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        for c in chunks:
            src_h = _u16(w.sources[c])
            bad += sum(ex.map(lambda gi: _check_group(h, src_h, w, c, gi, rule, check_out),
                              range(w.cfg.groups_per_chunk)), [])
            del src_h
    return bad


def _all_group_amax(w):
    cfg = w.cfg
    want = []
    for c in range(cfg.chunks):
        s = w.sources[c].view(cfg.groups_per_chunk, -1)
        want.append(s.abs().amax(dim=1).float())
    return torch.cat(want)


def test_full_cache_read_30_layers_every_group():
    """30 layers x K,V x 32760 tokens x 12 heads x 128, mse-quantized in 7 chunks of 4680:
    all 420 groups (3,019,161,600 elements) -- codes, scale bytes, amax and the bf16 output
    of the one whole-cache dequantize launch -- bit for bit against the oracle."""
    t0 = time.perf_counter()
    cfg = synth.C3
    w = bench.CacheWorkload(cfg, "mse", DEV, keep_sources=True)
    w.append()
    w.dequantize_all()
    torch.cuda.synchronize()
    assert torch.equal(w.amax, _all_group_amax(w))
    h = _host_cache(w)
    bad = _check_chunks(w, h, range(cfg.chunks), "mse", check_out=True)
    assert not bad, bad[:10]
    print(f"C3 whole cache: {w.n_groups} groups checked in {time.perf_counter() - t0:.1f} s "
          f"on {THREADS} threads")


def test_rollout_step_5b_every_rule_every_group():
    """30 layers, 24 heads, 36960-token cache (14 chunks of 2640): the appended chunk's 60
    groups under each rule, then the whole static_6 cache (840 groups, 6,812,467,200
    elements) and its whole-cache dequantize, every byte against the oracle."""
    t0 = time.perf_counter()
    cfg = synth.C4
    w = bench.CacheWorkload(cfg, "static_6", DEV, keep_sources=True)
    last = cfg.chunks - 1
    for rule in ("static_6", "static_4", "mse"):
        w.rule = rule
        w.append()
        torch.cuda.synchronize()
        h = _host_cache(w, with_out=False)
        bad = _check_chunks(w, h, [last], rule, check_out=False)
        assert not bad, (rule, bad[:10])
    w.rule = "static_6"
    w.append()
    w.dequantize_all()
    torch.cuda.synchronize()
    assert torch.equal(w.amax, _all_group_amax(w))
    h = _host_cache(w)
    bad = _check_chunks(w, h, range(cfg.chunks), "static_6", check_out=True)
    assert not bad, bad[:10]
    print(f"C4 appends (3 rules) + whole cache: {w.n_groups} groups checked in "
          f"{time.perf_counter() - t0:.1f} s on {THREADS} threads")
