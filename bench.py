#!/usr/bin/env python3
"""bench.py -- NVFP4 KV-cache quantize + dequantize throughput on one MI355X.

One step of the default workload (the 30-layer full-cache read) is one pass of the whole
hot path: quantize-on-append of the newest 4680-token chunk for every layer's K and V
(group amax, block scales, E2M1 codes; mse rule) into its slab of the packed cache, then
dequantization of the whole packed cache (30 layers x K,V x 32760 tokens x 12 heads x 128)
to bf16.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is algorithmic bytes per step / time per step, where the
bytes per element are bf16 (2) + codes (0.5) + scales (0.0625), plus 4 B per group amax.
Beside the step it reports (each on its own workload, skippable with --no-*): the same
cache read as per-layer launches, float32 dequantize and fake quantization, the RTN
INT4/INT2 caches, the paged-cache gather, the fused dequantize + attention, and the CPU
oracle on bounded samples.

    python bench.py [--steps K] [--warmup W] [--config C3|C4|C2|C1] [--rule R] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV FP4 quant+dequant GB/s (bf16+packed bytes) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 16.0
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_fp4_amd", "csrc", f)
                  for f in ("kvfp4.hip", "kvfp4_device.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C3", choices=["C1", "C2", "C3", "C4"])
    ap.add_argument("--rule", default=None, choices=["static_6", "static_4", "mse"],
                    help="append rule (default: mse for C3, static_6 otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rtn", action="store_true",
                    help="skip the RTN INT4/INT2 timing (reported beside the step)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache gather timing (reported beside the step)")
    ap.add_argument("--no-f32-fake", action="store_true",
                    help="skip the float32-output dequantize and fake-quantize timings")
    ap.add_argument("--no-attend", action="store_true",
                    help="skip the fused dequantize+attention timing (reported beside the step)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the one-layer chunk append and the 5B-shaped rollout step "
                         "(reported beside the step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args(argv)


# ---- workload ---------------------------------------------------------------------------

class CacheWorkload:
    """Packed cache laid out as append slabs: [chunk][layer][K/V][tokens*heads rows][head_dim].
    Group g = (chunk, layer, kv) in that order, so one chunk's append for every layer is one
    contiguous quantize call and the whole cache is one contiguous dequantize call."""

    def __init__(self, cfg, rule, device, keep_sources=False):
        import torch

        import kv_cache_fp4_amd as kv
        import synth
        self.cfg, self.rule, self.device = cfg, rule, device
        D, rpg = cfg.head_dim, cfg.rows_per_group
        self.rpg = rpg
        self.slab_rows = cfg.groups_per_chunk * rpg
        self.rows = cfg.chunks * self.slab_rows
        self.n_groups = cfg.chunks * cfg.groups_per_chunk
        self.codes = torch.empty((self.rows, D // 2), dtype=torch.uint8, device=device)
        self.scales = torch.empty((self.rows, D // 16), dtype=torch.uint8, device=device)
        self.amax = torch.empty((self.n_groups,), dtype=torch.float32, device=device)
        self.out = torch.empty((self.rows, D), dtype=torch.bfloat16, device=device)
        self.sources = {}
        for c in range(cfg.chunks):
            src = synth.chunk_all_layers(cfg, c, device=device)
            self.quantize_chunk(c, src)
            if keep_sources or c == cfg.chunks - 1:
                self.sources[c] = src
            else:
                del src
        torch.cuda.synchronize(device)
        self.append_src = self.sources[cfg.chunks - 1]
        self.kv = kv

    def slab(self, c):
        r0, r1 = c * self.slab_rows, (c + 1) * self.slab_rows
        g0, g1 = c * self.cfg.groups_per_chunk, (c + 1) * self.cfg.groups_per_chunk
        return self.codes[r0:r1], self.scales[r0:r1], self.amax[g0:g1]

    def quantize_chunk(self, c, src, opts=None):
        import kv_cache_fp4_amd as kv
        codes, scales, amax = self.slab(c)
        kv.kvfp4_quantize(src, self.rpg, self.rule, codes, scales, amax, opts=opts)

    def append(self, opts=None):
        self.quantize_chunk(self.cfg.chunks - 1, self.append_src, opts)

    def dequantize_all(self):
        self.kv.kvfp4_dequantize(self.codes, self.scales, self.amax, self.rpg, y=self.out)

    @property
    def append_elems(self):
        return self.slab_rows * self.cfg.head_dim

    @property
    def cache_elems(self):
        return self.rows * self.cfg.head_dim

    def append_bytes(self):
        return self.append_elems * BYTES_PER_ELEM + 4 * self.cfg.groups_per_chunk

    def dequant_bytes(self):
        return self.cache_elems * BYTES_PER_ELEM + 4 * self.n_groups


class PagedWorkload:
    """Paged cache of 30 layers x K,V x 2048 pages of 16 tokens x 12 heads x 128 (static_6),
    physical pages in a seeded random order; the timed calls gather every page to dense bf16
    and quantize every block into its page."""

    def __init__(self, device):
        import numpy as np
        import torch

        import kv_cache_fp4_amd as kv
        import synth
        cfg = synth.P1
        self.cfg, self.kv = cfg, kv
        D = cfg.head_dim
        self.rpp = cfg.chunk_tokens * cfg.heads
        self.n_blocks = cfg.layers * 2 * cfg.chunks
        self.src = torch.cat([synth.paged_tensor(cfg, l, k, device=device).reshape(-1, D)
                              for l in range(cfg.layers) for k in (0, 1)])
        perm = np.random.default_rng(cfg.seed).permutation(self.n_blocks).astype(np.int32)
        self.table = torch.from_numpy(perm).to(device)
        self.codes = torch.empty((self.n_blocks, self.rpp, D // 2), dtype=torch.uint8, device=device)
        self.scales = torch.empty((self.n_blocks, self.rpp, D // 16), dtype=torch.uint8, device=device)
        self.amax = torch.empty((self.n_blocks,), dtype=torch.float32, device=device)
        self.out = torch.empty((self.n_blocks * self.rpp, D), dtype=torch.bfloat16, device=device)
        kv.kvfp4_quantize_paged(self.src, self.table, self.rpp, self.codes, self.scales,
                                self.amax, "static_6")
        torch.cuda.synchronize(device)

    def dequantize_all(self):
        self.kv.kvfp4_dequantize_paged(self.codes, self.scales, self.amax, self.table, self.rpp,
                                       y=self.out)

    def dequant_bytes(self):
        return self.out.numel() * BYTES_PER_ELEM + 4 * self.n_blocks


def bench_paged(device, steps=20, warmup=3):
    import torch
    w = PagedWorkload(device)
    for _ in range(warmup):
        w.dequantize_all()
    stream = torch.cuda.current_stream(device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize(device)
    for a, b in ev:
        a.record(stream)
        w.dequantize_all()
        b.record(stream)
    torch.cuda.synchronize(device)
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    gbs = w.dequant_bytes() / (ms * 1e-3) / 1e9
    res = {"workload": (f"{w.cfg.name}: gather {w.n_blocks} pages of 16 tokens x 12 heads x 128 "
                        "(random physical order, static_6) to dense bf16"),
           "ms_per_call": round(ms, 4), "bytes_per_call": w.dequant_bytes(),
           "GBps": round(gbs, 2), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    # Quantizing every block into its page (same bytes), in both quantize forms.
    for form, key in (("auto", "quantize"), ("three_kernel", "quantize_three_kernel")):
        opts = w.kv.quantize_opts(form)
        quant = lambda: w.kv.kvfp4_quantize_paged(w.src, w.table, w.rpp, w.codes, w.scales,  # noqa: E731
                                                  w.amax, "static_6", opts=opts)
        qms = _time_calls(quant, device, max(steps // 2, 3), 2)
        res[key] = {"ms": round(qms, 4), "GBps": round(w.dequant_bytes() / (qms * 1e-3) / 1e9, 2)}
    del w
    torch.cuda.empty_cache()
    return res


def bench_rtn(device, steps=20, warmup=3):
    """RTN INT4 and INT2 caches of the full-cache size (30 x 2 x 32760 x 12 x 128 elements,
    one tensor): quantize and dequantize rates.  Algorithmic bytes per element: 2 (bf16) +
    bits/8 (codes) + 2/16 (bf16 block scale)."""
    import torch

    import kv_cache_fp4_amd as kv
    import synth
    cfg = synth.C3
    rows = cfg.layers * 2 * cfg.cache_tokens * cfg.heads
    g = torch.Generator(device=device).manual_seed(7)
    x = torch.randn((rows, cfg.head_dim), generator=g, device=device).to(torch.bfloat16)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream(device)
    res = {"workload": f"rtn_full_cache_{rows}x{cfg.head_dim}: symmetric blockwise RTN, block 16"}
    for bits in (4, 2):
        codes, scales = kv.kvfp4_rtn_quantize(x, bits)
        per = 2.0 + bits / 8.0 + 2.0 / 16.0
        nbytes = x.numel() * per
        for name, fn in (("quantize", lambda: kv.kvfp4_rtn_quantize(x, bits, codes, scales)),
                         ("dequantize", lambda: kv.kvfp4_rtn_dequantize(codes, scales, bits, y=out))):
            for _ in range(warmup):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            torch.cuda.synchronize(device)
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize(device)
            ms = sum(a.elapsed_time(b) for a, b in ev) / steps
            gbs = nbytes / (ms * 1e-3) / 1e9
            res[f"int{bits}_{name}"] = {"ms": round(ms, 4), "GBps": round(gbs, 2),
                                        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        del codes, scales
    del x, out
    torch.cuda.empty_cache()
    return res


# ---- the other configurations: one-layer chunk append, 5B-shaped rollout step ----------------

MALL_BYTES = 1 << 30  # buffer sets rotated over at least this many bytes (Infinity Cache: 256 MB)


def bench_chunk_append(device, calls=300, warmup=30):
    """One layer's chunk append: K and V [4680, 12, 128] bf16 quantized with static_6 (one
    scale group per tensor, one quantize call for both).  Each call reads its own copy of the
    input and writes its own outputs, rotating over sets that total >= 1 GiB, so neither the
    input nor the outputs are served from the Infinity Cache.  Algorithmic bytes per call:
    14,376,960 elements x 2.5625 + 4 per group; the rate includes the call's three kernel
    launches."""
    import torch

    import kv_cache_fp4_amd as kv
    import synth
    cfg = synth.C2
    x0 = torch.cat([synth.chunk_group(cfg, 0, kv_, 0, device=device).reshape(-1, cfg.head_dim)
                    for kv_ in (0, 1)])
    rows, D, rpg = x0.shape[0], cfg.head_dim, cfg.rows_per_group
    nbytes = rows * D * BYTES_PER_ELEM + 4 * 2
    n_sets = -(-MALL_BYTES // int(nbytes))
    sets = [(x0.clone(), torch.empty((rows, D // 2), dtype=torch.uint8, device=device),
             torch.empty((rows, D // 16), dtype=torch.uint8, device=device),
             torch.empty((2,), dtype=torch.float32, device=device)) for _ in range(n_sets)]
    k = [0]

    def call():
        x, c, sc, a = sets[k[0] % n_sets]
        k[0] += 1
        kv.kvfp4_quantize(x, rpg, "static_6", c, sc, a)

    for _ in range(warmup):
        call()
    ms = _time_calls(lambda: [call() for _ in range(calls)], device, 3, 0) / calls
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": (f"{cfg.name}: quantize one {cfg.chunk_tokens}-token chunk of one layer's K "
                        f"and V ({cfg.heads} heads x {cfg.head_dim}, static_6, one group per "
                        f"tensor), {n_sets} rotating buffer sets ({n_sets * nbytes / 2**30:.2f} GiB)"),
           "us_per_call": round(ms * 1e3, 2), "bytes_per_call": nbytes,
           "GBps": round(gbs, 2), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    del sets, x0
    torch.cuda.empty_cache()
    return res


def bench_rollout_5b(device, steps=10, warmup=3):
    """5B-shaped rollout step: 30 layers, 24 heads, head_dim 128, a 36,960-token cache in 14
    chunks of 2,640 tokens (static_6).  Appending one chunk for every layer's K and V under
    each of static_6, static_4 and mse (one quantize call each), and dequantizing the whole
    cache (one call).  Per rule: the append, and the step = append + whole-cache dequantize."""
    import torch

    import synth
    cfg = synth.C4
    w = CacheWorkload(cfg, "static_6", device)
    dq_ms = _time_calls(w.dequantize_all, device, steps, warmup)
    dq_bytes = w.dequant_bytes()
    res = {"workload": (f"{cfg.name}: append one {cfg.chunk_tokens}-token chunk for {cfg.layers} "
                        f"layers x K,V ({cfg.heads} heads x {cfg.head_dim}) + dequantize the whole "
                        f"{cfg.cache_tokens}-token cache"),
           "dequantize": {"ms": round(dq_ms, 4), "bytes": dq_bytes,
                          "GBps": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 2),
                          "pct_of_hbm_peak": round(100 * dq_bytes / (dq_ms * 1e-3) / 1e9
                                                   / HBM_PEAK_GBS, 2)}}
    for rule in ("static_6", "static_4", "mse"):
        w.rule = rule
        ap_ms = _time_calls(w.append, device, steps, warmup)
        ap_bytes = w.append_bytes()
        step_gbs = (ap_bytes + dq_bytes) / ((ap_ms + dq_ms) * 1e-3) / 1e9
        res[rule] = {"append_ms": round(ap_ms, 4), "append_bytes": ap_bytes,
                     "append_GBps": round(ap_bytes / (ap_ms * 1e-3) / 1e9, 2),
                     "append_pct_of_hbm_peak": round(100 * ap_bytes / (ap_ms * 1e-3) / 1e9
                                                     / HBM_PEAK_GBS, 2),
                     "step_ms": round(ap_ms + dq_ms, 4), "step_GBps": round(step_gbs, 2),
                     "step_pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2)}
    del w
    torch.cuda.empty_cache()
    return res


# ---- CPU baseline (the oracle on the host's threads and on one) -------------------------

def _host_threads():
    """Worker threads for the parallel oracle runs: the host's cores, at most 16 (the CPU
    share of one GPU on the machines this runs on)."""
    return max(1, min(16, os.cpu_count() or 1))


def _parallel(work, threads, budget_s):
    """Run work(deadline, i) -> units for i = 1..threads, all at once (the oracle's C calls
    release the GIL); returns (total units, wall seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        done = sum(ex.map(lambda i: work(t0 + budget_s, i), range(1, threads + 1)))
    return done, time.perf_counter() - t0


def cpu_baseline(cfg, rule, budget_s=8.0):
    """Time the oracle on a bounded sample with the step's byte mix: quantize one scale group
    (one chunk of one tensor) with the step's rule, then dequantize it `chunks` times (the
    whole-cache read is `chunks` times the append).  Run once single-threaded and once with
    one independent sample per host thread (value = the all-thread rate)."""
    import numpy as np

    import oracle
    import synth
    x = synth.chunk_group(cfg, 0, 0, 0).reshape(-1, cfg.head_dim)
    xh = x.view(__import__("torch").int16).numpy().view(np.uint16)
    n = xh.size

    def work(deadline, _i=0):
        done = 0
        while True:
            c, s, a = oracle.quantize(xh, cfg.rows_per_group, rule)
            done += n
            for _ in range(cfg.chunks):
                oracle.dequantize(c, s, a, cfg.rows_per_group)
                done += n
            if time.perf_counter() > deadline:
                return done

    t0 = time.perf_counter()
    done1 = work(t0 + budget_s)
    dt1 = time.perf_counter() - t0
    threads = _host_threads()
    doneN, dtN = _parallel(work, threads, budget_s)
    per = 1 + cfg.chunks  # elements counted per quantized element
    sample = (f"(quantize one {cfg.chunk_tokens}x{cfg.heads}x{cfg.head_dim} group, {rule}, then "
              f"dequantize it {cfg.chunks} times) repeated")
    return {"value": round(doneN * BYTES_PER_ELEM / dtN / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{sample} {doneN // (n * per)} times over {threads} threads, "
                       f"{doneN} elements in {dtN:.1f} s, C oracle"),
            "single_thread": {"value": round(done1 * BYTES_PER_ELEM / dt1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1,
                              "sample": f"{sample} {done1 // (n * per)} times, {done1} elements in "
                                        f"{dt1:.1f} s"}}


# ---- float32 output and fake quantization (on the step's own workload) ------------------------

def _time_calls(fn, device, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream(device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize(device)
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize(device)
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def bench_f32_fake(w, device, steps=20, warmup=3):
    """(1) dequantize the whole packed cache to float32 (algorithmic bytes 0.5625 + 4 per
    element + 4 per group); (2) fake-quantize the appended chunk of every layer's K and V
    with the step's rule (bf16 in, bf16 out: 4 B per element + 4 per group)."""
    import torch
    y32 = torch.empty((w.rows, w.cfg.head_dim), dtype=torch.float32, device=device)
    ms = _time_calls(lambda: w.kv.kvfp4_dequantize_f32(w.codes, w.scales, w.amax, w.rpg, y=y32),
                     device, steps, warmup)
    nb = w.cache_elems * (0.5 + 1.0 / 16.0 + 4.0) + 4 * w.n_groups
    res = {"dequantize_f32": {"workload": f"{w.cfg.name}: whole cache to float32",
                              "ms": round(ms, 4), "bytes": nb,
                              "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                              "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}}
    del y32
    yf = torch.empty_like(w.append_src)
    af = torch.empty((w.cfg.groups_per_chunk,), dtype=torch.float32, device=device)
    ms = _time_calls(lambda: w.kv.kvfp4_fake_quantize(w.append_src, w.rpg, w.rule, y=yf,
                                                      group_amax=af), device, steps, warmup)
    nb = w.append_elems * 4.0 + 4 * w.cfg.groups_per_chunk
    res["fake_quantize"] = {"workload": (f"{w.cfg.name}: one {w.cfg.chunk_tokens}-token chunk of "
                                         f"every layer's K and V ({w.rule}), bf16 to bf16"),
                            "ms": round(ms, 4), "bytes": nb,
                            "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                            "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    del yf, af
    torch.cuda.empty_cache()
    return res


def cpu_baseline_attend(budget_s=5.0):
    """The attention oracle (double precision softmax(QK^T)V over the oracle's own bf16
    dequantization of the static_6 cache) on a sample of query rows of the attention
    workload; quantize/dequantize of K and V happen before the clock.  Single-threaded and
    with independent row samples on every host thread (value = the all-thread rate)."""
    import numpy as np
    import torch

    import oracle
    import synth
    cfg = synth.C5
    H, D, Tk = cfg.heads, cfg.head_dim, cfg.cache_tokens
    kvh = []
    for kv_ in (0, 1):
        x = torch.cat([synth.chunk_group(cfg, 0, kv_, c) for c in range(cfg.chunks)])
        xh = x.reshape(-1, D).view(torch.int16).numpy().view(np.uint16)
        c, s_, a = oracle.quantize(xh, cfg.rows_per_group, "static_6")
        kvh.append(oracle.dequantize(c, s_, a, cfg.rows_per_group).reshape(Tk, H, D))
    q = synth.c5_query().view(torch.int16).numpy().view(np.uint16)

    def work(deadline, i=0):
        rng = np.random.default_rng(5 + i)
        done = 0
        while time.perf_counter() < deadline:
            rows = rng.integers(0, synth.C5_Q_TOKENS * H, 8)
            oracle.attend_rows(q, kvh[0], kvh[1], D ** -0.5, rows)
            done += rows.size
        return done

    t0 = time.perf_counter()
    done1 = work(t0 + budget_s)
    dt1 = time.perf_counter() - t0
    threads = _host_threads()
    doneN, dtN = _parallel(work, threads, budget_s)
    fl = 4.0 * Tk * D  # flop per query row
    what = f"query rows (of {synth.C5_Q_TOKENS * H}) of {cfg.name}, each against all {Tk} keys"
    return {"value": round(doneN * fl / dtN / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{doneN} {what}, over {threads} threads in {dtN:.1f} s, C oracle (double)",
            "single_thread": {"value": round(done1 * fl / dt1 / 1e9, 3), "unit": "GFLOP/s",
                              "cores": 1, "sample": f"{done1} {what} in {dt1:.1f} s"}}


# ---- fused dequantize + attention (its own workload) ---------------------------------------

MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_attend(device, steps=50, warmup=50):
    """Q [4680, 12, 128] against the 32760-token NVFP4 K/V cache (7 groups of 4680 tokens,
    static_6), non-causal, softmax scale 1/sqrt(128): 4*Tq*Tk*H*D flops per call.  The MFMA
    clock takes some 40 calls (~40 ms) to settle from idle, hence the long warmup."""
    import torch

    import kv_cache_fp4_amd as kv
    import synth
    cfg = synth.C5
    q = synth.c5_query(device=device)
    packed = []
    for kv_ in (0, 1):
        x = torch.cat([synth.chunk_group(cfg, 0, kv_, c, device=device) for c in range(cfg.chunks)])
        packed.append(kv.kvfp4_quantize(x, cfg.rows_per_group, "static_6"))
    (kc, ks, ka), (vc, vs, va) = packed
    out = torch.empty_like(q)
    scale = cfg.head_dim ** -0.5
    call = lambda: kv.kvfp4_attend(q, kc, ks, ka, vc, vs, va, cfg.chunk_tokens, scale, out=out)  # noqa: E731
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream(device)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(device)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize(device)
    ms = a.elapsed_time(b) / steps
    tq, tk = synth.C5_Q_TOKENS, cfg.cache_tokens
    flops = 4.0 * tq * tk * cfg.heads * cfg.head_dim
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": (f"{cfg.name}: non-causal attention, Q {tq}x{cfg.heads}x{cfg.head_dim} bf16 "
                         f"over an NVFP4 K/V cache of {tk} tokens (static_6, {cfg.chunks} groups)"),
            "ms_per_call": round(ms, 4), "flops_per_call": flops, "steps": steps,
            "roofline": {"bound": "mfma", "kernel": "attend_kernel<128>", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}}


# ---- counters ----------------------------------------------------------------------------

def _source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload_name):
    """HBM bytes per dequant launch from the committed counter summary, or None when the
    summary is missing, is for another workload, or predates the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != _source_hash() or t.get("workload") != workload_name:
        return None
    return t.get("dequant_bytes_per_launch")


# ---- main -----------------------------------------------------------------------------------

def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); sharded by heads, the "
              "dequantize and attention paths need no communication and the quantize path one "
              "max-allreduce of the group amax per append, which is not built", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    cfg = synth.CONFIGS[args.config]
    rule = args.rule or ("mse" if args.config == "C3" else "static_6")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: building {cfg.name} ({rule}) on {torch.cuda.get_device_name(dev)}", file=sys.stderr,
          flush=True)
    w = CacheWorkload(cfg, rule, dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize(dev)

    for _ in range(args.warmup):
        w.append()
        w.dequantize_all()
    torch.cuda.synchronize(dev)
    print(f"bench: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    start, end = ev(), ev()
    dq = [(ev(), ev()) for _ in range(args.steps)]
    ap = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    start.record(stream)
    for i in range(args.steps):
        ap[i][0].record(stream)
        w.append()
        ap[i][1].record(stream)
        dq[i][0].record(stream)
        w.dequantize_all()
        dq[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    ms_dq = sum(a.elapsed_time(b) for a, b in dq) / args.steps
    ms_ap = sum(a.elapsed_time(b) for a, b in ap) / args.steps

    # The same cache read as 60 launches of one layer-tensor each (7 groups, contiguous), as a
    # model that attends layer by layer would issue them.
    gpl = cfg.chunks  # groups per layer-tensor
    n_launch = w.n_groups // gpl
    rpl = gpl * w.rpg

    def per_layer():
        for i in range(n_launch):
            r0, r1 = i * rpl, (i + 1) * rpl
            w.kv.kvfp4_dequantize(w.codes[r0:r1], w.scales[r0:r1], w.amax[i * gpl:(i + 1) * gpl],
                                  w.rpg, y=w.out[r0:r1])
    ms_pl = _time_calls(per_layer, dev, max(args.steps // 3, 3), 2)

    # The append again in the three-kernel form (clear, group amax, encode) for comparison
    # with the one-kernel form the step used.
    three = w.kv.quantize_opts("three_kernel")
    ms_ap3 = _time_calls(lambda: w.append(three), dev, max(args.steps, 3), 2)

    step_bytes = w.append_bytes() + w.dequant_bytes()
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    dq_gbs = w.dequant_bytes() / (ms_dq * 1e-3) / 1e9
    ap_gbs = w.append_bytes() / (ms_ap * 1e-3) / 1e9
    workload = (f"{cfg.name}: append one {cfg.chunk_tokens}-token chunk for {cfg.layers} layers x K,V "
                f"({rule}) + dequantize the whole {cfg.cache_tokens}-token cache "
                f"({cfg.layers} x 2 x {cfg.cache_tokens} x {cfg.heads} x {cfg.head_dim})")
    traffic = traffic_for(cfg.name)
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "layers": cfg.layers, "heads": cfg.heads,
                   "head_dim": cfg.head_dim, "cache_tokens": cfg.cache_tokens,
                   "chunk_tokens": cfg.chunk_tokens, "rule": rule,
                   "elements_per_step": w.append_elems + w.cache_elems,
                   "bytes_per_step": step_bytes, "generator_version": synth.GENERATOR_VERSION},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        # the same step counted without the scale bytes (bf16 + codes only, 2.5 B/element)
        "GBps_without_scale_bytes": round((w.append_elems + w.cache_elems) * 2.5 / (ms_step * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "dequant_kernel",
                     "achieved": round(dq_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dq_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": w.dequant_bytes(), "ms_per_launch": round(ms_dq, 4)},
        "breakdown": {"append_ms": round(ms_ap, 4), "append_GBps": round(ap_gbs, 2),
                      "append_bytes": w.append_bytes(),
                      "append_form": "one-kernel",
                      "append_three_kernel_ms": round(ms_ap3, 4),
                      "dequant_ms": round(ms_dq, 4), "dequant_GBps": round(dq_gbs, 2)},
        "per_layer_dequant": {"launches": n_launch, "ms_total": round(ms_pl, 4),
                              "us_per_launch": round(1e3 * ms_pl / n_launch, 2),
                              "GBps": round(w.dequant_bytes() / (ms_pl * 1e-3) / 1e9, 2)},
    }
    if not args.no_f32_fake:
        print("bench: timing float32 dequantize and fake quantize", file=sys.stderr, flush=True)
        res.update(bench_f32_fake(w, dev))
    del w
    torch.cuda.empty_cache()
    if not args.no_configs:
        print("bench: timing the one-layer chunk append and the 5B-shaped rollout step",
              file=sys.stderr, flush=True)
        res["chunk_append"] = bench_chunk_append(dev)
        res["rollout_5b"] = bench_rollout_5b(dev)
    if not args.no_rtn:
        print("bench: timing the RTN INT4/INT2 caches", file=sys.stderr, flush=True)
        res["rtn"] = bench_rtn(dev)
    if not args.no_paged:
        print("bench: timing the paged-cache gather", file=sys.stderr, flush=True)
        res["paged"] = bench_paged(dev)
    if not args.no_attend:
        print("bench: timing fused dequantize + attention", file=sys.stderr, flush=True)
        res["attend"] = bench_attend(dev)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, rule)
        res["cpu_baseline"]["host_threads_available"] = os.cpu_count()
        if not args.no_attend:
            res["attend"]["cpu_baseline"] = cpu_baseline_attend()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
