"""GPU parity of the paged-cache entry points against the oracle (bit for bit): permuted
block tables with spare pages, skipped entries on both the write and the read side, pages
gathered twice, every rule, both quantize forms (one kernel with the hand-off in each page;
three kernels), and a full-size paged cache (16-token pages, 12 heads, 128 dims) on sampled
pages."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _opts(fused):
    import kv_cache_fp4_amd as kv
    return kv.quantize_opts("one_kernel" if fused else "three_kernel")


@pytest.mark.parametrize("fused", [1, 0], ids=["one_kernel", "three_kernels"])
@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
@pytest.mark.parametrize("nb,rpp,d", [(37, 16 * 12, 128), (5, 64, 64), (200, 16 * 4, 256),
                                      (9, 1, 64)])
def test_paged_round_trip_matches_oracle(fused, rule, nb, rpp, d):
    import kv_cache_fp4_amd as kv
    npg = nb + 7
    x = synth.gauss_outliers((nb * rpp, d), seed=nb + rpp + d)
    tab = np.random.default_rng(nb).permutation(npg)[:nb].astype(np.int32)
    codes = torch.full((npg, rpp, d // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((npg, rpp, d // 16), 0x33, dtype=torch.uint8, device=DEV)
    amax = torch.full((npg,), -3.0, dtype=torch.float32, device=DEV)
    ttab = torch.from_numpy(tab).to(DEV)
    kv.kvfp4_quantize_paged(x.to(DEV), ttab, rpp, codes, scales, amax, rule, opts=_opts(fused))
    y = kv.kvfp4_dequantize_paged(codes, scales, amax, ttab, rpp)
    torch.cuda.synchronize()
    oc = np.full((npg, rpp, d // 2), 0x5A, np.uint8)
    os_ = np.full((npg, rpp, d // 16), 0x33, np.uint8)
    oa = np.full(npg, -3.0, np.float32)
    oracle.quantize_paged(_u16(x), tab, rpp, npg, rule, oc, os_, oa)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(amax.cpu().numpy(), oa)
    assert np.array_equal(_u16(y), oracle.dequantize_paged(oc, os_, oa, tab, rpp))


@pytest.mark.parametrize("fused", [1, 0], ids=["one_kernel", "three_kernels"])
def test_paged_quantize_skips_entries(fused):
    """Write-side table entries outside [0, n_pages) are skipped: their blocks write nothing
    and every page not named keeps its old bytes."""
    import kv_cache_fp4_amd as kv
    nb, rpp, d, npg = 6, 192, 128, 5
    x = synth.gauss_outliers((nb * rpp, d), seed=11)
    tab = np.array([3, -1, 0, npg + 2, 1, 4], dtype=np.int32)
    codes = torch.full((npg, rpp, d // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((npg, rpp, d // 16), 0x33, dtype=torch.uint8, device=DEV)
    amax = torch.full((npg,), -3.0, dtype=torch.float32, device=DEV)
    kv.kvfp4_quantize_paged(x.to(DEV), torch.from_numpy(tab).to(DEV), rpp, codes, scales, amax,
                            "mse", opts=_opts(fused))
    torch.cuda.synchronize()
    oc = np.full((npg, rpp, d // 2), 0x5A, np.uint8)
    os_ = np.full((npg, rpp, d // 16), 0x33, np.uint8)
    oa = np.full(npg, -3.0, np.float32)
    oracle.quantize_paged(_u16(x), tab, rpp, npg, "mse", oc, os_, oa)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(amax.cpu().numpy(), oa)
    assert np.all(oc[2] == 0x5A) and oa[2] == -3.0  # page 2 is named by no valid entry


def test_paged_gather_skips_and_repeats():
    import kv_cache_fp4_amd as kv
    nb, rpp, d = 6, 192, 128
    x = synth.gauss_outliers((nb * rpp, d), seed=3)
    tab = np.arange(nb, dtype=np.int32)
    ttab = torch.from_numpy(tab).to(DEV)
    codes = torch.zeros((nb, rpp, d // 2), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((nb, rpp, d // 16), dtype=torch.uint8, device=DEV)
    amax = torch.zeros((nb,), dtype=torch.float32, device=DEV)
    kv.kvfp4_quantize_paged(x.to(DEV), ttab, rpp, codes, scales, amax, "mse")
    gather = np.array([5, -1, 5, nb, 0, 2, 2], dtype=np.int32)
    y = torch.full((gather.size * rpp, d), 0x1234, dtype=torch.int16, device=DEV)
    kv.kvfp4_dequantize_paged(codes, scales, amax, torch.from_numpy(gather).to(DEV), rpp,
                              y=y.view(torch.bfloat16))
    torch.cuda.synchronize()
    oc, os_, oa = oracle.quantize_paged(_u16(x), tab, rpp, nb, "mse")
    want = oracle.dequantize_paged(oc, os_, oa, gather, rpp,
                                   y=np.full((gather.size * rpp, d), 0x1234, np.uint16))
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want)


def test_full_size_paged_cache_every_page():
    """30 layers x K,V x 2048 pages of 16 tokens (32768 tokens) x 12 heads x 128, pages in a
    random physical order: all 122,880 pages (codes, scale bytes, page amax) and the whole
    gather to dense bf16, bit for bit against the oracle, which quantizes and gathers the
    same blocks through the same table on the host's threads (each thread a run of blocks;
    the table is a permutation, so their pages are disjoint)."""
    import os
    import time
    from concurrent.futures import ThreadPoolExecutor

    import bench
    t0 = time.perf_counter()
    w = bench.PagedWorkload(DEV)
    w.dequantize_all()
    torch.cuda.synchronize()
    tab = w.table.cpu().numpy()
    assert np.array_equal(np.sort(tab), np.arange(w.n_blocks))
    xh = _u16(w.src)
    D = xh.shape[1]
    oc = np.zeros((w.n_blocks, w.rpp, D // 2), np.uint8)
    os_ = np.zeros((w.n_blocks, w.rpp, D // 16), np.uint8)
    oa = np.zeros(w.n_blocks, np.float32)
    threads = max(1, min(16, os.cpu_count() or 1))
    parts = np.array_split(np.arange(w.n_blocks), threads * 4)

    def quant(p):
        b0, b1 = int(p[0]), int(p[-1]) + 1
        oracle.quantize_paged(xh[b0 * w.rpp:b1 * w.rpp], tab[b0:b1], w.rpp, w.n_blocks,
                              "static_6", oc, os_, oa)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(quant, parts))
    assert np.array_equal(w.codes.cpu().numpy(), oc)
    assert np.array_equal(w.scales.cpu().numpy(), os_)
    assert np.array_equal(w.amax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
    gy = _u16(w.out)

    def gather_ok(p):
        b0, b1 = int(p[0]), int(p[-1]) + 1
        oy = oracle.dequantize_paged(oc, os_, oa, tab[b0:b1], w.rpp)
        return np.array_equal(gy[b0 * w.rpp:b1 * w.rpp], oy)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        assert all(ex.map(gather_ok, parts))
    print(f"paged cache: {w.n_blocks} pages checked in {time.perf_counter() - t0:.1f} s on "
          f"{threads} threads")
