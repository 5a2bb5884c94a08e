"""Exhaustive GPU parity against the oracle, bit for bit.

Quantize: every finite bf16 bit pattern (65,280 of them, 510 rows of 128) under every rule,
in both quantize forms (one kernel; three kernels), arranged as
  - patterns in order, one group per row: each row holds 128 consecutive patterns (part of
    one binade's mantissas, one sign), so every row sits at its own magnitude;
  - patterns in order in groups of 8 rows (128 units, so the one-kernel form applies, also
    to the first groups, whose amax is small enough for s_enc and inv to overflow);
  - a seeded permutation, one group per row: blocks that mix magnitudes over the whole bf16
    range, so underflowing elements sit next to the block maximum;
  - the same permutation in groups of 7 rows (ragged last group of 6);
  - every pattern in one group (A = the largest finite bf16: most blocks underflow).
Checked: codes, scale bytes, group amax, the bf16 dequantization of the GPU's own packed
output, and fake quantization.

Paged: the patterns in order as logical blocks written into pages in a random order (pages
of 1 and 6 rows, both forms), gathered back to bf16 and float32.

RTN INT4 / INT2: every finite pattern in order and permuted; codes, bf16 scales and the
dequantization.

Dequantize: every code byte (both nibbles) with every scale byte 0x00..0x7E, under group
amax values that put the products from the float32 subnormal range to near the bf16
maximum; bf16 and float32 outputs.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RULES = ["static_6", "static_4", "mse"]
D = 128


def _finite_patterns():
    p = np.arange(65536, dtype=np.uint32)
    return p[(p & 0x7F80) != 0x7F80].astype(np.uint16)


def _arrangements():
    p = _finite_patterns()
    assert p.size == 510 * D
    perm = p[np.random.default_rng(0).permutation(p.size)]
    return {
        "in_order/1": (p.reshape(-1, D), 1),
        "in_order/8": (p.reshape(-1, D), 8),
        "permuted/1": (perm.reshape(-1, D), 1),
        "permuted/7": (perm.reshape(-1, D), 7),
        "in_order/all": (p.reshape(-1, D), 510),
    }


ARR = _arrangements()


@pytest.fixture
def options():
    import kv_cache_fp4_amd as kv
    return kv


def _opts(kv, fused):
    return kv.quantize_opts("one_kernel" if fused else "three_kernel")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fused", [1, 0], ids=["one_kernel", "three_kernels"])
@pytest.mark.parametrize("name", list(ARR))
def test_every_finite_bf16_pattern(options, name, fused):
    kv = options
    opts = _opts(kv, fused)
    xh, rpg = ARR[name]
    x = torch.from_numpy(xh.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    for rule in RULES:
        c, s, a = kv.kvfp4_quantize(x, rpg, rule, opts=opts)
        y = kv.kvfp4_dequantize(c, s, a, rpg)
        fy, fa = kv.kvfp4_fake_quantize(x, rpg, rule, opts=opts)
        torch.cuda.synchronize()
        oc, os_, oa = oracle.quantize(xh, rpg, rule)
        what = (name, fused, rule)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), oa.view(np.uint32)), what
        assert np.array_equal(s.cpu().numpy(), os_), what
        assert np.array_equal(c.cpu().numpy(), oc), what
        assert np.array_equal(_u16(y), oracle.dequantize(oc, os_, oa, rpg)), what
        ofy, ofa = oracle.fake_quantize(xh, rpg, rule)
        assert np.array_equal(fa.cpu().numpy().view(np.uint32), ofa.view(np.uint32)), what
        assert np.array_equal(_u16(fy), ofy), what


@pytest.mark.parametrize("fused", [1, 0], ids=["one_kernel", "three_kernels"])
@pytest.mark.parametrize("rows_per_page", [1, 6])
def test_every_finite_bf16_pattern_paged(options, rows_per_page, fused):
    """The patterns in order as logical blocks of a paged cache, written into pages in a
    seeded random order (every page its own scale group, from subnormal-amax pages up), then
    gathered back to dense bf16 and float32."""
    kv = options
    opts = _opts(kv, fused)
    xh = ARR["in_order/1"][0]
    n_blocks = xh.shape[0] // rows_per_page
    xh = xh[: n_blocks * rows_per_page]
    n_pages = n_blocks + 3
    table = np.random.default_rng(1).permutation(n_pages)[:n_blocks].astype(np.int32)
    x = torch.from_numpy(xh.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    td = torch.from_numpy(table).to(DEV)
    for rule in RULES:
        codes = torch.zeros((n_pages, rows_per_page, D // 2), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((n_pages, rows_per_page, D // 16), dtype=torch.uint8, device=DEV)
        amax = torch.zeros((n_pages,), dtype=torch.float32, device=DEV)
        kv.kvfp4_quantize_paged(x, td, rows_per_page, codes, scales, amax, rule, opts=opts)
        y = kv.kvfp4_dequantize_paged(codes, scales, amax, td, rows_per_page)
        y32 = kv.kvfp4_dequantize_paged_f32(codes, scales, amax, td, rows_per_page)
        torch.cuda.synchronize()
        oc, os_, oa = oracle.quantize_paged(xh, table, rows_per_page, n_pages, rule)
        what = (rows_per_page, fused, rule)
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), oa.view(np.uint32)), what
        assert np.array_equal(scales.cpu().numpy(), os_), what
        assert np.array_equal(codes.cpu().numpy(), oc), what
        ref = oracle.dequantize_paged(oc, os_, oa, table, rows_per_page)
        assert np.array_equal(_u16(y), ref), what
        ref32 = oracle.dequantize_paged_f32(oc, os_, oa, table, rows_per_page)
        assert np.array_equal(y32.cpu().numpy().view(np.uint32), ref32.view(np.uint32)), what


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("name", ["in_order/1", "permuted/1"])
def test_every_finite_bf16_pattern_rtn(name, bits):
    """RTN INT4/INT2 (no group amax): per-block bf16 scales at every magnitude, from blocks of
    subnormals (reciprocal +inf) to blocks at the bf16 maximum."""
    import kv_cache_fp4_amd as kv
    xh, _ = ARR[name]
    x = torch.from_numpy(xh.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    c, s = kv.kvfp4_rtn_quantize(x, bits)
    y = kv.kvfp4_rtn_dequantize(c, s, bits)
    torch.cuda.synchronize()
    oc, os_ = oracle.rtn_quantize(xh, bits)
    assert np.array_equal(_u16(s), os_), (name, bits)
    assert np.array_equal(c.cpu().numpy(), oc), (name, bits)
    assert np.array_equal(_u16(y), oracle.rtn_dequantize(oc, os_, bits)), (name, bits)


# Group amax values: s_dec = A/2688 exactly 1; ordinary; tiny (products in the float32
# subnormal range and below bf16's smallest subnormal); huge (products near the bf16
# maximum, the largest finite bf16); a value that is not a power of two; zero (every
# product 0).
AMAX = [2688.0, 1.0, 0.1, 3.0e-35, 1.0e-41, 2.5e35, 3.3895314e38, 7.389, 0.0]


def _every_code_and_scale():
    """Rows of 64 code bytes and 8 scale bytes covering each (code byte, scale byte) pair:
    256 code bytes = 32 blocks of 8 bytes per scale byte, 127 scale bytes."""
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(32, 8), (127, 1))  # [4064, 8]
    scales = np.repeat(np.arange(127, dtype=np.uint8), 32)                      # [4064]
    return codes.reshape(-1, D // 2), scales.reshape(-1, D // 16)               # 508 rows


def test_every_code_and_scale_byte_dequantizes_exactly():
    import kv_cache_fp4_amd as kv
    codes, scales = _every_code_and_scale()
    rows = codes.shape[0]
    amax = np.array([AMAX[r % len(AMAX)] for r in range(rows)], dtype=np.float32)
    cd = torch.from_numpy(codes).to(DEV)
    sd = torch.from_numpy(scales).to(DEV)
    ad = torch.from_numpy(amax).to(DEV)
    y = kv.kvfp4_dequantize(cd, sd, ad, 1)
    y32 = kv.kvfp4_dequantize_f32(cd, sd, ad, 1)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(y), oracle.dequantize(codes, scales, amax, 1))
    ref32 = oracle.dequantize_f32(codes, scales, amax, 1)
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
