"""Pins for the oracle's float32 dequantize output and its fake quantization (quantize then
dequantize to bf16 without a packed store), no GPU.

Pages: "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference", "Stage 3"
(the dequantize kernel emits float32 or bf16) and "Stage 1" (the fake-quant variant of the
block-scale path).

What each test would catch if the oracle were wrong:
  - W2 float32 values: a product order other than (E4M3(sf) * s_dec) * E2M1(c) changes the
    last bit of 1.9285716 or 1.5 (the fixture lists the values the other order gives);
  - exhaustive A = 2688: a wrong decode table entry, a lost sign or an extra rounding;
  - exhaustive rounding bound: a wrong global scale (missing or inverted s_dec);
  - bf16 of the float32 output vs the bf16 path: a float32 path that drifted from the bf16
    one (they must differ only by the final rounding);
  - fake quantization: the worked examples' dequantized bytes and amax.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import goldens
from tests.test_oracle_quant import E4M3, GRID, _bf16


def _exhaustive_rows():
    sf = np.arange(0x7F, dtype=np.uint8)
    c = np.arange(16, dtype=np.uint8)
    cc, ss = (t.reshape(-1) for t in np.meshgrid(c, sf, indexing="ij"))
    codes = np.repeat((cc | (cc << 4)).astype(np.uint8)[:, None], 8, axis=1)
    return cc, ss, codes, ss[:, None].astype(np.uint8)


@pytest.mark.parametrize("name", goldens.ALL)
def test_worked_examples_f32_and_fake(name):
    g = goldens.load(name)
    for case in g["cases"]:
        codes, scales, amax = oracle.quantize(g["x"], g["rows_per_group"], case["rule"])
        yf = oracle.dequantize_f32(codes, scales, amax, g["rows_per_group"])
        if case["dequant_f32"] is not None:
            assert np.array_equal(yf.reshape(-1).view(np.uint32), case["dequant_f32"]), \
                (name, case["rule"])
        y, a = oracle.fake_quantize(g["x"], g["rows_per_group"], case["rule"])
        assert np.array_equal(y.reshape(-1), case["dequant"]), (name, case["rule"])
        assert a[0] == np.float32(g["amax"])


def test_w2_has_f32_values():
    assert all(c["dequant_f32"] is not None for c in goldens.load("w2_four_over_six.txt")["cases"])


def test_f32_exhaustive_exact_when_global_scale_is_one():
    cc, ss, codes, scales = _exhaustive_rows()
    y = oracle.dequantize_f32(codes, scales, np.float32([2688.0]), cc.size)
    want = GRID[cc] * E4M3[ss]                  # exact in binary32 (2 x 4 significant bits)
    got = y[:, 0].astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(y, np.repeat(y[:, :1], 16, axis=1))


@pytest.mark.parametrize("A", [1.0, 6.0, 20.0, 0.037, 3.0e4])
def test_f32_exhaustive_within_rounding_bound(A):
    cc, ss, codes, scales = _exhaustive_rows()
    y = oracle.dequantize_f32(codes, scales, np.float32([A]), cc.size)
    exact = GRID[cc] * E4M3[ss] * (float(np.float32(A)) / 2688.0)
    got = y[:, 0].astype(np.float64)
    # three binary32 roundings: s_dec, S, v * S
    tol = np.abs(exact) * (3.0001 * 2.0 ** -24)
    assert np.all(np.abs(got - exact) <= tol)


@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_bf16_of_f32_output_is_the_bf16_output(rule):
    g = torch.Generator().manual_seed(11)
    x = _bf16((torch.randn((300, 128), generator=g) * 3).numpy())
    codes, scales, amax = oracle.quantize(x, 128, rule)
    yf = oracle.dequantize_f32(codes, scales, amax, 128)
    yb = oracle.dequantize(codes, scales, amax, 128)
    assert np.array_equal(_bf16(yf), yb)
    assert np.array_equal(oracle.float_to_bf16(yf.reshape(-1)).reshape(yb.shape), yb)


def test_f32_paged_gathers_pages():
    g = torch.Generator().manual_seed(12)
    rpp, d, n_pages = 8, 64, 5
    x = _bf16(torch.randn((n_pages * rpp, d), generator=g).numpy())
    ident = np.arange(n_pages, dtype=np.int32)
    codes, scales, amax = oracle.quantize_paged(x, ident, rpp, n_pages, "static_6")
    table = np.array([3, -1, 0, 3, 7], np.int32)
    y = oracle.dequantize_paged_f32(codes, scales, amax, table, rpp)
    for b, pg in enumerate(table):
        blk = y[b * rpp:(b + 1) * rpp]
        if 0 <= pg < n_pages:
            want = oracle.dequantize_rows_f32(codes[pg], scales[pg], amax[pg])
            assert np.array_equal(blk.view(np.uint32), want.view(np.uint32))
        else:
            assert not blk.any()          # skipped entry: the given (zero) buffer untouched


@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_fake_quantize_groups_and_ragged_tail(rule):
    g = torch.Generator().manual_seed(13)
    x = _bf16((torch.randn((70, 64), generator=g) * torch.linspace(0.1, 9, 70)[:, None]).numpy())
    y, amax = oracle.fake_quantize(x, 32, rule)
    assert amax.size == 3
    for gi, r0 in enumerate(range(0, 70, 32)):
        xs = x[r0:r0 + 32]
        assert amax[gi] == oracle.group_amax(xs)
        c, s = oracle.quantize_rows(xs, amax[gi], rule)
        assert np.array_equal(y[r0:r0 + 32], oracle.dequantize_rows(c, s, amax[gi]))
