"""GPU parity of the RTN INT4/INT2 entry points against the oracle (bit for bit): worked
examples, ragged shapes, K2/V4 (2-bit keys, 4-bit values), the bf16 recent tail copied
behind the dequantized prefix, and a full-cache-sized INT4/INT2 cache on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_oracle_rtn import _load_w6

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["w6_rtn.txt", "w7_rtn_bf16_scale.txt"])
def test_worked_examples_on_gpu(name):
    import kv_cache_fp4_amd as kv
    x16, cases = _load_w6(name)
    x = np.zeros((1, 64), np.uint16)
    x[:, :16] = x16
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    for c in cases:
        codes, scales = kv.kvfp4_rtn_quantize(xt, c["bits"])
        y = kv.kvfp4_rtn_dequantize(codes, scales, c["bits"])
        torch.cuda.synchronize()
        nbytes = 16 * c["bits"] // 8
        assert codes.cpu().numpy()[0, :nbytes].tolist() == [int(t, 16) for t in c["codes"].split()]
        assert _u16(scales)[0, :1].tolist() == [int(t, 16) for t in c["scales"].split()]
        assert _u16(y)[0, :16].tolist() == [int(t, 16) for t in c["dequant_bf16"].split()]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("rows,d,tail", [(1, 64, 0), (37, 128, 5), (1000, 256, 0), (4099, 64, 130),
                                         (20000, 128, 3)])
def test_rtn_matches_oracle(bits, rows, d, tail):
    import kv_cache_fp4_amd as kv
    x = synth.student_t_mix((rows, d), seed=rows + d + bits, p=0.01)
    t = synth.gauss_outliers((tail, d), seed=tail + 1) if tail else None
    codes, scales = kv.kvfp4_rtn_quantize(x.to(DEV), bits)
    y = kv.kvfp4_rtn_dequantize(codes, scales, bits, tail=None if t is None else t.to(DEV))
    torch.cuda.synchronize()
    oc, os_ = oracle.rtn_quantize(_u16(x), bits)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(_u16(scales), os_)
    want = oracle.rtn_dequantize(oc, os_, bits)
    if t is not None:
        want = np.concatenate([want, _u16(t)])
    assert np.array_equal(_u16(y), want)


def test_k2_v4_pair():
    import kv_cache_fp4_amd as kv
    k = synth.gauss_outliers((2000, 128), seed=71)
    v = synth.gauss_outliers((2000, 128), seed=72)
    kc, ks = kv.kvfp4_rtn_quantize(k.to(DEV), 2)
    vc, vs = kv.kvfp4_rtn_quantize(v.to(DEV), 4)
    assert kc.shape == (2000, 32) and vc.shape == (2000, 64)
    ky = kv.kvfp4_rtn_dequantize(kc, ks, 2)
    vy = kv.kvfp4_rtn_dequantize(vc, vs, 4)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(ky), oracle.rtn_dequantize(*oracle.rtn_quantize(_u16(k), 2), 2))
    assert np.array_equal(_u16(vy), oracle.rtn_dequantize(*oracle.rtn_quantize(_u16(v), 4), 4))


@pytest.mark.parametrize("bits", [2, 4])
def test_full_cache_sized_rtn_sampled(bits):
    """30 layers x K,V x 32760 tokens x 12 heads x 128 as one tensor; 2048 sampled rows."""
    import kv_cache_fp4_amd as kv
    cfg = synth.C3
    rows = cfg.layers * 2 * cfg.cache_tokens * cfg.heads
    g = torch.Generator(device=DEV).manual_seed(bits)
    x = (torch.randn((rows, 128), generator=g, device=DEV) * 2).to(torch.bfloat16)
    codes, scales = kv.kvfp4_rtn_quantize(x, bits)
    y = kv.kvfp4_rtn_dequantize(codes, scales, bits)
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(bits).integers(0, rows, 2046)]))).to(DEV)
    xs = _u16(x.index_select(0, idx))
    oc, os_ = oracle.rtn_quantize(xs, bits)
    assert np.array_equal(codes.index_select(0, idx).cpu().numpy(), oc)
    assert np.array_equal(_u16(scales.index_select(0, idx)), os_)
    assert np.array_equal(_u16(y.index_select(0, idx)), oracle.rtn_dequantize(oc, os_, bits))
