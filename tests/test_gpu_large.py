"""Beyond 32-bit unit indexing: one tensor of 2^27 + 4133 rows x 128 (2.15e9 eight-element
units, 34 GB of bf16) quantized in C3-sized groups (56,160 rows: the one-kernel form, a
ragged last group) and dequantized in one call each, then checked:
  - every full group's amax against a max over its rows on the GPU;
  - the groups on both sides of unit 2^31 (row 2^27), the first group and the ragged last
    group: codes, scale bytes, amax and the bf16 dequantization against the oracle;
  - RTN INT4 over the same tensor: rows on both sides of unit 2^31 and the last rows
    against the oracle.
About 90 GB of device memory.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D = 128
ROWS = (1 << 27) + 4133
RPG = 4680 * 12


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def big():
    torch.cuda.empty_cache()   # blocks cached by earlier tests count as used
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 120 * 2 ** 30:
        pytest.skip(f"needs about 100 GB of free device memory, {free / 2 ** 30:.0f} GiB free")
    g = torch.Generator(device=DEV).manual_seed(31)
    x = torch.empty((ROWS, D), dtype=torch.bfloat16, device=DEV)
    step = 1 << 23
    for r0 in range(0, ROWS, step):
        r1 = min(r0 + step, ROWS)
        x[r0:r1] = torch.randn((r1 - r0, D), generator=g, device=DEV, dtype=torch.float32) \
            .to(torch.bfloat16)
    yield x
    del x
    torch.cuda.empty_cache()


def test_quantize_dequantize_beyond_2_31_units(big):
    import kv_cache_fp4_amd as kv
    x = big
    assert ROWS * D // 8 > 2 ** 31
    codes, scales, amax = kv.kvfp4_quantize(x, RPG, "mse")
    y = kv.kvfp4_dequantize(codes, scales, amax, RPG)
    torch.cuda.synchronize()
    ng = -(-ROWS // RPG)
    assert amax.numel() == ng
    full = ROWS // RPG
    for g0 in range(0, full, 256):   # max |x| per group, 256 groups (3.7 GB) at a time
        g1 = min(g0 + 256, full)
        ref = x[g0 * RPG:g1 * RPG].view(g1 - g0, RPG * D).abs().amax(dim=1).float()
        assert torch.equal(amax[g0:g1], ref), g0
    g_cross = (1 << 27) // RPG       # the group holding row 2^27 (unit 2^31)
    for g in sorted({0, g_cross - 1, g_cross, g_cross + 1, ng - 1} & set(range(ng))):
        r0, r1 = g * RPG, min((g + 1) * RPG, ROWS)
        xh = _u16(x[r0:r1])
        oc, os_, oa = oracle.quantize(xh, RPG, "mse")
        assert oa.view(np.uint32)[0] == amax[g:g + 1].cpu().numpy().view(np.uint32)[0], g
        assert np.array_equal(scales[r0:r1].cpu().numpy(), os_), g
        assert np.array_equal(codes[r0:r1].cpu().numpy(), oc), g
        assert np.array_equal(_u16(y[r0:r1]), oracle.dequantize(oc, os_, oa, RPG)), g
    del codes, scales, amax, y
    torch.cuda.empty_cache()


def test_rtn_beyond_2_31_units(big):
    import kv_cache_fp4_amd as kv
    x = big
    codes, scales = kv.kvfp4_rtn_quantize(x, 4)
    y = kv.kvfp4_rtn_dequantize(codes, scales, 4)
    torch.cuda.synchronize()
    for r0, r1 in (((1 << 27) - 64, (1 << 27) + 64), (ROWS - 64, ROWS)):
        xh = _u16(x[r0:r1])
        oc, os_ = oracle.rtn_quantize(xh, 4)
        assert np.array_equal(_u16(scales[r0:r1]), os_), r0
        assert np.array_equal(codes[r0:r1].cpu().numpy(), oc), r0
        assert np.array_equal(_u16(y[r0:r1]), oracle.rtn_dequantize(oc, os_, 4)), r0
    del codes, scales, y
    torch.cuda.empty_cache()
