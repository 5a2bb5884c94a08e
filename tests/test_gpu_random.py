"""Randomized GPU parity: 40 seeded cases of random shape (rows, head_dim, rows_per_group),
rule and per-group value range (group amax from 2^-60 to 2^100, inside the contract), with
zero blocks, zero groups and a few huge outliers mixed in.  Every output -- codes, scale
bytes, group amax, bf16 and float32 dequantize, fake quantization -- must equal the
oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RULES = ["static_6", "static_4", "mse"]


def _case(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.integers(1, 17)) * 64
    rows = int(rng.integers(1, max(2, 600_000 // d)))
    rpg = int(rng.integers(1, rows + 1)) if rng.random() < 0.7 else rows
    rule = RULES[int(rng.integers(0, 3))]
    ng = -(-rows // rpg)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    # per-group scale 2^e, e in [-60, 100]: every group amax stays in [2^-64, bf16 max)
    e = rng.integers(-60, 101, ng).astype(np.float32)
    x *= np.repeat(np.exp2(e), rpg)[:rows, None]
    blocks = x.reshape(rows, d // 16, 16)
    blocks[rng.random((rows, d // 16)) < 0.03] = 0.0           # zero blocks
    if ng > 2 and rng.random() < 0.5:
        g = int(rng.integers(0, ng))
        x[g * rpg:(g + 1) * rpg] = 0.0                            # a zero group
    hit = rng.random(x.shape) < 1e-4                              # outliers x 2^6
    x[hit] *= 64.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xb = torch.where(torch.isinf(xb), torch.zeros_like(xb), xb)   # keep every value finite
    return xb, rpg, rule


@pytest.mark.parametrize("seed", list(range(40)))
def test_random_case_matches_oracle(seed):
    import kv_cache_fp4_amd as kv
    xb, rpg, rule = _case(1000 + seed)
    rows, d = xb.shape
    xh = xb.view(torch.int16).numpy().view(np.uint16)
    oc, os_, oa = oracle.quantize(xh, rpg, rule)
    oy = oracle.dequantize(oc, os_, oa, rpg)
    of = oracle.dequantize_f32(oc, os_, oa, rpg)
    ofy, ofa = oracle.fake_quantize(xh, rpg, rule)

    xd = xb.to(DEV)
    c, s, a = kv.kvfp4_quantize(xd, rpg, rule)
    y = kv.kvfp4_dequantize(c, s, a, rpg)
    y32 = kv.kvfp4_dequantize_f32(c, s, a, rpg)
    fy, fa = kv.kvfp4_fake_quantize(xd, rpg, rule)
    torch.cuda.synchronize()
    what = f"seed {seed}: rows {rows} d {d} rpg {rpg} {rule}"
    assert np.array_equal(a.cpu().numpy().view(np.uint32), oa.view(np.uint32)), what
    assert np.array_equal(s.cpu().numpy(), os_), what
    assert np.array_equal(c.cpu().numpy(), oc), what
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), oy), what
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), of.view(np.uint32)), what
    assert np.array_equal(fa.cpu().numpy().view(np.uint32), ofa.view(np.uint32)), what
    assert np.array_equal(fy.view(torch.int16).cpu().numpy().view(np.uint16), ofy), what
