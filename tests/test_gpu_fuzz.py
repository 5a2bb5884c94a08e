"""Structured fuzz against the oracle, bit for bit: blocks built from an alphabet of special
values at random scales, so that block contexts near every rounding boundary occur.

Each seeded case draws head_dim (64..1024), rows, rows_per_group and a rule, then fills each
group with blocks whose elements are, around a per-group binade 2^e (e from the bf16
subnormal range to near the bf16 maximum):
  - +-0;
  - E2M1 grid values and the midpoints between them, times a per-block scale, and the bf16
    neighbours of those (one ulp either side) -- codes decided by a tie or by one ulp;
  - bf16 subnormals;
  - block maxima placed so that m/6 falls on a midpoint of the E4M3 grid relative to the
    group's binade, or one bf16 ulp beside it (the scale rounding near a tie; exact ties
    where the group's s_enc is a power of two);
  - rare outliers 2^8 .. 2^16 times larger (blocks that saturate the 4-max candidate).
Checked in both quantize forms: codes, scale bytes, group amax, dequantize (bf16 and float32)
of the GPU's own packed output, fake quantization; every third case also through RTN INT4
and INT2.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RULES = ["static_6", "static_4", "mse"]
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MIDS = (GRID[1:] + GRID[:-1]) / 2


def _bf16_bits(f):
    return torch.from_numpy(np.asarray(f, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _case(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 192, 256, 512, 1024]))
    rows = int(rng.integers(1, 400))
    rpg = int(rng.integers(1, rows + 1))
    rule = RULES[seed % 3]
    n = rows * d
    nb = n // 16
    # per-group binade, then per-block scale inside it
    groups = np.arange(rows) // rpg
    e_group = rng.integers(-135, 120, size=groups.max() + 1)
    e_row = np.repeat(e_group[groups], d // 16)                 # per block
    kind = rng.integers(0, 6, size=(nb, 16))
    base = np.where(kind == 0, 0.0,
           np.where(kind == 1, rng.choice(GRID, size=(nb, 16)),
           np.where(kind == 2, rng.choice(MIDS, size=(nb, 16)),
           np.where(kind == 3, rng.uniform(0, 6, size=(nb, 16)),
           np.where(kind == 4, rng.choice(MIDS, size=(nb, 16)) * (1 + 2.0 ** -8),
                    rng.choice(MIDS, size=(nb, 16)) * (1 - 2.0 ** -8))))))
    block_scale = np.exp2(e_row[:, None] + rng.integers(-6, 3, size=(nb, 1)))
    x = base * block_scale * rng.choice([-1.0, 1.0], size=(nb, 16))
    # block maxima near a tie of the E4M3 rounding of m/6 * s_enc: m/6 on a midpoint between
    # two E4M3 values relative to the group binade, or one bf16 ulp beside it
    tie = rng.random(nb) < 0.1
    e4_mid = (1.0 + (2 * rng.integers(0, 8, size=nb) + 1) / 16.0) \
        * np.exp2(rng.integers(-6, 8, size=nb))
    nudge = rng.choice([1 - 2.0 ** -8, 1.0, 1 + 2.0 ** -8], size=tie.sum())
    x[tie, 0] = (6.0 * e4_mid * np.exp2(e_row - 8))[tie] * nudge
    # bf16 subnormals and outliers
    sub = rng.random((nb, 16)) < 0.02
    x[sub] = (rng.integers(1, 128, size=sub.sum()) * 2.0 ** -133
              * rng.choice([-1, 1], size=sub.sum()))
    out = rng.random((nb, 16)) < 0.002
    x[out] *= np.exp2(rng.integers(8, 17, size=out.sum()))
    x = np.clip(x, -3.38e38, 3.38e38)
    xh = _bf16_bits(x.reshape(rows, d).astype(np.float32))
    # bf16 rounding can make new infinities only beyond the clip; keep every pattern finite
    assert np.all((xh & 0x7F80) != 0x7F80)
    return xh, rpg, rule


@pytest.fixture
def options():
    import kv_cache_fp4_amd as kv
    return kv


def _opts(kv, fused):
    return kv.quantize_opts("one_kernel" if fused else "three_kernel")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("seed", range(60))
def test_fuzz_matches_oracle(options, seed):
    kv = options
    xh, rpg, rule = _case(seed)
    x = torch.from_numpy(xh.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    oc, os_, oa = oracle.quantize(xh, rpg, rule)
    oy = oracle.dequantize(oc, os_, oa, rpg)
    oy32 = oracle.dequantize_f32(oc, os_, oa, rpg)
    ofy, ofa = oracle.fake_quantize(xh, rpg, rule)
    for fused in (1, 0):
        opts = _opts(kv, fused)
        c, s, a = kv.kvfp4_quantize(x, rpg, rule, opts=opts)
        y = kv.kvfp4_dequantize(c, s, a, rpg)
        y32 = kv.kvfp4_dequantize_f32(c, s, a, rpg)
        fy, fa = kv.kvfp4_fake_quantize(x, rpg, rule, opts=opts)
        torch.cuda.synchronize()
        what = (seed, xh.shape, rpg, rule, fused)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), oa.view(np.uint32)), what
        assert np.array_equal(s.cpu().numpy(), os_), what
        assert np.array_equal(c.cpu().numpy(), oc), what
        assert np.array_equal(_u16(y), oy), what
        assert np.array_equal(y32.cpu().numpy().view(np.uint32), oy32.view(np.uint32)), what
        assert np.array_equal(fa.cpu().numpy().view(np.uint32), ofa.view(np.uint32)), what
        assert np.array_equal(_u16(fy), ofy), what


@pytest.mark.parametrize("seed", range(0, 60, 3))
@pytest.mark.parametrize("bits", [4, 2])
def test_fuzz_rtn_matches_oracle(seed, bits):
    """The same blocks through RTN INT4/INT2 (per-block bf16 scale, round half to even):
    codes, scales and the dequantization."""
    import kv_cache_fp4_amd as kv
    xh, _, _ = _case(seed)
    x = torch.from_numpy(xh.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    c, s = kv.kvfp4_rtn_quantize(x, bits)
    y = kv.kvfp4_rtn_dequantize(c, s, bits)
    torch.cuda.synchronize()
    oc, os_ = oracle.rtn_quantize(xh, bits)
    what = (seed, xh.shape, bits)
    assert np.array_equal(_u16(s), os_), what
    assert np.array_equal(c.cpu().numpy(), oc), what
    assert np.array_equal(_u16(y), oracle.rtn_dequantize(oc, os_, bits)), what
