"""Pins for the oracle's quantize / dequantize against worked examples, closed forms,
invariants and brute force (no GPU).

What each test would catch if the oracle were wrong:
  - worked examples W1-W3: a wrong nibble order, divisor, global-scale formula, FP8 rounding
    or sign handling changes at least one byte;
  - scaled W1: a scale that is not carried exactly through powers of two;
  - static invariants: a divisor swapped between static_6 and static_4;
  - mse brute force: a wrong error definition, a flipped comparison or a wrong tie rule;
  - group tests: a wrong group index or amax scope;
  - exhaustive dequant: a wrong E2M1 or E4M3 decode entry or a wrong product order;
  - zero times infinity: a NaN (or a sign taken from it) where a zero element or an all-zero
    block meets an overflowed s_enc or inv.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import goldens


def _grid():
    vals = {}
    import os
    with open(os.path.join(goldens.GOLDEN_DIR, "e2m1_grid.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line and not line.startswith("code"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)])


GRID = _grid()
E4M3 = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _from_bf16(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


# ---- worked examples ------------------------------------------------------------------

@pytest.mark.parametrize("name", goldens.ALL)
def test_worked_examples(name):
    g = goldens.load(name)
    for case in g["cases"]:
        codes, scales, amax = oracle.quantize(g["x"], g["rows_per_group"], case["rule"])
        assert amax[0] == np.float32(g["amax"])
        assert np.array_equal(scales.reshape(-1), case["scales"]), (name, case["rule"])
        assert np.array_equal(codes.reshape(-1), case["codes"]), (name, case["rule"])
        y = oracle.dequantize(codes, scales, amax, g["rows_per_group"])
        assert np.array_equal(y.reshape(-1), case["dequant"]), (name, case["rule"])


@pytest.mark.parametrize("k", list(range(-20, 21)))
def test_w1_scaled_by_powers_of_two(k):
    g = goldens.load("w1_grid_roundtrip.txt")
    x = _bf16(_from_bf16(g["x"]) * np.float32(2.0 ** k)).reshape(g["x"].shape)
    for rule in ("static_6", "mse"):
        codes, scales, amax = oracle.quantize(x, 1, rule)
        assert scales[0, 0] == 0x7E
        assert np.array_equal(codes.reshape(-1), g["cases"][0]["codes"])
        assert np.array_equal(oracle.dequantize(codes, scales, amax, 1), x)


# ---- invariants on Gaussian data with outliers ----------------------------------------

def _gauss(rows, d, seed, outlier_p=0.01, outlier_mul=20.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, d)).astype(np.float32)
    z = np.where(rng.random((rows, d)) < outlier_p, z * outlier_mul, z)
    return _bf16(z).reshape(rows, d)


def _block_view(codes, scales, d):
    c = _unpack(codes).reshape(codes.shape[0], d // 16, 16)
    return c & 7, scales


def test_static_rules_put_block_amax_on_6_and_4():
    x = _gauss(512, 128, 1)
    for rule, top in (("static_6", 7), ("static_4", 6)):
        codes, scales, amax = oracle.quantize(x, 512, rule)
        mag, sf = _block_view(codes, scales, 128)
        xb = np.abs(_from_bf16(x)).reshape(512, 8, 16)
        m = xb.max(-1)
        s_enc = np.float32(2688.0) / amax[0]
        dv = np.float32(6.0 if rule == "static_6" else 4.0)
        u = (m / dv).astype(np.float32) * s_enc
        normal = (sf >= 0x08) & (u < 448.0) & (m > 0)
        assert normal.sum() > 3000
        assert np.all(mag.max(-1)[normal] == top), rule
        if rule == "static_4":
            assert not np.any(mag[normal] == 7)


def _margin(xb, cb, sf, s_dec):
    """Bound on |binary32 error sum - exact error sum| for one candidate: each r = fl(v*S)
    is off by at most |r| 2^-24, which moves d^2 by about 2|d||r| 2^-24; the difference and
    the fma chain of 8 terms add a few ulps of the sum."""
    S = (E4M3[sf].astype(np.float32) * s_dec).astype(np.float64)[..., None]
    r = GRID[cb] * S
    d = xb - r
    e = (d * d).sum(-1)
    return (2 * np.abs(d) * np.abs(r) * 2.0 ** -23).sum(-1) + e * 2.0 ** -19


def test_mse_is_one_of_the_static_candidates_and_not_worse():
    x = _gauss(256, 128, 2)
    A = oracle.group_amax(x)
    c6, s6, _ = oracle.quantize(x, 256, "static_6")
    c4, s4, _ = oracle.quantize(x, 256, "static_4")
    cm, sm, _ = oracle.quantize(x, 256, "mse")
    c6b, c4b, cmb = (_unpack(c).reshape(256, 8, 16) for c in (c6, c4, cm))
    is6 = np.all(cmb == c6b, -1) & (sm == s6)
    is4 = np.all(cmb == c4b, -1) & (sm == s4)
    assert np.all(is6 | is4)
    # independent double-precision errors of each candidate
    s_dec = np.float32(A) / np.float32(2688.0)
    xb = _from_bf16(x).astype(np.float64).reshape(256, 8, 16)

    def err(cb, sf):
        S = (E4M3[sf].astype(np.float32) * s_dec).astype(np.float64)
        return ((xb - GRID[cb] * S[..., None]) ** 2).sum(-1)

    e6, e4 = err(c6b, s6), err(c4b, s4)
    clear = np.abs(e4 - e6) > _margin(xb, c6b, s6, s_dec) + _margin(xb, c4b, s4, s_dec)
    chose4 = is4 & ~is6
    assert np.all(chose4[clear] == (e4 < e6)[clear])
    assert (chose4 & clear).sum() > 50 and (~chose4 & clear).sum() > 50


def test_mse_exhaustive_two_element_blocks():
    # blocks [a, b, 0 x 14] on a 64 x 64 grid, plus one row that fixes the group amax at 8
    vals = np.linspace(-7.9, 7.9, 64).astype(np.float32)
    a, b = np.meshgrid(vals, vals, indexing="ij")
    rows = np.zeros((64 * 64 + 1, 16), dtype=np.float32)
    rows[:-1, 0] = a.reshape(-1)
    rows[:-1, 1] = b.reshape(-1)
    rows[-1, 0] = 8.0
    x = _bf16(rows).reshape(rows.shape)
    A = oracle.group_amax(x)
    assert A == 8.0
    cm, sm, _ = oracle.quantize(x, x.shape[0], "mse")
    c6, s6, _ = oracle.quantize(x, x.shape[0], "static_6")
    c4, s4, _ = oracle.quantize(x, x.shape[0], "static_4")
    s_dec = np.float32(A) / np.float32(2688.0)
    xf = _from_bf16(x).astype(np.float64)

    def err(c, s):
        S = (E4M3[s[:, 0]].astype(np.float32) * s_dec).astype(np.float64)
        return ((xf - GRID[_unpack(c)] * S[:, None]) ** 2).sum(-1)

    e6, e4 = err(c6, s6), err(c4, s4)
    want4 = e4 < e6
    m6 = _margin(xf[:, None, :], _unpack(c6)[:, None, :], s6, s_dec)[:, 0]
    m4 = _margin(xf[:, None, :], _unpack(c4)[:, None, :], s4, s_dec)[:, 0]
    clear = np.abs(e4 - e6) > m6 + m4
    got4 = np.all(cm == c4, -1) & (sm[:, 0] == s4[:, 0]) & ~(np.all(cm == c6, -1) & (sm[:, 0] == s6[:, 0]))
    assert np.array_equal(got4[clear], want4[clear])
    # exact ties keep the 6-max candidate
    tie = (e4 == e6)
    assert np.all(np.all(cm[tie] == c6[tie], -1))


# ---- zero, underflow, groups ----------------------------------------------------------

@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_all_zero_group(rule):
    x = np.zeros((8, 64), dtype=np.uint16)
    x[1, 3] = 0x8000  # a negative zero
    codes, scales, amax = oracle.quantize(x, 8, rule)
    assert amax[0] == 0.0 and not np.any(scales)
    c = _unpack(codes)
    assert c[1, 3] == 8 and np.count_nonzero(c) == 1
    y = oracle.dequantize(codes, scales, amax, 8)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_underflowing_block_is_zero(rule):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1000.0            # block 0 sets A = 1000
    x[0, 16:] = 1e-4            # block 1: u = (1e-4/6) * 2.688 < 2^-10 -> sf 0
    x[0, 17] = -1e-4
    xb = _bf16(x).reshape(1, 32)
    codes, scales, amax = oracle.quantize(xb, 1, rule)
    assert scales[0, 1] == 0
    c = _unpack(codes)[0, 16:]
    assert c[1] == 8 and np.all(np.delete(c, 1) == 0)
    y = oracle.dequantize(codes, scales, amax, 1)[0, 16:]
    assert y[1] == 0x8000 and np.all(np.delete(y, 1) == 0)


@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_zero_times_infinity_is_zero(rule):
    """A group whose amax is 2^-129 (bf16 pattern 0x0010 = 16 * 2^-133): s_enc = 2688 * 2^129
    overflows to +inf, so a nonzero block gets u = inf -> scale byte 0x7E; S = 448 * A/2688
    (about 2^-129/6, a float32 subnormal) has 1/S > FLT_MAX, so inv = +inf: nonzero elements
    go to +-inf and saturate (code 7 | sign), zero elements stay +-0 (codes 0x0 / 0x8); the
    all-zero second block gets u = 0 -> scale byte 0x00.  Derived by hand from the reading
    that a product with a zero operand is zero (binary32 would give 0 * inf = NaN)."""
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, :5] = [0x0010, 0x0000, 0x8000, 0x0001, 0x8001]   # 2^-129, +0, -0, 2^-133, -2^-133
    codes, scales, amax = oracle.quantize(x, 1, rule)
    assert amax.view(np.uint32)[0] == 0x00100000
    assert scales.tolist() == [[0x7E, 0x00]]
    assert codes.tolist() == [[0x07, 0x78, 0x0F, 0, 0, 0, 0, 0] + [0] * 8]


def test_groups_are_independent_and_ragged_tail():
    x = _gauss(37, 64, 3)
    codes, scales, amax = oracle.quantize(x, 10, "mse")
    assert amax.shape == (4,)
    for g in range(4):
        r0, r1 = 10 * g, min(10 * g + 10, 37)
        assert amax[g] == np.abs(_from_bf16(x[r0:r1])).max()
        c, s, a = oracle.quantize(x[r0:r1], r1 - r0, "mse")
        assert np.array_equal(codes[r0:r1], c) and np.array_equal(scales[r0:r1], s)
        assert a[0] == amax[g]
    y = oracle.dequantize(codes, scales, amax, 10)
    for g in range(4):
        r0, r1 = 10 * g, min(10 * g + 10, 37)
        assert np.array_equal(y[r0:r1], oracle.dequantize_rows(codes[r0:r1], scales[r0:r1], amax[g]))


def test_quantize_rows_matches_whole_group():
    x = _gauss(64, 128, 4)
    codes, scales, amax = oracle.quantize(x, 64, "static_6")
    c, s = oracle.quantize_rows(x[17:40], amax[0], "static_6")
    assert np.array_equal(c, codes[17:40]) and np.array_equal(s, scales[17:40])


# ---- dequantization -------------------------------------------------------------------

def test_dequant_exhaustive_exact_when_global_scale_is_one():
    # A = 2688 makes s_dec = 1, so every output is E2M1(c) * E4M3(sf), exact in bf16.
    sf = np.arange(0x7F, dtype=np.uint8)
    c = np.arange(16, dtype=np.uint8)
    cc, ss = np.meshgrid(c, sf, indexing="ij")            # [16, 127]
    n = cc.size
    cc = cc.reshape(-1)
    ss = ss.reshape(-1)
    # one 16-element row per (code, sf): all 16 elements carry the same code
    codes = np.repeat((cc | (cc << 4)).astype(np.uint8)[:, None], 8, axis=1)
    scales = ss[:, None].astype(np.uint8)
    y = oracle.dequantize(codes, scales, np.float32([2688.0]), n)
    want = GRID[cc] * E4M3[ss]
    got = _from_bf16(y[:, 0]).astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("A", [1.0, 6.0, 20.0, 0.037])
def test_dequant_exhaustive_within_rounding_bound(A):
    sf = np.arange(0x7F, dtype=np.uint8)
    c = np.arange(16, dtype=np.uint8)
    cc, ss = (t.reshape(-1) for t in np.meshgrid(c, sf, indexing="ij"))
    codes = np.repeat((cc | (cc << 4)).astype(np.uint8)[:, None], 8, axis=1)
    y = oracle.dequantize(codes, ss[:, None].astype(np.uint8), np.float32([A]), cc.size)
    exact = GRID[cc] * E4M3[ss] * (A / 2688.0)
    got = _from_bf16(y[:, 0]).astype(np.float64)
    # three binary32 roundings (s_dec, S, v*S) then one bf16 rounding
    tol = np.abs(exact) * (2.0 ** -8 + 4 * 2.0 ** -24) + 1e-300
    assert np.all(np.abs(got - exact) <= tol)


@pytest.mark.parametrize("rule", ["static_6", "static_4", "mse"])
def test_round_trip_error_bound(rule):
    x = _gauss(256, 128, 5)
    codes, scales, amax = oracle.quantize(x, 256, rule)
    y = oracle.dequantize(codes, scales, amax, 256)
    xf = _from_bf16(x).astype(np.float64).reshape(256, 8, 16)
    yf = _from_bf16(y).astype(np.float64).reshape(256, 8, 16)
    s_dec = np.float32(amax[0]) / np.float32(2688.0)
    S = (E4M3[scales].astype(np.float32) * s_dec).astype(np.float64)[..., None]
    yv = np.abs(xf) / np.where(S > 0, S, 1)
    # half the E2M1 spacing around |y| (0.25 below 2, 0.5 below 4, 1 up to 6), or the
    # saturation excess above 6
    half_gap = np.where(yv < 2, 0.25, np.where(yv < 4, 0.5, 1.0))
    bound = S * np.maximum(half_gap, yv - 6.0) * (1 + 1e-5) + np.abs(yf) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(xf - yf) <= bound)


def test_storage_is_4p5_bits_per_element():
    rows, d = 1000, 128
    codes, scales, amax = oracle.quantize(np.zeros((rows, d), np.uint16), rows, "static_6")
    bits = 8 * (codes.nbytes + scales.nbytes) / (rows * d)
    assert bits == 4.5
