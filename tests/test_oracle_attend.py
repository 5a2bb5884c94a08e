"""Pins for the oracle's attention over a dequantized cache (no GPU).

Checked against the textbook definition evaluated by torch in float64 (an independent
library routine), and against special cases with closed forms: one key gives O = V,
identical keys give O = mean(V), a dominant key selects its value row.
"""
import numpy as np
import torch

import oracle


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _all_rows(tq, heads):
    return np.arange(tq * heads, dtype=np.int64)


def test_attend_vs_torch_float64():
    rng = np.random.default_rng(21)
    tq, tk, H, d = 7, 53, 3, 64
    q = _bf16(rng.standard_normal((tq, H, d)) * 0.5).reshape(tq, H, d)
    k = _bf16(rng.standard_normal((tk, H, d))).reshape(tk, H, d)
    v = _bf16(rng.standard_normal((tk, H, d))).reshape(tk, H, d)
    scale = 1.0 / np.sqrt(d)
    got = _f(oracle.attend_rows(q, k, v, scale, _all_rows(tq, H))).reshape(tq, H, d)
    Q, K, V = (torch.from_numpy(_f(t).astype(np.float64)).permute(1, 0, 2) for t in (q, k, v))
    P = torch.softmax((Q @ K.transpose(1, 2)) * scale, dim=-1)
    ref = (P @ V).permute(1, 0, 2).numpy()
    # one bf16 rounding (plus a binary32 rounding) separates the two
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-12)


def test_single_key_returns_value_row():
    rng = np.random.default_rng(22)
    q = _bf16(rng.standard_normal((5, 2, 128))).reshape(5, 2, 128)
    k = _bf16(rng.standard_normal((1, 2, 128))).reshape(1, 2, 128)
    v = _bf16(rng.standard_normal((1, 2, 128))).reshape(1, 2, 128)
    got = oracle.attend_rows(q, k, v, 0.1, _all_rows(5, 2)).reshape(5, 2, 128)
    for t in range(5):
        assert np.array_equal(got[t], v[0])


def test_identical_keys_average_values():
    rng = np.random.default_rng(23)
    tk = 40
    q = _bf16(rng.standard_normal((3, 1, 64))).reshape(3, 1, 64)
    k = np.repeat(_bf16(rng.standard_normal((1, 1, 64))).reshape(1, 1, 64), tk, axis=0)
    v = _bf16(rng.standard_normal((tk, 1, 64))).reshape(tk, 1, 64)
    got = _f(oracle.attend_rows(q, k, v, 1.0, _all_rows(3, 1))).reshape(3, 64)
    mean = _f(v).astype(np.float64).mean(0)[0]
    for t in range(3):
        assert np.all(np.abs(got[t] - mean) <= np.abs(mean) * 2.0 ** -8 + 1e-12)


def test_dominant_key_selects_its_value():
    tk, d = 16, 64
    k = np.zeros((tk, 1, d), np.float32)
    k[5, 0, 0] = 1.0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    v = np.random.default_rng(24).standard_normal((tk, 1, d)).astype(np.float32)
    qb, kb, vb = _bf16(q).reshape(q.shape), _bf16(k).reshape(k.shape), _bf16(v).reshape(v.shape)
    got = oracle.attend_rows(qb, kb, vb, 200.0, np.array([0], np.int64)).reshape(d)
    assert np.array_equal(got, vb[5, 0])  # exp(-200) is far below half a bf16 ulp


def test_row_subset_equals_full():
    rng = np.random.default_rng(25)
    tq, tk, H, d = 6, 20, 4, 64
    q = _bf16(rng.standard_normal((tq, H, d))).reshape(tq, H, d)
    k = _bf16(rng.standard_normal((tk, H, d))).reshape(tk, H, d)
    v = _bf16(rng.standard_normal((tk, H, d))).reshape(tk, H, d)
    full = oracle.attend_rows(q, k, v, 0.125, _all_rows(tq, H))
    sub = np.array([3, 17, 22], np.int64)
    assert np.array_equal(oracle.attend_rows(q, k, v, 0.125, sub), full[sub])


# ---- the output's single rounding (double -> bf16) -------------------------------------------

def _nearest_bf16_exact(v):
    """Nearest bf16 pattern to the double v by exact rational comparison against every
    non-negative finite bf16 value (ties to the even pattern; beyond the largest finite value
    the IEEE overflow rule: 2^128 stands for infinity)."""
    from fractions import Fraction
    pats = np.arange(0, 0x7F81, dtype=np.uint32)            # +0 .. 0x7F7F, then 0x7F80 = inf
    vals = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vals[-1] = 2.0 ** 128
    a = abs(v)
    i = int(np.searchsorted(vals, a))
    if i < len(vals) and vals[i] == a:
        p = i
    else:
        lo, hi = i - 1, i
        dlo, dhi = Fraction(a) - Fraction(vals[lo]), Fraction(vals[hi]) - Fraction(a)
        p = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
    return np.uint16(p | (0x8000 if np.signbit(v) else 0))


def test_double_to_bf16_vs_exact_nearest():
    rng = np.random.default_rng(24)
    v = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 127, 3000)),
        # doubles within a few ulps of bf16 midpoints, on both sides
        ((rng.integers(0x0001, 0x7F7F, 2000).astype(np.uint32) << 16 | 0x8000)
         .view(np.float32).astype(np.float64) * (1.0 + rng.integers(-3, 4, 2000) * 2.0 ** -52)),
        [0.0, -0.0, 2.0 ** -134, 2.0 ** -133, 1.5 * 2.0 ** -133, 3.3895313892515355e38,
         3.3961e38, 3.4e38, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40],
    ])
    got = oracle.double_to_bf16(v)
    want = np.array([_nearest_bf16_exact(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_double_to_bf16_agrees_with_float_rounding_on_floats():
    """On doubles that are binary32 values the one-step rounding is the binary32 -> bf16
    rounding, which is pinned against torch."""
    rng = np.random.default_rng(25)
    bits = rng.integers(0, 0x7F7FFFFF, 200_000, dtype=np.uint32)
    f = bits.view(np.float32)
    assert np.array_equal(oracle.double_to_bf16(f.astype(np.float64)), oracle.float_to_bf16(f))


def test_attend_rounds_the_double_result_once():
    """Three keys with equal scores average their values: (3 + 3*2^-8 + 2^-23) / 3 =
    1 + 2^-8 + 2^-23/3 lies just above the bf16 midpoint 1 + 2^-8, so it rounds up to
    0x3F81.  Rounding through binary32 first would land exactly on the midpoint
    (2^-23/3 < half a binary32 ulp) and then tie to the even 0x3F80."""
    tk, d = 3, 64
    q = _bf16(np.ones((1, 1, d))).reshape(1, 1, d)
    k = _bf16(np.full((tk, 1, d), 0.25)).reshape(tk, 1, d)       # identical keys
    vcol = np.array([3.0, 3 * 2.0 ** -8, 2.0 ** -23])          # each exactly a bf16 value
    v = _bf16(np.repeat(vcol[:, None], d, axis=1)).reshape(tk, 1, d)
    assert np.array_equal(_f(v)[:, 0, 0].astype(np.float64), vcol)
    got = oracle.attend_rows(q, k, v, 1.0 / np.sqrt(d), _all_rows(1, 1)).reshape(d)
    assert np.all(got == 0x3F81)
    mean = vcol.sum() / 3
    assert oracle.float_to_bf16(np.float32(mean))[0] == 0x3F80   # the double-rounding path
