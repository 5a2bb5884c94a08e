"""Pins for the oracle's format conversions (E2M1, E4M3, bf16).

Each conversion is checked against something other than the oracle itself: the grid and
landmark fixtures (format definitions cited in tests/golden/), the round-to-nearest-even
threshold table that follows from the grid, and torch's own float8_e4m3fn / bfloat16
conversions (independent library routines).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.goldens import GOLDEN_DIR


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN_DIR, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line or line.startswith(("code", "byte")):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _bits(f):
    return np.asarray(f, dtype=np.float32).view(np.uint32)


# ---- E2M1 ------------------------------------------------------------------------------

def test_e2m1_grid_values_and_signed_zero():
    for code, val in _table("e2m1_grid.txt"):
        got = oracle.e2m1_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_grid_round_trips():
    vals = np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float32)
    assert np.array_equal(oracle.e2m1_encode(vals), np.arange(16, dtype=np.uint8))


def _threshold_codes(y):
    """Round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6}: a tie goes to the even code, so the
    midpoints 0.25, 1.25, 2.5, 5 round down and 0.75, 1.75, 3.5 round up; saturate at 6."""
    a = np.abs(y.astype(np.float64))
    c = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
         + (a >= 3.5) + (a > 5.0))
    return (c | (np.signbit(y).astype(np.uint8) << 3)).astype(np.uint8)


def test_e2m1_encode_vs_threshold_table():
    rng = np.random.default_rng(11)
    # a strided sweep over every binary32 pattern in [0, 8]
    top = int(_bits(np.float32(8.0)))
    sweep = np.arange(0, top + 1, 61, dtype=np.uint32)
    # +-64 ulps around each midpoint and grid point, and the saturation region
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 7.0]
    near = np.concatenate([int(_bits(np.float32(p))) + np.arange(-64, 65) for p in pts]).astype(np.uint32)
    rand = rng.integers(0, top, 2_000_000, dtype=np.uint32)
    y = _f32(np.concatenate([sweep, near, rand]))
    y = np.concatenate([y, -y, np.float32([1e30, -1e30, 6.5, -100.0])])
    assert np.array_equal(oracle.e2m1_encode(y), _threshold_codes(y))


def test_e2m1_negative_tiny_is_code8():
    y = np.float32([-0.0, -1e-30, -0.25, -0.1])
    assert list(oracle.e2m1_encode(y)) == [8, 8, 8, 8]


# ---- E4M3 ------------------------------------------------------------------------------

def test_e4m3_landmarks():
    for byte, val in _table("e4m3_landmarks.txt"):
        assert oracle.e4m3_value(byte) == val, hex(byte)


def test_e4m3_decode_vs_torch_float8():
    b = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(i) for i in range(0x7F)])
    assert np.array_equal(got, ref)
    assert np.all(np.diff(got) > 0)  # strictly increasing: 127 distinct finite values


def _torch_e4m3(u):
    return torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_vs_torch_float8():
    rng = np.random.default_rng(12)
    vals = np.array([oracle.e4m3_value(i) for i in range(0x7F)], dtype=np.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)  # exact in binary32
    ulps = np.arange(-16, 17)
    near = np.concatenate([int(b) + ulps for b in _bits(np.concatenate([mids, vals.astype(np.float32)]))])
    near = near[(near >= 0)].astype(np.uint32)
    top = int(_bits(np.float32(448.0)))
    rand = rng.integers(0, top, 1_000_000, dtype=np.uint32)
    u = _f32(np.concatenate([near, rand]))
    u = u[u < 448.0]
    assert np.array_equal(oracle.e4m3_encode(u), _torch_e4m3(u))


def test_e4m3_encode_every_binary32_in_range():
    """Brute force: every binary32 value in [2^-12, 2^10] (about 1.8e8 values, the whole range
    a block scale's encode operand u takes in ordinary groups and then some).  Below 448 the
    oracle's table scan equals torch's float8_e4m3fn conversion (an independent
    implementation of round-to-nearest-even into OCP E4M3); from 448 up it saturates to
    0x7E, the reading of the pages' FP8 block scale taken here (torch has no saturating
    mode).  Chunks run on the host's threads (the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    lo = int(_bits(np.float32(2.0 ** -12)))
    hi = int(_bits(np.float32(2.0 ** 10)))
    sat = int(_bits(np.float32(448.0)))
    step = 1 << 22

    def chunk(b0):
        b = np.arange(b0, min(b0 + step, hi + 1), dtype=np.uint32)
        u = _f32(b)
        got = oracle.e4m3_encode(u)
        below = b < sat
        ok = np.array_equal(got[below], _torch_e4m3(u[below]))
        return ok and bool(np.all(got[~below] == 0x7E)), int(b.size)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(chunk, range(lo, hi + 1, step)))
    assert all(ok for ok, _ in res)
    assert sum(n for _, n in res) == hi - lo + 1 == 22 * (1 << 23) + 1


def test_e4m3_saturates_at_448():
    u = np.float32([448.0, 448.5, 463.9, 464.0, 1000.0, 3.0e38, np.inf])
    assert np.all(oracle.e4m3_encode(u) == 0x7E)


def test_e4m3_underflow():
    # below half the smallest subnormal (2^-10) everything rounds to 0; the tie goes to 0
    u = np.float32([0.0, 1e-30, 2.0 ** -11, 2.0 ** -10])
    assert np.all(oracle.e4m3_encode(u) == 0)
    assert oracle.e4m3_encode(np.float32([2.0 ** -10 * 1.0000001]))[0] == 1


# ---- bf16 ------------------------------------------------------------------------------

def test_bf16_vs_torch():
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 32, 3_000_000, dtype=np.uint64).astype(np.uint32)
    f = _f32(bits)
    f = f[np.isfinite(f)]
    # exact ties: low half 0x8000 with even and odd upper halves
    ties = _f32((rng.integers(0, 0x7F00, 20000, dtype=np.uint32) << 16) | 0x8000)
    f = np.concatenate([f, ties, -ties, np.float32([0.0, -0.0, 3.3895e38, 1e-40, -1e-45])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.float_to_bf16(f), ref)


def test_bf16_widening_is_exact():
    h = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    h = h[((h & 0x7F80) != 0x7F80)]  # finite patterns
    f = oracle.bf16_to_float(h)
    assert np.array_equal(oracle.float_to_bf16(f), h)
