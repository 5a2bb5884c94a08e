"""Pins for the oracle's round-to-nearest symmetric blockwise INT4/INT2 (no GPU): a worked
example derived by hand (tests/golden/w6_rtn.txt), the realized compression printed by the
Self-Forcing study (tests/golden/rtn_compression.txt), exact round trips of integer
multiples, sign symmetry, the clamp, and the half-step error bound."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.goldens import GOLDEN_DIR


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _load_w6(name="w6_rtn.txt"):
    head, cases, cur = {}, [], None
    for line in open(os.path.join(GOLDEN_DIR, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = (t.strip() for t in line.split(":", 1))
        if k == "bits":
            cur = {"bits": int(v)}
            cases.append(cur)
        elif cur is None:
            head[k] = v
        else:
            cur[k] = v
    x = np.array([int(t, 16) for t in head["x_bf16"].split()], np.uint16).reshape(1, -1)
    return x, cases


@pytest.mark.parametrize("name", ["w6_rtn.txt", "w7_rtn_bf16_scale.txt"])
def test_worked_example(name):
    x, cases = _load_w6(name)
    for c in cases:
        codes, scales = oracle.rtn_quantize(x, c["bits"])
        assert codes.reshape(-1).tolist() == [int(t, 16) for t in c["codes"].split()], c["bits"]
        assert scales.reshape(-1).tolist() == [int(t, 16) for t in c["scales"].split()]
        y = oracle.rtn_dequantize(codes, scales, c["bits"])
        assert y.reshape(-1).tolist() == [int(t, 16) for t in c["dequant_bf16"].split()]


def test_zero_times_infinity_is_zero():
    """INT4 block with max 7 * 2^-130 (bf16 pattern 0x0038): s = bf16(m/7) = 2^-130 (pattern
    0x0008) and 1/s = 2^130 > FLT_MAX, so inv = +inf: nonzero elements go to +-inf and clamp
    to +-7, zero elements (either sign) give q = 0.  Derived by hand from the reading that a
    product with a zero operand is zero (binary32 would give rint(0 * inf) = NaN)."""
    x = np.zeros((1, 16), dtype=np.uint16)
    x[0, :5] = [0x0038, 0x0000, 0x8000, 0x0001, 0x8001]  # 7*2^-130, +-0, +-2^-133
    codes, scales = oracle.rtn_quantize(x, 4)
    assert scales.tolist() == [[0x0008]]
    # q = 7, 0, 0, 7, -7 (0x9), then zeros; element 2j in the low nibble
    assert codes.tolist() == [[0x07, 0x70, 0x09, 0, 0, 0, 0, 0]]


def test_int2_compression_matches_the_study():
    vals = {}
    for line in open(os.path.join(GOLDEN_DIR, "rtn_compression.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (t.strip() for t in line.split(":", 1))
            vals[k] = v
    x = _bf16(np.random.default_rng(1).standard_normal((100, 128))).reshape(100, 128)
    codes, scales = oracle.rtn_quantize(x, 2)
    bits = 8 * (codes.nbytes + scales.nbytes) / x.size
    assert round(16 / bits, 2) == float(vals["comp_moviegen"]) == float(vals["comp_storyeval"])


@pytest.mark.parametrize("bits", [2, 4])
def test_integer_multiples_round_trip(bits):
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits)
    q = rng.integers(-qmax, qmax + 1, (64, 64))
    q[:, ::16] = qmax                       # every block reaches qmax, so s = m / qmax
    s = 2.0 ** rng.integers(-6, 7, (64, 4))  # powers of two: m / qmax and q * s are exact
    x = (q.reshape(64, 4, 16) * s[..., None]).reshape(64, 64).astype(np.float32)
    xb = _bf16(x).reshape(64, 64)
    codes, scales = oracle.rtn_quantize(xb, bits)
    assert np.array_equal(oracle.rtn_dequantize(codes, scales, bits), _bf16(x).reshape(64, 64) | 0)


@pytest.mark.parametrize("bits", [2, 4])
def test_sign_symmetry_and_error_bound(bits):
    qmax = (1 << (bits - 1)) - 1
    x = _bf16(np.random.default_rng(5).standard_normal((200, 128)) * 3).reshape(200, 128)
    codes, scales = oracle.rtn_quantize(x, bits)
    y = _f(oracle.rtn_dequantize(codes, scales, bits)).astype(np.float64)
    yn = _f(oracle.rtn_dequantize(*oracle.rtn_quantize(x ^ 0x8000, bits), bits)).astype(np.float64)
    assert np.array_equal(yn, -y + 0.0)
    xf = _f(x).astype(np.float64).reshape(200, 8, 16)
    sv = _f(scales).astype(np.float64)[..., None]
    m = np.abs(xf).max(-1, keepdims=True)
    err = np.abs(xf - y.reshape(200, 8, 16))
    # half a step, plus the clamp excess when s was rounded down, plus the bf16 rounding
    bound = sv * 0.5 * (1 + 2.0 ** -20) + np.maximum(m - qmax * sv, 0) + np.abs(y.reshape(200, 8, 16)) * 2.0 ** -8
    assert np.all(err <= bound + 1e-30)
    q = np.rint(y.reshape(200, 8, 16) / np.where(sv > 0, sv, 1))
    assert np.all(np.abs(q) <= qmax)
