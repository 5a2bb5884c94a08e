"""GPU sweeps of the device conversion helpers (E2M1, E4M3, bf16) against the oracle at
binary32 inputs the quantize path reaches only rarely: every midpoint and grid point with
+-64 neighbouring ulps, the saturation region, signed zeros and large random samples.

The helpers are applied by the test-only probe library (tests/gpu_probe), which includes
the library's own device header, so these are the exact instructions the kernels use."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_probe", "libconv_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        pytest.fail("conversion probe not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE)
    P, i64 = ctypes.c_void_p, ctypes.c_int64
    for n in ("probe_e2m1_encode", "probe_e2m1_decode", "probe_e4m3_encode", "probe_e4m3_decode",
              "probe_bf16_pack"):
        getattr(L, n).argtypes = [P, i64, P, P]
        getattr(L, n).restype = ctypes.c_int
    return L


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _bits(f):
    return np.asarray(f, dtype=np.float32).view(np.uint32)


def _near(points, k=64):
    b = _bits(np.asarray(points, np.float32)).astype(np.int64)
    out = (b[:, None] + np.arange(-k, k + 1)[None, :]).reshape(-1)
    return _f32(out[(out >= 0) & (out < 0x7F800000)].astype(np.uint32))


def _run(fn, inp: np.ndarray, n_arg: int, out_dtype, out_count: int):
    dev = torch.device("cuda:0")
    x = torch.from_numpy(np.ascontiguousarray(inp)).to(dev)
    out = torch.zeros(out_count, dtype=out_dtype, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    assert fn(x.data_ptr(), n_arg, out.data_ptr(), s) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_e2m1_encode_hardware_matches_oracle(probe):
    rng = np.random.default_rng(31)
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 7.0, 1e-30]
    y = np.concatenate([_near(pts), _f32(rng.integers(0, 0x41000000, 4_000_000, dtype=np.uint32))])
    y = np.concatenate([y, -y, np.float32([0.0, -0.0, 6.5, -6.5, 100.0, -1e30, 3e38, -3e38])])
    y = np.concatenate([y, np.zeros((-y.size) % 8, np.float32)]).astype(np.float32)
    words = _run(probe.probe_e2m1_encode, y, y.size // 8, torch.int32, y.size // 8).view(np.uint32)
    nib = np.stack([(words >> (4 * j)) & 15 for j in range(8)], axis=1).reshape(-1).astype(np.uint8)
    want = oracle.e2m1_encode(y)
    bad = np.nonzero(nib != want)[0]
    assert bad.size == 0, [(float(y[i]), int(nib[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_decode_hardware_matches_oracle(probe):
    words = np.array([0x76543210, 0xFEDCBA98, 0x8F80F808], dtype=np.uint32)
    got = _run(probe.probe_e2m1_decode, words.view(np.int32), words.size, torch.float32, 8 * words.size)
    codes = np.stack([(words >> (4 * j)) & 15 for j in range(8)], axis=1).reshape(-1)
    want = np.array([oracle.e2m1_value(int(c)) for c in codes], np.float32)
    assert np.array_equal(_bits(got), _bits(want))  # bit-equal, so -0.0 must stay -0.0


def test_e4m3_encode_matches_oracle(probe):
    rng = np.random.default_rng(32)
    vals = np.array([oracle.e4m3_value(i) for i in range(0x7F)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    u = np.concatenate([_near(mids, 16), _near(vals.astype(np.float32), 16),
                        _f32(rng.integers(0, 0x44000000, 2_000_000, dtype=np.uint32)),
                        np.float32([0.0, 448.0, 460.0, 464.0, 1e6, 3e38, 1e-40, 1e-45])])
    u = u[np.isfinite(u) & (u >= 0)].astype(np.float32)
    got = _run(probe.probe_e4m3_encode, u, u.size, torch.uint8, u.size)
    want = oracle.e4m3_encode(u)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(u[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_decode_matches_oracle(probe):
    b = np.arange(0x7F, dtype=np.uint8)
    got = _run(probe.probe_e4m3_decode, b, b.size, torch.float32, b.size)
    want = np.array([oracle.e4m3_value(int(i)) for i in b], np.float32)
    assert np.array_equal(_bits(got), _bits(want))


def test_bf16_pack_matches_oracle(probe):
    rng = np.random.default_rng(33)
    f = _f32(rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32))
    f = f[np.isfinite(f)]
    ties = _f32((rng.integers(0, 0x7F00, 100_000, dtype=np.uint32) << 16) | 0x8000)
    f = np.concatenate([f, ties, -ties, np.float32([0.0, -0.0, 1e-40, -1e-45, 3.3e38])])
    f = np.concatenate([f, np.zeros(f.size % 2, np.float32)]).astype(np.float32)
    got = _run(probe.probe_bf16_pack, f, f.size // 2, torch.int32, f.size // 2).view(np.uint32)
    halves = np.stack([got & 0xFFFF, got >> 16], axis=1).reshape(-1).astype(np.uint16)
    want = oracle.float_to_bf16(f)
    bad = np.nonzero(halves != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(halves[i]), hex(want[i])) for i in bad[:10]]


def test_mfma_32x32x16_bf16_lane_layout(probe):
    """The operand and accumulator lane layout the attention kernel is written against."""
    probe.probe_mfma_32x32x16_bf16.argtypes = [ctypes.c_void_p] * 4
    probe.probe_mfma_32x32x16_bf16.restype = ctypes.c_int
    rng = np.random.default_rng(34)
    # small integers are exact in bf16 and their products/sums exact in fp32
    a = rng.integers(-4, 5, (32, 16)).astype(np.float32)
    b = rng.integers(-4, 5, (16, 32)).astype(np.float32)
    dev = torch.device("cuda:0")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    td = torch.zeros((32, 32), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    assert probe.probe_mfma_32x32x16_bf16(ta.data_ptr(), tb.data_ptr(), td.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert np.array_equal(td.cpu().numpy(), a @ b)
