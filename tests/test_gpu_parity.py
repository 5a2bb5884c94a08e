"""GPU parity: the HIP quantize / dequantize path (through the C ABI) against the oracle,
element by element and bit for bit (codes, scale bytes, group amax, bf16 output).

Sizes: the tiny workload whole; ragged shapes that span several slices and groups with a
short last group; edge cases (zero, underflow, tiny and huge amax, worked examples);
guard bytes around every output; appends into a larger cache at row offsets; the one-layer
chunk append whole; and the full-size multi-layer caches in the launch configuration the
benchmark times, on sampled groups and rows the oracle recomputes from the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import goldens

pytestmark = pytest.mark.gpu

RULES = ["static_6", "static_4", "mse"]
DEV = torch.device("cuda:0")


def kvmod():
    import kv_cache_fp4_amd as kv
    return kv


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_roundtrip(x_cpu_bf16, rpg, rule, guard=64):
    """Quantize + dequantize on the GPU into guarded buffers; check the guards."""
    kv = kvmod()
    x2 = x_cpu_bf16.reshape(-1, x_cpu_bf16.shape[-1])
    rows, d = x2.shape
    ng = -(-rows // rpg) if rows else 0
    xd = x2.to(DEV)
    G = guard

    def guarded(n, dtype, fill):
        b = torch.full((n + 2 * G,), fill, dtype=dtype, device=DEV)
        return b, b[G:G + n]

    cb, codes = guarded(rows * d // 2, torch.uint8, 0xA5)
    sb, scales = guarded(rows * d // 16, torch.uint8, 0x5A)
    ab, amax = guarded(ng, torch.float32, -7.0)
    yb, y = guarded(rows * d, torch.int16, 0x3C3C)
    kv.kvfp4_quantize(xd, rpg, rule, codes, scales, amax)
    kv.kvfp4_dequantize(codes.view(rows, d // 2), scales.view(rows, d // 16), amax, rpg,
                        y=y.view(torch.bfloat16).view(rows, d))
    torch.cuda.synchronize()
    for b, fill in ((cb, 0xA5), (sb, 0x5A), (ab, -7.0), (yb, 0x3C3C)):
        head, tail = b[:G].cpu(), b[-G:].cpu()
        assert torch.all(head == fill) and torch.all(tail == fill), "output guard overwritten"
    return (codes.cpu().numpy().reshape(rows, d // 2), scales.cpu().numpy().reshape(rows, d // 16),
            amax.cpu().numpy(), y.cpu().numpy().view(np.uint16).reshape(rows, d))


def assert_parity(x_cpu_bf16, rpg, rule):
    xh = _u16(x_cpu_bf16).reshape(-1, x_cpu_bf16.shape[-1])
    g = gpu_roundtrip(x_cpu_bf16, rpg, rule)
    o = oracle.quantize(xh, rpg, rule)
    oy = oracle.dequantize(*o, rpg)
    for name, a, b in zip(("codes", "scales", "amax"), g[:3], o):
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)[:5]
            raise AssertionError(f"{name} differ ({rule}) at {idx.tolist()}")
    if not np.array_equal(g[3], oy):
        idx = np.argwhere(g[3] != oy)[:5]
        raise AssertionError(f"dequant differs ({rule}) at {idx.tolist()}")


# ---- worked examples through the GPU ---------------------------------------------------

@pytest.mark.parametrize("name", ["w2_four_over_six.txt", "w3_outlier.txt", "w4_exact_tie.txt",
                                  "w5_midpoint_ties.txt"])
def test_worked_examples_on_gpu(name):
    gl = goldens.load(name)
    # the library needs head_dim >= 64: pad each example row with zero blocks (a zero
    # block does not change the group amax or the other blocks' bytes)
    d = gl["d"]
    x = np.zeros((gl["x"].shape[0], 64), np.uint16)
    x[:, :d] = gl["x"]
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    for case in gl["cases"]:
        codes, scales, amax, y = gpu_roundtrip(xt, gl["rows_per_group"], case["rule"])
        assert amax[0] == np.float32(gl["amax"])
        assert np.array_equal(scales[:, : d // 16].reshape(-1), case["scales"])
        assert np.array_equal(codes[:, : d // 2].reshape(-1), case["codes"])
        assert np.array_equal(y[:, :d].reshape(-1), case["dequant"])
        assert not codes[:, d // 2:].any() and not scales[:, d // 16:].any()


def test_w1_grid_on_gpu_all_scales():
    gl = goldens.load("w1_grid_roundtrip.txt")
    base = (gl["x"].astype(np.uint32) << 16).view(np.float32).reshape(-1)
    rows = []
    for k in range(-20, 21):
        row = np.zeros(64, np.float32)
        row[:16] = base * np.float32(2.0 ** k)
        rows.append(row)
    xt = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    for rule in RULES:
        codes, scales, amax, y = gpu_roundtrip(xt, 1, rule)
        assert np.all(scales[:, 0] == 0x7E)
        assert np.all(codes[:, :8] == gl["cases"][0]["codes"][None, :])
        assert np.array_equal(y, _u16(xt))


# ---- the tiny workload and ragged shapes ---------------------------------------------------

@pytest.mark.parametrize("rule", RULES)
def test_tiny_workload(rule):
    cfg = synth.C1
    x = torch.cat([synth.chunk_group(cfg, 0, kv_, 0).reshape(-1, cfg.head_dim) for kv_ in (0, 1)])
    assert_parity(x, cfg.rows_per_group, rule)


SHAPES = [  # rows, head_dim, rows_per_group
    (1, 64, 1), (1, 128, 5), (3, 256, 2), (37, 64, 10), (1000, 256, 333), (3001, 128, 3001),
    (50, 1024, 7), (40000, 128, 20000), (12345, 64, 4096), (777, 192, 100), (2, 128, 1),
]


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("rows,d,rpg", SHAPES)
def test_ragged_shapes(rows, d, rpg, rule):
    x = synth.gauss_outliers((rows, d), seed=rows * 7 + d + rpg)
    assert_parity(x, rpg, rule)


@pytest.mark.parametrize("rule", RULES)
def test_student_t_and_channel_outliers(rule):
    x1 = synth.student_t_mix((4096, 128), seed=41, p=0.01)
    assert_parity(x1, 1024, rule)
    f = synth.channel_factors(8, 128, 42)
    x2 = synth.channel_lognormal(512, 8, 128, 43, f)
    assert_parity(x2.reshape(-1, 128), 1024, rule)


# ---- edge cases ------------------------------------------------------------------------------

@pytest.mark.parametrize("rule", RULES)
def test_zero_and_signed_zero_group(rule):
    x = torch.zeros((256, 128), dtype=torch.float32)
    x[3, 5] = -0.0
    x[100:] = torch.randn((156, 128), generator=torch.Generator().manual_seed(5))
    xb = x.to(torch.bfloat16)
    assert_parity(xb, 100, rule)  # group 0 (rows 0..99) is all zero (one -0)


@pytest.mark.parametrize("rule", RULES)
def test_underflowing_blocks_and_huge_amax(rule):
    g = torch.Generator().manual_seed(6)
    x = torch.randn((512, 128), generator=g) * 1e-3
    x[0, 0] = 3.0e4               # group amax dominates: most blocks underflow to sf 0
    x[300, 7] = -2.5e38           # near the bf16 maximum
    assert_parity(x.to(torch.bfloat16), 256, rule)


@pytest.mark.parametrize("rule", RULES)
def test_tiny_amax(rule):
    g = torch.Generator().manual_seed(7)
    x = torch.randn((256, 64), generator=g) * 1e-18   # amax ~ 4e-18 > 2^-64
    assert_parity(x.to(torch.bfloat16), 256, rule)


@pytest.mark.parametrize("rule", RULES)
def test_tiny_blocks_and_bf16_subnormals(rule):
    # block maxima below 2^-123 (and bf16 subnormals) in a group whose amax is 1e-19
    g = torch.Generator().manual_seed(11)
    x = torch.randn((128, 64), generator=g) * 1e-38
    x[:, 32:] = torch.randn((128, 32), generator=g) * 1e-39
    x[0, 0] = 1e-19
    x[5, 40] = -2.0e-20
    assert_parity(x.to(torch.bfloat16), 128, rule)


@pytest.mark.parametrize("rule", RULES)
def test_exact_grid_multiples(rule):
    # values that land exactly on E2M1 midpoints after scaling stress the tie rules
    g = torch.Generator().manual_seed(8)
    grid = torch.tensor([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0])
    idx = torch.randint(0, grid.numel(), (1024, 128), generator=g)
    sign = torch.where(torch.rand((1024, 128), generator=g) < 0.5, -1.0, 1.0)
    x = grid[idx] * sign
    x[:, ::16] = 6.0   # every block's amax is 6 -> S = 1 for static_6
    assert_parity(x.to(torch.bfloat16), 1024, rule)


def test_append_into_cache_at_row_offset():
    """Quantize a chunk straight into rows [r0, r1) of a bigger cache; rows outside stay."""
    kv = kvmod()
    d, rpg = 128, 600
    cache_rows, r0 = 3000, 1200
    x = synth.gauss_outliers((rpg, d), seed=9)
    codes = torch.full((cache_rows, d // 2), 0x11, dtype=torch.uint8, device=DEV)
    scales = torch.full((cache_rows, d // 16), 0x22, dtype=torch.uint8, device=DEV)
    amax = torch.full((5,), -1.0, dtype=torch.float32, device=DEV)
    kv.kvfp4_quantize(x.to(DEV), rpg, "mse", codes[r0:r0 + rpg], scales[r0:r0 + rpg], amax[2:3])
    torch.cuda.synchronize()
    oc, os_, oa = oracle.quantize(_u16(x), rpg, "mse")
    c, s, a = codes.cpu().numpy(), scales.cpu().numpy(), amax.cpu().numpy()
    assert np.array_equal(c[r0:r0 + rpg], oc) and np.array_equal(s[r0:r0 + rpg], os_)
    assert a[2] == oa[0] and np.all(np.delete(a, 2) == -1.0)
    assert np.all(np.delete(c, np.s_[r0:r0 + rpg], 0) == 0x11)
    assert np.all(np.delete(s, np.s_[r0:r0 + rpg], 0) == 0x22)


def test_repeat_calls_are_deterministic():
    kv = kvmod()
    x = synth.gauss_outliers((20000, 128), seed=10).to(DEV)
    outs = []
    for _ in range(3):
        c, s, a = kv.kvfp4_quantize(x, 5000, "mse")
        y = kv.kvfp4_dequantize(c, s, a, 5000)
        torch.cuda.synchronize()
        outs.append((c.cpu(), s.cpu(), a.cpu(), y.view(torch.int16).cpu()))
    for o in outs[1:]:
        assert all(torch.equal(p, q) for p, q in zip(o, outs[0]))


def test_bad_arguments_raise_before_launch():
    kv = kvmod()
    x = torch.zeros((10, 80), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):  # the binding refuses head_dim 80 before any C call
        kv.kvfp4_quantize(x, 10, "static_6")
    x = torch.zeros((10, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        kv.kvfp4_quantize(x, 0, "static_6")


# ---- the one-layer chunk append, whole -----------------------------------------------------

@pytest.mark.parametrize("rule", RULES)
def test_chunk_append_whole(rule):
    cfg = synth.C2
    x = torch.cat([synth.chunk_group(cfg, 0, kv_, 0).reshape(-1, cfg.head_dim) for kv_ in (0, 1)])
    assert_parity(x, cfg.rows_per_group, rule)
