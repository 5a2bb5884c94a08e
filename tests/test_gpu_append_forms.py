"""The two forms of a quantize call -- the one-kernel append (group amax and encode in one
launch, with a hand-off through three words of each group's output) and the three-kernel
form (clear, group amax, encode) -- each bit-exact against the oracle: codes, scale bytes,
group amax, and for fake quantization the bf16 output.

Cases: shapes on both sides of the one-kernel form's applicability bound (every group,
the last included, at least 66 units of 8 elements), ragged last groups, many small groups,
one large group, every head_dim class; guard bytes around each output; the one-kernel form
with a zero wait bound (every encode workgroup that finds its group amax unpublished
computes it itself: the failure path of the bounded wait, forced from the host); the
default form, which picks between the two by input size; fake quantization in place
(always three kernels) and not in place.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RULES = ["static_6", "static_4", "mse"]

# (rows, head_dim, rows_per_group): units per group = rpg * head_dim / 8
SHAPES = [
    (66 * 8 // 64 + 1, 64, 9),        # one group of 72 units (>= 66: one kernel)
    (8 * 3 + 1, 64, 8),               # groups of 64 units and a 8-unit tail (three kernels)
    (33 * 9, 64, 9),                  # 33 groups of 72 units
    (4000, 128, 37),                  # many groups, ragged last (4000 = 108*37 + 4: 64-unit tail)
    (4000 + 29, 128, 37),             # ragged last of 33 rows (528 units)
    (7001, 256, 7001),                # one group of 224032 units (several tiles of each kind)
    (20000, 128, 4680),               # 4 full groups + a 1280-row tail, lag < groups
    (3000, 1024, 1000),               # head_dim 1024
    (60000, 128, 2000),               # 30 groups of 32000 units
]


def _x(rows, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, d), generator=g) * torch.exp2(torch.randint(-30, 30, (rows, 1), generator=g).float())
    x[torch.rand((rows, d), generator=g) < 1e-3] *= 64.0
    return x.to(torch.bfloat16)


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _guarded(n, dtype, fill, G=64):
    b = torch.full((n + 2 * G,), fill, dtype=dtype, device=DEV)
    return b, b[G:G + n]


def _guards_ok(b, fill, G=64):
    return bool(torch.all(b[:G] == fill)) and bool(torch.all(b[-G:] == fill))


def _one_kernel_applies(rows, d, rpg):
    upg = min(rpg, rows) * d // 8
    ng = -(-rows // rpg)
    return rows * d // 8 - (ng - 1) * upg >= 66


@pytest.fixture
def kv():
    import kv_cache_fp4_amd
    return kv_cache_fp4_amd


def _form_opts(kv, form):
    name = {"three_kernels": "three_kernel", "auto": "auto"}.get(form, "one_kernel")
    return kv.quantize_opts(name, 0 if form == "one_kernel_no_wait" else 20000)


@pytest.mark.parametrize("form", ["one_kernel", "three_kernels", "one_kernel_no_wait", "auto"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{d}/{g}" for r, d, g in SHAPES])
def test_quantize_forms_match_oracle(kv, shape, form):
    opts = _form_opts(kv, form)
    rows, d, rpg = shape
    x = _x(rows, d, rows + d)
    xh = _u16(x)
    xd = x.to(DEV)
    ng = -(-rows // rpg)
    for rule in RULES:
        cb, codes = _guarded(rows * d // 2, torch.uint8, 0xA5)
        sb, scales = _guarded(rows * d // 16, torch.uint8, 0x5A)
        ab, amax = _guarded(ng, torch.float32, -7.0)
        kv.kvfp4_quantize(xd, rpg, rule, codes, scales, amax, opts=opts)
        fb, fy = _guarded(rows * d, torch.int16, 0x3C3C)
        fab, famax = _guarded(ng, torch.float32, -7.0)
        kv.kvfp4_fake_quantize(xd, rpg, rule, y=fy.view(rows, d).view(torch.bfloat16),
                               group_amax=famax, opts=opts)
        torch.cuda.synchronize()
        oc, os_, oa = oracle.quantize(xh, rpg, rule)
        ofy, ofa = oracle.fake_quantize(xh, rpg, rule)
        what = (shape, form, rule, _one_kernel_applies(rows, d, rpg))
        for b, fill in ((cb, 0xA5), (sb, 0x5A), (ab, -7.0), (fb, 0x3C3C), (fab, -7.0)):
            assert _guards_ok(b, fill), what
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), oa.view(np.uint32)), what
        assert np.array_equal(scales.cpu().numpy().reshape(os_.shape), os_), what
        assert np.array_equal(codes.cpu().numpy().reshape(oc.shape), oc), what
        assert np.array_equal(famax.cpu().numpy().view(np.uint32), ofa.view(np.uint32)), what
        assert np.array_equal(_u16(fy).reshape(ofy.shape), ofy), what


def test_fake_quantize_in_place_matches_oracle(kv):
    rows, d, rpg = 9000, 128, 3000
    x = _x(rows, d, 5)
    xh = _u16(x)
    for rule in RULES:
        xd = x.to(DEV)
        kv.kvfp4_fake_quantize(xd, rpg, rule, y=xd)
        torch.cuda.synchronize()
        ofy, _ = oracle.fake_quantize(xh, rpg, rule)
        assert np.array_equal(_u16(xd).reshape(ofy.shape), ofy), rule


def test_append_into_cache_slab_both_forms_agree(kv):
    """A chunk appended into views of a larger cache (the benchmark's call pattern):
    the two forms write the same bytes, touch nothing outside the chunk's rows and group,
    and match the oracle."""
    H, D, T, chunks = 12, 128, 1170, 4
    rpg = T * H
    rows = rpg * chunks
    base = _x(rows, D, 11)
    src = _x(rpg, D, 12)
    out = {}
    for fused in (0, 1):
        opts = kv.quantize_opts("one_kernel" if fused else "three_kernel")
        codes, scales, amax = kv.kvfp4_quantize(base.to(DEV), rpg, "mse", opts=opts)
        last = slice(2 * rpg, 3 * rpg)
        kv.kvfp4_quantize(src.to(DEV), rpg, "mse", codes[last], scales[last], amax[2:3],
                          opts=opts)
        torch.cuda.synchronize()
        out[fused] = (codes.cpu(), scales.cpu(), amax.cpu())
    for a, b in zip(out[0], out[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    merged = base.clone()
    merged[2 * rpg:3 * rpg] = src
    oc, os_, oa = oracle.quantize(_u16(merged), rpg, "mse")
    assert np.array_equal(out[1][0].numpy(), oc)
    assert np.array_equal(out[1][1].numpy(), os_)
    assert np.array_equal(out[1][2].numpy().view(np.uint32), oa.view(np.uint32))


def test_concurrent_appends_on_two_streams(kv):
    """Two one-kernel appends enqueued back to back on two streams, so that they can run at
    the same time (different inputs and outputs): each call's hand-off lives in its own
    output, so both match the oracle."""
    rows, d, rpg = 60000, 128, 6000
    xs = [_x(rows, d, 100 + i) for i in range(2)]
    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
    xd = [x.to(DEV) for x in xs]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        outs = []
        for x, st in zip(xd, streams):
            with torch.cuda.stream(st):
                outs.append(kv.kvfp4_quantize(x, rpg, "mse", stream=st))
        torch.cuda.synchronize()
    for x, (c, s, a) in zip(xs, outs):
        oc, os_, oa = oracle.quantize(_u16(x), rpg, "mse")
        assert np.array_equal(c.cpu().numpy(), oc)
        assert np.array_equal(s.cpu().numpy(), os_)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), oa.view(np.uint32))
