"""The library under HIP graph capture: the entry points allocate nothing, never synchronize
and clear the group amax words with a kernel (no memset node), so an append + whole-cache
read + fused attention can be captured once and replayed, with the append in either quantize
form.  Each replay gets new input values (copied into the captured buffers between replays,
with eager work and a synchronization in between) and must match the eager result for those
values bit for bit.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _x(rows, d, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((rows, d), generator=g) * torch.exp(torch.randn((1, d), generator=g))).to(
        torch.bfloat16)


@pytest.mark.parametrize("form", ["one_kernel", "three_kernel"])
def test_capture_append_read_attend_and_replay(form):
    import kv_cache_fp4_amd as kv
    opts = kv.quantize_opts(form)
    H, D, tpg, chunks = 4, 128, 300, 3
    rpg = tpg * H
    rows = rpg * chunks
    # static buffers: the appended chunk (last group), the packed cache, outputs, a query
    src = _x(rpg, D, 1).to(DEV)
    base = _x(rows, D, 2).to(DEV)
    codes, scales, amax = kv.kvfp4_quantize(base, rpg, "mse")
    y = torch.empty((rows, D), dtype=torch.bfloat16, device=DEV)
    q = synth.query((200, H, D), 3, 1.0, device=DEV)
    vc, vs, va = kv.kvfp4_quantize(_x(rows, D, 4).to(DEV), rpg, "static_6")
    att = torch.empty((200, H, D), dtype=torch.bfloat16, device=DEV)
    last = slice((chunks - 1) * rpg, rows)

    def step():
        kv.kvfp4_quantize(src, rpg, "mse", codes[last], scales[last], amax[chunks - 1:],
                          opts=opts)
        kv.kvfp4_dequantize(codes, scales, amax, rpg, y=y)
        kv.kvfp4_attend(q, codes, scales, amax, vc, vs, va, tpg, D ** -0.5, out=att)

    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        src.copy_(_x(rpg, D, 10 + rep).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (codes, scales, amax, y, att)]
        step()  # eager on the same inputs
        torch.cuda.synchronize()
        for a, b, name in zip(got, (codes, scales, amax, y, att),
                              ("codes", "scales", "amax", "dequant", "attend")):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, name)
        # the replay really used the new chunk: its group amax is the new input's
        assert amax[chunks - 1].item() == src.abs().max().float().item()
