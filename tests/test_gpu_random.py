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


def _f(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("seed", list(range(12)))
def test_random_attention_case(seed):
    """Random (q_tokens, kv_tokens, heads, head_dim, tokens_per_group, query scale); 64 sampled
    query rows against the oracle's double-precision attention over its own dequantized
    cache, within the attention tolerance (max |err| <= 2e-2 of max(1, max |O|), relative
    RMS <= 1e-2)."""
    import kv_cache_fp4_amd as kv
    rng = np.random.default_rng(2000 + seed)
    tq, tk = int(rng.integers(1, 700)), int(rng.integers(1, 2500))
    H, D = int(rng.integers(1, 6)), int(rng.choice([64, 128]))
    tpg = int(rng.integers(1, tk + 1)) if rng.random() < 0.8 else tk
    qs = float(rng.choice([D ** -0.5, 1.0, 4.0]))
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((tq, H, D), generator=g) * qs).to(torch.bfloat16)
    k = torch.randn((tk, H, D), generator=g).to(torch.bfloat16)
    v = (torch.randn((tk, H, D), generator=g) * 3).to(torch.bfloat16)
    rpg = tpg * H
    kc, ks, ka = kv.kvfp4_quantize(k.to(DEV), rpg, "static_6")
    vc, vs, va = kv.kvfp4_quantize(v.to(DEV), rpg, "static_6")
    o = kv.kvfp4_attend(q.to(DEV), kc, ks, ka, vc, vs, va, tpg, D ** -0.5)
    torch.cuda.synchronize()
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    kd = oracle.dequantize(*oracle.quantize(u16(k).reshape(-1, D), rpg, "static_6"), rpg)
    vd = oracle.dequantize(*oracle.quantize(u16(v).reshape(-1, D), rpg, "static_6"), rpg)
    rows = np.unique(np.concatenate([[0, tq * H - 1], rng.integers(0, tq * H, 62)])).astype(np.int64)
    ref = _f(oracle.attend_rows(u16(q), kd.reshape(tk, H, D), vd.reshape(tk, H, D), D ** -0.5, rows))
    got = _f(u16(o.cpu()).reshape(-1, D)[rows])
    err = np.abs(got - ref).max() / max(1.0, np.abs(ref).max())
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= 2e-2 and rel <= 1e-2, (seed, tq, tk, H, D, tpg, qs, err, rel)


@pytest.mark.parametrize("seed", list(range(12)))
def test_random_rtn_case(seed):
    import kv_cache_fp4_amd as kv
    rng = np.random.default_rng(3000 + seed)
    d = int(rng.integers(1, 17)) * 64
    rows, tail_rows = int(rng.integers(0, 200_000 // d)), int(rng.integers(0, 300))
    bits = int(rng.choice([2, 4]))
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((rows, d), generator=g) * float(2.0 ** rng.integers(-40, 40))).to(torch.bfloat16)
    tail = torch.randn((tail_rows, d), generator=g).to(torch.bfloat16)
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    oc, os_ = oracle.rtn_quantize(u16(x), bits)
    oy = oracle.rtn_dequantize(oc, os_, bits)
    c, s = kv.kvfp4_rtn_quantize(x.to(DEV), bits)
    y = kv.kvfp4_rtn_dequantize(c, s, bits, tail=tail.to(DEV) if tail_rows else None)
    torch.cuda.synchronize()
    what = (seed, rows, d, bits, tail_rows)
    assert np.array_equal(c.cpu().numpy(), oc), what
    assert np.array_equal(u16(s.cpu()), os_), what
    assert np.array_equal(u16(y.cpu()), np.concatenate([oy.reshape(rows, d), u16(tail)])), what
