"""The Python binding checks every tensor before it calls the C ABI: dtype, element count
against the packed sizes the call implies, layout, device, and the scalar arguments.  A
mismatch raises ValueError and no C entry point is reached (the library is swapped for a
recorder that fails on any use), so a short or mistyped buffer can never become an
out-of-bounds device access.  Runs on the CPU: the checks come before any device work."""
import pytest
import torch

import kv_cache_fp4_amd as kv

bf, u8, f32, i32 = torch.bfloat16, torch.uint8, torch.float32, torch.int32


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"C entry point {name} reached")


@pytest.fixture(autouse=True)
def no_c_calls(monkeypatch):
    monkeypatch.setattr(kv, "lib", _NoCalls())


def z(n, dtype, *shape):
    return torch.zeros(shape or (n,), dtype=dtype)


ROWS, D, RPG = 48, 128, 16          # 3 groups
NC, NS, NG = ROWS * D // 2, ROWS * D // 16, 3


def _raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


# ---- quantize ----------------------------------------------------------------------------

def test_quantize_checks_x():
    _raises("x must be torch.bfloat16", kv.kvfp4_quantize, z(0, f32, ROWS, D), RPG)
    _raises("head_dim 80", kv.kvfp4_quantize, z(0, bf, ROWS, 80), RPG)
    _raises("contiguous", kv.kvfp4_quantize, z(0, bf, D, ROWS).t(), RPG)
    _raises("rows_per_group", kv.kvfp4_quantize, z(0, bf, ROWS, D), 0)
    _raises("unknown rule", kv.kvfp4_quantize, z(0, bf, ROWS, D), RPG, "static_5")
    _raises("on a GPU", kv.kvfp4_quantize, z(0, bf, ROWS, D), RPG)


@pytest.mark.parametrize("kw,match", [
    (dict(codes=z(NC - 1, u8)), "codes has"),
    (dict(codes=z(NC, torch.int8)), "codes must be torch.uint8"),
    (dict(scales=z(NS + 16, u8)), "scales has"),
    (dict(scales=z(NS, bf)), "scales must be torch.uint8"),
    (dict(group_amax=z(NG - 1, f32)), "group_amax has"),
    (dict(group_amax=z(NG, torch.float64)), "group_amax must be torch.float32"),
])
def test_quantize_checks_outputs(kw, match):
    _raises(match, kv.kvfp4_quantize, z(0, bf, ROWS, D), RPG, "mse", **kw)


def test_quantize_checks_options():
    _raises("quantize_opts", kv.kvfp4_quantize, z(0, bf, ROWS, D), RPG, opts=(0, 1))


# ---- dequantize (bf16 and float32) ---------------------------------------------------------

@pytest.mark.parametrize("fn,ydt", [(kv.kvfp4_dequantize, bf), (kv.kvfp4_dequantize_f32, f32)])
@pytest.mark.parametrize("codes,scales,amax,y,match", [
    (z(NC, u8), z(NS, u8), z(NG, f32), None, "codes must be a 2-D"),
    (z(0, u8, ROWS, D // 2), z(NS - 1, u8), z(NG, f32), None, "scales has"),
    (z(0, u8, ROWS, D // 2), z(NS, u8), z(NG + 1, f32), None, "group_amax has"),
    (z(0, u8, ROWS, D // 2), z(NS, u8), z(NG, f32), z(ROWS * D - 8, None), "y has"),
    (z(0, u8, ROWS, 40), z(NS, u8), z(NG, f32), None, "head_dim 80"),
    (z(0, u8, ROWS, D // 2), z(NS, u8), z(NG, f32), None, "on a GPU"),
])
def test_dequantize_checks(fn, ydt, codes, scales, amax, y, match):
    if y is not None:
        y = y.to(ydt)
    _raises(match, fn, codes, scales, amax, RPG, y=y)


def test_dequantize_checks_output_dtype():
    _raises("y must be torch.bfloat16", kv.kvfp4_dequantize, z(0, u8, ROWS, D // 2), z(NS, u8),
            z(NG, f32), RPG, y=z(ROWS * D, f32))
    _raises("y must be torch.float32", kv.kvfp4_dequantize_f32, z(0, u8, ROWS, D // 2),
            z(NS, u8), z(NG, f32), RPG, y=z(ROWS * D, bf))


# ---- fake quantization -----------------------------------------------------------------------

def test_fake_quantize_checks():
    x = z(0, bf, ROWS, D)
    _raises("y has", kv.kvfp4_fake_quantize, x, RPG, y=z(ROWS * D - 1, bf))
    _raises("y must be torch.bfloat16", kv.kvfp4_fake_quantize, x, RPG, y=z(ROWS * D, torch.int16))
    _raises("group_amax has", kv.kvfp4_fake_quantize, x, RPG, group_amax=z(NG - 1, f32))
    _raises("on a GPU", kv.kvfp4_fake_quantize, x, RPG)


# ---- paged cache -----------------------------------------------------------------------------

NB, RPP, NP = 4, 24, 6


def _pages(dc=0, ds=0, da=0):
    return (z(0, u8, NP * RPP + dc, D // 2), z(NP * RPP * D // 16 + ds, u8), z(NP + da, f32))


@pytest.mark.parametrize("pages,tab,match", [
    (_pages(ds=-1), z(NB, i32), "scales has"),
    (_pages(dc=1), z(NB, i32), "codes has"),
    (_pages(), z(NB, torch.int64), "block_table must be torch.int32"),
    (_pages(), z(NB, i32), "on a GPU"),
])
def test_paged_checks(pages, tab, match):
    c, s, a = pages
    _raises(match, kv.kvfp4_dequantize_paged, c, s, a, tab, RPP)
    _raises(match, kv.kvfp4_dequantize_paged_f32, c, s, a, tab, RPP)
    _raises(match, kv.kvfp4_quantize_paged, z(NB * RPP * D, bf), tab, RPP, c, s, a)


def test_paged_quantize_checks_x_and_rows_per_page():
    c, s, a = _pages()
    _raises("rows_per_page", kv.kvfp4_quantize_paged, z(NB * RPP * D, bf), z(NB, i32), 0, c, s, a)
    _raises("x has", kv.kvfp4_quantize_paged, z(NB * RPP * D - D, bf), z(NB, i32), RPP, c, s, a)
    _raises("x must be torch.bfloat16", kv.kvfp4_quantize_paged, z(NB * RPP * D, f32),
            z(NB, i32), RPP, c, s, a)
    _raises("head_dim", kv.kvfp4_quantize_paged, z(0, bf, NB * RPP * 2, D // 2), z(NB, i32), RPP,
            c, s, a)
    _raises("y has", kv.kvfp4_dequantize_paged, c, s, a, z(NB, i32), RPP, y=z(NB * RPP * D + 1, bf))
    _raises("on a GPU", kv.kvfp4_quantize_paged, z(NB * RPP * D, bf), z(NB, i32), RPP, c, s, a)


# ---- RTN -------------------------------------------------------------------------------------

def test_rtn_checks():
    x = z(0, bf, ROWS, D)
    _raises("bits must be 2 or 4", kv.kvfp4_rtn_quantize, x, 3)
    _raises("codes has", kv.kvfp4_rtn_quantize, x, 4, codes=z(ROWS * D // 4, u8))
    _raises("scales must be torch.bfloat16", kv.kvfp4_rtn_quantize, x, 2,
            scales=z(ROWS * D // 16, u8))
    _raises("on a GPU", kv.kvfp4_rtn_quantize, x, 4)
    sc = z(0, bf, ROWS, D // 16)
    _raises("codes has", kv.kvfp4_rtn_dequantize, z(ROWS * D // 2, u8), sc, 2)
    _raises("whole rows", kv.kvfp4_rtn_dequantize, z(ROWS * D // 4, u8), sc, 2,
            tail=z(D + 3, bf))
    _raises("scales must be a 2-D", kv.kvfp4_rtn_dequantize, z(ROWS * D // 4, u8),
            z(ROWS * D // 16, bf), 2)
    _raises("on a GPU", kv.kvfp4_rtn_dequantize, z(ROWS * D // 4, u8), sc, 2)


# ---- attention -------------------------------------------------------------------------------

TQ, H, TK, TPG = 10, 2, 40, 16     # 3 K/V groups
KC, KS, KG = TK * H * D // 2, TK * H * D // 16, 3


def _att(**kw):
    a = dict(q=z(0, bf, TQ, H, D), k_codes=z(KC, u8), k_scales=z(KS, u8), k_amax=z(KG, f32),
             v_codes=z(KC, u8), v_scales=z(KS, u8), v_amax=z(KG, f32))
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,match", [
    (dict(k_scales=z(KS - 1, u8)), "k_scales has"),
    (dict(v_scales=z(KS + 4, u8)), "v_scales has"),
    (dict(v_codes=z(KC - D // 2, u8)), "v_codes has"),
    (dict(k_codes=z(KC + 1, u8)), "whole"),
    (dict(k_amax=z(KG - 1, f32)), "k_amax has"),
    (dict(v_amax=z(KG + 1, f32)), "v_amax has"),
    (dict(v_amax=z(KG, bf)), "v_amax must be torch.float32"),
    (dict(q=z(0, bf, TQ, H * D)), "3-D"),
    (dict(q=z(0, bf, TQ, H, 96)), "head_dim 64 or 128"),
    (dict(q=z(0, f32, TQ, H, D)), "q must be torch.bfloat16"),
    (dict(), "on a GPU"),
])
def test_attend_checks(kw, match):
    a = _att(**kw)
    _raises(match, kv.kvfp4_attend, a["q"], a["k_codes"], a["k_scales"], a["k_amax"],
            a["v_codes"], a["v_scales"], a["v_amax"], TPG)


def test_attend_checks_out_and_group_size():
    a = _att()
    args = (a["q"], a["k_codes"], a["k_scales"], a["k_amax"], a["v_codes"], a["v_scales"],
            a["v_amax"])
    _raises("tokens_per_group", kv.kvfp4_attend, *args, 0)
    _raises("out has", kv.kvfp4_attend, *args, TPG, out=z(TQ * H * D - 1, bf))
