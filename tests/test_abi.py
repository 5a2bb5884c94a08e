"""C-ABI checks that need no GPU: the library loads, exports every function its header
declares, and rejects bad arguments on the host before enqueueing anything."""
import ctypes
import os
import re

import pytest

import kv_cache_fp4_amd as kv
from kv_cache_fp4_amd import (KVFP4_EALIGN, KVFP4_EINVAL, KVFP4_EUNSUPPORTED, KVFP4_OK, lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            txt = open(os.path.join(inc, f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(kvfp4_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"kvfp4_quantize", "kvfp4_dequantize", "kvfp4_packed_sizes", "kvfp4_status_str",
            "kvfp4_abi_version", "kvfp4_last_hip_error"} <= set(names)
    raw = ctypes.CDLL(kv.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_abi_version_and_status_strings():
    assert lib.kvfp4_abi_version() == 2
    for s in range(5):
        assert lib.kvfp4_status_str(s)
    assert b"unknown" in lib.kvfp4_status_str(99)


A16 = 1 << 20  # a fake, 16-byte aligned address: validation never dereferences it


def q(x=A16, rows=64, d=128, rpg=64, rule=0, codes=A16, scales=A16, amax=A16):
    return lib.kvfp4_quantize(x, rows, d, rpg, rule, codes, scales, amax, None)


def dq(codes=A16, scales=A16, amax=A16, rows=64, d=128, rpg=64, y=A16):
    return lib.kvfp4_dequantize(codes, scales, amax, rows, d, rpg, y, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), KVFP4_EINVAL),
    (dict(rpg=0), KVFP4_EINVAL),
    (dict(rpg=-5), KVFP4_EINVAL),
    (dict(rule=3), KVFP4_EINVAL),
    (dict(rule=-1), KVFP4_EINVAL),
    (dict(x=None), KVFP4_EINVAL),
    (dict(codes=None), KVFP4_EINVAL),
    (dict(scales=None), KVFP4_EINVAL),
    (dict(amax=None), KVFP4_EINVAL),
    (dict(d=48), KVFP4_EUNSUPPORTED),
    (dict(d=96), KVFP4_EUNSUPPORTED),
    (dict(d=2048), KVFP4_EUNSUPPORTED),
    (dict(d=0), KVFP4_EUNSUPPORTED),
    (dict(x=A16 + 8), KVFP4_EALIGN),
    (dict(codes=A16 + 4), KVFP4_EALIGN),
    (dict(scales=A16 + 2), KVFP4_EALIGN),
    (dict(amax=A16 + 2), KVFP4_EALIGN),
    (dict(rows=1 << 50), KVFP4_EINVAL),
])
def test_quantize_rejects(kw, want):
    assert q(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-3), KVFP4_EINVAL),
    (dict(rpg=0), KVFP4_EINVAL),
    (dict(codes=None), KVFP4_EINVAL),
    (dict(y=None), KVFP4_EINVAL),
    (dict(d=16), KVFP4_EUNSUPPORTED),
    (dict(y=A16 + 2), KVFP4_EALIGN),
    (dict(codes=A16 + 1), KVFP4_EALIGN),
    (dict(scales=A16 + 1), KVFP4_EALIGN),
])
def test_dequantize_rejects(kw, want):
    assert dq(**kw) == want


def test_zero_rows_is_a_noop_even_with_null_pointers():
    assert q(rows=0, x=None, codes=None, scales=None, amax=None) == KVFP4_OK
    assert dq(rows=0, codes=None, scales=None, amax=None, y=None) == KVFP4_OK


def test_packed_sizes():
    assert kv.kvfp4_packed_sizes(56160 * 2, 128, 56160) == (56160 * 2 * 64, 56160 * 2 * 8, 2)
    assert kv.kvfp4_packed_sizes(37, 64, 10) == (37 * 32, 37 * 4, 4)
    assert kv.kvfp4_packed_sizes(0, 64, 10) == (0, 0, 0)
    with pytest.raises(kv.KVFP4Error):
        kv.kvfp4_packed_sizes(10, 80, 10)


def at(q=A16, tq=10, kc=A16, ks=A16, ka=A16, vc=A16, vs=A16, va=A16, tk=10, h=2, d=128, tpg=5,
       scale=0.1, out=A16):
    return lib.kvfp4_attend(q, tq, kc, ks, ka, vc, vs, va, tk, h, d, tpg, scale, out, None)


@pytest.mark.parametrize("kw,want", [
    (dict(tq=-1), KVFP4_EINVAL),
    (dict(tk=0), KVFP4_EINVAL),
    (dict(h=0), KVFP4_EINVAL),
    (dict(tpg=0), KVFP4_EINVAL),
    (dict(scale=float("inf")), KVFP4_EINVAL),
    (dict(scale=float("nan")), KVFP4_EINVAL),
    (dict(scale=0.0), KVFP4_EINVAL),
    (dict(scale=-0.5), KVFP4_EINVAL),
    (dict(d=256), KVFP4_EUNSUPPORTED),
    (dict(d=96), KVFP4_EUNSUPPORTED),
    (dict(q=None), KVFP4_EINVAL),
    (dict(va=None), KVFP4_EINVAL),
    (dict(out=None), KVFP4_EINVAL),
    (dict(q=A16 + 8), KVFP4_EALIGN),
    (dict(kc=A16 + 4), KVFP4_EALIGN),
    (dict(vs=A16 + 2), KVFP4_EALIGN),
    (dict(out=A16 + 2), KVFP4_EALIGN),
    (dict(h=70000), KVFP4_EINVAL),
])
def test_attend_rejects(kw, want):
    assert at(**kw) == want


def test_attend_zero_queries_is_a_noop():
    assert at(tq=0, q=None, kc=None, ks=None, ka=None, vc=None, vs=None, va=None, out=None) == KVFP4_OK


def qp(x=A16, nb=4, rpp=24, d=128, rule=0, tab=A16, npg=8, codes=A16, scales=A16, amax=A16):
    return lib.kvfp4_quantize_paged(x, nb, rpp, d, rule, tab, npg, codes, scales, amax, None)


def dqp(codes=A16, scales=A16, amax=A16, tab=A16, nb=4, rpp=24, d=128, npg=8, y=A16):
    return lib.kvfp4_dequantize_paged(codes, scales, amax, tab, nb, rpp, d, npg, y, None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=-1), KVFP4_EINVAL), (dict(rpp=0), KVFP4_EINVAL), (dict(npg=-1), KVFP4_EINVAL),
    (dict(rule=5), KVFP4_EINVAL), (dict(tab=None), KVFP4_EINVAL), (dict(x=None), KVFP4_EINVAL),
    (dict(d=100), KVFP4_EUNSUPPORTED), (dict(tab=A16 + 2), KVFP4_EALIGN),
    (dict(codes=A16 + 8), KVFP4_EALIGN), (dict(amax=A16 + 1), KVFP4_EALIGN),
    (dict(nb=1 << 40, rpp=1 << 20), KVFP4_EINVAL),
    (dict(npg=1 << 40, rpp=1 << 10), KVFP4_EINVAL),
])
def test_quantize_paged_rejects(kw, want):
    assert qp(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(nb=-1), KVFP4_EINVAL), (dict(rpp=-2), KVFP4_EINVAL), (dict(tab=None), KVFP4_EINVAL),
    (dict(y=None), KVFP4_EINVAL), (dict(d=32), KVFP4_EUNSUPPORTED), (dict(y=A16 + 4), KVFP4_EALIGN),
    (dict(scales=A16 + 3), KVFP4_EALIGN), (dict(npg=1 << 40, rpp=1 << 10), KVFP4_EINVAL),
])
def test_dequantize_paged_rejects(kw, want):
    assert dqp(**kw) == want


def test_paged_zero_blocks_is_a_noop():
    assert qp(nb=0, x=None, tab=None, codes=None, scales=None, amax=None) == KVFP4_OK
    assert dqp(nb=0, codes=None, scales=None, amax=None, tab=None, y=None) == KVFP4_OK


@pytest.mark.parametrize("kw,want", [
    (dict(bits=3), KVFP4_EINVAL), (dict(bits=8), KVFP4_EINVAL), (dict(rows=-1), KVFP4_EINVAL),
    (dict(x=None), KVFP4_EINVAL), (dict(d=80), KVFP4_EUNSUPPORTED), (dict(codes=A16 + 2), KVFP4_EALIGN),
    (dict(scales=A16 + 2), KVFP4_EALIGN),
])
def test_rtn_quantize_rejects(kw, want):
    a = dict(x=A16, rows=10, d=128, bits=4, codes=A16, scales=A16)
    a.update(kw)
    assert lib.kvfp4_rtn_quantize(a["x"], a["rows"], a["d"], a["bits"], a["codes"], a["scales"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(bits=1), KVFP4_EINVAL), (dict(tail_rows=-1), KVFP4_EINVAL), (dict(tail=None), KVFP4_EINVAL),
    (dict(y=None), KVFP4_EINVAL), (dict(tail=A16 + 8), KVFP4_EALIGN), (dict(d=16), KVFP4_EUNSUPPORTED),
])
def test_rtn_dequantize_rejects(kw, want):
    a = dict(codes=A16, scales=A16, rows=10, d=128, bits=2, tail=A16, tail_rows=3, y=A16)
    a.update(kw)
    assert lib.kvfp4_rtn_dequantize(a["codes"], a["scales"], a["rows"], a["d"], a["bits"], a["tail"],
                                    a["tail_rows"], a["y"], None) == want


def test_rtn_zero_rows_is_a_noop():
    assert lib.kvfp4_rtn_quantize(None, 0, 128, 4, None, None, None) == KVFP4_OK
    assert lib.kvfp4_rtn_dequantize(None, None, 0, 128, 4, None, 0, None, None) == KVFP4_OK


def dqf(codes=A16, scales=A16, amax=A16, rows=64, d=128, rpg=64, y=A16):
    return lib.kvfp4_dequantize_f32(codes, scales, amax, rows, d, rpg, y, None)


def dqpf(codes=A16, scales=A16, amax=A16, tab=A16, nb=4, rpp=24, d=128, npg=8, y=A16):
    return lib.kvfp4_dequantize_paged_f32(codes, scales, amax, tab, nb, rpp, d, npg, y, None)


def fq(x=A16, rows=64, d=128, rpg=64, rule=0, amax=A16, y=A16):
    return lib.kvfp4_fake_quantize(x, rows, d, rpg, rule, amax, y, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-3), KVFP4_EINVAL), (dict(rpg=0), KVFP4_EINVAL), (dict(codes=None), KVFP4_EINVAL),
    (dict(amax=None), KVFP4_EINVAL), (dict(y=None), KVFP4_EINVAL), (dict(d=16), KVFP4_EUNSUPPORTED),
    (dict(y=A16 + 4), KVFP4_EALIGN), (dict(codes=A16 + 1), KVFP4_EALIGN),
    (dict(scales=A16 + 1), KVFP4_EALIGN),
])
def test_dequantize_f32_rejects(kw, want):
    assert dqf(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(nb=-1), KVFP4_EINVAL), (dict(tab=None), KVFP4_EINVAL), (dict(y=None), KVFP4_EINVAL),
    (dict(d=32), KVFP4_EUNSUPPORTED), (dict(y=A16 + 8), KVFP4_EALIGN),
    (dict(amax=A16 + 2), KVFP4_EALIGN),
])
def test_dequantize_paged_f32_rejects(kw, want):
    assert dqpf(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), KVFP4_EINVAL), (dict(rpg=0), KVFP4_EINVAL), (dict(rule=3), KVFP4_EINVAL),
    (dict(x=None), KVFP4_EINVAL), (dict(amax=None), KVFP4_EINVAL), (dict(y=None), KVFP4_EINVAL),
    (dict(d=96), KVFP4_EUNSUPPORTED), (dict(x=A16 + 8), KVFP4_EALIGN),
    (dict(y=A16 + 2), KVFP4_EALIGN), (dict(amax=A16 + 2), KVFP4_EALIGN),
    (dict(rows=1 << 50), KVFP4_EINVAL),
])
def test_fake_quantize_rejects(kw, want):
    assert fq(**kw) == want


def test_f32_and_fake_zero_rows_are_noops():
    assert dqf(rows=0, codes=None, scales=None, amax=None, y=None) == KVFP4_OK
    assert dqpf(nb=0, codes=None, scales=None, amax=None, tab=None, y=None) == KVFP4_OK
    assert fq(rows=0, x=None, amax=None, y=None) == KVFP4_OK


def qx(opts, **kw):
    a = dict(x=A16, rows=64, d=128, rpg=64, rule=0, codes=A16, scales=A16, amax=A16)
    a.update(kw)
    return lib.kvfp4_quantize_ex(a["x"], a["rows"], a["d"], a["rpg"], a["rule"], a["codes"],
                                 a["scales"], a["amax"], opts, None)


@pytest.mark.parametrize("form,wait,want", [
    (3, 20000, KVFP4_EINVAL), (-1, 20000, KVFP4_EINVAL), (0, -1, KVFP4_EINVAL),
    (1, 60000001, KVFP4_EINVAL), (0, 1 << 40, KVFP4_EINVAL),
])
def test_quantize_options_rejected_per_call(form, wait, want):
    """Bad per-call options are argument errors of that call, found before anything is
    enqueued (the pointers here are fake: nothing may be launched), on every _ex entry."""
    o = ctypes.byref(kv.QuantizeOpts(form, wait))
    assert qx(o) == want
    assert lib.kvfp4_quantize_paged_ex(A16, 4, 24, 128, 0, A16, 8, A16, A16, A16, o, None) == want
    assert lib.kvfp4_fake_quantize_ex(A16, 64, 128, 64, 0, A16, A16, o, None) == want


@pytest.mark.parametrize("form,wait", [(0, 0), (0, 20000), (1, 0), (1, 60000000), (2, 0),
                                       (2, 20000)])
def test_quantize_options_accepted(form, wait):
    """Valid options with zero rows: accepted, nothing to do (no device needed)."""
    o = ctypes.byref(kv.QuantizeOpts(form, wait))
    assert qx(o, rows=0, x=None, codes=None, scales=None, amax=None) == KVFP4_OK
    assert lib.kvfp4_quantize_paged_ex(None, 0, 24, 128, 0, None, 8, None, None, None, o,
                                       None) == KVFP4_OK
    assert lib.kvfp4_fake_quantize_ex(None, 0, 128, 64, 0, None, None, o, None) == KVFP4_OK
    # NULL options are the defaults
    assert qx(None, rows=0, x=None, codes=None, scales=None, amax=None) == KVFP4_OK


def test_ex_entries_check_arguments_like_the_plain_ones():
    o = ctypes.byref(kv.quantize_opts())
    assert qx(o, rule=3) == KVFP4_EINVAL
    assert qx(o, d=96) == KVFP4_EUNSUPPORTED
    assert qx(o, x=A16 + 8) == KVFP4_EALIGN
    assert qx(o, rpg=0) == KVFP4_EINVAL


def test_library_keeps_no_mutable_global_state():
    """The only writable object the library defines in its own namespace is the thread-local
    last HIP error; every other kvfp4:: object is a kernel's host-side launch handle (a
    function signature).  Read from the ELF symbol table of the built library."""
    import subprocess
    out = subprocess.run(["readelf", "-sW", kv.LIB_PATH], check=True, capture_output=True,
                         text=True).stdout
    dem = subprocess.run(["c++filt"], input=out, check=True, capture_output=True, text=True).stdout
    objs = []
    for line in dem.splitlines():
        f = line.split(None, 7)
        if len(f) == 8 and f[3] in ("OBJECT", "TLS") and f[6] != "UND" and "kvfp4" in f[7]:
            objs.append((f[3], f[7]))
    tls = [n for t, n in objs if t == "TLS"]
    assert tls == ["kvfp4::(anonymous namespace)::g_last_hip_error"], tls
    others = [n for t, n in objs if t == "OBJECT"]
    assert others, "expected the kernels' launch handles"
    for n in others:
        assert "_kernel" in n and "(" in n, n
