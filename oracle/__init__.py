"""CPU oracle for NVFP4 KV-cache quantize / dequantize / attention (ctypes loader).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``; never by the ``kv_cache_fp4_amd`` package.  The
arithmetic lives in ``kvfp4_oracle.c`` (plain C, one IEEE binary32 operation per step);
this module only moves numpy arrays in and out of it.

Every function here is "parity pinned" by ``tests/test_oracle_*.py`` against closed forms,
worked examples, brute force and library routines; see the header of ``kvfp4_oracle.c``
for the page citations of each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvfp4_oracle.c")
# KVFP4_ORACLE_LIB lets the mutation tests load a deliberately broken build of the oracle.
_LIB = os.environ.get("KVFP4_ORACLE_LIB") or os.path.join(_HERE, "libkvfp4_oracle.so")

RULES = {"static_6": 0, "static_4": 1, "mse": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.kvfp4_oracle_e2m1_value.argtypes = [i32]
        L.kvfp4_oracle_e2m1_value.restype = f64
        L.kvfp4_oracle_e2m1_encode.argtypes = [f32]
        L.kvfp4_oracle_e2m1_encode.restype = i32
        L.kvfp4_oracle_e4m3_value.argtypes = [i32]
        L.kvfp4_oracle_e4m3_value.restype = f64
        L.kvfp4_oracle_e4m3_encode.argtypes = [f32]
        L.kvfp4_oracle_e4m3_encode.restype = i32
        L.kvfp4_oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.kvfp4_oracle_bf16_to_float.restype = f32
        L.kvfp4_oracle_float_to_bf16.argtypes = [f32]
        L.kvfp4_oracle_float_to_bf16.restype = ctypes.c_uint16
        L.kvfp4_oracle_group_amax.argtypes = [P, i64]
        L.kvfp4_oracle_group_amax.restype = f32
        L.kvfp4_oracle_quantize_rows.argtypes = [P, i64, i32, f32, i32, P, P]
        L.kvfp4_oracle_quantize_rows.restype = i32
        L.kvfp4_oracle_quantize.argtypes = [P, i64, i32, i64, i32, P, P, P]
        L.kvfp4_oracle_quantize.restype = i32
        L.kvfp4_oracle_dequantize_rows.argtypes = [P, P, i64, i32, f32, P]
        L.kvfp4_oracle_dequantize_rows.restype = i32
        L.kvfp4_oracle_dequantize.argtypes = [P, P, P, i64, i32, i64, P]
        L.kvfp4_oracle_dequantize.restype = i32
        L.kvfp4_oracle_dequantize_rows_f32.argtypes = [P, P, i64, i32, f32, P]
        L.kvfp4_oracle_dequantize_rows_f32.restype = i32
        L.kvfp4_oracle_dequantize_f32.argtypes = [P, P, P, i64, i32, i64, P]
        L.kvfp4_oracle_dequantize_f32.restype = i32
        L.kvfp4_oracle_dequantize_paged_f32.argtypes = [P, P, P, P, i64, i64, i32, i64, P]
        L.kvfp4_oracle_dequantize_paged_f32.restype = i32
        L.kvfp4_oracle_fake_quantize.argtypes = [P, i64, i32, i64, i32, P, P]
        L.kvfp4_oracle_fake_quantize.restype = i32
        L.kvfp4_oracle_attend_rows.argtypes = [P, P, P, i64, i32, i32, f64, P, i64, P, P]
        L.kvfp4_oracle_attend_rows.restype = i32
        L.kvfp4_oracle_quantize_paged.argtypes = [P, i64, i64, i32, i32, P, i64, P, P, P]
        L.kvfp4_oracle_quantize_paged.restype = i32
        L.kvfp4_oracle_dequantize_paged.argtypes = [P, P, P, P, i64, i64, i32, i64, P]
        L.kvfp4_oracle_dequantize_paged.restype = i32
        L.kvfp4_oracle_rtn_quantize.argtypes = [P, i64, i32, i32, P, P]
        L.kvfp4_oracle_rtn_quantize.restype = i32
        L.kvfp4_oracle_rtn_dequantize.argtypes = [P, P, i64, i32, i32, P]
        L.kvfp4_oracle_rtn_dequantize.restype = i32
        for name in ("kvfp4_oracle_e2m1_encode_n", "kvfp4_oracle_e4m3_encode_n",
                     "kvfp4_oracle_float_to_bf16_n", "kvfp4_oracle_double_to_bf16_n"):
            getattr(L, name).argtypes = [P, i64, P]
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _rule(rule) -> int:
    return RULES[rule] if isinstance(rule, str) else int(rule)


# ---- formats -------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().kvfp4_oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().kvfp4_oracle_e4m3_value(int(byte))


def e2m1_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    out = np.empty(y.size, dtype=np.uint8)
    lib().kvfp4_oracle_e2m1_encode_n(_p(y), y.size, _p(out))
    return out


def e4m3_encode(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.float32).reshape(-1)
    out = np.empty(u.size, dtype=np.uint8)
    lib().kvfp4_oracle_e4m3_encode_n(_p(u), u.size, _p(out))
    return out


def float_to_bf16(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32).reshape(-1)
    out = np.empty(f.size, dtype=np.uint16)
    lib().kvfp4_oracle_float_to_bf16_n(_p(f), f.size, _p(out))
    return out


def double_to_bf16(f) -> np.ndarray:
    """Round doubles to bf16 in one step (the attention output's rounding)."""
    f = np.ascontiguousarray(f, dtype=np.float64).reshape(-1)
    out = np.empty(f.size, dtype=np.uint16)
    lib().kvfp4_oracle_double_to_bf16_n(_p(f), f.size, _p(out))
    return out


def bf16_to_float(h) -> np.ndarray:
    """Exact widening (a bf16 pattern is the high half of a binary32 pattern)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---- quantize / dequantize -----------------------------------------------------------

def group_amax(x_bf16: np.ndarray) -> float:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1)
    return float(lib().kvfp4_oracle_group_amax(_p(x), x.size))


def quantize(x_bf16: np.ndarray, rows_per_group: int, rule="static_6"):
    """x_bf16: uint16 [rows, d].  Returns (codes u8 [rows, d/2], scales u8 [rows, d/16],
    group_amax f32 [ceil(rows/rows_per_group)])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, d = x.shape
    ng = -(-rows // rows_per_group) if rows else 0
    codes = np.zeros((rows, d // 2), dtype=np.uint8)
    scales = np.zeros((rows, d // 16), dtype=np.uint8)
    amax = np.zeros(ng, dtype=np.float32)
    rc = lib().kvfp4_oracle_quantize(_p(x), rows, d, rows_per_group, _rule(rule), _p(codes),
                                     _p(scales), _p(amax))
    if rc:
        raise ValueError("oracle quantize: bad arguments")
    return codes, scales, amax


def quantize_rows(x_bf16: np.ndarray, amax: float, rule="static_6"):
    """Quantize rows that belong to one group whose amax is already known."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, d = x.shape
    codes = np.zeros((rows, d // 2), dtype=np.uint8)
    scales = np.zeros((rows, d // 16), dtype=np.uint8)
    rc = lib().kvfp4_oracle_quantize_rows(_p(x), rows, d, float(amax), _rule(rule), _p(codes),
                                          _p(scales))
    if rc:
        raise ValueError("oracle quantize_rows: bad arguments")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, amax: np.ndarray,
               rows_per_group: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    rows, half = codes.shape
    d = half * 2
    y = np.zeros((rows, d), dtype=np.uint16)
    rc = lib().kvfp4_oracle_dequantize(_p(codes), _p(scales), _p(amax), rows, d, rows_per_group,
                                       _p(y))
    if rc:
        raise ValueError("oracle dequantize: bad arguments")
    return y


def dequantize_f32(codes: np.ndarray, scales: np.ndarray, amax: np.ndarray,
                   rows_per_group: int) -> np.ndarray:
    """Float32 output: the binary32 products before the bf16 rounding."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    rows, half = codes.shape
    d = half * 2
    y = np.zeros((rows, d), dtype=np.float32)
    rc = lib().kvfp4_oracle_dequantize_f32(_p(codes), _p(scales), _p(amax), rows, d,
                                           rows_per_group, _p(y))
    if rc:
        raise ValueError("oracle dequantize_f32: bad arguments")
    return y


def dequantize_rows_f32(codes: np.ndarray, scales: np.ndarray, amax: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    d = half * 2
    y = np.zeros((rows, d), dtype=np.float32)
    rc = lib().kvfp4_oracle_dequantize_rows_f32(_p(codes), _p(scales), rows, d, float(amax),
                                                _p(y))
    if rc:
        raise ValueError("oracle dequantize_rows_f32: bad arguments")
    return y


def fake_quantize(x_bf16: np.ndarray, rows_per_group: int, rule="static_6"):
    """Quantize then dequantize to bf16: (y u16 [rows, d], group_amax f32 [groups])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, d = x.shape
    ng = (rows + rows_per_group - 1) // rows_per_group
    y = np.zeros((rows, d), dtype=np.uint16)
    amax = np.zeros(ng, dtype=np.float32)
    rc = lib().kvfp4_oracle_fake_quantize(_p(x), rows, d, rows_per_group, _rule(rule), _p(amax),
                                          _p(y))
    if rc:
        raise ValueError("oracle fake_quantize: bad arguments")
    return y, amax


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, amax: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    d = half * 2
    y = np.zeros((rows, d), dtype=np.uint16)
    rc = lib().kvfp4_oracle_dequantize_rows(_p(codes), _p(scales), rows, d, float(amax), _p(y))
    if rc:
        raise ValueError("oracle dequantize_rows: bad arguments")
    return y


def quantize_paged(x_bf16: np.ndarray, table: np.ndarray, rows_per_page: int, n_pages: int,
                   rule="static_6", codes=None, scales=None, page_amax=None):
    """Dense x [n_blocks*rows_per_page, d] into pages named by table (int32 [n_blocks]).
    Pages not named keep the contents of the given (or zero) buffers."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    table = np.ascontiguousarray(table, dtype=np.int32)
    d = x.shape[1]
    if codes is None:
        codes = np.zeros((n_pages, rows_per_page, d // 2), np.uint8)
    if scales is None:
        scales = np.zeros((n_pages, rows_per_page, d // 16), np.uint8)
    if page_amax is None:
        page_amax = np.zeros(n_pages, np.float32)
    rc = lib().kvfp4_oracle_quantize_paged(_p(x), table.size, rows_per_page, d, _rule(rule),
                                           _p(table), n_pages, _p(codes), _p(scales),
                                           _p(page_amax))
    if rc:
        raise ValueError("oracle quantize_paged: bad arguments")
    return codes, scales, page_amax


def dequantize_paged(codes, scales, page_amax, table, rows_per_page: int, y=None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    page_amax = np.ascontiguousarray(page_amax, dtype=np.float32)
    table = np.ascontiguousarray(table, dtype=np.int32)
    d = codes.shape[-1] * 2
    if y is None:
        y = np.zeros((table.size * rows_per_page, d), np.uint16)
    rc = lib().kvfp4_oracle_dequantize_paged(_p(codes), _p(scales), _p(page_amax), _p(table),
                                             table.size, rows_per_page, d, page_amax.size, _p(y))
    if rc:
        raise ValueError("oracle dequantize_paged: bad arguments")
    return y


def dequantize_paged_f32(codes, scales, page_amax, table, rows_per_page: int, y=None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    page_amax = np.ascontiguousarray(page_amax, dtype=np.float32)
    table = np.ascontiguousarray(table, dtype=np.int32)
    d = codes.shape[-1] * 2
    if y is None:
        y = np.zeros((table.size * rows_per_page, d), np.float32)
    rc = lib().kvfp4_oracle_dequantize_paged_f32(_p(codes), _p(scales), _p(page_amax),
                                                 _p(table), table.size, rows_per_page, d,
                                                 page_amax.size, _p(y))
    if rc:
        raise ValueError("oracle dequantize_paged_f32: bad arguments")
    return y


def rtn_quantize(x_bf16: np.ndarray, bits: int):
    """Symmetric blockwise RTN: codes u8 [rows, d*bits/8], scales bf16 bits u16 [rows, d/16]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, d = x.shape
    codes = np.zeros((rows, d * bits // 8), np.uint8)
    scales = np.zeros((rows, d // 16), np.uint16)
    if lib().kvfp4_oracle_rtn_quantize(_p(x), rows, d, bits, _p(codes), _p(scales)):
        raise ValueError("oracle rtn_quantize: bad arguments")
    return codes, scales


def rtn_dequantize(codes: np.ndarray, scales: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    rows = codes.shape[0]
    d = codes.shape[1] * 8 // bits
    y = np.zeros((rows, d), np.uint16)
    if lib().kvfp4_oracle_rtn_dequantize(_p(codes), _p(scales), rows, d, bits, _p(y)):
        raise ValueError("oracle rtn_dequantize: bad arguments")
    return y


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                rows: np.ndarray) -> np.ndarray:
    """q [tq, H, d], k/v [tk, H, d] (bf16 as uint16).  rows: int64 indices token*H+head.
    Returns bf16 [len(rows), d]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    tk, heads, d = k.shape
    out = np.zeros((rows.size, d), dtype=np.uint16)
    scratch = np.zeros(tk, dtype=np.float64)
    rc = lib().kvfp4_oracle_attend_rows(_p(q), _p(k), _p(v), tk, heads, d, float(scale),
                                        _p(rows), rows.size, _p(out), _p(scratch))
    if rc:
        raise ValueError("oracle attend: bad arguments")
    return out
