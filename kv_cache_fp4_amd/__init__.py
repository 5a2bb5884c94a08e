"""kv_cache_fp4_amd -- NVFP4 KV-cache compression for MI355X (gfx950).

Thin Python binding over the C ABI of ``libkvfp4.so`` (declared in ``include/kvfp4.h``).
The functions below have the same names as the C entry points and only marshal
arguments: tensor pointers, sizes and the caller's HIP stream.  torch supplies device
memory and streams; every step of the computation runs in the HIP kernels.  There is no
fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (libamdhip64.so.7 with an $ORIGIN rpath).  Importing it
# first makes this library bind to that same runtime instead of loading a second copy from
# /opt/rocm, which would give the process two HIP runtimes with separate device contexts.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvfp4.so")

RULES = {"static_6": 0, "static_4": 1, "mse": 2}

KVFP4_OK, KVFP4_EINVAL, KVFP4_EALIGN, KVFP4_EUNSUPPORTED, KVFP4_EHIP = range(5)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libkvfp4.so not found at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.kvfp4_quantize.argtypes = [P, i64, i32, i64, i32, P, P, P, P]
    L.kvfp4_quantize.restype = ctypes.c_int
    L.kvfp4_dequantize.argtypes = [P, P, P, i64, i32, i64, P, P]
    L.kvfp4_dequantize.restype = ctypes.c_int
    L.kvfp4_quantize_paged.argtypes = [P, i64, i64, i32, i32, P, i64, P, P, P, P]
    L.kvfp4_quantize_paged.restype = ctypes.c_int
    L.kvfp4_dequantize_paged.argtypes = [P, P, P, P, i64, i64, i32, i64, P, P]
    L.kvfp4_dequantize_paged.restype = ctypes.c_int
    L.kvfp4_dequantize_f32.argtypes = [P, P, P, i64, i32, i64, P, P]
    L.kvfp4_dequantize_f32.restype = ctypes.c_int
    L.kvfp4_dequantize_paged_f32.argtypes = [P, P, P, P, i64, i64, i32, i64, P, P]
    L.kvfp4_dequantize_paged_f32.restype = ctypes.c_int
    L.kvfp4_fake_quantize.argtypes = [P, i64, i32, i64, i32, P, P, P]
    L.kvfp4_fake_quantize.restype = ctypes.c_int
    L.kvfp4_rtn_quantize.argtypes = [P, i64, i32, i32, P, P, P]
    L.kvfp4_rtn_quantize.restype = ctypes.c_int
    L.kvfp4_rtn_dequantize.argtypes = [P, P, i64, i32, i32, P, i64, P, P]
    L.kvfp4_rtn_dequantize.restype = ctypes.c_int
    L.kvfp4_attend.argtypes = [P, i64, P, P, P, P, P, P, i64, i32, i32, i64, ctypes.c_float, P, P]
    L.kvfp4_attend.restype = ctypes.c_int
    L.kvfp4_packed_sizes.argtypes = [i64, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
    L.kvfp4_packed_sizes.restype = ctypes.c_int
    L.kvfp4_status_str.argtypes = [ctypes.c_int]
    L.kvfp4_status_str.restype = ctypes.c_char_p
    L.kvfp4_abi_version.argtypes = []
    L.kvfp4_abi_version.restype = ctypes.c_int
    L.kvfp4_last_hip_error.argtypes = []
    L.kvfp4_last_hip_error.restype = ctypes.c_int
    L.kvfp4_set_option.argtypes = [i32, i64]
    L.kvfp4_set_option.restype = ctypes.c_int
    L.kvfp4_get_option.argtypes = [i32, ctypes.POINTER(i64)]
    L.kvfp4_get_option.restype = ctypes.c_int
    return L


lib = _load()


class KVFP4Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = lib.kvfp4_status_str(status).decode()
        if status == KVFP4_EHIP:
            msg += f" (hipError {lib.kvfp4_last_hip_error()})"
        super().__init__(msg)


def _check(rc: int) -> None:
    if rc != KVFP4_OK:
        raise KVFP4Error(rc)


def _rule(rule) -> int:
    return RULES[rule] if isinstance(rule, str) else int(rule)


def _ptr(t) -> int:
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("kvfp4: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def kvfp4_packed_sizes(rows: int, head_dim: int, rows_per_group: int):
    """(codes_bytes, scales_bytes, n_groups) for a tensor of `rows` rows."""
    c, s, g = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.kvfp4_packed_sizes(rows, head_dim, rows_per_group, ctypes.byref(c),
                                  ctypes.byref(s), ctypes.byref(g)))
    return c.value, s.value, g.value


OPTIONS = {"append_fused": 1, "append_wait_us": 2}


def kvfp4_set_option(name, value: int) -> None:
    """Set a process-wide option ("append_fused" 0/1, "append_wait_us" >= 0)."""
    _check(lib.kvfp4_set_option(OPTIONS[name] if isinstance(name, str) else int(name), int(value)))


def kvfp4_get_option(name) -> int:
    v = ctypes.c_int64()
    _check(lib.kvfp4_get_option(OPTIONS[name] if isinstance(name, str) else int(name),
                                ctypes.byref(v)))
    return v.value


def kvfp4_quantize(x, rows_per_group: int, rule="static_6", codes=None, scales=None,
                   group_amax=None, stream=None):
    """Quantize bf16 rows ``x`` [..., head_dim] (contiguous, on the GPU).

    Returns (codes uint8 [rows, head_dim/2], scales uint8 [rows, head_dim/16],
    group_amax float32 [n_groups]); outputs that are passed in are written in place
    (e.g. views into a cache at the appended chunk's rows)."""
    import torch
    head_dim = x.shape[-1]
    rows = x.numel() // head_dim if head_dim else 0
    cb, sb, ng = kvfp4_packed_sizes(rows, head_dim, rows_per_group)
    if codes is None:
        codes = torch.empty((rows, head_dim // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, head_dim // 16), dtype=torch.uint8, device=x.device)
    if group_amax is None:
        group_amax = torch.empty((ng,), dtype=torch.float32, device=x.device)
    _check(lib.kvfp4_quantize(_ptr(x), rows, head_dim, rows_per_group, _rule(rule), _ptr(codes),
                              _ptr(scales), _ptr(group_amax), _stream(stream, x.device)))
    return codes, scales, group_amax


def kvfp4_dequantize(codes, scales, group_amax, rows_per_group: int, y=None, stream=None):
    """Dequantize a packed tensor to bf16 [rows, head_dim] (written into ``y`` if given)."""
    import torch
    rows = codes.shape[0]
    head_dim = codes.shape[1] * 2 if codes.dim() == 2 else 0
    if y is None:
        y = torch.empty((rows, head_dim), dtype=torch.bfloat16, device=codes.device)
    _check(lib.kvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(group_amax), rows, head_dim,
                                rows_per_group, _ptr(y), _stream(stream, codes.device)))
    return y


def kvfp4_dequantize_f32(codes, scales, group_amax, rows_per_group: int, y=None, stream=None):
    """Dequantize a packed tensor to float32 [rows, head_dim] (the products before bf16
    rounding; written into ``y`` if given)."""
    import torch
    rows = codes.shape[0]
    head_dim = codes.shape[1] * 2 if codes.dim() == 2 else 0
    if y is None:
        y = torch.empty((rows, head_dim), dtype=torch.float32, device=codes.device)
    _check(lib.kvfp4_dequantize_f32(_ptr(codes), _ptr(scales), _ptr(group_amax), rows, head_dim,
                                    rows_per_group, _ptr(y), _stream(stream, codes.device)))
    return y


def kvfp4_fake_quantize(x, rows_per_group: int, rule="static_6", y=None, group_amax=None,
                        stream=None):
    """bf16 ``x`` [..., head_dim] -> (dequantize(quantize(x)) as bf16 [rows, head_dim],
    group_amax float32 [n_groups]) without a packed copy.  ``y`` may be ``x`` (in place)."""
    import torch
    head_dim = x.shape[-1]
    rows = x.numel() // head_dim if head_dim else 0
    _, _, ng = kvfp4_packed_sizes(rows, head_dim, rows_per_group)
    if y is None:
        y = torch.empty((rows, head_dim), dtype=torch.bfloat16, device=x.device)
    if group_amax is None:
        group_amax = torch.empty((ng,), dtype=torch.float32, device=x.device)
    _check(lib.kvfp4_fake_quantize(_ptr(x), rows, head_dim, rows_per_group, _rule(rule),
                                   _ptr(group_amax), _ptr(y), _stream(stream, x.device)))
    return y, group_amax


def kvfp4_quantize_paged(x, block_table, rows_per_page: int, codes, scales, page_amax,
                         rule="static_6", stream=None):
    """Quantize dense bf16 rows ``x`` [n_blocks*rows_per_page, head_dim] into the pages of a
    paged cache (codes [n_pages, rows_per_page, head_dim/2], scales [..., head_dim/16],
    page_amax [n_pages]) named by ``block_table`` (int32 [n_blocks], on the GPU)."""
    head_dim = x.shape[-1]
    n_blocks = block_table.numel()
    n_pages = page_amax.numel()
    _check(lib.kvfp4_quantize_paged(_ptr(x), n_blocks, rows_per_page, head_dim, _rule(rule),
                                    _ptr(block_table), n_pages, _ptr(codes), _ptr(scales),
                                    _ptr(page_amax), _stream(stream, x.device)))
    return codes, scales, page_amax


def kvfp4_dequantize_paged(codes, scales, page_amax, block_table, rows_per_page: int, y=None,
                           stream=None):
    """Gather the pages named by ``block_table`` into dense bf16 [n_blocks*rows_per_page,
    head_dim]."""
    import torch
    head_dim = codes.shape[-1] * 2
    n_blocks = block_table.numel()
    n_pages = page_amax.numel()
    if y is None:
        y = torch.empty((n_blocks * rows_per_page, head_dim), dtype=torch.bfloat16,
                        device=codes.device)
    _check(lib.kvfp4_dequantize_paged(_ptr(codes), _ptr(scales), _ptr(page_amax),
                                      _ptr(block_table), n_blocks, rows_per_page, head_dim,
                                      n_pages, _ptr(y), _stream(stream, codes.device)))
    return y


def kvfp4_dequantize_paged_f32(codes, scales, page_amax, block_table, rows_per_page: int,
                               y=None, stream=None):
    """As kvfp4_dequantize_paged, with float32 output."""
    import torch
    head_dim = codes.shape[-1] * 2
    n_blocks = block_table.numel()
    n_pages = page_amax.numel()
    if y is None:
        y = torch.empty((n_blocks * rows_per_page, head_dim), dtype=torch.float32,
                        device=codes.device)
    _check(lib.kvfp4_dequantize_paged_f32(_ptr(codes), _ptr(scales), _ptr(page_amax),
                                          _ptr(block_table), n_blocks, rows_per_page, head_dim,
                                          n_pages, _ptr(y), _stream(stream, codes.device)))
    return y


def kvfp4_rtn_quantize(x, bits: int, codes=None, scales=None, stream=None):
    """Symmetric blockwise RTN of bf16 rows ``x`` [..., head_dim]: returns (codes uint8
    [rows, head_dim*bits/8], scales bf16 [rows, head_dim/16])."""
    import torch
    head_dim = x.shape[-1]
    rows = x.numel() // head_dim if head_dim else 0
    if codes is None:
        codes = torch.empty((rows, head_dim * bits // 8), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, head_dim // 16), dtype=torch.bfloat16, device=x.device)
    _check(lib.kvfp4_rtn_quantize(_ptr(x), rows, head_dim, int(bits), _ptr(codes), _ptr(scales),
                                  _stream(stream, x.device)))
    return codes, scales


def kvfp4_rtn_dequantize(codes, scales, bits: int, tail=None, y=None, stream=None):
    """bf16 [rows + tail_rows, head_dim]: the dequantized rows followed by ``tail`` (bf16
    [tail_rows, head_dim], the recent rows kept unquantized)."""
    import torch
    rows = codes.shape[0]
    head_dim = scales.shape[1] * 16
    tail_rows = 0 if tail is None else tail.numel() // head_dim
    if y is None:
        y = torch.empty((rows + tail_rows, head_dim), dtype=torch.bfloat16, device=codes.device)
    _check(lib.kvfp4_rtn_dequantize(_ptr(codes), _ptr(scales), rows, head_dim, int(bits),
                                    _ptr(tail), tail_rows, _ptr(y), _stream(stream, codes.device)))
    return y


def kvfp4_attend(q, k_codes, k_scales, k_amax, v_codes, v_scales, v_amax,
                 tokens_per_group: int, softmax_scale=None, out=None, stream=None):
    """Attention of bf16 ``q`` [q_tokens, heads, head_dim] over a packed K/V cache
    (codes [kv_tokens*heads, head_dim/2], scales [kv_tokens*heads, head_dim/16], one amax per
    ``tokens_per_group`` tokens), dequantized on chip.  Returns bf16 [q_tokens, heads, head_dim]."""
    import math

    import torch
    q_tokens, heads, head_dim = q.shape
    kv_tokens = k_codes.numel() * 2 // (heads * head_dim) if heads * head_dim else 0
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    if out is None:
        out = torch.empty((q_tokens, heads, head_dim), dtype=torch.bfloat16, device=q.device)
    _check(lib.kvfp4_attend(_ptr(q), q_tokens, _ptr(k_codes), _ptr(k_scales), _ptr(k_amax),
                            _ptr(v_codes), _ptr(v_scales), _ptr(v_amax), kv_tokens, heads,
                            head_dim, tokens_per_group, float(softmax_scale), _ptr(out),
                            _stream(stream, q.device)))
    return out


__all__ = ["kvfp4_quantize", "kvfp4_dequantize", "kvfp4_dequantize_f32", "kvfp4_fake_quantize",
           "kvfp4_quantize_paged", "kvfp4_dequantize_paged", "kvfp4_dequantize_paged_f32",
           "kvfp4_rtn_quantize", "kvfp4_rtn_dequantize", "kvfp4_attend", "kvfp4_packed_sizes",
           "kvfp4_set_option", "kvfp4_get_option", "KVFP4Error", "RULES", "OPTIONS", "lib",
           "LIB_PATH"]
