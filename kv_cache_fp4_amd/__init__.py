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


FORMS = {"auto": 0, "three_kernel": 1, "one_kernel": 2}


class QuantizeOpts(ctypes.Structure):
    """struct kvfp4_quantize_opts: how a quantize call enqueues its work (never its bytes)."""
    _fields_ = [("form", ctypes.c_int32), ("wait_us", ctypes.c_int64)]


def quantize_opts(form="auto", wait_us: int = 20000) -> QuantizeOpts:
    """Options for the quantize calls: ``form`` "auto" (one kernel where it applies and the
    input is large enough for it to be faster), "one_kernel" (wherever it applies) or
    "three_kernel"; ``wait_us`` bounds the one-kernel form's wait for a group amax."""
    return QuantizeOpts(FORMS[form] if isinstance(form, str) else int(form), int(wait_us))


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
    O = ctypes.POINTER(QuantizeOpts)
    L.kvfp4_quantize_ex.argtypes = [P, i64, i32, i64, i32, P, P, P, O, P]
    L.kvfp4_quantize_ex.restype = ctypes.c_int
    L.kvfp4_quantize_paged_ex.argtypes = [P, i64, i64, i32, i32, P, i64, P, P, P, O, P]
    L.kvfp4_quantize_paged_ex.restype = ctypes.c_int
    L.kvfp4_fake_quantize_ex.argtypes = [P, i64, i32, i64, i32, P, P, O, P]
    L.kvfp4_fake_quantize_ex.restype = ctypes.c_int
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
    if isinstance(rule, str):
        if rule not in RULES:
            raise ValueError(f"kvfp4: unknown rule {rule!r} (one of {sorted(RULES)})")
        return RULES[rule]
    return int(rule)


# ---- argument checks (the C ABI sees bare pointers and sizes, so the binding checks every
# tensor's dtype, device, layout and element count before any C call) ------------------------

def _need(t, name, dtype, numel):
    """Check that tensor ``t`` is a contiguous ``dtype`` tensor with exactly ``numel``
    elements (``numel`` -1: any count); raise ValueError otherwise.  Devices are checked
    afterwards by ``_gpu``."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"kvfp4: {name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"kvfp4: {name} must be {dtype}, got {t.dtype}")
    if numel >= 0 and t.numel() != numel:
        raise ValueError(f"kvfp4: {name} has {t.numel()} elements, the call needs {numel}")
    if not t.is_contiguous():
        raise ValueError(f"kvfp4: {name} must be contiguous")
    return t


def _gpu(**tensors):
    """All the given tensors (None skipped) on one GPU; returns that device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"kvfp4: {name} must be on a GPU, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"kvfp4: {name} is on {t.device}, the call's other tensors on {dev}")
    return dev


def _head_dim(d, name):
    if d < 64 or d > 1024 or d % 64:
        raise ValueError(f"kvfp4: {name} gives head_dim {d}; it must be a multiple of 64 in "
                         "[64, 1024]")
    return d


def _groups(rows, rows_per_group):
    if rows_per_group <= 0:
        raise ValueError(f"kvfp4: rows_per_group must be > 0, got {rows_per_group}")
    return -(-rows // rows_per_group)


def _rows_of(x, name):
    """(rows, head_dim) of a tensor viewed as [..., head_dim]."""
    if x.dim() < 1:
        raise ValueError(f"kvfp4: {name} needs a head_dim axis")
    d = _head_dim(int(x.shape[-1]), name)
    return x.numel() // d, d


def _stream(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _opts(opts):
    if opts is None:
        return None
    if not isinstance(opts, QuantizeOpts):
        raise ValueError("kvfp4: opts must come from quantize_opts()")
    if opts.form not in FORMS.values() or not 0 <= opts.wait_us <= 60_000_000:
        raise ValueError(f"kvfp4: bad quantize options (form {opts.form}, wait_us {opts.wait_us})")
    return ctypes.byref(opts)


def kvfp4_packed_sizes(rows: int, head_dim: int, rows_per_group: int):
    """(codes_bytes, scales_bytes, n_groups) for a tensor of `rows` rows."""
    c, s, g = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.kvfp4_packed_sizes(rows, head_dim, rows_per_group, ctypes.byref(c),
                                  ctypes.byref(s), ctypes.byref(g)))
    return c.value, s.value, g.value


def kvfp4_quantize(x, rows_per_group: int, rule="static_6", codes=None, scales=None,
                   group_amax=None, stream=None, opts=None):
    """Quantize bf16 rows ``x`` [..., head_dim] (contiguous, on the GPU).

    Returns (codes uint8 [rows, head_dim/2], scales uint8 [rows, head_dim/16],
    group_amax float32 [n_groups]); outputs that are passed in are written in place
    (e.g. views into a cache at the appended chunk's rows).  ``opts`` (from
    ``quantize_opts``) selects the enqueue form; None = the defaults."""
    import torch
    r = _rule(rule)
    _need(x, "x", torch.bfloat16, x.numel() if isinstance(x, torch.Tensor) else -1)
    rows, d = _rows_of(x, "x")
    ng = _groups(rows, rows_per_group)
    for t, name, dt, n in ((codes, "codes", torch.uint8, rows * d // 2),
                           (scales, "scales", torch.uint8, rows * d // 16),
                           (group_amax, "group_amax", torch.float32, ng)):
        if t is not None:
            _need(t, name, dt, n)
    o = _opts(opts)
    dev = _gpu(x=x, codes=codes, scales=scales, group_amax=group_amax)
    if codes is None:
        codes = torch.empty((rows, d // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, d // 16), dtype=torch.uint8, device=dev)
    if group_amax is None:
        group_amax = torch.empty((ng,), dtype=torch.float32, device=dev)
    args = (x.data_ptr(), rows, d, rows_per_group, r, codes.data_ptr(), scales.data_ptr(),
            group_amax.data_ptr())
    if o is None:
        _check(lib.kvfp4_quantize(*args, _stream(stream, dev)))
    else:
        _check(lib.kvfp4_quantize_ex(*args, o, _stream(stream, dev)))
    return codes, scales, group_amax


def _packed_in(codes, scales, group_amax, rows_per_group, y, y_dtype):
    """Checks of a packed tensor given as codes [rows, head_dim/2] and of the output ``y``
    (if given); returns (rows, head_dim, device)."""
    import torch
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError("kvfp4: codes must be a 2-D tensor [rows, head_dim/2]")
    rows, d = int(codes.shape[0]), _head_dim(int(codes.shape[1]) * 2, "codes")
    ng = _groups(rows, rows_per_group)
    _need(codes, "codes", torch.uint8, rows * d // 2)
    _need(scales, "scales", torch.uint8, rows * d // 16)
    _need(group_amax, "group_amax", torch.float32, ng)
    if y is not None:
        _need(y, "y", y_dtype, rows * d)
    return rows, d, _gpu(codes=codes, scales=scales, group_amax=group_amax, y=y)


def kvfp4_dequantize(codes, scales, group_amax, rows_per_group: int, y=None, stream=None):
    """Dequantize a packed tensor to bf16 [rows, head_dim] (written into ``y`` if given)."""
    import torch
    rows, d, dev = _packed_in(codes, scales, group_amax, rows_per_group, y, torch.bfloat16)
    if y is None:
        y = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
    _check(lib.kvfp4_dequantize(codes.data_ptr(), scales.data_ptr(), group_amax.data_ptr(), rows,
                                d, rows_per_group, y.data_ptr(), _stream(stream, dev)))
    return y


def kvfp4_dequantize_f32(codes, scales, group_amax, rows_per_group: int, y=None, stream=None):
    """Dequantize a packed tensor to float32 [rows, head_dim] (the products before bf16
    rounding; written into ``y`` if given)."""
    import torch
    rows, d, dev = _packed_in(codes, scales, group_amax, rows_per_group, y, torch.float32)
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=dev)
    _check(lib.kvfp4_dequantize_f32(codes.data_ptr(), scales.data_ptr(), group_amax.data_ptr(),
                                    rows, d, rows_per_group, y.data_ptr(), _stream(stream, dev)))
    return y


def kvfp4_fake_quantize(x, rows_per_group: int, rule="static_6", y=None, group_amax=None,
                        stream=None, opts=None):
    """bf16 ``x`` [..., head_dim] -> (dequantize(quantize(x)) as bf16 [rows, head_dim],
    group_amax float32 [n_groups]) without a packed copy.  ``y`` may be ``x`` (in place)."""
    import torch
    r = _rule(rule)
    _need(x, "x", torch.bfloat16, x.numel() if isinstance(x, torch.Tensor) else -1)
    rows, d = _rows_of(x, "x")
    ng = _groups(rows, rows_per_group)
    if y is not None:
        _need(y, "y", torch.bfloat16, rows * d)
    if group_amax is not None:
        _need(group_amax, "group_amax", torch.float32, ng)
    o = _opts(opts)
    dev = _gpu(x=x, y=y, group_amax=group_amax)
    if y is None:
        y = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
    if group_amax is None:
        group_amax = torch.empty((ng,), dtype=torch.float32, device=dev)
    args = (x.data_ptr(), rows, d, rows_per_group, r, group_amax.data_ptr(), y.data_ptr())
    if o is None:
        _check(lib.kvfp4_fake_quantize(*args, _stream(stream, dev)))
    else:
        _check(lib.kvfp4_fake_quantize_ex(*args, o, _stream(stream, dev)))
    return y, group_amax


def _paged(codes, scales, page_amax, block_table, rows_per_page, dense=None, dense_name="y",
           dense_dtype=None):
    """Checks of a paged cache (codes [n_pages, rows_per_page, head_dim/2] ...), its block
    table and the dense side (if given); returns (n_blocks, n_pages, head_dim, device)."""
    import torch
    if rows_per_page <= 0:
        raise ValueError(f"kvfp4: rows_per_page must be > 0, got {rows_per_page}")
    for t, name in ((codes, "codes"), (page_amax, "page_amax"), (block_table, "block_table")):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"kvfp4: {name} must be a torch.Tensor")
    n_pages = page_amax.numel()
    d = _head_dim(int(codes.shape[-1]) * 2, "codes")
    _need(codes, "codes", torch.uint8, n_pages * rows_per_page * d // 2)
    _need(scales, "scales", torch.uint8, n_pages * rows_per_page * d // 16)
    _need(page_amax, "page_amax", torch.float32, n_pages)
    n_blocks = block_table.numel()
    _need(block_table, "block_table", torch.int32, n_blocks)
    if dense is not None:
        _need(dense, dense_name, dense_dtype, n_blocks * rows_per_page * d)
        if int(dense.shape[-1]) != d and dense.dim() > 1:
            raise ValueError(f"kvfp4: {dense_name} has head_dim {dense.shape[-1]}, the pages {d}")
    dev = _gpu(codes=codes, scales=scales, page_amax=page_amax, block_table=block_table,
               **{dense_name: dense})
    return n_blocks, n_pages, d, dev


def kvfp4_quantize_paged(x, block_table, rows_per_page: int, codes, scales, page_amax,
                         rule="static_6", stream=None, opts=None):
    """Quantize dense bf16 rows ``x`` [n_blocks*rows_per_page, head_dim] into the pages of a
    paged cache (codes [n_pages, rows_per_page, head_dim/2], scales [..., head_dim/16],
    page_amax [n_pages]) named by ``block_table`` (int32 [n_blocks], on the GPU)."""
    import torch
    r = _rule(rule)
    if x is None:
        raise ValueError("kvfp4: x must be a torch.Tensor")
    o = _opts(opts)
    n_blocks, n_pages, d, dev = _paged(codes, scales, page_amax, block_table, rows_per_page,
                                       x, "x", torch.bfloat16)
    args = (x.data_ptr(), n_blocks, rows_per_page, d, r, block_table.data_ptr(), n_pages,
            codes.data_ptr(), scales.data_ptr(), page_amax.data_ptr())
    if o is None:
        _check(lib.kvfp4_quantize_paged(*args, _stream(stream, dev)))
    else:
        _check(lib.kvfp4_quantize_paged_ex(*args, o, _stream(stream, dev)))
    return codes, scales, page_amax


def kvfp4_dequantize_paged(codes, scales, page_amax, block_table, rows_per_page: int, y=None,
                           stream=None):
    """Gather the pages named by ``block_table`` into dense bf16 [n_blocks*rows_per_page,
    head_dim]."""
    import torch
    n_blocks, n_pages, d, dev = _paged(codes, scales, page_amax, block_table, rows_per_page,
                                       y, "y", torch.bfloat16)
    if y is None:
        y = torch.empty((n_blocks * rows_per_page, d), dtype=torch.bfloat16, device=dev)
    _check(lib.kvfp4_dequantize_paged(codes.data_ptr(), scales.data_ptr(), page_amax.data_ptr(),
                                      block_table.data_ptr(), n_blocks, rows_per_page, d, n_pages,
                                      y.data_ptr(), _stream(stream, dev)))
    return y


def kvfp4_dequantize_paged_f32(codes, scales, page_amax, block_table, rows_per_page: int,
                               y=None, stream=None):
    """As kvfp4_dequantize_paged, with float32 output."""
    import torch
    n_blocks, n_pages, d, dev = _paged(codes, scales, page_amax, block_table, rows_per_page,
                                       y, "y", torch.float32)
    if y is None:
        y = torch.empty((n_blocks * rows_per_page, d), dtype=torch.float32, device=dev)
    _check(lib.kvfp4_dequantize_paged_f32(codes.data_ptr(), scales.data_ptr(),
                                          page_amax.data_ptr(), block_table.data_ptr(), n_blocks,
                                          rows_per_page, d, n_pages, y.data_ptr(),
                                          _stream(stream, dev)))
    return y


def _bits(bits):
    if bits not in (2, 4):
        raise ValueError(f"kvfp4: bits must be 2 or 4, got {bits}")
    return int(bits)


def kvfp4_rtn_quantize(x, bits: int, codes=None, scales=None, stream=None):
    """Symmetric blockwise RTN of bf16 rows ``x`` [..., head_dim]: returns (codes uint8
    [rows, head_dim*bits/8], scales bf16 [rows, head_dim/16])."""
    import torch
    b = _bits(bits)
    _need(x, "x", torch.bfloat16, x.numel() if isinstance(x, torch.Tensor) else -1)
    rows, d = _rows_of(x, "x")
    if codes is not None:
        _need(codes, "codes", torch.uint8, rows * d * b // 8)
    if scales is not None:
        _need(scales, "scales", torch.bfloat16, rows * d // 16)
    dev = _gpu(x=x, codes=codes, scales=scales)
    if codes is None:
        codes = torch.empty((rows, d * b // 8), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, d // 16), dtype=torch.bfloat16, device=dev)
    _check(lib.kvfp4_rtn_quantize(x.data_ptr(), rows, d, b, codes.data_ptr(), scales.data_ptr(),
                                  _stream(stream, dev)))
    return codes, scales


def kvfp4_rtn_dequantize(codes, scales, bits: int, tail=None, y=None, stream=None):
    """bf16 [rows + tail_rows, head_dim]: the dequantized rows followed by ``tail`` (bf16
    [tail_rows, head_dim], the recent rows kept unquantized)."""
    import torch
    b = _bits(bits)
    if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
        raise ValueError("kvfp4: scales must be a 2-D tensor [rows, head_dim/16]")
    rows, d = int(scales.shape[0]), _head_dim(int(scales.shape[1]) * 16, "scales")
    _need(scales, "scales", torch.bfloat16, rows * d // 16)
    _need(codes, "codes", torch.uint8, rows * d * b // 8)
    tail_rows = 0
    if tail is not None:
        if not isinstance(tail, torch.Tensor) or tail.numel() % d:
            raise ValueError(f"kvfp4: tail must hold whole rows of {d} elements")
        tail_rows = tail.numel() // d
        _need(tail, "tail", torch.bfloat16, tail_rows * d)
    if y is not None:
        _need(y, "y", torch.bfloat16, (rows + tail_rows) * d)
    dev = _gpu(scales=scales, codes=codes, tail=tail, y=y)
    if y is None:
        y = torch.empty((rows + tail_rows, d), dtype=torch.bfloat16, device=dev)
    _check(lib.kvfp4_rtn_dequantize(codes.data_ptr(), scales.data_ptr(), rows, d, b,
                                    tail.data_ptr() if tail is not None else 0, tail_rows,
                                    y.data_ptr(), _stream(stream, dev)))
    return y


def kvfp4_attend(q, k_codes, k_scales, k_amax, v_codes, v_scales, v_amax,
                 tokens_per_group: int, softmax_scale=None, out=None, stream=None):
    """Attention of bf16 ``q`` [q_tokens, heads, head_dim] over a packed K/V cache
    (codes [kv_tokens*heads, head_dim/2], scales [kv_tokens*heads, head_dim/16], one amax per
    ``tokens_per_group`` tokens), dequantized on chip.  Returns bf16 [q_tokens, heads, head_dim]."""
    import math

    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("kvfp4: q must be a 3-D tensor [q_tokens, heads, head_dim]")
    q_tokens, heads, d = (int(v) for v in q.shape)
    if d not in (64, 128):
        raise ValueError(f"kvfp4: attention supports head_dim 64 or 128, got {d}")
    if heads <= 0:
        raise ValueError("kvfp4: q has no heads")
    if tokens_per_group <= 0:
        raise ValueError(f"kvfp4: tokens_per_group must be > 0, got {tokens_per_group}")
    _need(q, "q", torch.bfloat16, q_tokens * heads * d)
    if not isinstance(k_codes, torch.Tensor) or k_codes.numel() % (heads * d // 2):
        raise ValueError("kvfp4: k_codes must hold whole [heads, head_dim/2] token rows")
    kv_tokens = k_codes.numel() // (heads * d // 2)
    ng = -(-kv_tokens // tokens_per_group)
    _need(k_codes, "k_codes", torch.uint8, kv_tokens * heads * d // 2)
    _need(v_codes, "v_codes", torch.uint8, kv_tokens * heads * d // 2)
    _need(k_scales, "k_scales", torch.uint8, kv_tokens * heads * d // 16)
    _need(v_scales, "v_scales", torch.uint8, kv_tokens * heads * d // 16)
    _need(k_amax, "k_amax", torch.float32, ng)
    _need(v_amax, "v_amax", torch.float32, ng)
    if out is not None:
        _need(out, "out", torch.bfloat16, q_tokens * heads * d)
    dev = _gpu(q=q, k_codes=k_codes, k_scales=k_scales, k_amax=k_amax, v_codes=v_codes,
               v_scales=v_scales, v_amax=v_amax, out=out)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((q_tokens, heads, d), dtype=torch.bfloat16, device=dev)
    _check(lib.kvfp4_attend(q.data_ptr(), q_tokens, k_codes.data_ptr(), k_scales.data_ptr(),
                            k_amax.data_ptr(), v_codes.data_ptr(), v_scales.data_ptr(),
                            v_amax.data_ptr(), kv_tokens, heads, d, tokens_per_group,
                            float(softmax_scale), out.data_ptr(), _stream(stream, dev)))
    return out


__all__ = ["kvfp4_quantize", "kvfp4_dequantize", "kvfp4_dequantize_f32", "kvfp4_fake_quantize",
           "kvfp4_quantize_paged", "kvfp4_dequantize_paged", "kvfp4_dequantize_paged_f32",
           "kvfp4_rtn_quantize", "kvfp4_rtn_dequantize", "kvfp4_attend", "kvfp4_packed_sizes",
           "quantize_opts", "QuantizeOpts", "KVFP4Error", "RULES", "FORMS", "lib", "LIB_PATH"]
