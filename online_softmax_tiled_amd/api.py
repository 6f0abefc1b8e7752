"""Thin Python binding over libattn.so (ctypes).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch when the caller passes none,
and raw device pointers plus torch's current HIP stream are handed to the
C ABI declared in include/attn.h. Every step of the computation runs in the
library's HIP kernels; there is no fallback. If the library is missing or
fails to load, every call raises.
"""

import contextlib
import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")
# The bounds-checking debug build of the same sources (see checked_library).
CHECKED_LIB_PATH = os.path.join(_HERE, "libattn_checked.so")

DTYPE_CODES = {torch.float16: 0, torch.bfloat16: 1}
HEAD_DIM = 128

_c_int, _c_float, _c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_SIGNATURES = {
    "attn_prefill_fwd": [_c_void_p] * 7 + [_c_int] * 7 + [_c_float, _c_int, _c_void_p],
    "attn_prefill_paged": [_c_void_p, _c_void_p, _c_int] + [_c_void_p] * 5 + [_c_int] * 8 + [_c_float, _c_int]
                          + [_c_void_p] * 3,
    "attn_decode_plan": [_c_int, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p],
    "attn_decode_plan_fixed": [_c_int, _c_void_p, _c_int, _c_void_p, _c_void_p],
    "attn_decode_split": [_c_void_p] * 4 + [_c_int] * 3 + [_c_void_p] + [_c_int] * 8 + [_c_float]
                         + [_c_void_p] * 4,
    "attn_merge_states": [_c_void_p] * 4 + [_c_int] * 5 + [_c_void_p, _c_void_p, _c_int, _c_void_p],
    "attn_decode": [_c_void_p] * 4 + [_c_int] * 3 + [_c_void_p] + [_c_int] * 8 + [_c_float] + [_c_void_p] * 6,
    "attn_decode_noalloc": [_c_void_p] * 4 + [_c_int] * 3 + [_c_void_p] + [_c_int] * 8 + [_c_float] + [_c_void_p] * 3,
    "attn_decode_split_fp8kv": [_c_void_p] * 4 + [_c_int] * 3 + [_c_void_p] + [_c_int] * 8 + [_c_float] * 3
                               + [_c_void_p] * 4,
    "attn_decode_fp8kv": [_c_void_p] * 4 + [_c_int] * 3 + [_c_void_p] + [_c_int] * 8 + [_c_float] * 3
                         + [_c_void_p] * 6,
    "attn_merge_lse": [_c_void_p] * 4 + [_c_int] * 2 + [_c_void_p, _c_void_p, _c_int, _c_void_p],
    "attn_paged_gather": [_c_void_p] * 3 + [_c_int] * 8 + [_c_void_p, _c_void_p],
    "attn_stream_read": [_c_void_p, ctypes.c_uint64, _c_int, _c_void_p, _c_void_p],
    "attn_check_report": [_c_void_p, _c_int],
    "attn_check_clear": [],
    "attn_check_selftest": [_c_void_p, _c_void_p],
    "attn_last_error": [],
    "attn_version": [],
}
EXPORTS = tuple(_SIGNATURES)
CHECK_SITES = 64   # ATTN_CHECK_SITES

_lib = None
_checked_lib = None
_active = None     # a library that load() returns instead (checked_library)


class AttnError(RuntimeError):
    """A libattn call returned an error code."""

    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m online_softmax_tiled_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("attn_last_error", "attn_version") else ctypes.c_int
    return lib


def load():
    """Load libattn.so once. torch is imported first so that the library's
    HIP runtime dependency (libamdhip64.so.7) binds to the copy torch already
    loaded: one runtime per process, so torch's streams are valid here.
    Inside ``checked_library()`` the debug library is returned instead."""
    global _lib
    if _active is not None:
        return _active
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def checked_library():
    """Route every call made in the block to libattn_checked.so, the build
    whose kernels test each raw global access against its tensor's extent
    (include/attn.h, attn_check_report). A test aid: the product library is
    used again after the block."""
    global _checked_lib, _active
    if _checked_lib is None:
        _checked_lib = _open(CHECKED_LIB_PATH)
    prev, _active = _active, _checked_lib
    try:
        yield _checked_lib
    finally:
        _active = prev


def check_clear():
    """Clear the access-check flags (checked library)."""
    _check("attn_check_clear", load().attn_check_clear())


def check_report():
    """Sites whose access checks failed since the last clear (checked
    library; the device is synchronised first)."""
    torch.cuda.synchronize()
    hits = (ctypes.c_uint32 * CHECK_SITES)()
    _check("attn_check_report", load().attn_check_report(ctypes.cast(hits, _c_void_p), CHECK_SITES))
    return [i for i in range(CHECK_SITES) if hits[i]]


def check_selftest(base):
    """Launch the checker's self-test on a device tensor's address."""
    _check("attn_check_selftest", load().attn_check_selftest(_ptr(base), _stream(base.device)))


def version():
    return load().attn_version().decode()


def last_error():
    return load().attn_last_error().decode()


def _check(name, code):
    if code != 0:
        raise AttnError(name, code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _want(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(t):
    if t.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {t.dtype} (float16 or bfloat16)")
    return DTYPE_CODES[t.dtype]


def prefill(q, k, v, causal=True, scale=None, key_mask=None, row_mask=None, out=None, lse=None,
            return_lse=True):
    """O = attention(q, k, v) and its per-row LSE via attn_prefill_fwd.

    q [B, h, T_q, 128], k/v [B, h_kv, T_k, 128] (fp16 or bf16); key_mask
    [B, T_k] and row_mask [B, T_q] optional uint8 (see include/attn.h)."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    B, h, T_q, d = q.shape
    h_kv, T_k = k.shape[1], k.shape[2]
    _want(k, "k", dt, (B, h_kv, T_k, d), dev)
    _want(v, "v", dt, (B, h_kv, T_k, d), dev)
    if key_mask is not None:
        _want(key_mask, "key_mask", torch.uint8, (B, T_k), dev)
    if row_mask is not None:
        _want(row_mask, "row_mask", torch.uint8, (B, T_q), dev)
    out = torch.empty_like(q) if out is None else _want(out, "out", dt, q.shape, dev)
    if return_lse and lse is None:
        lse = torch.empty((B, h, T_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _want(lse, "lse", torch.float32, (B, h, T_q), dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_prefill_fwd", lib.attn_prefill_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(key_mask), _ptr(row_mask), _ptr(out), _ptr(lse),
        B, h, h_kv, T_q, T_k, d, _dtype_code(q), scale, 1 if causal else 0, _stream(dev)))
    return out, lse


def prefill_paged(q, cu_seqlens_q, max_q, k_pool, v_pool, block_table, seq_lens_k, causal=True, scale=None,
                  out=None, lse=None, seq_lens_k_host=None):
    """Variable-length prefill against a paged KV cache via attn_prefill_paged.

    q [total_q, h, 128] token-major, cu_seqlens_q [B+1] int32 (device),
    max_q >= every sequence's query count (host int), pools
    [num_pages, page_size, h_kv, 128], block_table [B, max_pages] int32,
    seq_lens_k [B] int32. ``seq_lens_k_host`` (optional, host ints) lets the
    library launch the longest contexts first. Returns (o [total_q, h, 128],
    lse [total_q, h])."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    total_q, h, d = q.shape
    _want(k_pool, "k_pool", dt, None, dev)
    num_pages, page_size, h_kv, _ = k_pool.shape
    _want(v_pool, "v_pool", dt, tuple(k_pool.shape), dev)
    _want(block_table, "block_table", torch.int32, None, dev)
    B, max_pages = block_table.shape
    _want(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,), dev)
    _want(seq_lens_k, "seq_lens_k", torch.int32, (B,), dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    _want(out, "out", dt, tuple(q.shape), dev)
    lse = torch.empty((total_q, h), dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, (total_q, h), dev)
    host = None
    if seq_lens_k_host is not None:
        host = np.ascontiguousarray(np.asarray(seq_lens_k_host, dtype=np.int32))
        if host.shape != (B,):
            raise ValueError(f"seq_lens_k_host has shape {host.shape}, expected ({B},)")
    _check("attn_prefill_paged", lib.attn_prefill_paged(
        _ptr(q), _ptr(cu_seqlens_q), int(max_q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(seq_lens_k), None if host is None else host.ctypes.data_as(_c_void_p), B, h, h_kv, d, page_size,
        max_pages, num_pages, _dtype_code(q), float(scale),
        int(bool(causal)), _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def decode_plan(seq_lens, h, h_kv, num_cus=None, d=HEAD_DIM, device=None):
    """(chunk_keys, max_splits) from attn_decode_plan. seq_lens: host ints."""
    lib = load()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(device or 0).multi_processor_count
    chunk, splits = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("attn_decode_plan", lib.attn_decode_plan(
        int(lens.size), lens.ctypes.data_as(ctypes.c_void_p), h, h_kv, d, int(num_cus),
        ctypes.byref(chunk), ctypes.byref(splits)))
    return chunk.value, splits.value


def decode_plan_fixed(seq_lens, split_keys=2048):
    """(chunk_keys, max_splits) from attn_decode_plan_fixed: a split length
    that does not depend on the batch, so each sequence's output bits depend
    only on its own query, keys and ``split_keys`` (batch-invariant decode).
    seq_lens: host ints; ``split_keys`` a positive multiple of 16."""
    lib = load()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    chunk, splits = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("attn_decode_plan_fixed", lib.attn_decode_plan_fixed(
        int(lens.size), lens.ctypes.data_as(ctypes.c_void_p), int(split_keys),
        ctypes.byref(chunk), ctypes.byref(splits)))
    return chunk.value, splits.value


def decode_split(q, k, v, seq_lens, chunk_keys, max_splits, block_table=None, page_size=16,
                 scale=None, part_o=None, part_m=None, part_l=None):
    """Stage 1 of split-KV decode via attn_decode_split.

    q [B, h, 128]; contiguous k/v [B, h_kv, s_max, 128] when block_table is
    None, else pools [num_pages, page_size, h_kv, 128] with block_table
    [B, max_pages] int32. seq_lens: int32 device tensor [B].
    Returns (part_o [B,h,S,128], part_m [B,h,S], part_l [B,h,S]) fp32."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    B, h, d = q.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if block_table is None:
        h_kv, s_max = k.shape[1], k.shape[2]
        _want(k, "k", dt, (B, h_kv, s_max, d), dev)
        _want(v, "v", dt, (B, h_kv, s_max, d), dev)
        max_pages, num_pages = 0, 0
    else:
        num_pages, page_size, h_kv = k.shape[0], k.shape[1], k.shape[2]
        _want(k, "k_pool", dt, (num_pages, page_size, h_kv, d), dev)
        _want(v, "v_pool", dt, (num_pages, page_size, h_kv, d), dev)
        _want(block_table, "block_table", torch.int32, None, dev)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        max_pages, s_max = block_table.shape[1], 0
    shp = (B, h, max_splits)
    part_o = torch.empty(shp + (d,), dtype=torch.float32, device=dev) if part_o is None else part_o
    part_m = torch.empty(shp, dtype=torch.float32, device=dev) if part_m is None else part_m
    part_l = torch.empty(shp, dtype=torch.float32, device=dev) if part_l is None else part_l
    _want(part_o, "part_o", torch.float32, shp + (d,), dev)
    _want(part_m, "part_m", torch.float32, shp, dev)
    _want(part_l, "part_l", torch.float32, shp, dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_decode_split", lib.attn_decode_split(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), max_pages, page_size, num_pages,
        _ptr(seq_lens), s_max, B, h, h_kv, d, int(chunk_keys), int(max_splits), _dtype_code(q),
        scale, _ptr(part_o), _ptr(part_m), _ptr(part_l), _stream(dev)))
    return part_o, part_m, part_l


def merge_states(part_o, part_m, part_l, seq_lens, chunk_keys, dtype, out=None, lse=None):
    """Stage 2 of split-KV decode via attn_merge_states -> (o [B,h,128], lse [B,h])."""
    lib = load()
    _want(part_o, "part_o", torch.float32)
    dev = part_o.device
    B, h, S, d = part_o.shape
    _want(part_m, "part_m", torch.float32, (B, h, S), dev)
    _want(part_l, "part_l", torch.float32, (B, h, S), dev)
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    out = torch.empty((B, h, d), dtype=dtype, device=dev) if out is None else out
    _want(out, "out", dtype, (B, h, d), dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, (B, h), dev)
    _check("attn_merge_states", lib.attn_merge_states(
        _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(seq_lens), int(chunk_keys), B, h, S, d,
        _ptr(out), _ptr(lse), _dtype_code(out), _stream(dev)))
    return out, lse


def _kv_geometry(q, k, v, block_table, page_size, kv_dtype=None):
    """(h_kv, s_max, max_pages, num_pages, page_size) of contiguous or paged K/V, checked
    (K/V elements of q's dtype, or of ``kv_dtype``)."""
    dev = q.device
    dt = q.dtype if kv_dtype is None else kv_dtype
    B, h, d = q.shape
    if block_table is None:
        h_kv, s_max = k.shape[1], k.shape[2]
        _want(k, "k", dt, (B, h_kv, s_max, d), dev)
        _want(v, "v", dt, (B, h_kv, s_max, d), dev)
        return h_kv, s_max, 0, 0, page_size
    num_pages, page_size, h_kv = k.shape[0], k.shape[1], k.shape[2]
    _want(k, "k_pool", dt, (num_pages, page_size, h_kv, d), dev)
    _want(v, "v_pool", dt, (num_pages, page_size, h_kv, d), dev)
    _want(block_table, "block_table", torch.int32, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    return h_kv, 0, block_table.shape[1], num_pages, page_size


def decode_call(q, k, v, seq_lens, chunk_keys, max_splits, block_table=None, page_size=16, scale=None,
                part_o=None, part_m=None, part_l=None, out=None, lse=None):
    """Both decode stages in one call of attn_decode; the partial buffers are
    allocated with torch when not given. Returns (o [B,h,128], lse [B,h])."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    B, h, d = q.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    h_kv, s_max, max_pages, num_pages, page_size = _kv_geometry(q, k, v, block_table, page_size)
    shp = (B, h, max_splits)
    part_o = torch.empty(shp + (d,), dtype=torch.float32, device=dev) if part_o is None else part_o
    part_m = torch.empty(shp, dtype=torch.float32, device=dev) if part_m is None else part_m
    part_l = torch.empty(shp, dtype=torch.float32, device=dev) if part_l is None else part_l
    _want(part_o, "part_o", torch.float32, shp + (d,), dev)
    _want(part_m, "part_m", torch.float32, shp, dev)
    _want(part_l, "part_l", torch.float32, shp, dev)
    out = torch.empty((B, h, d), dtype=dt, device=dev) if out is None else out
    _want(out, "out", dt, (B, h, d), dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, (B, h), dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_decode", lib.attn_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), max_pages, page_size, num_pages,
        _ptr(seq_lens), s_max, B, h, h_kv, d, int(chunk_keys), int(max_splits), _dtype_code(q),
        scale, _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def _partials(B, h, max_splits, d, dev, part_o, part_m, part_l):
    shp = (B, h, max_splits)
    part_o = torch.empty(shp + (d,), dtype=torch.float32, device=dev) if part_o is None else part_o
    part_m = torch.empty(shp, dtype=torch.float32, device=dev) if part_m is None else part_m
    part_l = torch.empty(shp, dtype=torch.float32, device=dev) if part_l is None else part_l
    _want(part_o, "part_o", torch.float32, shp + (d,), dev)
    _want(part_m, "part_m", torch.float32, shp, dev)
    _want(part_l, "part_l", torch.float32, shp, dev)
    return part_o, part_m, part_l


def decode_split_fp8kv(q, k, v, seq_lens, chunk_keys, max_splits, k_scale, v_scale, block_table=None,
                       page_size=16, scale=None, part_o=None, part_m=None, part_l=None):
    """Stage 1 of split-KV decode over 8-bit E4M3 K/V (uint8 codes, layouts
    as decode_split) with per-tensor scales, via attn_decode_split_fp8kv.
    Returns (part_o, part_m, part_l) fp32."""
    lib = load()
    _want(q, "q")
    dev = q.device
    B, h, d = q.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    h_kv, s_max, max_pages, num_pages, page_size = _kv_geometry(q, k, v, block_table, page_size, torch.uint8)
    part_o, part_m, part_l = _partials(B, h, max_splits, d, dev, part_o, part_m, part_l)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_decode_split_fp8kv", lib.attn_decode_split_fp8kv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), max_pages, page_size, num_pages,
        _ptr(seq_lens), s_max, B, h, h_kv, d, int(chunk_keys), int(max_splits), _dtype_code(q),
        scale, float(k_scale), float(v_scale), _ptr(part_o), _ptr(part_m), _ptr(part_l), _stream(dev)))
    return part_o, part_m, part_l


def decode_fp8kv_call(q, k, v, seq_lens, chunk_keys, max_splits, k_scale, v_scale, block_table=None,
                      page_size=16, scale=None, part_o=None, part_m=None, part_l=None, out=None, lse=None):
    """Both decode stages over 8-bit E4M3 K/V in one call of
    attn_decode_fp8kv. Returns (o [B,h,128], lse [B,h])."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    B, h, d = q.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    h_kv, s_max, max_pages, num_pages, page_size = _kv_geometry(q, k, v, block_table, page_size, torch.uint8)
    part_o, part_m, part_l = _partials(B, h, max_splits, d, dev, part_o, part_m, part_l)
    out = torch.empty((B, h, d), dtype=dt, device=dev) if out is None else out
    _want(out, "out", dt, (B, h, d), dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, (B, h), dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_decode_fp8kv", lib.attn_decode_fp8kv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), max_pages, page_size, num_pages,
        _ptr(seq_lens), s_max, B, h, h_kv, d, int(chunk_keys), int(max_splits), _dtype_code(q),
        scale, float(k_scale), float(v_scale), _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(out), _ptr(lse),
        _stream(dev)))
    return out, lse


def decode_fp8kv(q, k, v, seq_lens, k_scale, v_scale, seq_lens_host=None, block_table=None, page_size=16,
                 scale=None, plan=None, num_cus=None):
    """Split-KV decode over 8-bit E4M3 K/V: plan (host, as decode), then
    attn_decode_fp8kv. Returns (o, lse, (chunk_keys, max_splits))."""
    B, h, _ = q.shape
    h_kv = k.shape[2] if block_table is not None else k.shape[1]
    if plan is None:
        lens = seq_lens.cpu().numpy() if seq_lens_host is None else np.asarray(seq_lens_host)
        plan = decode_plan(lens, h, h_kv, num_cus=num_cus, device=q.device)
    chunk, splits = plan
    o, lse = decode_fp8kv_call(q, k, v, seq_lens, chunk, splits, k_scale, v_scale, block_table=block_table,
                               page_size=page_size, scale=scale)
    return o, lse, plan


def decode_noalloc(q, k, v, seq_lens, chunk_keys, max_splits, block_table=None, page_size=16, scale=None,
                   out=None, lse=None):
    """Both decode stages via attn_decode_noalloc: the partial states live in
    the library's per-GPU device scratch (the call allocates nothing; ``out``
    and ``lse`` are allocated here only when not given). Returns (o, lse)."""
    lib = load()
    _want(q, "q")
    dev, dt = q.device, q.dtype
    B, h, d = q.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    h_kv, s_max, max_pages, num_pages, page_size = _kv_geometry(q, k, v, block_table, page_size)
    out = torch.empty((B, h, d), dtype=dt, device=dev) if out is None else out
    _want(out, "out", dt, (B, h, d), dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, (B, h), dev)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(scale)
    _check("attn_decode_noalloc", lib.attn_decode_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), max_pages, page_size, num_pages,
        _ptr(seq_lens), s_max, B, h, h_kv, d, int(chunk_keys), int(max_splits), _dtype_code(q),
        scale, _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def decode(q, k, v, seq_lens, seq_lens_host=None, block_table=None, page_size=16, scale=None,
           plan=None, num_cus=None, one_call=True):
    """Split-KV decode: plan (host), then both stages on the device -- in one
    call of attn_decode (``one_call``) or as attn_decode_split followed by
    attn_merge_states. Returns (o [B,h,128], lse [B,h], (chunk_keys, max_splits))."""
    B, h, _ = q.shape
    h_kv = k.shape[1] if block_table is None else k.shape[2]
    if plan is None:
        lens = seq_lens.cpu().numpy() if seq_lens_host is None else seq_lens_host
        plan = decode_plan(lens, h, h_kv, num_cus=num_cus, device=q.device)
    chunk, splits = plan
    if one_call:
        o, lse = decode_call(q, k, v, seq_lens, chunk, splits, block_table, page_size, scale)
        return o, lse, plan
    po, pm, pl = decode_split(q, k, v, seq_lens, chunk, splits, block_table, page_size, scale)
    o, lse = merge_states(po, pm, pl, seq_lens, chunk, q.dtype)
    return o, lse, plan


def merge_lse(o_a, lse_a, o_b, lse_b, out=None, lse=None):
    """(O, LSE) of the union of two disjoint key ranges via attn_merge_lse.
    o_* [..., 128] and lse_* [...] over the same leading shape; ``out`` / ``lse``
    may be o_a / lse_a (in place)."""
    lib = load()
    _want(o_a, "o_a")
    dev, dt = o_a.device, o_a.dtype
    lead = tuple(o_a.shape[:-1])
    d = o_a.shape[-1]
    _want(o_b, "o_b", dt, tuple(o_a.shape), dev)
    _want(lse_a, "lse_a", torch.float32, lead, dev)
    _want(lse_b, "lse_b", torch.float32, lead, dev)
    out = torch.empty_like(o_a) if out is None else out
    _want(out, "out", dt, tuple(o_a.shape), dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if lse is None else lse
    _want(lse, "lse", torch.float32, lead, dev)
    rows = int(np.prod(lead)) if lead else 1
    _check("attn_merge_lse", lib.attn_merge_lse(
        _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, d, _ptr(out), _ptr(lse),
        _dtype_code(out), _stream(dev)))
    return out, lse


def paged_gather(pool, block_table, seq_lens, s_max, out=None):
    """Contiguous [B, h_kv, s_max, 128] copy of a paged pool via attn_paged_gather;
    positions past each sequence's length keep the contents of ``out``."""
    lib = load()
    _want(pool, "pool")
    dev, dt = pool.device, pool.dtype
    num_pages, page_size, h_kv, d = pool.shape
    _want(block_table, "block_table", torch.int32, None, dev)
    B, max_pages = block_table.shape
    _want(seq_lens, "seq_lens", torch.int32, (B,), dev)
    out = torch.zeros((B, h_kv, s_max, d), dtype=dt, device=dev) if out is None else out
    _want(out, "out", dt, (B, h_kv, s_max, d), dev)
    _check("attn_paged_gather", lib.attn_paged_gather(
        _ptr(pool), _ptr(block_table), _ptr(seq_lens), B, h_kv, d, page_size, max_pages, num_pages,
        s_max, _dtype_code(pool), _ptr(out), _stream(dev)))
    return out


def stream_read(src, chunks=1024, out=None):
    """Read ``src`` (a contiguous device tensor) once via attn_stream_read, a
    measurement aid for the attainable read rate; returns out [chunks] int32."""
    lib = load()
    _want(src, "src")
    nbytes = src.numel() * src.element_size()
    out = torch.empty(chunks, dtype=torch.int32, device=src.device) if out is None else out
    _want(out, "out", torch.int32, (chunks,), src.device)
    _check("attn_stream_read", lib.attn_stream_read(_ptr(src), nbytes, int(chunks), _ptr(out), _stream(src.device)))
    return out
