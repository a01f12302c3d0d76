"""Thin Python binding of libkvc (ctypes).  Argument marshalling only: every
step of the compression runs in the HIP kernels behind the C ABI declared in
``include/kvc.h``.  torch provides device memory and the current stream.

The library must have been built (``python -m kv_cache_compression_pool_amd._build``);
importing this module does not load it, the first call does, and a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK = 0
KVC_ERR_NULL = -1
KVC_ERR_SHAPE = -2
KVC_ERR_UNSUPPORTED = -3
KVC_ERR_PLAN = -4
KVC_ERR_HIP = -5

PLAN_DTYPE = np.dtype([("ragged_id", "<u4"), ("batch_id", "<u4"), ("position", "<u4"),
                       ("window_len", "<u4")])
PLAN_SENTINEL = 0xFFFFFFFF
ITEM_DTYPE = np.dtype([("compress", PLAN_DTYPE), ("write", PLAN_DTYPE)])

EXPORTS = ("kvc_version", "kvc_last_error", "kvc_plan_pool_prefill", "kvc_c128_plan_prefill",
           "kvc_compress_prefill", "kvc_compress_prefill_paged", "kvc_compress_decode_ring",
           "kvc_compress_decode_ring_paged", "kvc_compress_decode_ring_layers",
           "kvc_seed_tail_ring",
           "kvc_c128_online_decode", "kvc_c128_online_decode_layers",
           "kvc_c128_online_decode_quant", "kvc_c128_online_prefill",
           "kvc_c128_online_prefill_quant", "kvc_c128_plan_prefill_fused",
           "kvc_c128_fused_capacity",
           "kvc_c128_online_prefill_fused", "kvc_diag_convert", "kvc_diag_stream_read",
           "kvc_diag_empty_launch")


class KvcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libkvc error {code}: {msg}")
        self.code = code


_lib = None
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_u32 = ctypes.c_uint32


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m kv_cache_compression_pool_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kvc_version.restype = _i32
        L.kvc_last_error.restype = ctypes.c_char_p
        L.kvc_plan_pool_prefill.argtypes = [_p, _i64, _i32, _p, _i64, _p]
        L.kvc_c128_plan_prefill.argtypes = [_p, _p, _i64, _i64, _p, _p, _i32, _p, _p]
        L.kvc_compress_prefill.argtypes = [_p, _i64, _p, _i64, _i64, _p, _i32, _p, _i64, _p, _p,
                                           _i32, _p, _p]
        L.kvc_compress_decode_ring.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _i64, _p,
                                               _p, _p, _i64, _i32, _i32, _p, _p, _i64, _i32, _p,
                                               _p]
        L.kvc_compress_decode_ring_layers.argtypes = [_p, _i64, _i64, _p, _p, _i64, _i64, _i64,
                                                      _p, _i64, _i64, _i64, _p, _i64, _p, _p,
                                                      _i64, _i32, _i32, _p, _p, _i64, _i64, _i32,
                                                      _p]
        L.kvc_compress_prefill_paged.argtypes = [_p, _i64, _p, _i64, _i64, _p, _i32, _p, _i64,
                                                 _p, _i64, _i32, _p, _p, _i32, _p]
        L.kvc_compress_decode_ring_paged.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _i64,
                                                     _p, _p, _p, _i64, _i32, _i32, _p, _i64, _i32,
                                                     _i32, _p]
        L.kvc_seed_tail_ring.argtypes = [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i32, _p]
        L.kvc_c128_online_decode.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _i64, _p]
        L.kvc_c128_online_prefill.argtypes = [_p, _i64, _p, _p, _i64, _p, _p, _p, _i64, _p, _u32,
                                              _p, _u32, _p]
        L.kvc_c128_online_decode_layers.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
                                                    _p, _p, _i64, _i64, _p]
        L.kvc_c128_online_decode_quant.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                                   _p]
        L.kvc_c128_online_prefill_quant.argtypes = [_p, _i64, _p, _p, _p, _i64, _p, _p, _p,
                                                    _i64, _p, _u32, _p, _u32, _i32, _p]
        L.kvc_c128_plan_prefill_fused.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _p]
        L.kvc_c128_fused_capacity.argtypes = [_i64, _i64]
        L.kvc_c128_online_prefill_fused.argtypes = [_p, _i64, _p, _p, _p, _p, _i32, _i64, _p, _p,
                                                    _p, _i64, _p, _u32, _p]
        L.kvc_diag_convert.argtypes = [_p, _p, _p, _i64, _p]
        L.kvc_diag_stream_read.argtypes = [_p, _i64, _p, _i64, _i32, _i32, _p]
        L.kvc_diag_empty_launch.argtypes = [_i64, _i32, _i32, _p]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = _i32
        L.kvc_c128_fused_capacity.restype = _i64
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != KVC_OK:
        raise KvcError(rc, lib().kvc_last_error().decode())


_capture = threading.local()


def _invoke(name, args, stream):
    """Call device entry point `name` with its marshalled arguments (all but
    the stream), or, inside prepare(), return them as a PreparedCall."""
    if getattr(_capture, "on", False):
        return PreparedCall(name, args, stream)
    _check(getattr(lib(), name)(*args, _stream(stream)))


class PreparedCall:
    """One device entry point with its arguments checked and marshalled once
    (see prepare()).  Calling it issues the C call and nothing else, so a
    loop that launches the same call on the same buffers pays only the ctypes
    call.  It holds references to the tensors it was prepared with."""

    __slots__ = ("_fn", "_args", "_stream", "_keep", "name")

    def __init__(self, name, args, stream):
        self.name = name
        fn = getattr(lib(), name)
        # converted to ctypes values once (NULL stays None) ...
        self._args = tuple(None if a is None else t(a) for t, a in zip(fn.argtypes, args))
        # ... and passed through a pointer to the same function that has no
        # argtypes, so ctypes takes them as they are instead of converting
        # each one again on every call (about 0.3 us of a ~1 us ctypes call).
        # Every value it gets is a ctypes instance or None, so each keeps its
        # declared C type.
        self._fn = ctypes.cast(fn, ctypes.CFUNCTYPE(fn.restype))
        self._fn.argtypes = None
        # a stream given at preparation is kept; None means torch's current
        # stream at each call
        self._stream = None if stream is None else ctypes.c_void_p(_stream(stream))
        self._keep = None

    def __call__(self, stream=None):
        if stream is not None:
            s = ctypes.c_void_p(_stream(stream))
        elif self._stream is not None:
            s = self._stream
        else:
            s = ctypes.c_void_p(_current_stream())
        rc = self._fn(*self._args, s)
        if rc != KVC_OK:
            _check(rc)


def prepare(entry_point, *args, **kwargs):
    """Validate and marshal the arguments of a device entry point of this
    module once; returns a PreparedCall that launches it.  The buffers must
    stay the same tensors with the same shapes (the call keeps references to
    them); their contents may change between calls.  A stream given here is
    used by every call, also under HIP-graph capture; without one each call
    launches on torch's current stream (the capture stream while capturing).
    Example:
        launch = kvc.prepare(kvc.kvc_compress_prefill, keys, scores, ape, rows,
                             n_pools, out, scale, True)
        launch()            # on torch's current stream
    """
    _capture.on = True
    try:
        call = entry_point(*args, **kwargs)
    finally:
        _capture.on = False
    if not isinstance(call, PreparedCall):
        raise TypeError(f"{getattr(entry_point, '__name__', entry_point)} is not a device "
                        "entry point of this module")
    call._keep = (args, kwargs)
    return call


_current_stream_fn = None


def _current_stream() -> int:
    """torch's current hipStream_t handle on the current device."""
    global _current_stream_fn
    if _current_stream_fn is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        if raw is not None and dev is not None:
            # the handle without building a Stream object (a few us per call)
            _current_stream_fn = lambda: raw(dev())
        else:
            _current_stream_fn = lambda: torch.cuda.current_stream().cuda_stream
    return _current_stream_fn()


def _stream(stream) -> int | None:
    """hipStream_t handle: None = torch's current stream; a torch.cuda.Stream
    or a raw integer handle is used as given."""
    if stream is None:
        return _current_stream()
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    return int(stream)


def _dptr(t, dtype, name, optional=False):
    """Device pointer of a CUDA/HIP tensor of the given torch dtype."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _shape_ok(t, shape, name, contiguous=True):
    """t has exactly ``shape`` (None = any extent) and is contiguous."""
    _need(t.dim() == len(shape) and all(e is None or t.shape[i] == e
                                        for i, e in enumerate(shape)),
          f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def _head(a: np.ndarray, n: int) -> np.ndarray:
    """A compact copy of the first n records of a structured array (copied
    as bytes: numpy copies structured records field by field, ~15x slower)."""
    out = np.empty(n, a.dtype)
    out.view(np.uint8)[:] = a[:n].view(np.uint8)
    return out


# ------------------------------------------------------------------ planners
def kvc_plan_pool_prefill(seq_lens, pool_size: int = 16) -> np.ndarray:
    """First row of every complete pool of a ragged batch (host int32 array)."""
    sl = np.ascontiguousarray(seq_lens, np.int64)
    n = ctypes.c_int64()
    cap = int(np.sum(np.maximum(sl, 0) // pool_size)) if pool_size > 0 else 0
    out = np.empty(max(cap, 1), np.int32)
    _check(lib().kvc_plan_pool_prefill(_np_ptr(sl), sl.size, pool_size, _np_ptr(out), cap,
                                       ctypes.byref(n)))
    return out[:n.value].copy()


def kvc_c128_plan_prefill(seq_lens, extend_lens, num_tokens: int, pad_to_capacity: bool = False):
    """(compress_plan, write_plan) host structured arrays of PLAN_DTYPE."""
    sl = np.ascontiguousarray(seq_lens, np.int64)
    el = np.ascontiguousarray(extend_lens, np.int64)
    if sl.size != el.size:
        raise ValueError("seq_lens and extend_lens differ in length")
    cap = max(int(num_tokens), 1)
    # capacity is one entry per token; only the entries written are returned,
    # so the buffers need no clearing (untouched pages are never faulted in)
    cp = np.empty(cap, PLAN_DTYPE)
    wp = np.empty(cap, PLAN_DTYPE)
    nc, nw = ctypes.c_uint32(), ctypes.c_uint32()
    _check(lib().kvc_c128_plan_prefill(_np_ptr(sl), _np_ptr(el), sl.size, int(num_tokens),
                                       _np_ptr(cp), _np_ptr(wp), int(pad_to_capacity),
                                       ctypes.byref(nc), ctypes.byref(nw)))
    return _head(cp, nc.value), _head(wp, nw.value)


def kvc_c128_fused_capacity(num_tokens: int, max_batch: int) -> int:
    """Upper bound on the single-launch work items of any batch of at most
    max_batch requests extending num_tokens tokens."""
    return int(lib().kvc_c128_fused_capacity(int(num_tokens), int(max_batch)))


def kvc_c128_plan_prefill_fused(seq_lens, extend_lens, num_tokens: int,
                                pad_to_capacity: bool = False, capacity=None):
    """Work items for kvc_c128_online_prefill_fused: host array of ITEM_DTYPE
    (fields compress / write, each a PLAN_DTYPE record; all-0xFFFFFFFF = none).
    capacity defaults to kvc_c128_fused_capacity(num_tokens, len(seq_lens))."""
    sl = np.ascontiguousarray(seq_lens, np.int64)
    el = np.ascontiguousarray(extend_lens, np.int64)
    if sl.size != el.size:
        raise ValueError("seq_lens and extend_lens differ in length")
    if capacity is None:
        capacity = kvc_c128_fused_capacity(num_tokens, sl.size)
    items = np.empty(max(int(capacity), 1), ITEM_DTYPE)
    n = ctypes.c_uint32()
    _check(lib().kvc_c128_plan_prefill_fused(_np_ptr(sl), _np_ptr(el), sl.size, int(num_tokens),
                                             _np_ptr(items), int(capacity), int(pad_to_capacity),
                                             ctypes.byref(n)))
    return _head(items, n.value)


# ------------------------------------------------------------------ device entry points
def kvc_compress_prefill(keys, scores, ape, pool_src_row, n_pools: int, out_fp8, out_scale,
                         round_scale: bool, dbg_pooled=None, pool_size: int = 16, stream=None):
    """keys/scores: device int16/uint16-viewed bf16 [rows, >=128] (or torch.bfloat16);
    ape fp32 [16,128]; pool_src_row int32 [n_pools] or None; out_fp8 uint8
    [n_pools,128]; out_scale fp32 [n_pools]."""
    import torch
    k = _bf16_view(keys, "keys")
    s = _bf16_view(scores, "scores")
    if k.shape[0] != s.shape[0]:
        raise ValueError("keys and scores must have the same number of rows")
    n_pools = int(n_pools)
    _shape_ok(ape, (pool_size, 128), "ape")
    _need(out_fp8.dim() == 2 and out_fp8.shape[0] >= n_pools and out_fp8.shape[1] == 128
          and out_fp8.is_contiguous(), "out_fp8 must be a contiguous [>=n_pools, 128] tensor")
    _need(out_scale.dim() == 1 and out_scale.shape[0] >= n_pools, "out_scale must hold n_pools")
    if pool_src_row is not None:
        _need(pool_src_row.dim() == 1 and pool_src_row.shape[0] >= n_pools
              and pool_src_row.is_contiguous(), "pool_src_row must hold n_pools entries")
    if dbg_pooled is not None:
        _need(dbg_pooled.dim() == 2 and dbg_pooled.shape[0] >= n_pools
              and dbg_pooled.shape[1] == 128 and dbg_pooled.is_contiguous(),
              "dbg_pooled must be a contiguous [>=n_pools, 128] tensor")
    return _invoke("kvc_compress_prefill", (
        k.data_ptr(), k.stride(0), s.data_ptr(), s.stride(0), k.shape[0],
        _dptr(ape, torch.float32, "ape"), pool_size,
        _dptr(pool_src_row, torch.int32, "pool_src_row", optional=True), int(n_pools),
        _dptr(out_fp8, torch.uint8, "out_fp8"), _dptr(out_scale, torch.float32, "out_scale"),
        int(round_scale), _dptr(dbg_pooled, torch.float32, "dbg_pooled", optional=True)), stream)


def kvc_compress_prefill_paged(keys, scores, ape, pool_src_row, n_pools: int, kv_cache, loc,
                               round_scale: bool, write_mask=None, pool_size: int = 16,
                               stream=None):
    """As kvc_compress_prefill, writing into a page-size-1 cache: kv_cache
    uint8 [pages, 132] (or [pages, 1, 132]); loc int64 [n_pools]; write_mask
    bool/uint8 [n_pools] or None."""
    import torch
    k = _bf16_view(keys, "keys")
    s = _bf16_view(scores, "scores")
    n_pools = int(n_pools)
    _need(k.shape[0] == s.shape[0], "keys and scores must have the same number of rows")
    _shape_ok(ape, (pool_size, 128), "ape")
    _need(kv_cache.is_contiguous() and kv_cache.shape[-1] == 132 and kv_cache.numel() %
          132 == 0, "kv_cache must be a contiguous [pages, 132] uint8 tensor")
    _need(loc.dim() == 1 and loc.shape[0] >= n_pools and loc.is_contiguous(),
          "loc must hold n_pools entries")
    if pool_src_row is not None:
        _need(pool_src_row.dim() == 1 and pool_src_row.shape[0] >= n_pools
              and pool_src_row.is_contiguous(), "pool_src_row must hold n_pools entries")
    wm = None
    if write_mask is not None:
        _need(write_mask.dim() == 1 and write_mask.shape[0] >= n_pools and write_mask.is_cuda
              and write_mask.element_size() == 1 and write_mask.is_contiguous(),
              "write_mask must be a contiguous 1-byte device tensor of n_pools entries")
        wm = write_mask.data_ptr()
    return _invoke("kvc_compress_prefill_paged", (
        k.data_ptr(), k.stride(0), s.data_ptr(), s.stride(0), k.shape[0],
        _dptr(ape, torch.float32, "ape"), pool_size,
        _dptr(pool_src_row, torch.int32, "pool_src_row", optional=True), n_pools,
        _dptr(kv_cache, torch.uint8, "kv_cache"), kv_cache.numel() // 132, 1,
        _dptr(loc, torch.int64, "loc"), wm, int(round_scale)), stream)


def kvc_compress_decode_ring_layers(tail_ring, tail_slot_mapping, key, score, ape, slot_mapping,
                                    positions, out_fp8, out_scale, round_scale: bool,
                                    pool_size: int = 16, stream=None):
    """Multi-layer ring decode: tail_ring bf16 [L,nb,2,16,128]; key/score bf16
    [L,R,next_n,128] (per-layer views with a common layer stride); ape fp32
    [L,16,128]; maps int32 [R,next_n] shared by all layers; out_fp8 uint8
    [L,num_out,128]; out_scale fp32 [L,num_out]."""
    import torch
    ring = _bf16_view(tail_ring, "tail_ring", min_last=None)
    k = _bf16_view(key, "key", min_last=None)
    s = _bf16_view(score, "score", min_last=None)
    _need(ring.dim() == 5 and ring.is_contiguous() and tuple(ring.shape[2:]) == (2, pool_size, 128),
          f"tail_ring must be a contiguous [L, nb, 2, {pool_size}, 128] tensor")
    L = ring.shape[0]
    _need(k.dim() == 4 and k.shape[0] == L and k.shape[3] == 128 and tuple(s.shape) == tuple(k.shape),
          "key and score must be [L, R, next_n, 128]")
    R, N = k.shape[1], k.shape[2]
    for name, t in (("tail_slot_mapping", tail_slot_mapping), ("slot_mapping", slot_mapping),
                    ("positions", positions)):
        if tuple(t.shape) != (R, N) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{R}, {N}] tensor")
    _need(ape.dim() == 3 and tuple(ape.shape) == (L, pool_size, 128) and ape.is_contiguous(),
          f"ape must be a contiguous [L, {pool_size}, 128] tensor")
    _need(out_fp8.dim() == 3 and out_fp8.shape[0] == L and out_fp8.shape[2] == 128
          and out_fp8.is_contiguous(), "out_fp8 must be a contiguous [L, num_out, 128] tensor")
    num_out = out_fp8.shape[1]
    _need(tuple(out_scale.shape) == (L, num_out) and out_scale.is_contiguous(),
          "out_scale must be a contiguous [L, num_out] tensor")
    return _invoke("kvc_compress_decode_ring_layers", (
        ring.data_ptr(), ring.stride(0), ring.shape[1],
        _dptr(tail_slot_mapping, torch.int32, "tail_slot_mapping"),
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
        s.data_ptr(), s.stride(0), s.stride(1), s.stride(2),
        _dptr(ape, torch.float32, "ape"), ape.stride(0),
        _dptr(slot_mapping, torch.int32, "slot_mapping"), _dptr(positions, torch.int32, "positions"),
        R, N, pool_size, _dptr(out_fp8, torch.uint8, "out_fp8"),
        _dptr(out_scale, torch.float32, "out_scale"), num_out, L, int(round_scale)), stream)


def kvc_compress_decode_ring_paged(tail_ring, tail_slot_mapping, key, score, ape, slot_mapping,
                                   positions, kv_cache, round_scale: bool, pool_size: int = 16,
                                   stream=None):
    """As kvc_compress_decode_ring, completions written into a page-size-1
    cache (kv_cache uint8 [pages, 132]) at page slot_mapping[r, t]."""
    import torch
    ring = _bf16_view(tail_ring, "tail_ring", min_last=None)
    k = _bf16_view(key, "key", min_last=None)
    s = _bf16_view(score, "score", min_last=None)
    R, N = k.shape[0], k.shape[1]
    for name, t in (("tail_slot_mapping", tail_slot_mapping), ("slot_mapping", slot_mapping),
                    ("positions", positions)):
        _shape_ok(t, (R, N), name)
    _need(ring.is_contiguous() and tuple(ring.shape[1:]) == (2, pool_size, 128),
          f"tail_ring must be a contiguous [nb, 2, {pool_size}, 128] tensor")
    _need(k.dim() == 3 and k.shape[2] == 128 and tuple(s.shape) == tuple(k.shape),
          "key and score must be [R, next_n, 128]")
    _shape_ok(ape, (pool_size, 128), "ape")
    _need(kv_cache.is_contiguous() and kv_cache.shape[-1] == 132 and kv_cache.numel() %
          132 == 0, "kv_cache must be a contiguous [pages, 132] uint8 tensor")
    return _invoke("kvc_compress_decode_ring_paged", (
        ring.data_ptr(), ring.shape[0], _dptr(tail_slot_mapping, torch.int32, "tail_slot_mapping"),
        k.data_ptr(), k.stride(0), k.stride(1), s.data_ptr(), s.stride(0), s.stride(1),
        _dptr(ape, torch.float32, "ape"), _dptr(slot_mapping, torch.int32, "slot_mapping"),
        _dptr(positions, torch.int32, "positions"), R, N, pool_size,
        _dptr(kv_cache, torch.uint8, "kv_cache"), kv_cache.numel() // 132, 1, int(round_scale)), stream)


def kvc_compress_decode_ring(tail_ring, tail_slot_mapping, key, score, ape, slot_mapping,
                             positions, out_fp8, out_scale, round_scale: bool,
                             pool_size: int = 16, stream=None, dbg_pooled=None):
    """tail_ring bf16 [nb,2,16,128] (updated); key/score bf16 [R,next_n,128];
    maps int32 [R,next_n]; out_fp8 uint8 [num_out,128]; out_scale fp32 [num_out];
    dbg_pooled fp32 [num_out,128] or None (pre-rounding means of completions)."""
    import torch
    ring = _bf16_view(tail_ring, "tail_ring", min_last=None)
    k = _bf16_view(key, "key", min_last=None)
    s = _bf16_view(score, "score", min_last=None)
    R, N = k.shape[0], k.shape[1]
    for name, t in (("tail_slot_mapping", tail_slot_mapping), ("slot_mapping", slot_mapping),
                    ("positions", positions)):
        if tuple(t.shape) != (R, N) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{R}, {N}] tensor")
    if not ring.is_contiguous() or tuple(ring.shape[1:]) != (2, pool_size, 128):
        raise ValueError(f"tail_ring must be a contiguous [nb, 2, {pool_size}, 128] tensor")
    _need(k.dim() == 3 and k.shape[2] == 128 and tuple(s.shape) == tuple(k.shape),
          "key and score must be [R, next_n, 128]")
    _shape_ok(ape, (pool_size, 128), "ape")
    _need(out_fp8.dim() == 2 and out_fp8.shape[1] == 128 and out_fp8.is_contiguous(),
          "out_fp8 must be a contiguous [num_out, 128] tensor")
    _need(out_scale.dim() == 1 and out_scale.shape[0] >= out_fp8.shape[0],
          "out_scale must hold num_out entries")
    if dbg_pooled is not None:
        _need(dbg_pooled.dim() == 2 and dbg_pooled.shape[0] >= out_fp8.shape[0]
              and dbg_pooled.shape[1] == 128 and dbg_pooled.is_contiguous(),
              "dbg_pooled must be a contiguous [num_out, 128] tensor")
    return _invoke("kvc_compress_decode_ring", (
        ring.data_ptr(), ring.shape[0], _dptr(tail_slot_mapping, torch.int32, "tail_slot_mapping"),
        k.data_ptr(), k.stride(0), k.stride(1), s.data_ptr(), s.stride(0), s.stride(1),
        _dptr(ape, torch.float32, "ape"), _dptr(slot_mapping, torch.int32, "slot_mapping"),
        _dptr(positions, torch.int32, "positions"), R, N, pool_size,
        _dptr(out_fp8, torch.uint8, "out_fp8"), _dptr(out_scale, torch.float32, "out_scale"),
        out_fp8.shape[0], int(round_scale),
        _dptr(dbg_pooled, torch.float32, "dbg_pooled", optional=True)), stream)


def kvc_seed_tail_ring(tail_ring, key, score, tslot, pool_size: int = 16, stream=None):
    """tail_ring bf16 [nb,2,16,128] (updated); key/score bf16 [n,>=128];
    tslot int32 [n]."""
    import torch
    ring = _bf16_view(tail_ring, "tail_ring", min_last=None)
    k = _bf16_view(key, "key")
    s = _bf16_view(score, "score")
    n = int(tslot.shape[0])
    _need(ring.is_contiguous() and tuple(ring.shape[1:]) == (2, pool_size, 128),
          f"tail_ring must be a contiguous [nb, 2, {pool_size}, 128] tensor")
    _need(k.dim() == 2 and s.dim() == 2 and k.shape[0] >= n and s.shape[0] >= n,
          "key and score must hold one row per token")
    _shape_ok(tslot, (n,), "tslot")
    return _invoke("kvc_seed_tail_ring", (ring.data_ptr(), ring.shape[0], k.data_ptr(), k.stride(0),
                                    s.data_ptr(), s.stride(0),
                                    _dptr(tslot, torch.int32, "tslot"), n, pool_size), stream)


def kvc_c128_online_decode(state, kv_score_in, out, ape, indices, seq_lens, stream=None):
    import torch
    B = kv_score_in.shape[0]
    _shape_ok(state, (None, 384), "state")
    _shape_ok(kv_score_in, (B, 256), "kv_score_in")
    _shape_ok(out, (B, 128), "out")
    _shape_ok(ape, (128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    _shape_ok(seq_lens, (B,), "seq_lens")
    return _invoke("kvc_c128_online_decode", (
        _dptr(state, torch.float32, "state"), state.shape[0],
        _dptr(kv_score_in, torch.float32, "kv_score_in"), _dptr(out, torch.float32, "out"),
        _dptr(ape, torch.float32, "ape"), _dptr(indices, torch.int32, "indices"),
        _dptr(seq_lens, torch.int32, "seq_lens"), kv_score_in.shape[0]), stream)


def kvc_c128_online_decode_layers(state, kv_score_in, out, ape, indices, seq_lens, stream=None):
    """Multi-layer decode: state [L,S,384], kv_score_in [L,B,256], out
    [L,B,128], ape [L,128,128] (contiguous); indices / seq_lens [B] shared."""
    import torch
    Lr, B = kv_score_in.shape[0], kv_score_in.shape[1]
    _shape_ok(state, (Lr, None, 384), "state")
    _shape_ok(kv_score_in, (Lr, B, 256), "kv_score_in")
    _shape_ok(out, (Lr, B, 128), "out")
    _shape_ok(ape, (Lr, 128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    _shape_ok(seq_lens, (B,), "seq_lens")
    return _invoke("kvc_c128_online_decode_layers", (
        _dptr(state, torch.float32, "state"), state.stride(0), state.shape[1],
        _dptr(kv_score_in, torch.float32, "kv_score_in"), kv_score_in.stride(0),
        _dptr(out, torch.float32, "out"), out.stride(0), _dptr(ape, torch.float32, "ape"),
        ape.stride(0), _dptr(indices, torch.int32, "indices"),
        _dptr(seq_lens, torch.int32, "seq_lens"), B, Lr), stream)


def kvc_c128_online_decode_quant(state, kv_score_in, out_fp8, out_scale, ape, indices, seq_lens,
                                 round_scale: bool, stream=None):
    """Decode with the rotate / e4m3 epilogue on emitted vectors: out_fp8
    uint8 [B,128], out_scale fp32 [B]."""
    import torch
    B = kv_score_in.shape[0]
    _shape_ok(state, (None, 384), "state")
    _shape_ok(kv_score_in, (B, 256), "kv_score_in")
    _shape_ok(out_fp8, (B, 128), "out_fp8")
    _shape_ok(out_scale, (B,), "out_scale")
    _shape_ok(ape, (128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    _shape_ok(seq_lens, (B,), "seq_lens")
    return _invoke("kvc_c128_online_decode_quant", (
        _dptr(state, torch.float32, "state"), state.shape[0],
        _dptr(kv_score_in, torch.float32, "kv_score_in"), _dptr(out_fp8, torch.uint8, "out_fp8"),
        _dptr(out_scale, torch.float32, "out_scale"), _dptr(ape, torch.float32, "ape"),
        _dptr(indices, torch.int32, "indices"), _dptr(seq_lens, torch.int32, "seq_lens"), B,
        int(round_scale)), stream)


def kvc_c128_online_prefill_quant(state, kv_score_in, out_fp8, out_scale, ape, indices,
                                  compress_plan, n_compress, write_plan, n_write,
                                  round_scale: bool, load_indices=None, stream=None):
    """Prefill with the rotate / e4m3 epilogue on chunk-closing vectors:
    out_fp8 uint8 [N,128], out_scale fp32 [N]."""
    import torch
    N, B = kv_score_in.shape[0], indices.shape[0]
    _shape_ok(state, (None, 384), "state")
    _shape_ok(kv_score_in, (N, 256), "kv_score_in")
    _shape_ok(out_fp8, (N, 128), "out_fp8")
    _shape_ok(out_scale, (N,), "out_scale")
    _shape_ok(ape, (128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    if load_indices is not None:
        _shape_ok(load_indices, (B,), "load_indices")
    _check_plans(compress_plan, n_compress, write_plan, n_write)
    return _invoke("kvc_c128_online_prefill_quant", (
        _dptr(state, torch.float32, "state"), state.shape[0],
        _dptr(kv_score_in, torch.float32, "kv_score_in"), _dptr(out_fp8, torch.uint8, "out_fp8"),
        _dptr(out_scale, torch.float32, "out_scale"), N, _dptr(ape, torch.float32, "ape"),
        _dptr(indices, torch.int32, "indices"),
        _dptr(load_indices, torch.int32, "load_indices", optional=True), B,
        None if compress_plan is None else compress_plan.data_ptr(), int(n_compress),
        None if write_plan is None else write_plan.data_ptr(), int(n_write), int(round_scale)), stream)


def _check_plans(compress_plan, n_compress, write_plan, n_write):
    for name, plan, n in (("compress_plan", compress_plan, n_compress),
                          ("write_plan", write_plan, n_write)):
        if int(n) > 0:
            _need(plan is not None and plan.is_cuda and plan.is_contiguous()
                  and plan.numel() * plan.element_size() >= 16 * int(n),
                  f"{name} must be a contiguous device tensor of at least {int(n)} entries")


def kvc_c128_online_prefill(state, kv_score_in, out, ape, indices, compress_plan, n_compress,
                            write_plan, n_write, load_indices=None, stream=None):
    """compress_plan / write_plan: device uint8 tensors of 16-byte entries (or
    int32 [n,4]); n_compress / n_write: entries to process."""
    import torch
    N, B = kv_score_in.shape[0], indices.shape[0]
    _shape_ok(state, (None, 384), "state")
    _shape_ok(kv_score_in, (N, 256), "kv_score_in")
    _shape_ok(out, (N, 128), "out")
    _shape_ok(ape, (128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    if load_indices is not None:
        _shape_ok(load_indices, (B,), "load_indices")
    _check_plans(compress_plan, n_compress, write_plan, n_write)
    cp = None if compress_plan is None else compress_plan.data_ptr()
    wp = None if write_plan is None else write_plan.data_ptr()
    return _invoke("kvc_c128_online_prefill", (
        _dptr(state, torch.float32, "state"), state.shape[0],
        _dptr(kv_score_in, torch.float32, "kv_score_in"), _dptr(out, torch.float32, "out"),
        kv_score_in.shape[0], _dptr(ape, torch.float32, "ape"),
        _dptr(indices, torch.int32, "indices"),
        _dptr(load_indices, torch.int32, "load_indices", optional=True), indices.shape[0],
        cp, int(n_compress), wp, int(n_write)), stream)


def kvc_c128_online_prefill_fused(state, kv_score_in, ape, indices, items, n_items, out=None,
                                  out_fp8=None, out_scale=None, round_scale: bool = True,
                                  load_indices=None, stream=None):
    """Single-launch prefill over device work items (see items_to_device);
    chunk-closing vectors go to out (fp32 [N,128]) or, with out_fp8 / out_scale,
    through the rotate / e4m3 epilogue."""
    import torch
    N, B = kv_score_in.shape[0], indices.shape[0]
    _shape_ok(state, (None, 384), "state")
    _shape_ok(kv_score_in, (N, 256), "kv_score_in")
    _shape_ok(ape, (128, 128), "ape")
    _shape_ok(indices, (B,), "indices")
    if load_indices is not None:
        _shape_ok(load_indices, (B,), "load_indices")
    _need((out is None) != (out_fp8 is None), "give either out or out_fp8 / out_scale")
    if out is not None:
        _shape_ok(out, (N, 128), "out")
    else:
        _shape_ok(out_fp8, (N, 128), "out_fp8")
        _shape_ok(out_scale, (N,), "out_scale")
    if int(n_items) > 0:
        _need(items is not None and items.is_cuda and items.is_contiguous()
              and items.numel() * items.element_size() >= 32 * int(n_items),
              f"items must be a contiguous device tensor of at least {int(n_items)} entries")
    return _invoke("kvc_c128_online_prefill_fused", (
        _dptr(state, torch.float32, "state"), state.shape[0],
        _dptr(kv_score_in, torch.float32, "kv_score_in"),
        _dptr(out, torch.float32, "out", optional=True),
        _dptr(out_fp8, torch.uint8, "out_fp8", optional=True),
        _dptr(out_scale, torch.float32, "out_scale", optional=True), int(round_scale), N,
        _dptr(ape, torch.float32, "ape"), _dptr(indices, torch.int32, "indices"),
        _dptr(load_indices, torch.int32, "load_indices", optional=True), B,
        None if items is None else items.data_ptr(), int(n_items)), stream)


def kvc_diag_convert(x, bf16_out=None, fp8_out=None, stream=None):
    import torch
    return _invoke("kvc_diag_convert", (
        _dptr(x, torch.float32, "x"), _dptr(bf16_out, torch.int16, "bf16_out", optional=True),
        _dptr(fp8_out, torch.uint8, "fp8_out", optional=True), x.numel()), stream)


def stream_read_sink_words(nbytes: int, loads_per_lane: int) -> int:
    """Sink words kvc_diag_stream_read needs: one per wave."""
    return 4 * -(-int(nbytes) // (4096 * int(loads_per_lane)))


def kvc_diag_stream_read(src, sink, loads_per_lane: int = 4, fold: bool = False, stream=None):
    """Plain streaming read of a device tensor's bytes (see kvc.h); sink is a
    device int32/uint32 tensor of at least stream_read_sink_words() entries;
    fold=True writes each wave's XOR of the words it read to the sink."""
    nbytes = src.numel() * src.element_size()
    nbytes -= nbytes % 16
    _need(src.is_cuda and src.is_contiguous(), "src must be a contiguous device tensor")
    _need(sink.is_cuda and sink.element_size() == 4 and sink.is_contiguous(),
          "sink must be a contiguous device tensor of 4-byte words")
    return _invoke("kvc_diag_stream_read", (src.data_ptr(), nbytes, sink.data_ptr(), sink.numel(),
                                            int(loads_per_lane), int(bool(fold))), stream)


def kvc_diag_empty_launch(workgroups: int, threads: int, arg_bytes: int = 0, stream=None):
    """Launch an empty kernel of the given grid (launch-floor measurements);
    arg_bytes (0, 64, 112, 136 or 448) sizes its unused argument block."""
    return _invoke("kvc_diag_empty_launch", (int(workgroups), int(threads), int(arg_bytes)),
                   stream)


def plans_to_device(plan: np.ndarray, device="cuda"):
    """Host PLAN_DTYPE array -> device uint8 tensor [n, 16] (16-byte aligned)."""
    import torch
    raw = np.ascontiguousarray(plan, PLAN_DTYPE).view(np.uint8).reshape(-1, 16)
    if raw.shape[0] == 0:
        return torch.empty((1, 16), dtype=torch.uint8, device=device)
    return torch.from_numpy(raw.copy()).to(device)


def items_to_device(items: np.ndarray, device="cuda"):
    """Host ITEM_DTYPE array -> device uint8 tensor [n, 32] (16-byte aligned)."""
    import torch
    raw = np.ascontiguousarray(items, ITEM_DTYPE).view(np.uint8).reshape(-1, 32)
    if raw.shape[0] == 0:
        return torch.empty((1, 32), dtype=torch.uint8, device=device)
    return torch.from_numpy(raw.copy()).to(device)


def _bf16_view(t, name, min_last=128):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    if t.dtype not in (torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 bit patterns (bfloat16/int16), got {t.dtype}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    if min_last is not None and t.shape[-1] < min_last:
        raise ValueError(f"{name} rows must hold at least {min_last} channels")
    return t
