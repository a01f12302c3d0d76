"""CPU oracle for softmax-gated token-pool KV compression (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and it shares no code with them.

The arithmetic lives in ``kvc_oracle.c`` (plain scalar C, built with
``-O2 -ffp-contract=off -fno-tree-vectorize``, no fast-math).  This module
only marshals numpy arrays into it.  Each wrapper names the page passage the
C function follows:

* kpool_compress page (vLLM ``vllm.models.glm5next.amd.ops.kpool_compress``):
  ``_kpool_softmax_rotate_write_cache_kernel`` (pool-16 prefill) and
  ``_kpool_decode_update_batched_kernel`` (tail-ring decode with verify tokens).
* c128_online.cuh page (SGLang ``deepseek_v4/c128_online.cuh``):
  ``flash_c128_online_decode``, ``flash_c128_online_prefill`` and
  ``plan_online_prefill_host``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "libkvc_oracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-tree-vectorize", "-fno-fast-math",
          "-std=c11", "-shared", "-fPIC"]


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float


def _declare(L):
    L.orc_bf16_rne.argtypes = [_f32]
    L.orc_bf16_rne.restype = ctypes.c_uint16
    L.orc_e4m3_encode.argtypes = [_f32]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_decode.restype = ctypes.c_double
    L.orc_bf16_rne_array.argtypes = [_p, _p, _i64]
    L.orc_e4m3_encode_array.argtypes = [_p, _p, _i64]
    L.orc_hadamard128.argtypes = [_p, _p]
    L.orc_softmax_mean.argtypes = [_p, _i64, _p, _i64, _p, _i32, _p]
    L.orc_pool_compress.argtypes = [_p, _i64, _p, _i64, _p, _i32, _i32, _p, _p, _p, _p]
    L.orc_compress_prefill.argtypes = [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i32, _i32,
                                       _p, _p, _p]
    L.orc_pool_epilogue_rows.argtypes = [_p, _i64, _i32, _p, _p]
    L.orc_pool_plan.argtypes = [_p, _i64, _i32, _p, _i64]
    L.orc_pool_plan.restype = _i64
    L.orc_ring_decode.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _i64, _p, _p, _p,
                                  _i64, _i32, _i32, _i32, _p, _p, _i64, _p, _p]
    L.orc_seed_tail_ring.argtypes = [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i32]
    L.orc_compress_prefill_paged.argtypes = [_p, _i64, _p, _i64, _p, _p, _i64, _i32, _i32, _p,
                                             _i64, _p, _p]
    L.orc_ring_decode_paged.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _i64, _p, _p, _p,
                                        _i64, _i32, _i32, _i32, _p, _i64]
    L.orc_c128_decode.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _i64]
    L.orc_c128_plan.argtypes = [_p, _p, _i64, _i64, _p, _p, _i32, _p, _p]
    L.orc_c128_plan.restype = _i32
    L.orc_c128_prefill.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _p, _u32, _p, _u32]


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars
def bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, nearest-even (the pages' ``.to(bfloat16)``)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.empty(x.size, np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_encode(q) -> np.ndarray:
    """fp32 -> OCP e4m3 code, nearest-even, saturating at 448."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32).ravel())
    out = np.empty(q.size, np.uint8)
    lib().orc_e4m3_encode_array(_ptr(q), _ptr(out), q.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8).ravel()
    f = lib().orc_e4m3_decode
    return np.array([f(int(v)) for v in c], dtype=np.float64)


def hadamard128(x) -> np.ndarray:
    """y = H x / sqrt(128), Sylvester order, correctly rounded to fp32."""
    x = _c(x, np.float32)
    assert x.shape == (128,)
    y = np.empty(128, np.float32)
    lib().orc_hadamard128(_ptr(x), _ptr(y))
    return y


# ---------------------------------------------------------------- pool-16
def softmax_mean(keys_bf16, scores_bf16, ape) -> np.ndarray:
    """Per-channel softmax(score+ape)-weighted mean of one pool's keys."""
    k = _c(keys_bf16, np.uint16)
    s = _c(scores_bf16, np.uint16)
    a = _c(ape, np.float32)
    P = k.shape[0]
    assert k.shape == s.shape == a.shape == (P, 128)
    x = np.empty(128, np.float32)
    lib().orc_softmax_mean(_ptr(k), 128, _ptr(s), 128, _ptr(a), P, _ptr(x))
    return x


def pool_compress(keys_bf16, scores_bf16, ape, round_scale: bool):
    """One pool -> (code[128] u8, scale f32, x[128] f32, y[128] f32)."""
    k = _c(keys_bf16, np.uint16)
    s = _c(scores_bf16, np.uint16)
    a = _c(ape, np.float32)
    P = k.shape[0]
    assert k.shape == s.shape == a.shape == (P, 128)
    code = np.empty(128, np.uint8)
    scale = np.empty(1, np.float32)
    x = np.empty(128, np.float32)
    y = np.empty(128, np.float32)
    lib().orc_pool_compress(_ptr(k), 128, _ptr(s), 128, _ptr(a), P, int(round_scale),
                            _ptr(code), _ptr(scale), _ptr(x), _ptr(y))
    return code, float(scale[0]), x, y


def pool_epilogue(x_rows, round_scale: bool):
    """Epilogue only (bf16, rotate, bf16, quantise) from given fp32 pooled
    vectors [n,128] -> (codes [n,128] u8, scales [n] f32)."""
    x = _c(x_rows, np.float32).reshape(-1, 128)
    n = x.shape[0]
    code = np.empty((n, 128), np.uint8)
    scale = np.empty(n, np.float32)
    if n:
        lib().orc_pool_epilogue_rows(_ptr(x), n, int(round_scale), _ptr(code), _ptr(scale))
    return code, scale


def pool_plan(seq_lens, pool_size: int = 16) -> np.ndarray:
    """Row of the first token of every complete pool in a ragged packing."""
    sl = _c(seq_lens, np.int64)
    cap = int(np.sum(sl // pool_size))
    out = np.empty(max(cap, 1), np.int32)
    n = lib().orc_pool_plan(_ptr(sl), sl.size, pool_size, _ptr(out), cap)
    assert n == cap
    return out[:n].copy()


def compress_prefill(keys_bf16, scores_bf16, ape, pool_src_row, round_scale: bool,
                     pool_size: int = 16, pool_range=None, out=None):
    """Ragged prefill.  keys/scores: [T,128] bf16 patterns; pool_src_row: [n]
    int32 or None (pool p at row p*P).  Returns (codes [n,128] u8,
    scales [n] f32, x [n,128] f32)."""
    k = _c(keys_bf16, np.uint16)
    s = _c(scores_bf16, np.uint16)
    a = _c(ape, np.float32)
    assert a.shape == (pool_size, 128)
    if pool_src_row is None:
        n = k.shape[0] // pool_size
        rows = None
    else:
        rows = _c(pool_src_row, np.int32)
        n = rows.size
    if out is None:
        out = (np.empty((n, 128), np.uint8), np.empty(n, np.float32),
               np.empty((n, 128), np.float32))
    code, scale, x = out
    b, e = (0, n) if pool_range is None else pool_range
    lib().orc_compress_prefill(_ptr(k), k.shape[1], _ptr(s), s.shape[1], _ptr(a), _ptr(rows),
                               b, e, pool_size, int(round_scale), _ptr(code), _ptr(scale),
                               _ptr(x))
    return code, scale, x


def ring_decode(ring, tail_slot_mapping, key, score, ape, slot_mapping, positions,
                num_out: int, round_scale: bool, pool_size: int = 16,
                out_code=None, out_scale=None, pools_out=None):
    """Tail-ring decode.  ``ring`` ([nb,2,P,128] u16) is updated in place.
    key/score: [R, next_n, 128] bf16 patterns; maps: [R, next_n] int32.
    Returns (out_code [num_out,128], out_scale [num_out]); rows not written
    keep the content of the supplied arrays (zeros if None).  ``pools_out``
    (optional pair of uint16 [num_out,P,128] arrays) receives the gathered
    keys / scores of every completion."""
    assert ring.dtype == np.uint16 and ring.flags["C_CONTIGUOUS"]
    nb = ring.shape[0]
    R, nn = key.shape[0], key.shape[1]
    k = _c(key, np.uint16)
    s = _c(score, np.uint16)
    ts = _c(tail_slot_mapping, np.int32)
    sm = _c(slot_mapping, np.int32)
    pos = _c(positions, np.int32)
    a = _c(ape, np.float32)
    if out_code is None:
        out_code = np.zeros((num_out, 128), np.uint8)
    if out_scale is None:
        out_scale = np.zeros(num_out, np.float32)
    lib().orc_ring_decode(_ptr(ring), nb, _ptr(ts), _ptr(k), nn * 128, 128, _ptr(s), nn * 128,
                          128, _ptr(a), _ptr(sm), _ptr(pos), R, nn, pool_size,
                          int(round_scale), _ptr(out_code), _ptr(out_scale), num_out,
                          _ptr(pools_out[0]) if pools_out else None,
                          _ptr(pools_out[1]) if pools_out else None)
    return out_code, out_scale


def compress_prefill_paged(keys_bf16, scores_bf16, ape, pool_src_row, round_scale: bool,
                           cache, loc, write_mask=None, pool_size: int = 16):
    """Pool-16 prefill into a page-size-1 cache ([pages,132] uint8, updated in
    place): codes at bytes 0..127 of page loc[p], fp32 scale at 128..131."""
    k = _c(keys_bf16, np.uint16)
    s = _c(scores_bf16, np.uint16)
    assert cache.dtype == np.uint8 and cache.flags["C_CONTIGUOUS"] and cache.shape[1] == 132
    lc = _c(loc, np.int64)
    rows = None if pool_src_row is None else _c(pool_src_row, np.int32)
    n = lc.size
    wm = None if write_mask is None else _c(write_mask, np.uint8)
    lib().orc_compress_prefill_paged(_ptr(k), k.shape[1], _ptr(s), s.shape[1],
                                     _ptr(_c(ape, np.float32)), _ptr(rows), n, pool_size,
                                     int(round_scale), _ptr(cache), cache.shape[0], _ptr(lc),
                                     _ptr(wm))
    return cache


def ring_decode_paged(ring, tail_slot_mapping, key, score, ape, slot_mapping, positions,
                      cache, round_scale: bool, pool_size: int = 16):
    """Ring decode writing completions into a page-size-1 cache."""
    assert ring.dtype == np.uint16 and ring.flags["C_CONTIGUOUS"]
    assert cache.dtype == np.uint8 and cache.flags["C_CONTIGUOUS"] and cache.shape[1] == 132
    R, nn = key.shape[0], key.shape[1]
    lib().orc_ring_decode_paged(_ptr(ring), ring.shape[0], _ptr(_c(tail_slot_mapping, np.int32)),
                                _ptr(_c(key, np.uint16)), nn * 128, 128,
                                _ptr(_c(score, np.uint16)), nn * 128, 128,
                                _ptr(_c(ape, np.float32)), _ptr(_c(slot_mapping, np.int32)),
                                _ptr(_c(positions, np.int32)), R, nn, pool_size,
                                int(round_scale), _ptr(cache), cache.shape[0])
    return cache


def seed_tail_ring(ring, key, score, tslot, pool_size: int = 16):
    """Seed the tail ring ([nb,2,P,128] u16, updated in place) from a prefill
    batch: key/score [n,128] bf16 patterns, tslot [n] int32."""
    assert ring.dtype == np.uint16 and ring.flags["C_CONTIGUOUS"]
    k = _c(key, np.uint16)
    s = _c(score, np.uint16)
    ts = _c(tslot, np.int32)
    lib().orc_seed_tail_ring(_ptr(ring), ring.shape[0], _ptr(k), k.shape[1], _ptr(s), s.shape[1],
                             _ptr(ts), ts.size, pool_size)
    return ring


# ---------------------------------------------------------------- pool-128 online
PLAN_DTYPE = np.dtype([("ragged_id", "<u4"), ("batch_id", "<u4"), ("position", "<u4"),
                       ("window_len", "<u4")])


def c128_decode(state, kv_score_in, ape, indices, seq_lens, out=None):
    """Online decode.  ``state`` ([S,384] f32) is updated in place.  Returns
    ``out`` ([B,128] f32); rows not emitted keep their content."""
    assert state.dtype == np.float32 and state.flags["C_CONTIGUOUS"]
    x = _c(kv_score_in, np.float32)
    B = x.shape[0]
    if out is None:
        out = np.zeros((B, 128), np.float32)
    lib().orc_c128_decode(_ptr(state), state.shape[0], _ptr(x), _ptr(out),
                          _ptr(_c(ape, np.float32)), _ptr(_c(indices, np.int32)),
                          _ptr(_c(seq_lens, np.int32)), B)
    return out


def c128_decode_quant(state, kv_score_in, ape, indices, seq_lens, round_scale: bool):
    """Decode, then the pool-16 epilogue (bf16, rotation, bf16, e4m3) on every
    emitted vector.  Returns (emitted row mask, codes [B,128], scales [B],
    fp32 out [B,128]); non-emitted rows of codes / scales are zero."""
    x = _c(kv_score_in, np.float32)
    B = x.shape[0]
    out = np.full((B, 128), np.nan, np.float32)
    c128_decode(state, x, ape, indices, seq_lens, out=out)
    emit = ~np.isnan(out[:, 0])
    codes = np.zeros((B, 128), np.uint8)
    scales = np.zeros(B, np.float32)
    codes[emit], scales[emit] = pool_epilogue(out[emit], round_scale)
    return emit, codes, scales, out


def c128_prefill_quant(state, kv_score_in, ape, indices, cplan, wplan, round_scale: bool,
                       load_indices=None):
    """Prefill, then the pool-16 epilogue on every chunk-closing vector.
    Returns (written row mask, codes [N,128], scales [N], fp32 out [N,128])."""
    x = _c(kv_score_in, np.float32)
    N = x.shape[0]
    out = np.full((max(N, 1), 128), np.nan, np.float32)
    c128_prefill(state, x, ape, indices, cplan, wplan, load_indices=load_indices, out=out)
    rows = ~np.isnan(out[:, 0])
    codes = np.zeros((out.shape[0], 128), np.uint8)
    scales = np.zeros(out.shape[0], np.float32)
    codes[rows], scales[rows] = pool_epilogue(out[rows], round_scale)
    return rows, codes, scales, out


def c128_plan(seq_lens, extend_lens, num_tokens: int, pad: bool = False):
    """Compress / write plan lists (structured arrays of PLAN_DTYPE)."""
    sl = _c(seq_lens, np.int64)
    el = _c(extend_lens, np.int64)
    cap = max(int(num_tokens), 1)
    cp = np.zeros(cap, PLAN_DTYPE)
    wp = np.zeros(cap, PLAN_DTYPE)
    nc = ctypes.c_uint32()
    nw = ctypes.c_uint32()
    rc = lib().orc_c128_plan(_ptr(sl), _ptr(el), sl.size, num_tokens, _ptr(cp), _ptr(wp),
                             int(pad), ctypes.byref(nc), ctypes.byref(nw))
    if rc != 0:
        raise ValueError("invalid c128 prefill lengths")
    return cp[:nc.value].copy(), wp[:nw.value].copy()


def c128_prefill(state, kv_score_in, ape, indices, cplan, wplan, load_indices=None,
                 out=None):
    """Online ragged prefill.  ``state`` updated in place; returns ``out``
    ([N,128] f32, only chunk-closing rows written)."""
    assert state.dtype == np.float32 and state.flags["C_CONTIGUOUS"]
    x = _c(kv_score_in, np.float32)
    N = x.shape[0]
    if out is None:
        out = np.zeros((max(N, 1), 128), np.float32)
    cp = np.ascontiguousarray(cplan, PLAN_DTYPE)
    wp = np.ascontiguousarray(wplan, PLAN_DTYPE)
    li = None if load_indices is None else _c(load_indices, np.int32)
    lib().orc_c128_prefill(_ptr(state), state.shape[0], _ptr(x), _ptr(out),
                           _ptr(_c(ape, np.float32)), _ptr(_c(indices, np.int32)), _ptr(li),
                           _ptr(cp) if cp.size else None, cp.size,
                           _ptr(wp) if wp.size else None, wp.size)
    return out
