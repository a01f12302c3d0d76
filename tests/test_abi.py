"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, its host planners agree with the oracle's independent planners, and
argument validation rejects bad calls before anything reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from kv_cache_compression_pool_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kvc.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(kvc.EXPORTS) == set(names)
    assert L.kvc_version() >= 100


def test_header_serves_a_plain_c_client(tmp_path):
    """include/kvc.h compiles as C11 and the library links into a C program
    (the client the GPU tests run; built here into a scratch path)."""
    from tests.c_abi import build_client
    out = build_client.build(str(tmp_path / "kvc_c_client"))
    assert os.access(out, os.X_OK)


def test_pool_planner_matches_oracle():
    g = np.random.default_rng(1)
    for _ in range(50):
        lens = g.integers(0, 300, int(g.integers(1, 9)))
        assert np.array_equal(kvc.kvc_plan_pool_prefill(lens), oracle.pool_plan(lens))


def test_c128_planner_matches_oracle():
    g = np.random.default_rng(2)
    for _ in range(300):
        B = int(g.integers(1, 6))
        el = g.integers(1, 700, B)
        sl = el + g.integers(0, 700, B)
        n = int(el.sum())
        for pad in (False, True):
            a = kvc.kvc_c128_plan_prefill(sl, el, n, pad)
            b = oracle.c128_plan(sl, el, n, pad)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _is_pad(rec):
    return int(rec["ragged_id"]) == kvc.PLAN_SENTINEL


def test_c128_fused_planner_matches_oracle_plans():
    """The fused work items hold exactly the oracle's plans, pair a request's
    first compress plan with its write plan only when that compress plan
    starts mid-chunk (the one state read a write can conflict with), and are
    ordered paired / compress-only / write-only, each in request order."""
    g = np.random.default_rng(3)
    key = lambda r: tuple(int(r[f]) for f in ("ragged_id", "batch_id", "position", "window_len"))
    for trial in range(300):
        B = int(g.integers(1, 7))
        el = g.integers(1, 700, B)
        sl = el + g.integers(0, 700, B)
        if trial % 3 == 0:                  # many chunk-aligned lengths
            sl = np.maximum(sl - sl % 128, 128) + 128 * (g.random(B) < 0.5)
            el = np.minimum(el, sl)
        n = int(el.sum())
        cp, wp = oracle.c128_plan(sl, el, n)
        items = kvc.kvc_c128_plan_prefill_fused(sl, el, n)
        assert items.size == cp.size + wp.size - sum(
            1 for it in items if not _is_pad(it["compress"]) and not _is_pad(it["write"]))
        got_c = [key(it["compress"]) for it in items if not _is_pad(it["compress"])]
        got_w = [key(it["write"]) for it in items if not _is_pad(it["write"])]
        assert sorted(got_c) == sorted(key(r) for r in cp)
        assert sorted(got_w) == sorted(key(r) for r in wp)
        kinds = []
        for it in items:
            c, w = it["compress"], it["write"]
            assert not (_is_pad(c) and _is_pad(w))
            if not _is_pad(c) and not _is_pad(w):
                b = int(c["batch_id"])
                assert int(w["batch_id"]) == b
                prefix = int(sl[b] - el[b])
                first_pos = int(c["position"]) - int(c["window_len"]) + 1
                assert first_pos == prefix and prefix % 128 != 0
                kinds.append(0)
            elif not _is_pad(c):
                b = int(c["batch_id"])
                first_pos = int(c["position"]) - int(c["window_len"]) + 1
                # a first, mid-chunk compress plan with a write plan must be paired
                assert not (first_pos % 128 != 0 and sl[b] % 128 != 0)
                kinds.append(1)
            else:
                b = int(w["batch_id"])
                first_pos = int(w["position"]) - int(w["window_len"]) + 1
                # an unpaired write plan: no compress plan of its request reads the state
                assert first_pos == int(sl[b] - el[b]) or int(sl[b] - el[b]) % 128 == 0
                kinds.append(2)
        assert kinds == sorted(kinds)
        for k in (0, 1, 2):
            sel = [it for it, kk in zip(items, kinds) if kk == k]
            half = "write" if k == 2 else "compress"
            bids = [(int(it[half]["batch_id"]), int(it[half]["position"])) for it in sel]
            assert bids == sorted(bids)
        cap = kvc.kvc_c128_fused_capacity(n, B)
        assert items.size <= cap <= n                       # the documented bound holds
        padded = kvc.kvc_c128_plan_prefill_fused(sl, el, n, pad_to_capacity=True)
        assert padded.size == cap
        assert np.array_equal(padded[:items.size], items)
        assert all(_is_pad(it["compress"]) and _is_pad(it["write"]) for it in padded[items.size:])
        wide = kvc.kvc_c128_plan_prefill_fused(sl, el, n, pad_to_capacity=True, capacity=n)
        assert wide.size == n and np.array_equal(wide[:items.size], items)
        if items.size > 1:
            with pytest.raises(kvc.KvcError) as e:
                kvc.kvc_c128_plan_prefill_fused(sl, el, n, capacity=items.size - 1)
            assert e.value.code == kvc.KVC_ERR_PLAN


def test_c128_fused_capacity_bound_exhaustive():
    """The documented item bound floor(N/128) + 2B holds for every single
    request with prefix and extend up to 400 tokens, and for pairs of them."""
    for prefix in range(0, 400, 7):
        for E in range(1, 400, 3):
            n = kvc.kvc_c128_plan_prefill_fused([prefix + E], [E], E).size
            assert n <= kvc.kvc_c128_fused_capacity(E, 1), (prefix, E)
    g = np.random.default_rng(5)
    for _ in range(500):
        el = g.integers(1, 400, 2)
        sl = el + g.integers(0, 400, 2)
        N = int(el.sum())
        assert kvc.kvc_c128_plan_prefill_fused(sl, el, N).size <= kvc.kvc_c128_fused_capacity(N, 2)


def test_planner_errors():
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_c128_plan_prefill([10], [11], 11)
    assert e.value.code == kvc.KVC_ERR_PLAN
    with pytest.raises(kvc.KvcError):
        kvc.kvc_c128_plan_prefill([10, 20], [5, 5], 11)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_plan_pool_prefill([10], pool_size=8)
    assert e.value.code == kvc.KVC_ERR_UNSUPPORTED
    L = kvc.lib()
    n = ctypes.c_int64()
    out = np.empty(1, np.int32)
    lens = np.array([64], np.int64)
    rc = L.kvc_plan_pool_prefill(lens.ctypes.data, 1, 16, out.ctypes.data, 1, ctypes.byref(n))
    assert rc == kvc.KVC_ERR_PLAN and n.value == 4          # capacity too small, count reported
    assert b"capacity" in L.kvc_last_error()


def test_device_entry_points_validate_before_launch():
    # Every call below must fail in host-side validation (nothing is enqueued,
    # no HIP call is made), so it is safe without a GPU.
    L = kvc.lib()
    p = ctypes.c_void_p(0x1000)          # aligned dummy, never dereferenced
    # unsupported pool size
    assert L.kvc_compress_prefill(p, 128, p, 128, 16, p, 8, None, 1, p, p, 1, None, None) \
        == kvc.KVC_ERR_UNSUPPORTED
    # NULL pointers
    assert L.kvc_compress_prefill(None, 128, p, 128, 16, p, 16, None, 1, p, p, 1, None, None) \
        == kvc.KVC_ERR_NULL
    # bad stride, misalignment, too few rows
    assert L.kvc_compress_prefill(p, 100, p, 128, 16, p, 16, None, 1, p, p, 1, None, None) \
        == kvc.KVC_ERR_SHAPE
    assert L.kvc_compress_prefill(ctypes.c_void_p(0x1002), 128, p, 128, 16, p, 16, None, 1, p, p,
                                  1, None, None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_compress_prefill(p, 128, p, 128, 15, p, 16, None, 1, p, p, 1, None, None) \
        == kvc.KVC_ERR_SHAPE
    # sizes and strides the kernels take as 32-bit values
    assert L.kvc_compress_prefill(p, 1 << 31, p, 128, 16, p, 16, None, 1, p, p, 1, None, None) \
        == kvc.KVC_ERR_SHAPE
    assert b"exceed 2^31-1" in L.kvc_last_error()
    assert L.kvc_compress_prefill_paged(p, 128, p, 128, 16, p, 16, None, 1, p, 1 << 31, 1, p,
                                        None, 1, None) == kvc.KVC_ERR_SHAPE
    assert b"num_pages" in L.kvc_last_error()
    # empty work is a no-op, even with NULL buffers
    assert L.kvc_compress_prefill(None, 0, None, 0, 0, None, 16, None, 0, None, None, 1, None,
                                  None) == kvc.KVC_OK
    assert L.kvc_compress_decode_ring(None, 0, None, None, 0, 0, None, 0, 0, None, None, None, 0,
                                      4, 16, None, None, 0, 1, None, None) == kvc.KVC_OK
    assert L.kvc_compress_decode_ring(p, 4, p, p, 512, 128, p, 512, 128, p, p, p, 4, 4, 12, p, p,
                                      4, 1, None, None) == kvc.KVC_ERR_UNSUPPORTED
    assert L.kvc_compress_decode_ring(p, 4, p, p, 500, 128, p, 512, 128, p, p, p, 4, 4, 16, p, p,
                                      4, 1, None, None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_compress_decode_ring(p, 4, p, p, 512, 128, p, 512, 128, p, p, p, 4, 4, 16, p, p,
                                      4, 1, ctypes.c_void_p(0x1008), None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_c128_online_decode(None, 0, None, None, None, None, None, 0, None) == kvc.KVC_OK
    assert L.kvc_c128_online_decode(p, 4, None, p, p, p, p, 2, None) == kvc.KVC_ERR_NULL
    assert L.kvc_c128_online_decode(p, 4, ctypes.c_void_p(0x1004), p, p, p, p, 2, None) \
        == kvc.KVC_ERR_SHAPE
    assert L.kvc_c128_online_prefill(p, 4, p, p, 8, p, p, None, 1, None, 0, None, 0, None) \
        == kvc.KVC_OK
    assert L.kvc_c128_online_prefill(p, 4, p, p, 8, p, p, None, 1, None, 3, None, 0, None) \
        == kvc.KVC_ERR_NULL
    assert L.kvc_c128_online_prefill(p, 4, p, p, 8, p, p, None, 1, ctypes.c_void_p(0x1008), 3,
                                     None, 0, None) == kvc.KVC_ERR_SHAPE
    # multi-layer c128 decode: layer strides that overlap layers, too many layers
    d = L.kvc_c128_online_decode_layers
    assert d(p, 4 * 384 - 4, 4, p, 2 * 256, p, 2 * 128, p, 128 * 128, p, p, 2, 3, None) \
        == kvc.KVC_ERR_SHAPE
    assert b"kvc_c128_online_decode_layers" in L.kvc_last_error()
    assert d(p, 4 * 384, 4, p, 2 * 256, p, 2 * 128 - 4, p, 128 * 128, p, p, 2, 3, None) \
        == kvc.KVC_ERR_SHAPE
    assert d(p, 4 * 384, 4, p, 2 * 256, p, 2 * 128, p, 128 * 128, p, p, 2, 70000, None) \
        == kvc.KVC_ERR_SHAPE
    assert d(p, 0, 4, p, 0, p, 0, p, 0, p, p, 2, 0, None) == kvc.KVC_OK
    # multi-layer ring decode: too many layers, layer strides that overlap layers
    r = L.kvc_compress_decode_ring_layers
    assert r(p, 4 * 4096, 4, p, p, 4 * 512, 512, 128, p, 4 * 512, 512, 128, p, 2048, p, p, 4, 4,
             16, p, p, 4, 70000, 1, None) == kvc.KVC_ERR_SHAPE
    assert r(p, 4 * 4096 - 8, 4, p, p, 4 * 512, 512, 128, p, 4 * 512, 512, 128, p, 2048, p, p, 4,
             4, 16, p, p, 4, 3, 1, None) == kvc.KVC_ERR_SHAPE
    assert r(p, 4 * 4096, 4, p, p, 4 * 512 - 8, 512, 128, p, 4 * 512, 512, 128, p, 2048, p, p, 4,
             4, 16, p, p, 4, 3, 1, None) == kvc.KVC_ERR_SHAPE
    assert r(p, 4 * 4096, 4, p, p, 4 * 512, 512, 128, p, 4 * 512, 512, 128, p, 2044, p, p, 4, 4,
             16, p, p, 4, 3, 1, None) == kvc.KVC_ERR_SHAPE
    assert r(p, 0, 4, p, p, 0, 512, 128, p, 0, 512, 128, p, 0, p, p, 4, 4, 16, p, p, 4, 0, 1,
             None) == kvc.KVC_OK
    # fused prefill: nothing to do, missing items, both / neither output, misaligned items
    f = L.kvc_c128_online_prefill_fused
    assert f(p, 4, p, p, None, None, 1, 8, p, p, None, 1, None, 0, None) == kvc.KVC_OK
    assert f(p, 4, p, p, None, None, 1, 8, p, p, None, 1, None, 2, None) == kvc.KVC_ERR_NULL
    assert f(p, 4, p, p, p, p, 1, 8, p, p, None, 1, p, 2, None) == kvc.KVC_ERR_NULL
    assert f(p, 4, p, None, None, None, 1, 8, p, p, None, 1, p, 2, None) == kvc.KVC_ERR_NULL
    assert f(p, 4, p, None, p, None, 1, 8, p, p, None, 1, p, 2, None) == kvc.KVC_ERR_NULL
    assert f(p, 4, p, p, None, None, 1, 8, p, p, None, 1, ctypes.c_void_p(0x1008), 2, None) \
        == kvc.KVC_ERR_SHAPE
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_c128_plan_prefill_fused([10], [11], 11)
    assert e.value.code == kvc.KVC_ERR_PLAN
    assert kvc.kvc_c128_fused_capacity(-1, 4) == 0
    assert kvc.kvc_c128_fused_capacity(1000, 4) == 1000 // 128 + 8
    assert kvc.kvc_c128_fused_capacity(10, 4) == 8
    assert kvc.kvc_c128_fused_capacity(5, 4) == 5
    assert L.kvc_diag_convert(p, None, None, 3, None) == kvc.KVC_ERR_SHAPE
    assert b"even" in L.kvc_last_error()
    # streaming read: size, load count, sink size; empty launch: grid checks
    sr = L.kvc_diag_stream_read
    assert sr(p, 40, p, 8, 8, 1, None) == kvc.KVC_ERR_SHAPE
    assert sr(p, 4096, p, 8, 6, 1, None) == kvc.KVC_ERR_UNSUPPORTED
    assert sr(p, 0, None, 0, 8, 0, None) == kvc.KVC_OK
    assert sr(p, 3 * 4096 * 8, p, 11, 8, 0, None) == kvc.KVC_ERR_SHAPE
    assert b"sink needs 12 words" in L.kvc_last_error()
    assert sr(ctypes.c_void_p(0x1008), 4096, p, 8, 8, 1, None) == kvc.KVC_ERR_SHAPE
    assert kvc.stream_read_sink_words(3 * 4096 * 8 + 16, 8) == 16
    assert L.kvc_diag_empty_launch(4, 0, 0, None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_diag_empty_launch(4, 1025, 0, None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_diag_empty_launch(-1, 64, 0, None) == kvc.KVC_ERR_SHAPE
    assert L.kvc_diag_empty_launch(4, 64, 100, None) == kvc.KVC_ERR_UNSUPPORTED
    assert L.kvc_diag_empty_launch(0, 64, 0, None) == kvc.KVC_OK


def test_last_error_is_per_thread():
    """Each host thread reads the message of its own last failed call, even
    while other threads fail differently at the same time."""
    import threading
    L = kvc.lib()
    n = ctypes.c_int64()
    bad_pool = np.array([32], np.int64)
    errors = []

    def fail_pool_size():
        for _ in range(500):
            rc = L.kvc_plan_pool_prefill(bad_pool.ctypes.data, 1, 8, None, 0, ctypes.byref(n))
            msg = L.kvc_last_error()
            if rc != kvc.KVC_ERR_UNSUPPORTED or b"pool_size 8" not in msg:
                errors.append(("pool", rc, msg))

    def fail_convert():
        for _ in range(500):
            rc = L.kvc_diag_convert(ctypes.c_void_p(0x1000), None, None, 3, None)
            msg = L.kvc_last_error()
            if rc != kvc.KVC_ERR_SHAPE or b"even" not in msg:
                errors.append(("convert", rc, msg))

    def succeed():
        out = np.empty(2, np.int32)
        for _ in range(500):
            rc = L.kvc_plan_pool_prefill(bad_pool.ctypes.data, 1, 16, out.ctypes.data, 2,
                                         ctypes.byref(ctypes.c_int64()))
            if rc != kvc.KVC_OK or L.kvc_last_error() != b"":
                errors.append(("ok", rc, L.kvc_last_error()))

    threads = [threading.Thread(target=f) for f in (fail_pool_size, fail_convert, succeed) * 2]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_plan_struct_layout():
    assert kvc.PLAN_DTYPE.itemsize == 16
    assert kvc.ITEM_DTYPE.itemsize == 32
    assert kvc.PLAN_DTYPE == oracle.PLAN_DTYPE


def test_prepare_accepts_device_entry_points_only():
    """prepare() returns a PreparedCall for device entry points; anything else
    (here a host planner, which simply runs) is refused."""
    with pytest.raises(TypeError):
        kvc.prepare(kvc.kvc_plan_pool_prefill, np.array([32], np.int64))
    assert callable(kvc.PreparedCall.__call__)


def test_prepared_call_passes_64_bit_values_and_null():
    """A PreparedCall hands its pre-converted values to the C function as
    their declared C types (no GPU work: each call stops at host validation).
    A 64-bit size whose low 32 bits are zero, a pointer above 4 GiB and a
    NULL each reach the library intact, or the error named would differ."""
    fn = "kvc_c128_online_decode_layers"
    hi = 1 << 32                                    # 16-byte aligned, above 4 GiB
    ptrs = dict(state=hi, kv=hi + 0x1000, out=hi + 0x2000, ape=hi + 0x3000,
                idx=hi + 0x4000, sl=hi + 0x5000)

    def call(state, num_slots, batch, num_layers, out):
        # state, state_ls, num_slots, in, in_ls, out, out_ls, ape, ape_ls, indices, seq_lens,
        # batch, num_layers (the stream is the call's own, here the null stream)
        return kvc.PreparedCall(fn, (state, 0, num_slots, ptrs["kv"], 0, out, 0, ptrs["ape"], 0,
                                     ptrs["idx"], ptrs["sl"], batch, num_layers), 0)

    with pytest.raises(kvc.KvcError, match="negative size"):
        call(ptrs["state"], 8, -(1 << 40), 1, ptrs["out"])()   # low 32 bits are 0
    with pytest.raises(kvc.KvcError, match="NULL pointer"):
        call(None, 8, 1, 1, ptrs["out"])()
    with pytest.raises(kvc.KvcError, match="num_layers exceeds 65535"):
        call(ptrs["state"], 8, 1, 70000, ptrs["out"])()       # out truncated would be NULL
