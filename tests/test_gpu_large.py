"""GPU parity at byte offsets beyond 4 GiB.

Every kernel forms its addresses in 64-bit arithmetic.  Each case places the
rows it checks past the first 4 GiB of a large device allocation (pool-16
keys and scores, prefill tokens and the tail ring, the pool-128 state and
ragged input), runs the kernel through the C ABI on the large buffers, and
compares the result with the oracle run on compact copies of the same seeded
rows.  The rest of each allocation is either never read or filled with
zeros, whose outputs are known exactly.  The device holds 288 GB; a case
allocates at most about 11 GB and releases it.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_pool_amd as kvc
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, rel_err_rows, seed_states
from tests.test_gpu_parity import (VEC_TOL, check_codes, check_scales, compare_state, dev, note,
                                   reference_for)

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("reps", [1, 4100])   # 6 pools: one per wave; 24,600: two per wave
def test_pool16_prefill_rows_past_4gib(reps):
    stride = 1 << 16                                  # elements per row: 128 KiB rows
    R = FOUR_GIB // (2 * stride) + 256                # 33,024 rows, 4.33 GB
    src = np.array([0, 16, R - 96, R - 64, R - 33, R - 16], np.int64)
    assert (src[2:] * stride * 2 >= FOUR_GIB).all()
    g = synth.rng(71, "large_pool16_prefill")
    n = src.size
    kb = synth.bf16_normal(g, (16 * n, 128))
    sb = synth.bf16_normal(g, (16 * n, 128))
    ape = synth.ape_pool16(g)
    note(f"pool16 prefill: {R} rows x {stride} elements, pools at rows {src.tolist()}")
    buf = torch.empty((R, stride), dtype=torch.int16, device="cuda")
    k_rows, s_rows = dev(kb, torch.int16), dev(sb, torch.int16)
    for p, r0 in enumerate(src):
        buf[r0:r0 + 16, :128] = k_rows[16 * p:16 * p + 16]
        buf[r0:r0 + 16, 128:256] = s_rows[16 * p:16 * p + 16]
    # every pool of the launch reads one of the six row groups
    srcs = np.tile(src, reps)
    m = srcs.size
    out = torch.full((m, 128), 0x7F, dtype=torch.uint8, device="cuda")
    scale = torch.full((m,), float("nan"), device="cuda")
    dbg = torch.full((m, 128), float("nan"), device="cuda")
    kvc.kvc_compress_prefill(buf[:, :128], buf[:, 128:256], dev(ape), dev(srcs.astype(np.int32)),
                             m, out, scale, True, dbg)
    torch.cuda.synchronize()
    gc, gs, gx = out.cpu().numpy(), scale.cpu().numpy(), dbg.cpu().numpy()
    del buf
    # repeats of a row group give the same bits; the six distinct pools are
    # then held to the oracle
    for a in (gc, gs, gx):
        rep = a.reshape(reps, n, -1)
        assert np.array_equal(rep.view(np.uint8), np.broadcast_to(rep[:1], rep.shape).view(np.uint8))
    gc, gs, gx = gc[:n], gs[:n], gx[:n]
    rc, rs, rx = oracle.compress_prefill(kb, sb, ape, None, True)
    assert rel_err_rows(gx, rx).max() <= VEC_TOL
    ref_c, ref_s, _ = reference_for(gx, rx, rc, rs, True, "pool16 prefill past 4 GiB")
    check_codes(gc, ref_c, "pool16 prefill past 4 GiB")
    check_scales(gs, ref_s, True, "pool16 prefill past 4 GiB")


def test_ring_decode_blocks_past_4gib():
    R, N = 8, 4
    d = synth.pool16_ring(seed=72, num_requests=R, next_n=N, pad_frac=0.0)
    # every request closes a pool at its third token (positions 16k+13 .. 16k+16)
    base = 16 * np.arange(1, R + 1, dtype=np.int64)[:, None] + 13
    pos = base + np.arange(N)[None, :]
    d["positions"] = pos.astype(np.int32)
    d["tail_slot_mapping"] = (np.arange(R)[:, None] * 16 + pos % 16).astype(np.int32)
    d["slot_mapping"] = np.where(pos % 16 == 15, np.arange(R)[:, None], -1).astype(np.int32)
    nb = FOUR_GIB // 8192 + 1024                      # 525,312 blocks of 8 KiB, 4.30 GB
    first = nb - R
    assert first * 8192 >= FOUR_GIB
    note(f"ring decode: {nb} ring blocks, requests on blocks {first}..{nb - 1}")
    # oracle on the compact ring (blocks 0..R-1)
    ring = d["ring"].copy()
    rc = np.full((R, 128), 0x33, np.uint8)
    rs = np.full(R, 5.0, np.float32)
    pk = np.zeros((R, 16, 128), np.uint16)
    ps = np.zeros((R, 16, 128), np.uint16)
    oracle.ring_decode(ring, d["tail_slot_mapping"], d["key"], d["score"], d["ape"],
                       d["slot_mapping"], d["positions"], R, True, out_code=rc, out_scale=rs,
                       pools_out=(pk, ps))
    # the device ring holds the same blocks at the far end
    big = torch.empty((nb, 2, 16, 128), dtype=torch.int16, device="cuda")
    big[first:] = dev(d["ring"], torch.int16)
    ts_big = d["tail_slot_mapping"] + np.int32(16 * first)
    go = torch.full((R, 128), 0x33, dtype=torch.uint8, device="cuda")
    gs = torch.full((R,), 5.0, device="cuda")
    gx = torch.full((R, 128), float("nan"), device="cuda")
    kvc.kvc_compress_decode_ring(big, dev(ts_big), dev(d["key"], torch.int16),
                                 dev(d["score"], torch.int16), dev(d["ape"]),
                                 dev(d["slot_mapping"]), dev(d["positions"]), go, gs, True,
                                 dbg_pooled=gx)
    torch.cuda.synchronize()
    gring = big[first:].cpu().numpy().view(np.uint16)
    gc, gsc, gx = go.cpu().numpy(), gs.cpu().numpy(), gx.cpu().numpy()
    del big
    assert np.array_equal(gring, ring)
    assert (rs != 5.0).all()                          # every request completed a pool
    _, _, ox = oracle.compress_prefill(pk.reshape(-1, 128), ps.reshape(-1, 128), d["ape"], None,
                                       True)
    assert rel_err_rows(gx, ox).max() <= VEC_TOL
    ref_c, ref_s, _ = reference_for(gx, ox, rc, rs, True, "ring decode past 4 GiB")
    check_codes(gc, ref_c, "ring decode past 4 GiB")
    check_scales(gsc, ref_s, True, "ring decode past 4 GiB")


def test_seed_tail_ring_rows_and_blocks_past_4gib():
    """The last request of a prefill batch: its 40 token rows sit past 4 GiB
    (128 KiB row stride) and its ring block past 4 GiB of the ring."""
    stride = 1 << 16
    T = FOUR_GIB // (2 * stride) + 256                # 33,024 tokens
    n_req = 40
    nb = FOUR_GIB // 8192 + 1024
    assert (T - n_req) * stride * 2 >= FOUR_GIB and (nb - 1) * 8192 >= FOUR_GIB
    g = synth.rng(76, "large_seed")
    kb = synth.bf16_normal(g, (n_req, 128))
    sb = synth.bf16_normal(g, (n_req, 128))
    ring0 = synth.bf16_normal(g, (1, 2, 16, 128))
    pos = np.arange(n_req)
    # compact oracle problem: one request, ring block 0
    ring = ring0.copy()
    oracle.seed_tail_ring(ring, kb, sb, (pos % 16).astype(np.int32))
    note(f"tail-ring seeding: {T} tokens x {stride} elements, ring block {nb - 1} of {nb}")
    buf = torch.empty((T, stride), dtype=torch.int16, device="cuda")
    buf[T - n_req:, :128] = dev(kb, torch.int16)
    buf[T - n_req:, 128:256] = dev(sb, torch.int16)
    tslot = np.full(T, -1, np.int32)                  # earlier tokens: padding, never copied
    tslot[T - n_req:] = 16 * (nb - 1) + pos % 16
    big = torch.empty((nb, 2, 16, 128), dtype=torch.int16, device="cuda")
    big[nb - 1:] = dev(ring0, torch.int16)
    kvc.kvc_seed_tail_ring(big, buf[:, :128], buf[:, 128:256], dev(tslot))
    torch.cuda.synchronize()
    got = big[nb - 1:].cpu().numpy().view(np.uint16)
    del buf, big
    assert np.array_equal(got, ring)
    assert not np.array_equal(ring, ring0)            # the request's last 16 tokens landed


def test_c128_decode_state_past_4gib():
    d = c128_decode_case(seed=73, batch=16, num_slots=64, emit_frac=0.3)
    S = FOUR_GIB // 1536 + 4096                       # 2,800,298 slots of 1.5 KiB, 4.30 GB
    first = S - d["num_slots"]
    assert first * 1536 >= FOUR_GIB
    note(f"c128 decode: {S} state slots, requests on slots {first}..{S - 1}")
    st = d["state"].copy()
    ref = np.full((16, 128), np.nan, np.float32)
    oracle.c128_decode(st, d["kv_score_in"], d["ape"], d["indices"], d["seq_lens"], out=ref)
    big = torch.empty((S, 384), device="cuda")
    big[first:] = dev(d["state"])
    gout = torch.full((16, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode(big, dev(d["kv_score_in"]), gout, dev(d["ape"]),
                               dev(d["indices"] + np.int32(first)), dev(d["seq_lens"]))
    torch.cuda.synchronize()
    gst, gout = big[first:].cpu().numpy(), gout.cpu().numpy()
    del big
    emit = ~np.isnan(ref[:, 0])
    assert emit.any() and not emit.all()
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    assert rel_err_rows(gout[emit], ref[emit]).max() <= VEC_TOL
    compare_state(gst, st, "c128 decode past 4 GiB")


def test_c128_decode_layers_past_4gib():
    """Two layers whose second state copy starts past 4 GiB."""
    d = c128_decode_case(seed=74, batch=16, num_slots=64, emit_frac=0.3)
    S = FOUR_GIB // 1536 + 64                         # layer 1 starts at byte S * 1536 > 4 GiB
    note(f"c128 decode layers: 2 x {S} state slots")
    st = d["state"].copy()
    ref = np.full((16, 128), np.nan, np.float32)
    oracle.c128_decode(st, d["kv_score_in"], d["ape"], d["indices"], d["seq_lens"], out=ref)
    big = torch.empty((2, S, 384), device="cuda")
    big[:, :d["num_slots"]] = dev(d["state"])
    x = dev(d["kv_score_in"]).unsqueeze(0).repeat(2, 1, 1).contiguous()
    a = dev(d["ape"]).unsqueeze(0).repeat(2, 1, 1).contiguous()
    gout = torch.full((2, 16, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode_layers(big, x, gout, a, dev(d["indices"]), dev(d["seq_lens"]))
    torch.cuda.synchronize()
    gst = big[:, :d["num_slots"]].cpu().numpy()
    gout = gout.cpu().numpy()
    del big
    emit = ~np.isnan(ref[:, 0])
    for layer in range(2):
        assert np.array_equal(np.isnan(gout[layer]), np.isnan(ref))
        assert rel_err_rows(gout[layer][emit], ref[emit]).max() <= VEC_TOL
        compare_state(gst[layer], st, f"c128 decode layer {layer} past 4 GiB")


@pytest.mark.parametrize("fused", [False, True])
def test_c128_prefill_rows_and_state_past_4gib(fused):
    """Request 0 extends 32,800 whole chunks from position 0 (4.2 GB of input:
    all zeros except its last chunk); request 1 starts mid-chunk, loads its
    open state from a slot past 4 GiB, closes three chunks and writes its
    state back there.  Its rows and request 0's last chunk lie past 4 GiB."""
    E0, prefix1, E1 = 128 * 32800, 1000, 300
    N = E0 + E1
    assert (E0 - 128) * 1024 >= FOUR_GIB
    g = synth.rng(75, "large_c128_prefill")
    rows0 = g.standard_normal((128, 256), dtype=np.float32)     # request 0's last chunk
    rows1 = g.standard_normal((E1, 256), dtype=np.float32)
    ape = g.standard_normal((128, 128), dtype=np.float32) * np.float32(0.1)
    prior = g.standard_normal((prefix1 % 128, 256), dtype=np.float32)
    # compact oracle problem: request 0' = the last chunk alone, request 1 as is
    state = synth.nan_state(2)
    seed_states(state, np.array([0, 1], np.int32), np.array([0, prefix1 % 128]), prior,
                np.array([128, prefix1]), ape)
    st_ref = state.copy()
    sl, el = np.array([128, prefix1 + E1]), np.array([128, E1])
    cp, wp = oracle.c128_plan(sl, el, 128 + E1)
    ref = np.full((128 + E1, 128), np.nan, np.float32)
    oracle.c128_prefill(st_ref, np.concatenate([rows0, rows1]), ape, np.array([0, 1], np.int32),
                        cp, wp, out=ref)
    closes_ref = np.nonzero(~np.isnan(ref[:, 0]))[0]
    assert closes_ref.tolist() == [127, 128 + 23, 128 + 151, 128 + 279]

    S = FOUR_GIB // 1536 + 4096
    idx = np.array([S - 2, S - 1], np.int32)
    note(f"c128 prefill ({'one launch' if fused else 'two launches'}): {N} tokens, "
         f"{S} state slots")
    big_state = torch.full((S, 384), float("nan"), device="cuda")
    big_state[S - 2:] = dev(state)
    x = torch.zeros((N, 256), device="cuda")
    x[E0 - 128:E0] = dev(rows0)
    x[E0:] = dev(rows1)
    out = torch.full((N, 128), float("nan"), device="cuda")
    seq, ext = np.array([E0, prefix1 + E1]), np.array([E0, E1])
    if fused:
        items = kvc.kvc_c128_plan_prefill_fused(seq, ext, N)
        kvc.kvc_c128_online_prefill_fused(big_state, x, dev(ape), dev(idx),
                                          kvc.items_to_device(items), items.size, out=out)
    else:
        gcp, gwp = kvc.kvc_c128_plan_prefill(seq, ext, N)
        kvc.kvc_c128_online_prefill(big_state, x, out, dev(ape), dev(idx),
                                    kvc.plans_to_device(gcp), gcp.size,
                                    kvc.plans_to_device(gwp), gwp.size)
    torch.cuda.synchronize()
    written = (~torch.isnan(out[:, 0])).nonzero().flatten().cpu().numpy()
    closes = np.concatenate([np.arange(127, E0, 128), E0 + np.array([23, 151, 279])])
    assert np.array_equal(written, closes)
    zero_chunks = out[127:E0 - 128:128]               # all-zero input: the mean is exactly 0
    assert bool((zero_chunks == 0).all())
    got = out[torch.from_numpy(closes[-4:]).cuda()].cpu().numpy()
    gst = big_state[S - 2:].cpu().numpy()
    del x, out, big_state
    assert rel_err_rows(got, ref[closes_ref]).max() <= VEC_TOL
    assert np.isnan(gst[0]).all()                     # request 0 closes every chunk: no write
    compare_state(gst[1:], st_ref[1:], "c128 prefill past 4 GiB")
