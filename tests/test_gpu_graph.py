"""HIP-graph capture and replay of the compression path.

The launches of one step (pool-16 prefill, ring decode, c128 prefill with
capacity-padded plans, c128 decode) are captured once and replayed several
times.  Between replays the program does its own eager work: it restores the
mutable buffers (ring, states), refills outputs with sentinels, and for the
c128 prefill uploads a different plan list of the same capacity (the padding
keeps the captured grid valid).  Every replay must equal the eager run on the
same inputs bit for bit, and each replay's outputs are also held to the CPU
oracle with the tolerances of the parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_pool_amd as kvc
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, rel_err_rows, seed_states
from tests.test_gpu_parity import (FLIP_ULPS_POOL16, VEC_TOL, check_codes, check_scales,
                                   compare_state, reference_for)

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _c128_prefill_inputs(seed, seq_lens, extend_lens, num_slots=64):
    g = np.random.default_rng(seed)
    B = len(seq_lens)
    N = int(np.sum(extend_lens))
    idx = g.permutation(num_slots)[:B].astype(np.int32)
    prior = np.asarray(seq_lens) - np.asarray(extend_lens)
    counts = prior % 128
    st = synth.nan_state(num_slots)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    prior_in = g.standard_normal((int(counts.sum()), 256)).astype(np.float32)
    seed_states(st, idx, counts, prior_in, prior, ape)
    x = g.standard_normal((N, 256)).astype(np.float32)
    return st, x, ape, idx


def test_graph_replay_matches_eager():
    # pool-16 prefill
    d2 = synth.pool16_ragged(seed=21, num_seqs=8, max_len=700)
    rows = kvc.kvc_plan_pool_prefill(d2["seq_lens"])
    n2 = rows.size
    k2, s2, a2, r2 = (dev(d2["keys"]), dev(d2["scores"]), dev(d2["ape"]), dev(rows))
    o2 = torch.empty((n2, 128), dtype=torch.uint8, device="cuda")
    sc2 = torch.empty((n2,), device="cuda")
    x2 = torch.empty((n2, 128), device="cuda")
    # ring decode
    d3 = synth.pool16_ring(seed=24, num_requests=40, next_n=4)
    ring0 = dev(d3["ring"])
    ring = ring0.clone()
    m3 = [dev(d3[k]) for k in ("tail_slot_mapping", "key", "score", "ape", "slot_mapping",
                               "positions")]
    o3 = torch.empty((40, 128), dtype=torch.uint8, device="cuda")
    sc3 = torch.empty((40,), device="cuda")
    x3 = torch.empty((40, 128), device="cuda")
    # c128 decode
    d4 = c128_decode_case(seed=23, batch=200, emit_frac=0.3)
    st4_0 = dev(d4["state"])
    st4 = st4_0.clone()
    x4, a4, i4, l4 = (dev(d4[k]) for k in ("kv_score_in", "ape", "indices", "seq_lens"))
    o4 = torch.empty((200, 128), device="cuda")
    # c128 prefill: two plan lists of the same capacity
    sl_a, el_a = np.array([700, 300, 129, 50]), np.array([600, 300, 2, 50])
    sl_b, el_b = np.array([900, 130, 377, 20]), np.array([500, 130, 302, 20])
    N = int(el_a.sum())
    assert int(el_b.sum()) == N
    st5_np, x5_np, a5_np, i5_np = _c128_prefill_inputs(25, sl_a, el_a)
    st5_0, x5, a5, i5 = dev(st5_np), dev(x5_np), dev(a5_np), dev(i5_np)
    st5 = st5_0.clone()
    plans = {}
    for name, sl, el in (("a", sl_a, el_a), ("b", sl_b, el_b)):
        cp, wp = kvc.kvc_c128_plan_prefill(sl, el, N, pad_to_capacity=True)
        assert cp.size == N and wp.size == N
        plans[name] = (kvc.plans_to_device(cp), kvc.plans_to_device(wp))
    cp_t = torch.empty_like(plans["a"][0])
    wp_t = torch.empty_like(plans["a"][1])
    o5 = torch.empty((N, 128), device="cuda")

    def step():
        kvc.kvc_compress_prefill(k2, s2, a2, r2, n2, o2, sc2, True, x2)
        kvc.kvc_compress_decode_ring(ring, *m3, o3, sc3, True, dbg_pooled=x3)
        kvc.kvc_c128_online_prefill(st5, x5, o5, a5, i5, cp_t, N, wp_t, N)
        kvc.kvc_c128_online_decode(st4, x4, o4, a4, i4, l4)

    outs = (o2, sc2, ring, o3, sc3, st5, o5, st4, o4, x2, x3)

    def reset(plan):
        ring.copy_(ring0)
        st4.copy_(st4_0)
        st5.copy_(st5_0)
        cp_t.copy_(plans[plan][0])
        wp_t.copy_(plans[plan][1])
        for t in (o2, o3):
            t.fill_(0x33)
        for t in (sc2, sc3, o4, o5, x2, x3):
            t.fill_(7.0)

    # the oracle's results for both plan lists
    rc2, rs2, rx2 = oracle.compress_prefill(d2["keys"], d2["scores"], d2["ape"], rows, True)
    ring_ref = d3["ring"].copy()
    rc3 = np.full((40, 128), 0x33, np.uint8)
    rs3 = np.full(40, 7.0, np.float32)
    pk = np.zeros((40, 16, 128), np.uint16)
    ps = np.zeros((40, 16, 128), np.uint16)
    oracle.ring_decode(ring_ref, d3["tail_slot_mapping"], d3["key"], d3["score"], d3["ape"],
                       d3["slot_mapping"], d3["positions"], 40, True, out_code=rc3,
                       out_scale=rs3, pools_out=(pk, ps))
    done3 = np.nonzero(rs3 != 7.0)[0]
    assert done3.size > 0
    _, _, rx3 = oracle.compress_prefill(pk[done3].reshape(-1, 128), ps[done3].reshape(-1, 128),
                                        d3["ape"], None, True)
    st4_ref = d4["state"].copy()
    o4_ref = np.full((200, 128), 7.0, np.float32)
    oracle.c128_decode(st4_ref, d4["kv_score_in"], d4["ape"], d4["indices"], d4["seq_lens"],
                       out=o4_ref)
    ref5 = {}
    for name, sl, el in (("a", sl_a, el_a), ("b", sl_b, el_b)):
        st = st5_np.copy()
        o = np.full((N, 128), 7.0, np.float32)
        cp, wp = oracle.c128_plan(sl, el, N)
        oracle.c128_prefill(st, x5_np, a5_np, i5_np, cp, wp, out=o)
        ref5[name] = (st, o)

    def check_oracle(got, plan, what):
        g2, gs2, gring, g3, gs3, gst5, go5, gst4, go4, gx2, gx3 = (t.numpy() for t in got)
        assert rel_err_rows(gx2, rx2).max() <= VEC_TOL, f"{what}: prefill means"
        ref_c, ref_s, _ = reference_for(gx2, rx2, rc2, rs2, True, f"{what} prefill")
        check_codes(g2, ref_c, f"{what} prefill")
        check_scales(gs2, ref_s, True, f"{what} prefill")
        assert np.array_equal(gring.view(np.uint16), ring_ref), f"{what}: ring stashes"
        assert np.array_equal(np.nonzero(gs3 != 7.0)[0], done3), f"{what}: ring completions"
        assert rel_err_rows(gx3[done3], rx3).max() <= VEC_TOL, f"{what}: ring means"
        c3, s3, _ = reference_for(gx3[done3], rx3, rc3[done3], rs3[done3], True,
                                  f"{what} ring", ulps=FLIP_ULPS_POOL16)
        check_codes(g3[done3], c3, f"{what} ring")
        check_scales(gs3[done3], s3, True, f"{what} ring")
        assert np.all(g3[np.setdiff1d(np.arange(40), done3)] == 0x33)
        st_r, o_r = ref5[plan]
        compare_state(gst5, st_r, f"{what} c128 prefill state")
        w = o_r[:, 0] != 7.0
        assert np.array_equal(go5[:, 0] != 7.0, w), f"{what}: c128 prefill rows written"
        assert rel_err_rows(go5[w], o_r[w]).max() <= VEC_TOL, f"{what}: c128 prefill out"
        compare_state(gst4, st4_ref, f"{what} c128 decode state")
        e = o4_ref[:, 0] != 7.0
        assert np.array_equal(go4[:, 0] != 7.0, e), f"{what}: c128 decode rows emitted"
        assert rel_err_rows(go4[e], o4_ref[e]).max() <= VEC_TOL, f"{what}: c128 decode out"

    eager = {}
    for plan in ("a", "b"):
        reset(plan)
        step()
        torch.cuda.synchronize()
        eager[plan] = [t.cpu().clone() for t in outs]
    assert not torch.equal(eager["a"][6], eager["b"][6])   # the plan lists differ

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    reset("a")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        step()                                               # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset("a")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep, plan in enumerate(("a", "b", "a", "b", "b")):
        reset(plan)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in outs]
        for i, (g_, e_) in enumerate(zip(got, eager[plan])):
            assert torch.equal(g_.view(torch.uint8), e_.view(torch.uint8)), \
                f"replay {rep} (plans {plan}): output {i} differs from eager"
        check_oracle(got, plan, f"replay {rep} (plans {plan})")
        _ = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()


def test_graph_replay_single_launch_prefill():
    """The single-launch c128 prefill captured once with capacity-padded work
    items; two item lists of the same capacity swapped between replays."""
    sl_a, el_a = np.array([700, 300, 129, 50]), np.array([600, 300, 2, 50])
    sl_b, el_b = np.array([900, 130, 377, 20]), np.array([500, 130, 302, 20])
    N = int(el_a.sum())
    st_np, x_np, a_np, i_np = _c128_prefill_inputs(26, sl_a, el_a)
    st0, x, a, idx = dev(st_np), dev(x_np), dev(a_np), dev(i_np)
    st = st0.clone()
    lists = {}
    cap = kvc.kvc_c128_fused_capacity(N, 4)        # the capture serves batches of up to 4
    for name, sl, el in (("a", sl_a, el_a), ("b", sl_b, el_b)):
        items = kvc.kvc_c128_plan_prefill_fused(sl, el, N, pad_to_capacity=True, capacity=cap)
        assert items.size == cap
        lists[name] = kvc.items_to_device(items)
    items_t = torch.empty_like(lists["a"])
    out = torch.empty((N, 128), device="cuda")

    def step():
        kvc.kvc_c128_online_prefill_fused(st, x, a, idx, items_t, cap, out=out)

    def reset(name):
        st.copy_(st0)
        items_t.copy_(lists[name])
        out.fill_(7.0)

    eager = {}
    for name in ("a", "b"):
        reset(name)
        step()
        torch.cuda.synchronize()
        eager[name] = (st.cpu().clone(), out.cpu().clone())
    assert not torch.equal(eager["a"][1], eager["b"][1])
    ref = {}
    for name, sl, el in (("a", sl_a, el_a), ("b", sl_b, el_b)):
        rst = st_np.copy()
        ro = np.full((N, 128), 7.0, np.float32)
        cp, wp = oracle.c128_plan(sl, el, N)
        oracle.c128_prefill(rst, x_np, a_np, i_np, cp, wp, out=ro)
        ref[name] = (rst, ro)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    reset("a")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset("a")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep, name in enumerate(("a", "b", "b", "a")):
        reset(name)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (st.cpu(), out.cpu())
        for i, (g_, e_) in enumerate(zip(got, eager[name])):
            assert torch.equal(g_.view(torch.uint8), e_.view(torch.uint8)), \
                f"replay {rep} (items {name}): output {i} differs from eager"
        rst, ro = ref[name]
        compare_state(got[0].numpy(), rst, f"replay {rep} (items {name}) state")
        w = ro[:, 0] != 7.0
        go = got[1].numpy()
        assert np.array_equal(go[:, 0] != 7.0, w), f"replay {rep}: rows written"
        assert rel_err_rows(go[w], ro[w]).max() <= VEC_TOL, f"replay {rep}: out vs oracle"
        _ = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
