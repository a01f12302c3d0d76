"""HIP-graph capture and replay of the compression path.

The launches of one step (pool-16 prefill, ring decode, c128 prefill with
capacity-padded plans, c128 decode) are captured once and replayed several
times.  Between replays the program does its own eager work: it restores the
mutable buffers (ring, states), refills outputs with sentinels, and for the
c128 prefill uploads a different plan list of the same capacity (the padding
keeps the captured grid valid).  Every replay must equal the eager run on the
same inputs bit for bit.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_pool_amd as kvc
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, seed_states

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
    # ring decode
    d3 = synth.pool16_ring(seed=24, num_requests=40, next_n=4)
    ring0 = dev(d3["ring"])
    ring = ring0.clone()
    m3 = [dev(d3[k]) for k in ("tail_slot_mapping", "key", "score", "ape", "slot_mapping",
                               "positions")]
    o3 = torch.empty((40, 128), dtype=torch.uint8, device="cuda")
    sc3 = torch.empty((40,), device="cuda")
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
        kvc.kvc_compress_prefill(k2, s2, a2, r2, n2, o2, sc2, True)
        kvc.kvc_compress_decode_ring(ring, *m3, o3, sc3, True)
        kvc.kvc_c128_online_prefill(st5, x5, o5, a5, i5, cp_t, N, wp_t, N)
        kvc.kvc_c128_online_decode(st4, x4, o4, a4, i4, l4)

    outs = (o2, sc2, ring, o3, sc3, st5, o5, st4, o4)

    def reset(plan):
        ring.copy_(ring0)
        st4.copy_(st4_0)
        st5.copy_(st5_0)
        cp_t.copy_(plans[plan][0])
        wp_t.copy_(plans[plan][1])
        for t in (o2, o3):
            t.fill_(0x33)
        for t in (sc2, sc3, o4, o5):
            t.fill_(7.0)

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
        for i, (g_, e_) in enumerate(zip((st.cpu(), out.cpu()), eager[name])):
            assert torch.equal(g_.view(torch.uint8), e_.view(torch.uint8)), \
                f"replay {rep} (items {name}): output {i} differs from eager"
        _ = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
