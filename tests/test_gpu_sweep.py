"""Randomised sweep: many small seeded shapes per kernel, each compared with
the oracle to the same bar as the fixed-case parity tests.  The shapes cross
the kernels' internal boundaries (pools per workgroup, requests per wave,
verify-batch kernel choice, chunk edges, segments per request) at random."""
import os

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_pool_amd as kvc
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, c128_prefill_case, rel_err_rows
from tests.test_gpu_parity import (VEC_TOL, check_codes, check_ring_layers, check_scales,
                                   compare_c128_prefill, compare_c128_prefill_fused,
                                   compare_prefill, compare_state, dev, irregular_ring_case, note,
                                   run_ring)

pytestmark = pytest.mark.gpu

# More cases on demand: KVC_SWEEP_CASES=N
CASES = int(os.environ.get("KVC_SWEEP_CASES", "12"))


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_pool16_prefill(case):
    g = np.random.default_rng(1000 + case)
    seed = 2000 + case
    while True:   # redraw until the batch holds at least one complete pool
        d = synth.pool16_ragged(seed=seed, num_seqs=int(g.integers(1, 24)),
                                max_len=int(g.integers(1, 700)))
        rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
        if rows.size:
            break
        seed += 100
    stride = None if case % 3 else int(128 + 8 * g.integers(1, 5))
    compare_prefill(d, rows, bool(case % 2), f"sweep prefill {case}", key_stride=stride)


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_ring_decode(case):
    g = np.random.default_rng(3000 + case)
    next_n = int(g.integers(1, 37))   # up to three 16-token windows
    d = synth.pool16_ring(seed=4000 + case, num_requests=int(g.integers(1, 70)), next_n=next_n,
                          pad_frac=float(g.uniform(0, 0.3)))
    d["round_scale"] = bool(case % 2)
    note(f"sweep ring {case}: {d['key'].shape[0]}x{next_n}")
    gring, gc, gs, ring, rc, rs = run_ring(d)
    assert np.array_equal(gring, ring)
    check_codes(gc, rc, "sweep ring codes")
    check_scales(gs, rs, d["round_scale"], "sweep ring scales")


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_ring_decode_layers(case):
    """Multi-layer launches (the instances that park token rows and stage
    ape in LDS) against single-layer calls and the oracle."""
    g = np.random.default_rng(9000 + case)
    next_n = int(g.integers(1, 9))
    R = int(g.integers(1, 90))
    if case % 2:
        base = irregular_ring_case(9500 + case, R, next_n)
    else:
        base = synth.pool16_ring(seed=9600 + case, num_requests=R, next_n=next_n,
                                 pad_frac=float(g.uniform(0, 0.3)))
        base["round_scale"] = bool(case % 4 == 0)
    check_ring_layers(base, int(g.integers(2, 7)), 9700 + case)


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_c128_decode(case):
    g = np.random.default_rng(5000 + case)
    B = int(g.integers(1, 300))
    d = c128_decode_case(seed=6000 + case, batch=B, num_slots=max(2 * B, 8),
                         max_seq=int(g.integers(1, 5000)), emit_frac=float(g.uniform(0, 0.5)))
    note(f"sweep c128 decode {case}: batch {B}")
    st = d["state"].copy()
    ref = np.full((B, 128), np.nan, np.float32)
    oracle.c128_decode(st, d["kv_score_in"], d["ape"], d["indices"], d["seq_lens"], out=ref)
    gst = dev(d["state"])
    gout = torch.full((B, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode(gst, dev(d["kv_score_in"]), gout, dev(d["ape"]),
                               dev(d["indices"]), dev(d["seq_lens"]))
    torch.cuda.synchronize()
    gout = gout.cpu().numpy()
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    emit = ~np.isnan(ref[:, 0])
    if emit.any():
        assert rel_err_rows(gout[emit], ref[emit]).max() <= VEC_TOL
    compare_state(gst.cpu().numpy(), st, f"sweep c128 decode {case}")


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_c128_prefill(case):
    g = np.random.default_rng(7000 + case)
    d = c128_prefill_case(seed=8000 + case, batch=int(g.integers(1, 9)),
                          max_prior=int(g.integers(0, 600)), max_extend=int(g.integers(1, 900)))
    compare_c128_prefill(d, f"sweep c128 prefill {case}", pad=bool(case % 2))
    compare_c128_prefill_fused(d, f"sweep c128 fused prefill {case}", pad=bool(case % 3 == 0))
