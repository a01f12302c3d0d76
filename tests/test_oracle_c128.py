"""Pins of the oracle's pool-128 online path (c128_online.cuh page:
``flash_c128_online_decode``, ``flash_c128_online_prefill`` and
``plan_online_prefill_host``).

The planner is checked against an independent per-token enumerator; decode
and prefill against a decimal brute force of the per-chunk softmax mean and
against each other (online folding == two-pass == split prefill).
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, c128_prefill_case, rel_err_rows


# ------------------------------------------------------------------ planner
def enumerate_plans(seq_lens, extend_lens):
    """Independent enumerator: walk every extend token, group consecutive
    tokens of one request by 128-chunk; a group whose last token sits at chunk
    position 127 closes the chunk."""
    comp, write = [], []
    row = 0
    for b, (L, E) in enumerate(zip(seq_lens, extend_lens)):
        groups = {}
        for pos in range(L - E, L):
            groups.setdefault(pos // 128, []).append((row, pos))
            row += 1
        for _, toks in sorted(groups.items()):
            last_row, last_pos = toks[-1]
            entry = (last_row, b, last_pos, len(toks))
            (comp if last_pos % 128 == 127 else write).append(entry)
    return comp, write


def _as_tuples(plans):
    return [tuple(int(v) for v in p) for p in plans]


def test_planner_matches_enumerator_exhaustive_small():
    for prefix in range(0, 300, 7):
        for extend in list(range(1, 300, 11)) + [127, 128, 129, 256]:
            sl, el = [prefix + extend], [extend]
            cp, wp = oracle.c128_plan(sl, el, extend)
            ec, ew = enumerate_plans(sl, el)
            assert _as_tuples(cp) == ec and _as_tuples(wp) == ew


def test_planner_matches_enumerator_random_batches_and_invariants():
    g = np.random.default_rng(31)
    for _ in range(200):
        B = int(g.integers(1, 5))
        el = g.integers(1, 400, B)
        sl = el + g.integers(0, 400, B)
        n = int(el.sum())
        cp, wp = oracle.c128_plan(sl, el, n)
        ec, ew = enumerate_plans(sl.tolist(), el.tolist())
        assert _as_tuples(cp) == ec and _as_tuples(wp) == ew
        assert np.all(cp["position"] % 128 == 127) and np.all(wp["position"] % 128 < 127)
        for p in np.concatenate([cp, wp]):
            assert 1 <= p["window_len"] <= 128
            assert p["position"] % 128 + 1 >= p["window_len"]     # one chunk
        assert np.bincount(wp["batch_id"], minlength=B).max(initial=0) <= 1
        assert int(cp["window_len"].sum() + wp["window_len"].sum()) == n


def test_planner_padding_and_errors():
    cp, wp = oracle.c128_plan([300], [300], 300, pad=True)
    assert cp.size == 300 and wp.size == 300
    real = cp[cp["ragged_id"] != 0xFFFFFFFF]
    assert real.size == 2 and np.all(cp[2:]["batch_id"] == 0xFFFFFFFF)
    assert (wp["ragged_id"] != 0xFFFFFFFF).sum() == 1
    with pytest.raises(ValueError):
        oracle.c128_plan([10], [0], 0)
    with pytest.raises(ValueError):
        oracle.c128_plan([10], [11], 11)
    with pytest.raises(ValueError):
        oracle.c128_plan([10, 20], [5, 5], 11)


# ------------------------------------------------------------------ brute force
def exact_chunk_mean(kv, score, ape_rows):
    """40-digit sum e^{s} k / sum e^{s} per channel; s = fp32(score + ape)."""
    getcontext().prec = 40
    s32 = (score.astype(np.float32) + ape_rows.astype(np.float32)).astype(np.float64)
    out = np.empty(128)
    for d in range(128):
        e = [Decimal(v).exp() for v in s32[:, d]]
        num = sum(ei * Decimal(float(k)) for ei, k in zip(e, kv[:, d]))
        out[d] = float(num / sum(e))
    return out


def test_decode_folding_a_chunk_equals_the_pool128_mean():
    g = np.random.default_rng(41)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    toks = g.standard_normal((130, 256)).astype(np.float32)
    state = synth.nan_state(4)
    out = np.full((1, 128), np.nan, np.float32)
    base = 128 * 5
    for t in range(128):
        before = state.copy()
        o = oracle.c128_decode(state, toks[t][None], ape, np.array([2], np.int32),
                               np.array([base + t + 1], np.int32), out=out)
        if t < 127:
            assert np.all(np.isnan(o))                            # nothing emitted
            s32 = toks[:t + 1, 128:] + ape[:t + 1]
            assert np.array_equal(state[2, :128], s32.max(axis=0))  # max is exact
        else:
            assert np.array_equal(state, before, equal_nan=True)  # closing token: state untouched
    ref = exact_chunk_mean(toks[:128, :128], toks[:128, 128:], ape)
    assert rel_err_rows(out, ref[None])[0] < 2e-5
    assert np.all(np.isnan(np.delete(state, 2, axis=0)))          # other slots never touched


def test_decode_skips_invalid_rows_and_leaves_other_outputs():
    g = np.random.default_rng(42)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    x = g.standard_normal((4, 256)).astype(np.float32)
    state = g.standard_normal((3, 384)).astype(np.float32)
    state[:, 128:256] = np.abs(state[:, 128:256]) + 1
    st0 = state.copy()
    out = np.full((4, 128), 7.0, np.float32)
    oracle.c128_decode(state, x, ape, np.array([0, -1, 5, 1], np.int32),
                       np.array([0, 5, 5, 1], np.int32), out=out)
    assert np.array_equal(state[0], st0[0]) and np.array_equal(state[2], st0[2])
    assert np.all(out == 7.0)
    # row 3: seq_len 1 -> chunk position 0 -> state := (s, 1, k)
    assert np.array_equal(state[1, :128], x[3, 128:] + ape[0])
    assert np.all(state[1, 128:256] == 1.0) and np.array_equal(state[1, 256:], x[3, :128])


def test_prefill_closed_chunks_and_open_state_match_bruteforce():
    g = np.random.default_rng(43)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    prior, extend = 200, 333                     # 72 prior tokens in the open chunk
    toks = g.standard_normal((prior + extend, 256)).astype(np.float32)
    state = synth.nan_state(8)
    idx = np.array([5], np.int32)
    cp, wp = oracle.c128_plan([prior], [prior % 128], prior % 128)
    oracle.c128_prefill(state, toks[128:prior], ape, idx, cp, wp)
    cp, wp = oracle.c128_plan([prior + extend], [extend], extend)
    out = np.full((extend, 128), np.nan, np.float32)
    oracle.c128_prefill(state, toks[prior:], ape, idx, cp, wp, out=out)
    closed = [c for c in range(prior // 128, (prior + extend) // 128) if (c + 1) * 128 <= prior + extend]
    assert [int(r) for r in cp["ragged_id"]] == [(c + 1) * 128 - 1 - prior for c in closed]
    for c in closed:
        ref = exact_chunk_mean(toks[c * 128:(c + 1) * 128, :128],
                               toks[c * 128:(c + 1) * 128, 128:], ape)
        assert rel_err_rows(out[(c + 1) * 128 - 1 - prior][None], ref[None])[0] < 1e-6
    written = np.zeros(extend, bool)
    written[cp["ragged_id"]] = True
    assert np.all(np.isnan(out[~written]))
    # open chunk: state = (max, sum of exp, mean) over its tokens
    lo = (prior + extend) // 128 * 128
    kv, sc = toks[lo:, :128], toks[lo:, 128:]
    s32 = sc + ape[:kv.shape[0]]
    assert np.array_equal(state[5, :128], s32.max(axis=0))
    ref = exact_chunk_mean(kv, sc, ape[:kv.shape[0]])
    assert rel_err_rows(state[5, 256:][None], ref[None])[0] < 1e-6
    ssum = np.exp(s32.astype(np.float64) - s32.max(axis=0)).sum(axis=0)
    assert rel_err_rows(state[5, 128:256][None], ssum[None])[0] < 1e-6


def test_prefill_split_and_decode_agree():
    g = np.random.default_rng(44)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    E = 300
    toks = g.standard_normal((E, 256)).astype(np.float32)
    idx = np.array([0], np.int32)

    def run_prefill(splits):
        state = synth.nan_state(1)
        outs = np.full((E, 128), np.nan, np.float32)
        done = 0
        for e in splits:
            cp, wp = oracle.c128_plan([done + e], [e], e)
            o = oracle.c128_prefill(state, toks[done:done + e], ape, idx, cp, wp)
            outs[done:done + e][cp["ragged_id"]] = o[cp["ragged_id"]]
            done += e
        return outs, state

    one, st1 = run_prefill([E])
    for splits in ([100, 200], [1, 127, 1, 171], [128, 128, 44], [5] * 60):
        o, st = run_prefill(splits)
        assert np.array_equal(np.isnan(o), np.isnan(one))
        rows = ~np.isnan(one[:, 0])
        assert rel_err_rows(o[rows], one[rows]).max() < 2e-6
        assert np.array_equal(st[0, :128], st1[0, :128])
        assert rel_err_rows(st[:, 128:], st1[:, 128:]).max() < 2e-6
    state = synth.nan_state(1)
    dec = np.full((E, 128), np.nan, np.float32)
    for t in range(E):
        o = np.full((1, 128), np.nan, np.float32)
        oracle.c128_decode(state, toks[t][None], ape, idx, np.array([t + 1], np.int32), out=o)
        dec[t] = o[0]
    rows = ~np.isnan(one[:, 0])
    assert np.array_equal(~np.isnan(dec[:, 0]), rows)
    assert rel_err_rows(dec[rows], one[rows]).max() < 2e-5
    assert np.array_equal(state[0, :128], st1[0, :128])


def test_prefill_reads_state_before_the_write_pass_and_skips_sentinels():
    # One request whose extend starts mid-chunk, closes it, and ends mid-chunk:
    # its compress plan reads slot 3 and its write plan rewrites slot 3.
    d = c128_prefill_case(seed=9, batch=3, max_prior=600, max_extend=500)
    st_a = d["state"].copy()
    oa = oracle.c128_prefill(st_a, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"])
    n = int(d["extend_lens"].sum())
    cp, wp = oracle.c128_plan(d["seq_lens"], d["extend_lens"], n, pad=True)
    st_b = d["state"].copy()
    ob = oracle.c128_prefill(st_b, d["kv_score_in"], d["ape"], d["indices"], cp, wp)
    assert np.array_equal(oa, ob) and np.array_equal(st_a, st_b, equal_nan=True)
    # brute force the first closed chunk of every request from raw tokens
    starts = synth.ragged_starts(d["extend_lens"])
    pstarts = synth.ragged_starts(d["prior_counts"])
    for b in range(3):
        prior = int(d["seq_lens"][b] - d["extend_lens"][b])
        first_close = (prior // 128 + 1) * 128
        if first_close > d["seq_lens"][b]:
            continue
        pc = int(d["prior_counts"][b])
        raw = np.concatenate([d["prior_in"][pstarts[b]:pstarts[b] + pc],
                              d["kv_score_in"][starts[b]:starts[b] + first_close - prior]])
        assert raw.shape[0] == 128
        ref = exact_chunk_mean(raw[:, :128], raw[:, 128:], d["ape"])
        row = starts[b] + first_close - 1 - prior
        assert rel_err_rows(oa[row][None], ref[None])[0] < 2e-6


def test_full_size_workloads_stay_finite():
    d = c128_decode_case(seed=0)
    st = d["state"].copy()
    out = np.full((1024, 128), np.nan, np.float32)
    oracle.c128_decode(st, d["kv_score_in"], d["ape"], d["indices"], d["seq_lens"], out=out)
    emit = (d["seq_lens"] - 1) % 128 == 127
    assert np.all(np.isfinite(out[emit])) and np.all(np.isnan(out[~emit]))
    touched = d["indices"][~emit]
    assert np.all(np.isfinite(st[touched]))
