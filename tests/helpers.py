"""Shared test helpers: workload assembly on top of the seeded generators.

Only oracle calls and plain numpy live here; nothing from the HIP path.
"""
import numpy as np

import oracle
from kv_cache_compression_pool_amd import synth


def seed_states(state, indices, prior_counts, prior_in, chunk_end_pos, ape):
    """Fold each request's prior chunk tokens into state row indices[b] with
    the oracle's prefill (one write plan per request with prior tokens)."""
    keep, sl, el = synth.state_seed_lengths(np.asarray(prior_counts), np.asarray(chunk_end_pos))
    if not keep.any():
        return state
    n = int(el.sum())
    cp, wp = oracle.c128_plan(sl, el, n)
    assert cp.size == 0 and wp.size == int(keep.sum())
    oracle.c128_prefill(state, prior_in[:n], ape, np.asarray(indices)[keep], cp, wp)
    return state


def c128_decode_case(seed=0, **kw):
    d = synth.c128_decode(seed=seed, **kw)
    st = synth.nan_state(d["num_slots"])
    seed_states(st, d["indices"], d["prior_counts"], d["prior_in"],
                d["seq_lens"].astype(np.int64) - 1, d["ape"])
    d["state"] = st
    return d


def c128_prefill_case(seed=0, **kw):
    d = synth.c128_prefill(seed=seed, **kw)
    st = synth.nan_state(d["num_slots"])
    prior = d["seq_lens"] - d["extend_lens"]
    seed_states(st, d["indices"], d["prior_counts"], d["prior_in"], prior, d["ape"])
    d["state"] = st
    d["cplan"], d["wplan"] = oracle.c128_plan(d["seq_lens"], d["extend_lens"],
                                              int(d["extend_lens"].sum()))
    return d


def rel_err_rows(got, ref):
    """Per-row max-abs error relative to the row's max-abs reference value."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return np.abs(got - ref).max(axis=-1) / den


def e4m3_ordinal(codes):
    """Map e4m3 codes to a magnitude-ordered integer line (+0 and -0 equal)."""
    c = np.asarray(codes, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)
