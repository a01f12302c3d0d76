"""Seeded synthetic inputs for the compression kernels and their checks.

This module draws random numbers and lays them out; it performs none of the
method's arithmetic (no softmax, rotation, rounding scheme or quantisation of
its own).  bf16 inputs are produced by casting fp32 normals with torch's CPU
conversion.  Both the GPU tests / benchmark and the CPU oracle tests consume
these arrays, so the two sides always see identical inputs.

Every generator takes a ``seed`` and uses its own numpy PCG64 stream
(``default_rng([seed, stream_id])``), so results are reproducible on any host.

Workloads (all head_dim 128):
  pool16_single   one sequence of 256 tokens, pool 16, round_scale off.
  pool16_ragged   64 sequences, lengths uniform in [1, 8192], pool 16,
                  tokens after the last full pool are not compressed,
                  round_scale on.
  pool16_ring     256 requests x 4 verify tokens, 16-slot tail ring per
                  request, positions base + t with base uniform in [0, 65535],
                  5% of entries padded with -1 (their key/score rows are NaN).
  c128_decode     1024 requests, one token each, 2048 state slots, seq_len
                  uniform in [1, 131072], prior chunk tokens to build the state.
  c128_prefill    32 sequences, prior uniform in [0, 32768], extend uniform in
                  [1, 16384], 2048 state slots, prior chunk tokens for the state.
  pool16_seed     a prefill batch (64 sequences, lengths uniform in [1, 8192])
                  whose last 16 tokens per request seed the tail rings.
"""
from __future__ import annotations

import numpy as np
import torch

HEAD_DIM = 128
BF16_NAN = np.uint16(0x7FC0)

_STREAMS = {"pool16_single": 1, "pool16_ragged": 2, "pool16_ring": 3,
            "c128_decode": 4, "c128_prefill": 5, "pool16_seed": 6, "misc": 99}


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAMS.get(name, 100)])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 patterns to fp32 (exact; bit placement only)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_normal(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    return to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def ape_pool16(g: np.random.Generator, pool: int = 16) -> np.ndarray:
    """[pool,128] position bias: N(0, 0.1) drawn as bf16, stored as fp32."""
    return bf16_bits_to_f32(bf16_normal(g, (pool, HEAD_DIM), 0.1))


def ragged_starts(lens: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


# ------------------------------------------------------------------ pool-16
def pool16_single(seed: int = 0, tokens: int = 256):
    g = rng(seed, "pool16_single")
    keys = bf16_normal(g, (tokens, HEAD_DIM))
    scores = bf16_normal(g, (tokens, HEAD_DIM))
    ape = ape_pool16(g)
    return dict(keys=keys, scores=scores, ape=ape,
                seq_lens=np.array([tokens], np.int64), round_scale=False)


def pool16_ragged(seed: int = 0, num_seqs: int = 64, max_len: int = 8192):
    g = rng(seed, "pool16_ragged")
    lens = g.integers(1, max_len, size=num_seqs, endpoint=True).astype(np.int64)
    T = int(lens.sum())
    keys = bf16_normal(g, (T, HEAD_DIM))
    scores = bf16_normal(g, (T, HEAD_DIM))
    ape = ape_pool16(g)
    return dict(keys=keys, scores=scores, ape=ape, seq_lens=lens, round_scale=True)


def pool16_ring(seed: int = 0, num_requests: int = 256, next_n: int = 4,
                pad_frac: float = 0.05, max_base: int = 65535, pool: int = 16):
    g = rng(seed, "pool16_ring")
    R, N = num_requests, next_n
    base = g.integers(0, max_base, size=R, endpoint=True).astype(np.int64)
    pos = (base[:, None] + np.arange(N)[None, :]).astype(np.int64)
    padded = g.random((R, N)) < pad_frac
    req = np.repeat(np.arange(R)[:, None], N, axis=1)
    positions = np.where(padded, -1, pos).astype(np.int32)
    tail_slot = np.where(padded, -1, req * pool + pos % pool).astype(np.int32)
    slot_mapping = np.where(~padded & (pos % pool == pool - 1), req, -1).astype(np.int32)
    ring = bf16_normal(g, (R, 2, pool, HEAD_DIM))
    key = bf16_normal(g, (R, N, HEAD_DIM))
    score = bf16_normal(g, (R, N, HEAD_DIM))
    key[padded] = BF16_NAN
    score[padded] = BF16_NAN
    ape = ape_pool16(g, pool)
    return dict(ring=ring, tail_slot_mapping=tail_slot, key=key, score=score, ape=ape,
                slot_mapping=slot_mapping, positions=positions, num_out=R,
                round_scale=True)


def pool16_seed(seed: int = 0, num_seqs: int = 64, max_len: int = 8192, pad_tokens: int = 0,
                pool: int = 16):
    """A prefill batch whose requests seed their tail rings: request b owns
    ring block b and seq_lens[b] consecutive tokens at positions 0..len-1;
    tail slot = 16*b + pos%16.  ``pad_tokens`` padding entries (slot -1, NaN
    rows) follow the last request."""
    g = rng(seed, "pool16_seed")
    lens = g.integers(1, max_len, size=num_seqs, endpoint=True).astype(np.int64)
    T = int(lens.sum()) + pad_tokens
    req = np.repeat(np.arange(num_seqs), lens)
    pos = np.concatenate([np.arange(n) for n in lens]) if num_seqs else np.zeros(0, np.int64)
    tslot = np.full(T, -1, np.int32)
    tslot[:req.size] = req * pool + pos % pool
    key = bf16_normal(g, (T, HEAD_DIM))
    score = bf16_normal(g, (T, HEAD_DIM))
    key[req.size:] = BF16_NAN
    score[req.size:] = BF16_NAN
    ring = bf16_normal(g, (num_seqs, 2, pool, HEAD_DIM))
    return dict(key=key, score=score, tslot=tslot, ring=ring, seq_lens=lens)


# ------------------------------------------------------------------ pool-128 online
def _prior_tokens(g, counts):
    """Raw kv|score rows for the tokens already in each open chunk."""
    n = int(np.sum(counts))
    return g.standard_normal((n, 2 * HEAD_DIM), dtype=np.float32)


def c128_decode(seed: int = 0, batch: int = 1024, num_slots: int = 2048,
                max_seq: int = 131072, emit_frac: float = 0.0, seq_lens=None):
    """Inputs for one decode step.  The state of request b must be built from
    ``prior_in`` rows (its first ``prior_counts[b]`` rows belong to b, in
    order) by folding them into an open chunk that ends at position
    seq_lens[b]-2; slots whose chunk is empty are never read.  ``emit_frac``
    of the requests are moved to a chunk-closing length (a multiple of 128);
    ``seq_lens`` overrides the drawn lengths."""
    g = rng(seed, "c128_decode")
    indices = g.permutation(num_slots)[:batch].astype(np.int32)
    drawn = g.integers(1, max_seq, size=batch, endpoint=True).astype(np.int32)
    closing = g.random(batch) < emit_frac
    drawn = np.where(closing, np.maximum(drawn // 128, 1) * 128, drawn).astype(np.int32)
    seq_lens = drawn if seq_lens is None else np.asarray(seq_lens, np.int32)
    kv_score = g.standard_normal((batch, 2 * HEAD_DIM), dtype=np.float32)
    ape = (g.standard_normal((128, HEAD_DIM), dtype=np.float32) * np.float32(0.1))
    prior_counts = ((seq_lens.astype(np.int64) - 1) % 128)
    prior_in = _prior_tokens(g, prior_counts)
    return dict(indices=indices, seq_lens=seq_lens, kv_score_in=kv_score, ape=ape,
                num_slots=num_slots, prior_counts=prior_counts, prior_in=prior_in)


def c128_prefill(seed: int = 0, batch: int = 32, num_slots: int = 2048,
                 max_prior: int = 32768, max_extend: int = 16384, seq_lens=None,
                 extend_lens=None):
    """Inputs for one ragged prefill.  ``prior_counts[b] = prior % 128`` raw
    tokens (rows of ``prior_in``) form the open chunk carried in the state.
    Explicit ``seq_lens`` / ``extend_lens`` replace the random lengths."""
    g = rng(seed, "c128_prefill")
    prior = g.integers(0, max_prior, size=batch, endpoint=True).astype(np.int64)
    extend = g.integers(1, max_extend, size=batch, endpoint=True).astype(np.int64)
    if seq_lens is not None:
        extend = np.asarray(extend_lens, np.int64)
        prior = np.asarray(seq_lens, np.int64) - extend
        batch = extend.size
    seq_lens = prior + extend
    N = int(extend.sum())
    indices = g.permutation(num_slots)[:batch].astype(np.int32)
    kv_score = g.standard_normal((N, 2 * HEAD_DIM), dtype=np.float32)
    ape = (g.standard_normal((128, HEAD_DIM), dtype=np.float32) * np.float32(0.1))
    prior_counts = prior % 128
    prior_in = _prior_tokens(g, prior_counts)
    return dict(seq_lens=seq_lens, extend_lens=extend, indices=indices,
                kv_score_in=kv_score, ape=ape, num_slots=num_slots,
                prior_counts=prior_counts, prior_in=prior_in)


def state_seed_lengths(prior_counts: np.ndarray, chunk_end_pos: np.ndarray):
    """(seq_lens, extend_lens) that fold each open chunk's prior tokens into a
    state with one planned prefill: the chunk's tokens end at position
    chunk_end_pos-1, so seq_len = chunk_end_pos and extend = prior_counts.
    Entries with no prior tokens are dropped (their slots are never read).
    Returns (keep_mask, seq_lens, extend_lens)."""
    keep = prior_counts > 0
    return keep, chunk_end_pos[keep].astype(np.int64), prior_counts[keep].astype(np.int64)


def nan_state(num_slots: int) -> np.ndarray:
    return np.full((num_slots, 3 * HEAD_DIM), np.nan, np.float32)
