"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Tolerances (the specification's bar):
  * fp32 vectors (pool-16 pre-rounding mean, pool-128 outputs and state kv /
    sum): per vector max-abs error <= 2e-3 of the vector's max-abs value.
  * pool-128 state max: bit-exact.
  * e4m3 codes: at most 1 step apart (ordered code line, +0 == -0) on at most
    0.1% of codes, identical elsewhere.
  * scales: bit-exact with power-of-two rounding; without it, identical except
    on at most 0.1% of vectors whose absmax moved by one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_pool_amd as kvc
from kv_cache_compression_pool_amd import synth
from tests.helpers import c128_decode_case, c128_prefill_case, e4m3_ordinal, rel_err_rows

pytestmark = pytest.mark.gpu

VEC_TOL = 2e-3
# Batches of at least this many codes are also held to the raw 0.1% bar.
RAW_CHECK_MIN_CODES = 100_000


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def note(msg):
    print(f"[gpu] {msg}", flush=True)


def check_codes(got, ref, what):
    d = np.abs(e4m3_ordinal(got) - e4m3_ordinal(ref))
    n_off = int((d != 0).sum())
    assert d.max(initial=0) <= 1, f"{what}: code off by {d.max()}"
    assert n_off <= 0.001 * d.size, f"{what}: {n_off} of {d.size} codes differ"
    return n_off


def check_scales(got, ref, round_scale, what):
    if round_scale:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
            f"{what}: {(got != ref).sum()} power-of-two scales differ"
    else:
        bad = got != ref
        assert bad.sum() <= max(1, 0.001 * got.size), f"{what}: {bad.sum()} scales differ"
        if bad.any():
            assert np.all(np.abs(got[bad] / ref[bad] - 1) <= 2.0**-7)


# Fp32 accumulation error allowed in a channel that rounds to a different
# bf16 value than the oracle's, in fp32 ulps (2^-23) of the vector's max-abs
# value.  A pool-16 mean sums 16 weighted terms (observed at most about 1.5
# ulps); a pool-128 mean sums 128 through several partial merges (observed
# at most about 1.5 ulps).
FLIP_ULPS_POOL16 = 8
FLIP_ULPS_POOL128 = 16
# Pools whose bf16 rounding differs anywhere: at most this share of the batch
# (observed 0.9% on the 64-sequence ragged batch), or FLIP_FLOOR pools.
FLIP_FRAC = 0.02
FLIP_FLOOR = 8


def reference_for(gx, rx, rc, rs, round_scale, what, ulps=FLIP_ULPS_POOL16):
    """Reference codes / scales for the GPU output.

    Where the GPU's fp32 pooled vector rounds to the same bf16 vector as the
    oracle's, the oracle's own codes are the reference.  Where some channel
    rounds to the neighbouring bf16 value (the exact mean sits within fp32
    rounding error of a bf16 rounding boundary, so both roundings are correct),
    the reference is the oracle's epilogue applied to the GPU's pooled vector;
    e4m3 resolves near-zero values far more finely than a one-bf16-ulp input
    change, so those codes cannot be compared directly.  Every such channel
    must be within `ulps` fp32 ulps of the vector's max-abs value of the
    oracle's mean, and such pools must stay rare."""
    n = rx.shape[0]
    gb = oracle.bf16_rne(gx.ravel()).reshape(n, 128)
    rb = oracle.bf16_rne(rx.ravel()).reshape(n, 128)
    ch = gb != rb
    flip = ch.any(axis=1)
    ref_c, ref_s = rc.copy(), rs.copy()
    worst = 0.0
    if flip.any():
        # fp32 accumulation error is absolute on the vector's scale, so
        # channels near zero (where bf16 values are closest) flip most
        vmax = np.abs(rx).max(axis=1, keepdims=True)
        err_ulps = np.abs(gx.astype(np.float64) - rx) / (2.0**-23 * vmax)
        worst = float(err_ulps[ch].max())
        assert worst <= ulps, \
            f"{what}: a channel rounds differently {worst:.1f} fp32 ulps from the oracle's mean"
        ref_c[flip], ref_s[flip] = oracle.pool_epilogue(gx[flip], round_scale)
    # A rounding-mode error would flip about half of all channels.
    nf = int(flip.sum())
    assert nf <= max(FLIP_FLOOR, FLIP_FRAC * n), f"{what}: {nf} of {n} pools round differently"
    note(f"{what}: {nf} of {n} vectors at a bf16 boundary ({int(ch.sum())} channels, "
         f"worst {worst:.2f} fp32 ulps of the vector max)")
    return ref_c, ref_s, nf


def check_raw_codes(got, ref, what):
    """The literal bar without the boundary rule: at most 0.1% of all codes
    differ from the oracle's (by any number of steps).  Applied to the
    full-size batches, where 0.1% is a meaningful count."""
    d = np.abs(e4m3_ordinal(got) - e4m3_ordinal(ref))
    n_off = int((d != 0).sum())
    note(f"{what}: raw vs oracle {n_off} of {d.size} codes differ, largest by {d.max(initial=0)}")
    assert n_off <= 0.001 * d.size, f"{what}: {n_off} of {d.size} codes differ from the oracle"
    return n_off


# ------------------------------------------------------------------ pool-16 prefill
def run_prefill_gpu(keys, scores, ape, rows, n_pools, round_scale, key_stride=None):
    T = keys.shape[0]
    if key_stride:
        kbuf = np.full((T, key_stride), synth.BF16_NAN, np.uint16)
        kbuf[:, :128] = keys
        sbuf = np.full((T, key_stride), synth.BF16_NAN, np.uint16)
        sbuf[:, :128] = scores
        kt, st = dev(kbuf, torch.int16), dev(sbuf, torch.int16)
    else:
        kt, st = dev(keys, torch.int16), dev(scores, torch.int16)
    rows_t = None if rows is None else dev(rows.astype(np.int32))
    out = torch.full((max(n_pools, 1), 128), 0x7F, dtype=torch.uint8, device="cuda")
    scale = torch.full((max(n_pools, 1),), float("nan"), device="cuda")
    dbg = torch.full((max(n_pools, 1), 128), float("nan"), device="cuda")
    kvc.kvc_compress_prefill(kt, st, dev(ape), rows_t, n_pools, out, scale, round_scale, dbg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), scale.cpu().numpy(), dbg.cpu().numpy()


def compare_prefill(d, rows, round_scale, what, key_stride=None):
    n = rows.size if rows is not None else d["keys"].shape[0] // 16
    note(f"{what}: {n} pools round_scale={round_scale}")
    gc, gs, gx = run_prefill_gpu(d["keys"], d["scores"], d["ape"], rows, n, round_scale, key_stride)
    rc, rs, rx = oracle.compress_prefill(d["keys"], d["scores"], d["ape"], rows, round_scale)
    err = rel_err_rows(gx[:n], rx)
    assert err.max() <= VEC_TOL, f"{what}: fp32 mean rel err {err.max():.3g}"
    ref_c, ref_s, flips = reference_for(gx[:n], rx, rc, rs, round_scale, what)
    n_off = check_codes(gc[:n], ref_c, what)
    check_scales(gs[:n], ref_s, round_scale, what)
    if n * 128 >= RAW_CHECK_MIN_CODES:
        check_raw_codes(gc[:n], rc, what)
    note(f"{what}: max rel err {err.max():.3g}, bf16-boundary pools {flips}, codes off by one "
         f"{n_off}")


def test_pool16_single_sequence_c1():
    d = synth.pool16_single(seed=0)
    compare_prefill(d, kvc.kvc_plan_pool_prefill(d["seq_lens"]), False, "pool16 1x256")


@pytest.mark.parametrize("round_scale", [True, False])
def test_pool16_ragged_prefill_full_size_c2(round_scale):
    d = synth.pool16_ragged(seed=0)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    assert np.array_equal(rows, oracle.pool_plan(d["seq_lens"]))
    compare_prefill(d, rows, round_scale, "pool16 ragged 64 seqs")


@pytest.mark.parametrize("round_scale", [True, False])
def test_pool16_ragged_prefill_128_sequences(round_scale):
    """Twice the configured batch (about 31k pools), both scale modes."""
    d = synth.pool16_ragged(seed=4, num_seqs=128)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    assert rows.size > 30000
    compare_prefill(d, rows, round_scale, "pool16 ragged 128 seqs")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_pool16_ragged_small_with_nan_tails(seed):
    d = synth.pool16_ragged(seed=seed, num_seqs=7, max_len=200)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    covered = np.zeros(d["keys"].shape[0], bool)
    for r in rows:
        covered[r:r + 16] = True
    d["keys"][~covered] = synth.BF16_NAN          # tail tokens must never be read
    d["scores"][~covered] = synth.BF16_NAN
    compare_prefill(d, rows, seed % 2 == 0, f"pool16 ragged small seed {seed}")


def test_pool16_null_rows_and_wide_row_stride():
    d = synth.pool16_single(seed=4, tokens=16 * 37)
    compare_prefill(d, None, True, "pool16 contiguous pools, NULL src rows")
    compare_prefill(d, np.arange(37, dtype=np.int32)[::-1] * 16, False,
                    "pool16 reversed pools, row stride 192", key_stride=192)


def test_pool16_extreme_values():
    g = np.random.default_rng(5)
    P = 9 * 16
    keys = np.zeros((P, 128), np.float32)
    scores = np.zeros((P, 128), np.float32)
    keys[0:16] = 0.0                                   # zero vector -> floor scale
    keys[16:32] = g.standard_normal((16, 128)) * 1e4   # large keys
    keys[32:48] = g.standard_normal((16, 128)) * 1e-6  # tiny keys
    keys[48:64] = 1.0                                  # constant keys
    scores[64:80] = g.standard_normal((16, 128)) * 60  # peaked softmax
    keys[64:80] = g.standard_normal((16, 128))
    scores[80:96, :] = -3e4                            # huge negative scores
    keys[80:96] = g.standard_normal((16, 128))
    keys[96:] = g.standard_normal((48, 128))
    scores[96:] = g.standard_normal((48, 128))
    d = dict(keys=synth.to_bf16_bits(keys), scores=synth.to_bf16_bits(scores),
             ape=synth.ape_pool16(g))
    for rs in (True, False):
        compare_prefill(d, None, rs, "pool16 extreme values")


def test_pool16_empty_and_invalid_rows_untouched():
    d = synth.pool16_single(seed=6, tokens=64)
    kt, st = dev(d["keys"], torch.int16), dev(d["scores"], torch.int16)
    out = torch.full((4, 128), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((4,), 3.0, device="cuda")
    kvc.kvc_compress_prefill(kt, st, dev(d["ape"]), None, 0, out, scale, True)
    rows = dev(np.array([0, 50, -16, 48], np.int32))     # 50 and -16 fall outside 64 rows
    kvc.kvc_compress_prefill(kt, st, dev(d["ape"]), rows, 4, out, scale, True)
    torch.cuda.synchronize()
    o, s = out.cpu().numpy(), scale.cpu().numpy()
    assert np.all(o[1] == 0x55) and np.all(o[2] == 0x55) and s[1] == 3.0 and s[2] == 3.0
    rc, rs, _ = oracle.compress_prefill(d["keys"], d["scores"], d["ape"],
                                        np.array([0, 48], np.int32), True)
    check_codes(o[[0, 3]], rc, "valid rows")
    check_scales(s[[0, 3]], rs, True, "valid rows")


# ------------------------------------------------------------------ number formats
def test_device_fp8_encoder_matches_oracle_on_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)].copy()
    if x.size % 2:
        x = x[:-1]
    xt = dev(x)
    f8 = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    kvc.kvc_diag_convert(xt, None, f8)
    torch.cuda.synchronize()
    got = f8.cpu().numpy()
    ref = oracle.e4m3_encode(x)
    assert np.array_equal(e4m3_ordinal(got), e4m3_ordinal(ref))
    nz = x != 0
    assert np.array_equal(got[nz], ref[nz])


def test_device_bf16_rounding_matches_oracle():
    g = np.random.default_rng(8)
    bits = g.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    ties = ((np.arange(1 << 16, dtype=np.uint32) << 16) | 0x8000)
    x = np.concatenate([bits, ties]).view(np.float32)
    x = x[np.isfinite(x)].copy()
    if x.size % 2:
        x = x[:-1]
    bf = torch.empty(x.size, dtype=torch.int16, device="cuda")
    kvc.kvc_diag_convert(dev(x), bf, None)
    torch.cuda.synchronize()
    assert np.array_equal(bf.cpu().numpy().view(np.uint16), oracle.bf16_rne(x))


# ------------------------------------------------------------------ pool-16 ring decode
def run_ring(d):
    """Run ring decode on both sides; return GPU ring / codes / scales and the
    reference ring / codes / scales (bf16-boundary aware, see reference_for:
    the ring kernel's own fp32 means, from its dbg_pooled output, decide which
    pools round differently)."""
    ring = d["ring"].copy()
    n_out = d["num_out"]
    rc = np.full((n_out, 128), 0x33, np.uint8)
    rs = np.full(n_out, 5.0, np.float32)
    pk = np.zeros((n_out, 16, 128), np.uint16)
    ps = np.zeros((n_out, 16, 128), np.uint16)
    oracle.ring_decode(ring, d["tail_slot_mapping"], d["key"], d["score"], d["ape"],
                       d["slot_mapping"], d["positions"], n_out, d["round_scale"],
                       out_code=rc, out_scale=rs, pools_out=(pk, ps))
    gring = dev(d["ring"], torch.int16)
    go = torch.full((n_out, 128), 0x33, dtype=torch.uint8, device="cuda")
    gs = torch.full((n_out,), 5.0, device="cuda")
    gx = torch.full((n_out, 128), float("nan"), device="cuda")
    kvc.kvc_compress_decode_ring(gring, dev(d["tail_slot_mapping"]), dev(d["key"], torch.int16),
                                 dev(d["score"], torch.int16), dev(d["ape"]),
                                 dev(d["slot_mapping"]), dev(d["positions"]), go, gs,
                                 d["round_scale"], dbg_pooled=gx)
    torch.cuda.synchronize()
    gc, gsc, gx = go.cpu().numpy(), gs.cpu().numpy(), gx.cpu().numpy()
    done = np.nonzero(rs != 5.0)[0]
    assert np.array_equal(np.nonzero(~np.isnan(gx[:, 0]))[0], done), "completed rows differ"
    ref_c, ref_s = rc.copy(), rs.copy()
    if done.size:
        # the oracle's pooled means of the same 16-slot pools
        _, _, ox = oracle.compress_prefill(pk[done].reshape(-1, 128), ps[done].reshape(-1, 128),
                                           d["ape"], None, d["round_scale"])
        e = rel_err_rows(gx[done], ox).max()
        assert e <= VEC_TOL, f"ring decode: fp32 mean rel err {e:.3g}"
        c2, s2, flips = reference_for(gx[done], ox, rc[done], rs[done], d["round_scale"],
                                      "ring decode")
        ref_c[done], ref_s[done] = c2, s2
    return gring.cpu().numpy().view(np.uint16), gc, gsc, ring, ref_c, ref_s


def test_ring_decode_full_size_c3():
    d = synth.pool16_ring(seed=0)
    note("ring decode 256x4")
    gring, gc, gs, ring, rc, rs = run_ring(d)
    assert np.array_equal(gring, ring)                 # stashes are exact copies
    done = np.unique(d["slot_mapping"][d["slot_mapping"] >= 0])
    assert done.size > 30
    check_codes(gc, rc, "ring codes")
    check_scales(gs, rs, True, "ring scales")
    untouched = np.setdiff1d(np.arange(d["num_out"]), done)
    assert np.all(gc[untouched] == 0x33) and np.all(gs[untouched] == 5.0)


# 1-4 and 5-8 take the whole-wave kernel with 4 / 8 prefetched tokens, longer
# batches its 16-token form, window by window past 16 (21: a ragged second
# window, 48: three full windows).
@pytest.mark.parametrize("next_n", [1, 2, 3, 5, 8, 9, 16, 21, 48])
def test_ring_decode_ordered_verify_tokens(next_n):
    d = synth.pool16_ring(seed=10 + next_n, num_requests=37, next_n=next_n, pad_frac=0.1)
    d["round_scale"] = next_n % 2 == 1
    note(f"ring decode 37x{next_n}")
    gring, gc, gs, ring, rc, rs = run_ring(d)
    assert np.array_equal(gring, ring)
    check_codes(gc, rc, "ring codes")
    check_scales(gs, rs, d["round_scale"], "ring scales")


def irregular_ring_case(seed, num_requests, next_n):
    """Positions drawn independently in [0, 60] (so a verify batch may close
    several pools, revisit a slot or go backwards), each token in one of its
    request's two ring blocks, 10% padding, 5% of valid tokens with a -1 tail
    slot (read block 0, which no request owns; nothing is stashed)."""
    g = np.random.default_rng(seed)
    R, N = num_requests, next_n
    pos = g.integers(0, 61, size=(R, N)).astype(np.int32)
    pad = g.random((R, N)) < 0.1
    blk = 1 + 2 * np.arange(R)[:, None] + g.integers(0, 2, size=(R, N))
    ts = (16 * blk + pos % 16).astype(np.int32)
    ts[~pad & (g.random((R, N)) < 0.05)] = -1
    closes = ~pad & (pos % 16 == 15) & (g.random((R, N)) < 0.9)
    loc = np.full((R, N), -1, np.int32)
    loc[closes] = g.permutation(int(closes.sum())).astype(np.int32)
    pos[pad], ts[pad], loc[pad] = -1, -1, -1
    key = synth.bf16_normal(g, (R, N, 128))
    score = synth.bf16_normal(g, (R, N, 128))
    key[pad] = synth.BF16_NAN
    score[pad] = synth.BF16_NAN
    return dict(ring=synth.bf16_normal(g, (2 * R + 1, 2, 16, 128)), tail_slot_mapping=ts,
                key=key, score=score, ape=synth.ape_pool16(g), slot_mapping=loc, positions=pos,
                num_out=int(closes.sum()) + 3, round_scale=bool(seed % 2))


@pytest.mark.parametrize("next_n", [4, 8, 13, 24])
def test_ring_decode_irregular_positions(next_n):
    """Several completions per verify batch, repeated slots and tokens in
    different blocks: every instance (4, 8, 16 tokens; windows past 16) keeps
    the per-request token order."""
    d = irregular_ring_case(70 + next_n, 24, next_n)
    note(f"ring decode irregular 24x{next_n}: {d['num_out'] - 3} completions")
    gring, gc, gs, ring, rc, rs = run_ring(d)
    assert np.array_equal(gring, ring)
    check_codes(gc, rc, "irregular ring codes")
    check_scales(gs, rs, d["round_scale"], "irregular ring scales")


def test_ring_decode_sentinel_tail_slot_and_out_of_range_loc():
    d = synth.pool16_ring(seed=3, num_requests=4, next_n=2, pad_frac=0.0)
    # requests own ring blocks 1..4; block 0 is read only through the sentinel
    d["ring"] = synth.bf16_normal(np.random.default_rng(33), (5, 2, 16, 128))
    d["positions"][:] = [[14, 15], [30, 31], [46, 47], [62, 63]]
    d["tail_slot_mapping"][:] = (np.arange(4)[:, None] + 1) * 16 + d["positions"] % 16
    d["tail_slot_mapping"][1, 1] = -1        # completion reads block 0, no stash
    d["slot_mapping"][:] = -1
    d["slot_mapping"][:, 1] = [0, 1, 2, 99]  # 99 >= num_out: skipped
    gring, gc, gs, ring, rc, rs = run_ring(d)
    assert np.array_equal(gring, ring)
    check_codes(gc, rc, "ring codes")
    check_scales(gs, rs, True, "ring scales")
    assert np.all(gc[3] == 0x33)


# ------------------------------------------------------------------ pool-128 decode
def test_c128_decode_full_size_c4():
    d = c128_decode_case(seed=0)
    note("c128 decode 1024")
    st = d["state"].copy()
    ref_out = np.full((1024, 128), np.nan, np.float32)
    oracle.c128_decode(st, d["kv_score_in"], d["ape"], d["indices"], d["seq_lens"], out=ref_out)
    gst = dev(d["state"])
    gout = torch.full((1024, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode(gst, dev(d["kv_score_in"]), gout, dev(d["ape"]),
                               dev(d["indices"]), dev(d["seq_lens"]))
    torch.cuda.synchronize()
    gst, gout = gst.cpu().numpy(), gout.cpu().numpy()
    emit = (d["seq_lens"] - 1) % 128 == 127
    assert np.array_equal(np.isnan(gout), np.isnan(ref_out))
    if emit.any():
        assert rel_err_rows(gout[emit], ref_out[emit]).max() <= VEC_TOL
    compare_state(gst, st, "c128 decode state")


def compare_state(g, r, what):
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN pattern differs"
    rows = ~np.isnan(r[:, 0])
    assert np.array_equal(g[rows, :128], r[rows, :128]), f"{what}: max not bit-exact"
    e_sum = rel_err_rows(g[rows, 128:256], r[rows, 128:256]).max(initial=0)
    e_kv = rel_err_rows(g[rows, 256:], r[rows, 256:]).max(initial=0)
    assert e_sum <= VEC_TOL and e_kv <= VEC_TOL, f"{what}: sum {e_sum:.3g} kv {e_kv:.3g}"
    note(f"{what}: sum err {e_sum:.3g}, kv err {e_kv:.3g}")


def test_c128_decode_chunk_edges_and_invalid_rows():
    g = np.random.default_rng(12)
    B = 9
    seq = np.array([1, 128, 129, 256, 2, 127, 0, 300, 5], np.int32)
    idx = np.array([0, 1, 2, 3, 4, 5, 6, -1, 99], np.int32)   # 7, 8 invalid slots; 6 seq 0
    state = g.standard_normal((8, 384)).astype(np.float32)
    state[:, 128:256] = np.abs(state[:, 128:256]) + 1
    x = g.standard_normal((B, 256)).astype(np.float32)
    ape = (g.standard_normal((128, 128)) * 0.1).astype(np.float32)
    st = state.copy()
    ref = np.full((B, 128), 9.0, np.float32)
    oracle.c128_decode(st, x, ape, idx, seq, out=ref)
    gst = dev(state)
    gout = torch.full((B, 128), 9.0, device="cuda")
    kvc.kvc_c128_online_decode(gst, dev(x), gout, dev(ape), dev(idx), dev(seq))
    torch.cuda.synchronize()
    gout = gout.cpu().numpy()
    assert np.array_equal(gout == 9.0, ref == 9.0)
    em = ref[:, 0] != 9.0
    assert rel_err_rows(gout[em], ref[em]).max() <= VEC_TOL
    compare_state(gst.cpu().numpy(), st, "c128 decode edges")


# ------------------------------------------------------------------ pool-128 prefill
def run_c128_prefill_gpu(d, state, pad=False, load_indices=None):
    n = int(d["extend_lens"].sum())
    cp, wp = kvc.kvc_c128_plan_prefill(d["seq_lens"], d["extend_lens"], n, pad_to_capacity=pad)
    gst = dev(state)
    gout = torch.full((n, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_prefill(gst, dev(d["kv_score_in"]), gout, dev(d["ape"]),
                                dev(d["indices"]), kvc.plans_to_device(cp), cp.size,
                                kvc.plans_to_device(wp), wp.size,
                                load_indices=None if load_indices is None else dev(load_indices))
    torch.cuda.synchronize()
    return gst.cpu().numpy(), gout.cpu().numpy(), cp, wp


def compare_c128_prefill(d, what, pad=False):
    note(what)
    st = d["state"].copy()
    ref = np.full((int(d["extend_lens"].sum()), 128), np.nan, np.float32)
    oracle.c128_prefill(st, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"],
                        out=ref)
    gst, gout, cp, wp = run_c128_prefill_gpu(d, d["state"], pad=pad)
    if not pad:
        assert np.array_equal(cp, d["cplan"]) and np.array_equal(wp, d["wplan"])
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    rows = ~np.isnan(ref[:, 0])
    e = rel_err_rows(gout[rows], ref[rows]).max(initial=0)
    assert e <= VEC_TOL, f"{what}: out err {e:.3g}"
    note(f"{what}: {rows.sum()} vectors, out err {e:.3g}")
    compare_state(gst, st, what + " state")


def test_c128_prefill_full_size_c5():
    compare_c128_prefill(c128_prefill_case(seed=0), "c128 prefill 32 seqs")


def test_c128_prefill_then_decode_equals_one_prefill():
    """A request prefilled up to some length and then decoded token by token
    ends where one prefill over all its tokens ends: every closed chunk's
    vector (from the prefill or from the decode step that closes it) and the
    open chunk's state agree (max bit-exact, sum and kv within tolerance)."""
    g = np.random.default_rng(31)
    T = np.array([1, 127, 128, 129, 300, 256, 385, 200], np.int64)     # total tokens
    P = np.array([1, 1, 100, 129, 130, 1, 256, 200], np.int64)         # prefilled part
    B, S = T.size, 16
    D = T - P                                                           # decoded one by one
    idx = g.permutation(S)[:B].astype(np.int32)
    x = [g.standard_normal((int(t), 256)).astype(np.float32) for t in T]
    ape = dev((g.standard_normal((128, 128)) * 0.1).astype(np.float32))
    note(f"c128 prefill then decode: totals {T.tolist()}, prefilled {P.tolist()}")

    def prefill(lens):
        st = torch.full((S, 384), float("nan"), device="cuda")
        n = int(lens.sum())
        xin = dev(np.concatenate([x[b][:int(lens[b])] for b in range(B)]))
        out = torch.full((n, 128), float("nan"), device="cuda")
        cp, wp = kvc.kvc_c128_plan_prefill(lens, lens, n)
        kvc.kvc_c128_online_prefill(st, xin, out, ape, dev(idx), kvc.plans_to_device(cp), cp.size,
                                    kvc.plans_to_device(wp), wp.size)
        return st, out

    # path A: prefill P, then decode the rest in steps
    stA, outA = prefill(P)
    emitted = {}
    for k in range(int(D.max())):
        act = np.nonzero(D > k)[0]
        xin = dev(np.stack([x[b][int(P[b]) + k] for b in act]))
        out = torch.full((act.size, 128), float("nan"), device="cuda")
        kvc.kvc_c128_online_decode(stA, xin, out, ape, dev(idx[act]),
                                   dev((P[act] + k + 1).astype(np.int32)))
        out = out.cpu().numpy()
        for j, b in enumerate(act):
            if (int(P[b]) + k) % 128 == 127:
                emitted[(b, int(P[b]) + k)] = out[j]
            else:
                assert np.isnan(out[j]).all()
    # path B: one prefill over every token
    stB, outB = prefill(T)
    torch.cuda.synchronize()
    outA, outB = outA.cpu().numpy(), outB.cpu().numpy()
    offA = np.concatenate([[0], np.cumsum(P)[:-1]])
    offB = np.concatenate([[0], np.cumsum(T)[:-1]])
    n_chunks = 0
    for b in range(B):
        for p in range(127, int(T[b]), 128):
            ref = outB[offB[b] + p]
            got = outA[offA[b] + p] if p < P[b] else emitted[(b, p)]
            assert rel_err_rows(got[None], ref[None]).max() <= VEC_TOL, f"request {b} chunk {p}"
            n_chunks += 1
    assert n_chunks == int((T // 128).sum())
    open_rows = idx[T % 128 != 0]
    compare_state(stA.cpu().numpy()[open_rows], stB.cpu().numpy()[open_rows],
                  "c128 prefill + decode vs one prefill")


@pytest.mark.parametrize("seed", [1, 2])
def test_c128_prefill_small_and_padded_plans(seed):
    d = c128_prefill_case(seed=seed, batch=5, max_prior=700, max_extend=900)
    compare_c128_prefill(d, f"c128 prefill small seed {seed}")
    compare_c128_prefill(d, f"c128 prefill small seed {seed} padded", pad=True)


def test_c128_prefill_distinct_load_indices():
    d = c128_prefill_case(seed=3, batch=6, max_prior=400, max_extend=300)
    # the open-chunk state lives in other slots than the ones written back
    load = np.setdiff1d(np.arange(d["num_slots"]), d["indices"])[:d["indices"].size]
    load = np.random.default_rng(4).permutation(load).astype(np.int32)
    state = d["state"].copy()
    state[load] = d["state"][d["indices"]]
    state[d["indices"]] = np.nan
    st = state.copy()
    ref = np.full((int(d["extend_lens"].sum()), 128), np.nan, np.float32)
    oracle.c128_prefill(st, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"],
                        load_indices=load, out=ref)
    gst, gout, _, _ = run_c128_prefill_gpu(d, state, load_indices=load)
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    rows = ~np.isnan(ref[:, 0])
    assert rel_err_rows(gout[rows], ref[rows]).max(initial=0) <= VEC_TOL
    compare_state(gst, st, "c128 prefill load_indices")


def run_c128_prefill_fused_gpu(d, state, pad=False, quant=False, round_scale=True,
                               load_indices=None):
    n = int(d["extend_lens"].sum())
    items = kvc.kvc_c128_plan_prefill_fused(d["seq_lens"], d["extend_lens"], n,
                                            pad_to_capacity=pad)
    gst = dev(state)
    kw = {}
    if quant:
        kw["out_fp8"] = torch.full((n, 128), 0x33, dtype=torch.uint8, device="cuda")
        kw["out_scale"] = torch.full((n,), 5.0, device="cuda")
        kw["round_scale"] = round_scale
    else:
        kw["out"] = torch.full((n, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_prefill_fused(gst, dev(d["kv_score_in"]), dev(d["ape"]),
                                      dev(d["indices"]), kvc.items_to_device(items), items.size,
                                      load_indices=None if load_indices is None
                                      else dev(load_indices), **kw)
    torch.cuda.synchronize()
    outs = [t.cpu().numpy() for k, t in kw.items() if k != "round_scale"]
    return gst.cpu().numpy(), outs, items


def compare_c128_prefill_fused(d, what, pad=False):
    """Single-launch prefill: within tolerance of the oracle and identical to
    the two-launch device path (same per-plan arithmetic)."""
    note(what)
    st = d["state"].copy()
    ref = np.full((int(d["extend_lens"].sum()), 128), np.nan, np.float32)
    oracle.c128_prefill(st, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"],
                        out=ref)
    gst, (gout,), items = run_c128_prefill_fused_gpu(d, d["state"], pad=pad)
    paired = int(sum(1 for it in items if it["compress"]["ragged_id"] != kvc.PLAN_SENTINEL
                     and it["write"]["ragged_id"] != kvc.PLAN_SENTINEL))
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    rows = ~np.isnan(ref[:, 0])
    e = rel_err_rows(gout[rows], ref[rows]).max(initial=0)
    assert e <= VEC_TOL, f"{what}: out err {e:.3g}"
    compare_state(gst, st, what + " state")
    gst2, gout2, _, _ = run_c128_prefill_gpu(d, d["state"])
    assert np.array_equal(gout, gout2, equal_nan=True), f"{what}: differs from two launches"
    assert np.array_equal(gst, gst2, equal_nan=True), f"{what}: state differs from two launches"
    note(f"{what}: {items.size} items ({paired} paired), {rows.sum()} vectors, out err {e:.3g}")
    return paired


@pytest.mark.parametrize("seed", [40, 41])
def test_c128_prefill_result_is_independent_of_plan_order(seed):
    """Race check: the plans (two launches) and work items (one launch) reach
    the GPU in several random orders, with load_indices passed explicitly and
    equal to indices, so the state rows a request reads are the rows it
    replaces.  The compress pass only reads the state and each write (or
    paired item) reads its own row before replacing it, so the outputs and
    states must be the same for every order, bit for bit, and equal the
    oracle's within tolerance."""
    d = c128_prefill_case(seed=seed, batch=12, max_prior=900, max_extend=1100)
    n = int(d["extend_lens"].sum())
    note(f"c128 prefill plan order, seed {seed}: {n} tokens")
    st = d["state"].copy()
    ref = np.full((n, 128), np.nan, np.float32)
    oracle.c128_prefill(st, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"],
                        out=ref)
    cp, wp = kvc.kvc_c128_plan_prefill(d["seq_lens"], d["extend_lens"], n)
    items = kvc.kvc_c128_plan_prefill_fused(d["seq_lens"], d["extend_lens"], n)
    assert wp.size > 0 and np.any(d["prior_counts"] > 0)
    x, ape, idx = dev(d["kv_score_in"]), dev(d["ape"]), dev(d["indices"])
    li = dev(d["indices"].copy())
    g = np.random.default_rng(seed)
    results = []
    for k in range(4):
        pc, pw, pi = (np.arange(a.size) if k == 0 else g.permutation(a.size)
                      for a in (cp, wp, items))
        gst = dev(d["state"])
        gout = torch.full((n, 128), float("nan"), device="cuda")
        kvc.kvc_c128_online_prefill(gst, x, gout, ape, idx, kvc.plans_to_device(cp[pc]), cp.size,
                                    kvc.plans_to_device(wp[pw]), wp.size, load_indices=li)
        fst = dev(d["state"])
        fout = torch.full((n, 128), float("nan"), device="cuda")
        kvc.kvc_c128_online_prefill_fused(fst, x, ape, idx, kvc.items_to_device(items[pi]),
                                          items.size, out=fout, load_indices=li)
        torch.cuda.synchronize()
        results.append([t.cpu().numpy() for t in (gst, gout, fst, fout)])
    for k, r in enumerate(results):
        for i, (a, b) in enumerate(zip(r, results[0])):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
                f"order {k}: output {i} differs from the planner's order"
        assert np.array_equal(r[1], r[3], equal_nan=True), f"order {k}: one launch != two"
        assert np.array_equal(r[0], r[2], equal_nan=True), f"order {k}: states differ"
    gst, gout = results[0][0], results[0][1]
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    rows = ~np.isnan(ref[:, 0])
    e = rel_err_rows(gout[rows], ref[rows]).max(initial=0)
    assert e <= VEC_TOL, f"plan order: out err {e:.3g}"
    compare_state(gst, st, "plan order state")


def test_c128_prefill_fused_full_size_c5():
    assert compare_c128_prefill_fused(c128_prefill_case(seed=0), "c128 fused prefill 32 seqs") > 0


@pytest.mark.parametrize("seed", [1, 2])
def test_c128_prefill_fused_small_and_padded(seed):
    d = c128_prefill_case(seed=seed, batch=5, max_prior=700, max_extend=900)
    compare_c128_prefill_fused(d, f"c128 fused prefill small seed {seed}")
    compare_c128_prefill_fused(d, f"c128 fused prefill small seed {seed} padded", pad=True)


def test_c128_prefill_fused_every_item_kind():
    # prior mid-chunk + closing + trailing (paired); prior aligned (compress-only
    # first segment); single mid-chunk segment (write-only); exact chunk ends.
    seq = np.array([300, 512, 70, 256, 1000, 129, 131, 200], np.int64)
    ext = np.array([250, 256, 10, 200, 990, 1, 130, 199], np.int64)
    d = c128_prefill_case(seed=7, seq_lens=seq, extend_lens=ext)
    assert compare_c128_prefill_fused(d, "c128 fused prefill item kinds") == 4


def test_c128_prefill_fused_quant():
    d = c128_prefill_case(seed=0)
    note("c128 fused prefill quant 32 seqs")
    N = int(d["extend_lens"].sum())
    for rs in (True, False):
        gst, (gc, gs), items = run_c128_prefill_fused_gpu(d, d["state"], quant=True,
                                                          round_scale=rs)
        cp, wp = kvc.kvc_c128_plan_prefill(d["seq_lens"], d["extend_lens"], N)
        g2 = dev(d["state"])
        c2 = torch.full((N, 128), 0x33, dtype=torch.uint8, device="cuda")
        s2 = torch.full((N,), 5.0, device="cuda")
        kvc.kvc_c128_online_prefill_quant(g2, dev(d["kv_score_in"]), c2, s2, dev(d["ape"]),
                                          dev(d["indices"]), kvc.plans_to_device(cp), cp.size,
                                          kvc.plans_to_device(wp), wp.size, rs)
        torch.cuda.synchronize()
        assert np.array_equal(gc, c2.cpu().numpy())
        assert np.array_equal(gs, s2.cpu().numpy())
        assert np.array_equal(gst, g2.cpu().numpy(), equal_nan=True)


def test_c128_prefill_segments_at_every_wave_boundary():
    """Segments that cover one token, one wave's 16 positions, a span across
    two waves, a full chunk, or close a chunk with one or two tokens: after the
    partials meet, each wave finishes its own 16 channels from lane groups
    whose partials may all be empty.  Both launch forms against the oracle,
    and the quantised forms against each other."""
    offs = np.array([0, 127, 16, 15, 62, 0, 127, 100, 126, 48, 112], np.int64)
    ext = np.array([1, 1, 16, 17, 3, 128, 129, 200, 2, 80, 16], np.int64)
    prior = np.array([0, 1, 2, 0, 3, 1, 0, 2, 5, 1, 0], np.int64) * 128 + offs
    d = c128_prefill_case(seed=11, seq_lens=prior + ext, extend_lens=ext)
    compare_c128_prefill(d, "c128 prefill wave-boundary segments")
    compare_c128_prefill_fused(d, "c128 fused prefill wave-boundary segments")
    compare_c128_prefill_fused(d, "c128 fused prefill wave-boundary segments padded", pad=True)
    N = int(ext.sum())
    gst, (gc, gs), _ = run_c128_prefill_fused_gpu(d, d["state"], quant=True)
    cp, wp = kvc.kvc_c128_plan_prefill(d["seq_lens"], d["extend_lens"], N)
    g2 = dev(d["state"])
    c2 = torch.full((N, 128), 0x33, dtype=torch.uint8, device="cuda")
    s2 = torch.full((N,), 5.0, device="cuda")
    kvc.kvc_c128_online_prefill_quant(g2, dev(d["kv_score_in"]), c2, s2, dev(d["ape"]),
                                      dev(d["indices"]), kvc.plans_to_device(cp), cp.size,
                                      kvc.plans_to_device(wp), wp.size, True)
    torch.cuda.synchronize()
    assert np.array_equal(gc, c2.cpu().numpy())
    assert np.array_equal(gs, s2.cpu().numpy())
    assert np.array_equal(gst, g2.cpu().numpy(), equal_nan=True)
    assert (gc != 0x33).any(axis=1).sum() == int((d["seq_lens"] // 128 - prior // 128).sum())


def test_c128_prefill_fused_distinct_load_indices():
    """Open-chunk states read from other slots than the ones written back (the
    single launch's precondition holds: no request reads a written slot)."""
    d = c128_prefill_case(seed=3, batch=6, max_prior=400, max_extend=300)
    load = np.setdiff1d(np.arange(d["num_slots"]), d["indices"])[:d["indices"].size]
    load = np.random.default_rng(4).permutation(load).astype(np.int32)
    state = d["state"].copy()
    state[load] = d["state"][d["indices"]]
    state[d["indices"]] = np.nan
    st = state.copy()
    ref = np.full((int(d["extend_lens"].sum()), 128), np.nan, np.float32)
    oracle.c128_prefill(st, d["kv_score_in"], d["ape"], d["indices"], d["cplan"], d["wplan"],
                        load_indices=load, out=ref)
    gst, (gout,), _ = run_c128_prefill_fused_gpu(d, state, load_indices=load)
    assert np.array_equal(np.isnan(gout), np.isnan(ref))
    rows = ~np.isnan(ref[:, 0])
    assert rel_err_rows(gout[rows], ref[rows]).max(initial=0) <= VEC_TOL
    compare_state(gst, st, "c128 fused prefill load_indices")
    gst2, gout2, _, _ = run_c128_prefill_gpu(d, state, load_indices=load)
    assert np.array_equal(gout, gout2, equal_nan=True) and np.array_equal(gst, gst2, equal_nan=True)


# ------------------------------------------------------------------ tail-ring seeding
@pytest.mark.parametrize("num_seqs,max_len,pad,blocks", [(64, 8192, 0, None), (30, 40, 13, None),
                                                         (7, 5, 0, None), (12, 100, 3, 9)])
def test_seed_tail_ring_bit_exact(num_seqs, max_len, pad, blocks):
    d = synth.pool16_seed(seed=num_seqs, num_seqs=num_seqs, max_len=max_len, pad_tokens=pad)
    ring0 = d["ring"] if blocks is None else d["ring"][:blocks].copy()
    note(f"seed tail ring: {num_seqs} seqs, {d['tslot'].size} tokens, {ring0.shape[0]} blocks")
    ref = ring0.copy()
    oracle.seed_tail_ring(ref, d["key"], d["score"], d["tslot"])
    g = dev(ring0, torch.int16)
    kvc.kvc_seed_tail_ring(g, dev(d["key"], torch.int16), dev(d["score"], torch.int16),
                           dev(d["tslot"]))
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy().view(np.uint16), ref)


def test_seed_then_decode_continues_the_sequence():
    """Seed rings from a prefill batch, then decode the next tokens: every pool
    completed in decode must equal the prefill-path compression of the same
    16 consecutive tokens."""
    d = synth.pool16_seed(seed=5, num_seqs=16, max_len=300)
    g = np.random.default_rng(6)
    ape = synth.ape_pool16(g)
    R, N = 16, 20
    lens = d["seq_lens"]
    nk = synth.bf16_normal(g, (R, N, 128))
    ns = synth.bf16_normal(g, (R, N, 128))
    pos = (lens[:, None] + np.arange(N)).astype(np.int32)
    ts = (np.arange(R)[:, None] * 16 + pos % 16).astype(np.int32)
    loc = np.where(pos % 16 == 15, np.arange(R)[:, None] * 2 + (pos // 16) % 2, -1).astype(np.int32)
    gring = dev(d["ring"], torch.int16)
    kvc.kvc_seed_tail_ring(gring, dev(d["key"], torch.int16), dev(d["score"], torch.int16),
                           dev(d["tslot"]))
    out = torch.full((2 * R, 128), 0x33, dtype=torch.uint8, device="cuda")
    scl = torch.full((2 * R,), 5.0, device="cuda")
    kvc.kvc_compress_decode_ring(gring, dev(ts), dev(nk, torch.int16), dev(ns, torch.int16),
                                 dev(ape), dev(loc), dev(pos), out, scl, True)
    torch.cuda.synchronize()
    gc, gs = out.cpu().numpy(), scl.cpu().numpy()
    starts = synth.ragged_starts(lens)
    checked = 0
    for r in range(R):
        allk = np.concatenate([d["key"][starts[r]:starts[r] + lens[r]], nk[r]])
        alls = np.concatenate([d["score"][starts[r]:starts[r] + lens[r]], ns[r]])
        for t in range(N):
            p = int(pos[r, t])
            if p % 16 != 15 or p < 15:
                continue
            rows = np.arange(p - 15, p + 1)
            rc, rs, rx = oracle.compress_prefill(allk[rows], alls[rows], ape, None, True)
            pc, ps, px = run_prefill_gpu(allk[rows], alls[rows], ape, None, 1, True)
            l = loc[r, t]
            assert np.array_equal(gc[l], pc[0]) and gs[l] == ps[0]
            ref_c, ref_s, _ = reference_for(px[:1], rx, rc, rs, True, "seeded ring")
            check_codes(gc[l][None], ref_c, "seeded ring")
            check_scales(gs[l:l + 1], ref_s, True, "seeded ring")
            checked += 1
    assert checked >= 16


# ------------------------------------------------------------------ paged cache output
def _paged_expect(codes, scales, loc, mask, pages, fill):
    cache = np.full((pages, 132), fill, np.uint8)
    for p in range(loc.size):
        if (mask is None or mask[p]) and 0 <= loc[p] < pages:
            cache[loc[p], :128] = codes[p]
            cache[loc[p], 128:] = np.frombuffer(np.float32(scales[p]).tobytes(), np.uint8)
    return cache


@pytest.mark.parametrize("round_scale,masked,num_seqs,max_len",
                         [(True, True, 9, 900), (False, False, 9, 900),
                          (True, True, 128, 8192)])
def test_paged_prefill_matches_packed_and_oracle(round_scale, masked, num_seqs, max_len):
    d = synth.pool16_ragged(seed=12, num_seqs=num_seqs, max_len=max_len)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    n = rows.size
    g = np.random.default_rng(13)
    pages = n + 37
    loc = g.permutation(pages)[:n].astype(np.int64)
    loc[1] = -5                                          # skipped: outside the cache
    mask = (g.random(n) < 0.75).astype(np.uint8) if masked else None
    note(f"paged prefill: {n} pools into {pages} pages, masked={masked}")
    # packed device result (already held to the oracle by the prefill tests)
    gc, gs, gx = run_prefill_gpu(d["keys"], d["scores"], d["ape"], rows, n, round_scale)
    rc, rs, rx = oracle.compress_prefill(d["keys"], d["scores"], d["ape"], rows, round_scale)
    ref_c, ref_s, _ = reference_for(gx[:n], rx, rc, rs, round_scale, "paged prefill")
    check_codes(gc[:n], ref_c, "paged prefill")
    check_scales(gs[:n], ref_s, round_scale, "paged prefill")
    cache = torch.full((pages, 132), 0xA5, dtype=torch.uint8, device="cuda")
    kvc.kvc_compress_prefill_paged(dev(d["keys"], torch.int16), dev(d["scores"], torch.int16),
                                   dev(d["ape"]), dev(rows), n, cache, dev(loc), round_scale,
                                   write_mask=None if mask is None else dev(mask))
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    assert np.array_equal(got, _paged_expect(gc[:n], gs[:n], loc, mask, pages, 0xA5))
    # layout and skip rules agree with the oracle's paged writer
    oc = np.full((pages, 132), 0xA5, np.uint8)
    oracle.compress_prefill_paged(d["keys"], d["scores"], d["ape"], rows, round_scale, oc, loc,
                                  mask)
    assert np.array_equal(np.all(got == 0xA5, axis=1), np.all(oc == 0xA5, axis=1))


def test_paged_ring_decode_matches_packed():
    d = synth.pool16_ring(seed=14, num_requests=64, next_n=6, pad_frac=0.05)
    note("paged ring decode 64x6")
    gring, gc, gsc, ring, ref_c, ref_s = run_ring(d)
    assert np.array_equal(gring, ring)
    check_codes(gc, ref_c, "ring codes")
    check_scales(gsc, ref_s, True, "ring scales")
    pring = dev(d["ring"], torch.int16)
    cache = torch.full((d["num_out"], 132), 0x5A, dtype=torch.uint8, device="cuda")
    kvc.kvc_compress_decode_ring_paged(pring, dev(d["tail_slot_mapping"]),
                                       dev(d["key"], torch.int16), dev(d["score"], torch.int16),
                                       dev(d["ape"]), dev(d["slot_mapping"]), dev(d["positions"]),
                                       cache, True)
    torch.cuda.synchronize()
    assert np.array_equal(pring.cpu().numpy().view(np.uint16), ring)
    written = ref_s != 5.0
    exp = _paged_expect(gc, gsc, np.arange(d["num_out"]), written, d["num_out"], 0x5A)
    assert np.array_equal(cache.cpu().numpy(), exp)


def check_ring_layers(base, L, seed):
    """One launch over L layers (own ring, keys, scores and ape per layer,
    shared maps) equals L single-layer calls, each checked against the
    oracle.  Layer 0 uses base's rows; the others draw their own."""
    R = base["key"].shape[0]
    rs_mode = bool(base["round_scale"])
    pad = base["positions"] < 0
    g = np.random.default_rng(seed)
    layers = []
    for l in range(L):
        d = dict(base)
        if l:
            d["ring"] = synth.bf16_normal(g, base["ring"].shape)
            d["key"] = synth.bf16_normal(g, base["key"].shape)
            d["score"] = synth.bf16_normal(g, base["score"].shape)
            d["key"][pad] = synth.BF16_NAN
            d["score"][pad] = synth.BF16_NAN
            d["ape"] = synth.ape_pool16(g)
        layers.append(d)
    note(f"ring decode layers {L}x{R}x{base['key'].shape[1]}")
    singles = []
    for l, d in enumerate(layers):
        gring, gc, gsc, ring, ref_c, ref_s = run_ring(d)
        assert np.array_equal(gring, ring)
        check_codes(gc, ref_c, f"ring layer {l} codes")
        check_scales(gsc, ref_s, rs_mode, f"ring layer {l} scales")
        singles.append((gring, gc, gsc))
    n_out = base["num_out"]
    mring = dev(np.stack([d["ring"] for d in layers]), torch.int16)
    mkey = dev(np.stack([d["key"] for d in layers]), torch.int16)
    mscore = dev(np.stack([d["score"] for d in layers]), torch.int16)
    mape = dev(np.stack([d["ape"] for d in layers]))
    mo = torch.full((L, n_out, 128), 0x33, dtype=torch.uint8, device="cuda")
    ms = torch.full((L, n_out), 5.0, device="cuda")
    kvc.kvc_compress_decode_ring_layers(mring, dev(base["tail_slot_mapping"]), mkey, mscore, mape,
                                        dev(base["slot_mapping"]), dev(base["positions"]), mo, ms,
                                        rs_mode)
    torch.cuda.synchronize()
    mring, mo, ms = mring.cpu().numpy().view(np.uint16), mo.cpu().numpy(), ms.cpu().numpy()
    for l, (gring, gc, gsc) in enumerate(singles):
        assert np.array_equal(mring[l], gring), f"layer {l}: ring differs"
        assert np.array_equal(mo[l], gc), f"layer {l}: codes differ"
        assert np.array_equal(ms[l].view(np.uint32), gsc.view(np.uint32)), f"layer {l}: scales"


@pytest.mark.parametrize("next_n,irregular", [(4, False), (6, False), (9, False), (4, True),
                                               (8, True)])
def test_ring_decode_layers_equal_separate_calls(next_n, irregular):
    """Covers the 4-, 8- and 16-token instances; the irregular cases close
    several pools per verify batch (a wave's later completions reuse the ape
    table it already holds in LDS)."""
    if irregular:
        base = irregular_ring_case(140 + next_n, 120, next_n)
        closing = (base["positions"] % 16 == 15) & (base["slot_mapping"] >= 0)
        assert (closing.sum(axis=1) >= 2).any()
    else:
        base = synth.pool16_ring(seed=40 + next_n, num_requests=37, next_n=next_n, pad_frac=0.1)
    check_ring_layers(base, 5, 41)


# ------------------------------------------------------------------ c128 layers / quantised epilogue
def _layer_case(seq_lens, indices, seed, num_slots=2048):
    from tests.helpers import seed_states
    d = synth.c128_decode(seed=seed, batch=indices.size, num_slots=num_slots, seq_lens=seq_lens)
    st = synth.nan_state(num_slots)
    seed_states(st, indices, d["prior_counts"], d["prior_in"], seq_lens.astype(np.int64) - 1,
                d["ape"])
    return st, d["kv_score_in"], d["ape"]


@pytest.mark.parametrize("num_layers", [5, 16])
def test_c128_decode_layers_equal_separate_calls(num_layers):
    """5 layers: workgroup (x, y) is group x of layer y; 16 layers (a multiple
    of 8): the XCD-major layout, here with 38 request groups per layer."""
    base = c128_decode_case(seed=3, batch=300, emit_frac=0.2)
    idx, sl = base["indices"], base["seq_lens"]
    layers = [(base["state"], base["kv_score_in"], base["ape"])]
    layers += [_layer_case(sl, idx, seed=40 + l) for l in range(num_layers - 1)]
    L = len(layers)
    note(f"c128 decode {L} layers x 300")
    st = np.stack([x[0] for x in layers])
    xin = np.stack([x[1] for x in layers])
    ape = np.stack([x[2] for x in layers])
    gst, gout = dev(st), torch.full((L, 300, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode_layers(gst, dev(xin), gout, dev(ape), dev(idx), dev(sl))
    torch.cuda.synchronize()
    gst, gout = gst.cpu().numpy(), gout.cpu().numpy()
    for l in range(L):
        rs = st[l].copy()
        ro = np.full((300, 128), np.nan, np.float32)
        oracle.c128_decode(rs, xin[l], ape[l], idx, sl, out=ro)
        assert np.array_equal(np.isnan(gout[l]), np.isnan(ro))
        e = ~np.isnan(ro[:, 0])
        assert e.sum() > 20
        assert rel_err_rows(gout[l][e], ro[e]).max() <= VEC_TOL
        compare_state(gst[l], rs, f"layer {l} state")


@pytest.mark.parametrize("round_scale", [True, False])
def test_c128_decode_quant_epilogue(round_scale):
    d = c128_decode_case(seed=5, batch=1024, emit_frac=0.5)
    note(f"c128 decode quant round_scale={round_scale}")
    B = 1024
    rs = d["state"].copy()
    emit, rc, rsc, ro = oracle.c128_decode_quant(rs, d["kv_score_in"], d["ape"], d["indices"],
                                                 d["seq_lens"], round_scale)
    args = (dev(d["kv_score_in"]),)
    g1 = dev(d["state"])
    gout = torch.full((B, 128), float("nan"), device="cuda")
    kvc.kvc_c128_online_decode(g1, args[0], gout, dev(d["ape"]), dev(d["indices"]),
                               dev(d["seq_lens"]))
    g2 = dev(d["state"])
    gcodes = torch.full((B, 128), 0x33, dtype=torch.uint8, device="cuda")
    gscale = torch.full((B,), 5.0, device="cuda")
    kvc.kvc_c128_online_decode_quant(g2, args[0], gcodes, gscale, dev(d["ape"]),
                                     dev(d["indices"]), dev(d["seq_lens"]), round_scale)
    torch.cuda.synchronize()
    assert np.array_equal(g1.cpu().numpy(), g2.cpu().numpy(), equal_nan=True)
    gout, gc, gs = gout.cpu().numpy(), gcodes.cpu().numpy(), gscale.cpu().numpy()
    assert np.array_equal(~np.isnan(gout[:, 0]), emit) and emit.sum() > 300
    assert np.all(gc[~emit] == 0x33) and np.all(gs[~emit] == 5.0)
    assert rel_err_rows(gout[emit], ro[emit]).max() <= VEC_TOL
    ref_c, ref_s, flips = reference_for(gout[emit], ro[emit], rc[emit], rsc[emit], round_scale,
                                        "c128 decode quant", ulps=FLIP_ULPS_POOL128)
    check_codes(gc[emit], ref_c, "c128 decode quant")
    check_scales(gs[emit], ref_s, round_scale, "c128 decode quant")
    note(f"c128 decode quant: {emit.sum()} vectors, bf16-boundary vectors {flips}")


def test_c128_prefill_quant_epilogue():
    d = c128_prefill_case(seed=0)
    N = int(d["extend_lens"].sum())
    note("c128 prefill quant 32 seqs")
    rs = d["state"].copy()
    rows, rc, rsc, ro = oracle.c128_prefill_quant(rs, d["kv_score_in"], d["ape"], d["indices"],
                                                  d["cplan"], d["wplan"], True)
    gst, gout, cp, wp = run_c128_prefill_gpu(d, d["state"])
    g2 = dev(d["state"])
    gcodes = torch.full((N, 128), 0x33, dtype=torch.uint8, device="cuda")
    gscale = torch.full((N,), 5.0, device="cuda")
    kvc.kvc_c128_online_prefill_quant(g2, dev(d["kv_score_in"]), gcodes, gscale, dev(d["ape"]),
                                      dev(d["indices"]), kvc.plans_to_device(cp), cp.size,
                                      kvc.plans_to_device(wp), wp.size, True)
    torch.cuda.synchronize()
    assert np.array_equal(gst, g2.cpu().numpy(), equal_nan=True)
    gc, gs = gcodes.cpu().numpy(), gscale.cpu().numpy()
    assert np.array_equal(~np.isnan(gout[:, 0]), rows[:N])
    assert np.all(gc[~rows[:N]] == 0x33)
    r = rows[:N]
    ref_c, ref_s, flips = reference_for(gout[r], ro[:N][r], rc[:N][r], rsc[:N][r], True,
                                        "c128 prefill quant", ulps=FLIP_ULPS_POOL128)
    check_codes(gc[r], ref_c, "c128 prefill quant")
    check_raw_codes(gc[r], rc[:N][r], "c128 prefill quant")
    check_scales(gs[r], ref_s, True, "c128 prefill quant")
    note(f"c128 prefill quant: {r.sum()} vectors, bf16-boundary vectors {flips}")


@pytest.mark.parametrize("loads", [2, 4, 8, 16])
def test_diag_stream_read_reads_every_word(loads):
    g = np.random.default_rng(30 + loads)
    words = g.integers(0, 2**32, size=(3 * 4096 * loads + 4 * 37), dtype=np.uint64).astype(np.uint32)
    src = dev(words.view(np.int32))
    nw = kvc.kvc.stream_read_sink_words(words.size * 4, loads)
    sink = torch.full((nw + 3,), 7, dtype=torch.int32, device="cuda")
    kvc.kvc.kvc_diag_stream_read(src, sink, loads, fold=False)   # the timing form: no stores
    torch.cuda.synchronize()
    assert torch.all(sink == 7)
    kvc.kvc.kvc_diag_stream_read(src, sink, loads, fold=True)
    torch.cuda.synchronize()
    blocks = nw // 4
    padded = np.zeros(blocks * 1024 * loads, np.uint32)
    padded[:words.size] = words
    # [workgroup, load u, wave, lane, word]: a wave's words of every load
    w5 = padded.reshape(blocks, loads, 4, 64, 4)
    exp = np.bitwise_xor.reduce(w5.transpose(0, 2, 1, 3, 4).reshape(blocks, 4, -1), axis=2)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:nw], exp.ravel())
    assert np.all(got[nw:] == 7)


def test_diag_empty_launch_runs():
    for arg_bytes in (0, 64, 112, 136, 448):
        kvc.kvc.kvc_diag_empty_launch(512, 64, arg_bytes)
    kvc.kvc.kvc_diag_empty_launch(0, 64)
    torch.cuda.synchronize()


def test_prepared_calls_equal_direct_calls():
    """A PreparedCall launches exactly what the direct call launches: the
    same results on the same buffers, new results after the buffers' contents
    change, and on an explicit stream."""
    d = synth.pool16_ragged(seed=51, num_seqs=6, max_len=600)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    n = rows.size
    k, s_, a, r = dev(d["keys"], torch.int16), dev(d["scores"], torch.int16), dev(d["ape"]), dev(rows)
    o1 = torch.zeros((n, 128), dtype=torch.uint8, device="cuda")
    c1 = torch.zeros((n,), device="cuda")
    kvc.kvc_compress_prefill(k, s_, a, r, n, o1, c1, True)
    o2 = torch.zeros_like(o1)
    c2 = torch.zeros_like(c1)
    launch = kvc.prepare(kvc.kvc_compress_prefill, k, s_, a, r, n, o2, c2, True)
    assert isinstance(launch, kvc.PreparedCall) and launch.name == "kvc_compress_prefill"
    launch()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2)
    k.copy_(dev(d["scores"], torch.int16))               # new contents, same buffers
    kvc.kvc_compress_prefill(k, s_, a, r, n, o1, c1, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    launch(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2)
    # the pool-128 decode, which updates its state in place, twice in a row
    dd = c128_decode_case(seed=52, batch=100, emit_frac=0.3)
    st1, st2 = dev(dd["state"]), dev(dd["state"])
    x, ap, ix, sl = (dev(dd[kk]) for kk in ("kv_score_in", "ape", "indices", "seq_lens"))
    out1 = torch.full((100, 128), 3.0, device="cuda")
    out2 = torch.full((100, 128), 3.0, device="cuda")
    step = kvc.prepare(kvc.kvc_c128_online_decode, st2, x, out2, ap, ix, sl)
    for _ in range(2):
        kvc.kvc_c128_online_decode(st1, x, out1, ap, ix, sl)
        step()
    torch.cuda.synchronize()
    assert torch.equal(st1.view(torch.int32), st2.view(torch.int32))   # NaN in unused slots
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    # captured in a HIP graph (no fixed stream: it launches on the capture
    # stream) and replayed: the same as two more direct calls
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                           # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    kvc.kvc_c128_online_decode(st1, x, out1, ap, ix, sl)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
        kvc.kvc_c128_online_decode(st1, x, out1, ap, ix, sl)
    torch.cuda.synchronize()
    assert torch.equal(st1.view(torch.int32), st2.view(torch.int32))
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))


def test_explicit_stream_argument():
    """Work is enqueued on the stream passed in (a torch.cuda.Stream or its raw
    handle), not on the current stream."""
    d = synth.pool16_single(seed=0)
    rows = kvc.kvc_plan_pool_prefill(d["seq_lens"])
    n = rows.size
    k, s, a, r = dev(d["keys"], torch.int16), dev(d["scores"], torch.int16), dev(d["ape"]), dev(rows)
    ref_c = torch.zeros((n, 128), dtype=torch.uint8, device="cuda")
    ref_s = torch.zeros((n,), device="cuda")
    kvc.kvc_compress_prefill(k, s, a, r, n, ref_c, ref_s, False)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for handle in (side, side.cuda_stream):
        c = torch.zeros((n, 128), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((n,), device="cuda")
        torch.cuda.synchronize()
        kvc.kvc_compress_prefill(k, s, a, r, n, c, sc, False, stream=handle)
        side.synchronize()
        assert torch.equal(c, ref_c) and torch.equal(sc, ref_s)


def test_concurrent_streams_match_serial_calls():
    """The library keeps no state between calls: pool-16 prefill, ring decode
    and pool-128 decode issued on three streams at once, each on its own
    buffers, give exactly what the same calls give one after another."""
    p = synth.pool16_ragged(seed=21, num_seqs=12, max_len=900)
    rows = kvc.kvc_plan_pool_prefill(p["seq_lens"])
    n = rows.size
    pk, ps, pa, pr = (dev(p["keys"], torch.int16), dev(p["scores"], torch.int16), dev(p["ape"]),
                      dev(rows))
    r = synth.pool16_ring(seed=22, num_requests=48, next_n=4)
    rmaps = [dev(r[k]) for k in ("tail_slot_mapping", "slot_mapping", "positions")]
    rk, rsc, ra = dev(r["key"], torch.int16), dev(r["score"], torch.int16), dev(r["ape"])
    c = c128_decode_case(seed=23, batch=200, num_slots=400, emit_frac=0.2)
    cx, ca, ci, cl = dev(c["kv_score_in"]), dev(c["ape"]), dev(c["indices"]), dev(c["seq_lens"])
    reps = 6

    def fresh():
        return dict(
            pc=[torch.zeros((n, 128), dtype=torch.uint8, device="cuda") for _ in range(reps)],
            ps=[torch.zeros((n,), device="cuda") for _ in range(reps)],
            ring=[dev(r["ring"], torch.int16) for _ in range(reps)],
            rc=[torch.zeros((r["num_out"], 128), dtype=torch.uint8, device="cuda")
                for _ in range(reps)],
            rs=[torch.zeros((r["num_out"],), device="cuda") for _ in range(reps)],
            st=[dev(c["state"]) for _ in range(reps)],
            co=[torch.zeros((200, 128), device="cuda") for _ in range(reps)])

    def run(b, i, streams):
        s0, s1, s2 = streams
        kvc.kvc_compress_prefill(pk, ps, pa, pr, n, b["pc"][i], b["ps"][i], True, stream=s0)
        kvc.kvc_compress_decode_ring(b["ring"][i], rmaps[0], rk, rsc, ra, rmaps[1], rmaps[2],
                                     b["rc"][i], b["rs"][i], True, stream=s1)
        kvc.kvc_c128_online_decode(b["st"][i], cx, b["co"][i], ca, ci, cl, stream=s2)

    serial = fresh()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    for i in range(reps):
        run(serial, i, (cur, cur, cur))
    torch.cuda.synchronize()
    conc = fresh()
    side = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    for i in range(reps):
        run(conc, i, side)
    torch.cuda.synchronize()
    for key in serial:
        for i in range(reps):
            assert torch.equal(serial[key][i].nan_to_num(7.0), conc[key][i].nan_to_num(7.0)), key
