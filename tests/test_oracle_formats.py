"""Pins of the oracle's number formats and rotation against library routines.

bf16 rounding is checked against torch's CPU cast, the OCP e4m3 codec against
torch.float8_e4m3fn and a brute-force nearest-code search, and the rotation
against scipy's Sylvester Hadamard matrix.  None of these share code with the
oracle.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random_patterns():
    g = np.random.default_rng(11)
    bits = g.integers(0, 2**32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.bf16_rne(x), _torch_bf16_bits(x))


def test_bf16_rne_matches_torch_on_every_tie_and_neighbour():
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).ravel()
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.bf16_rne(x), _torch_bf16_bits(x))


def _torch_e4m3_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def test_e4m3_decode_every_code_matches_torch():
    ref = _torch_e4m3_decode_all()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0**-6 and got[0x01] == 2.0**-9


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def _finite_e4m3_values():
    v = oracle.e4m3_decode(np.arange(0, 0x7F))  # non-negative finite codes 0..0x7E
    return v


def test_e4m3_encode_midpoints_tie_to_even():
    v = _finite_e4m3_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)  # exact in fp32
    got = oracle.e4m3_encode(mids)
    lower = np.arange(0, 0x7E)
    expect = np.where(lower % 2 == 0, lower, lower + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(oracle.e4m3_encode(-mids), expect | 0x80)


def test_e4m3_encode_matches_torch_and_bruteforce():
    g = np.random.default_rng(12)
    q = np.concatenate([
        g.uniform(-448, 448, 400_000),
        np.sign(g.standard_normal(400_000)) * np.exp2(g.uniform(-12, 8.8, 400_000)),
        g.uniform(-2.0**-6, 2.0**-6, 200_000),
    ]).astype(np.float32)
    q = np.clip(q, -448, 448)
    got = oracle.e4m3_encode(q)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # independent brute force on a subset: nearest finite value, ties to even code
    v = _finite_e4m3_values()
    sub = q[:20000].astype(np.float64)
    a = np.abs(sub)
    dist = np.abs(a[:, None] - v[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(v.size)
    pick = np.where(cand, codes[None, :] % 2 == 0, False).any(axis=1)
    idx = np.where(pick, np.argmax(cand & (codes[None, :] % 2 == 0), axis=1),
                   np.argmax(cand, axis=1))
    sign = np.signbit(sub).astype(np.uint8) << 7
    assert np.array_equal(got[:20000], idx.astype(np.uint8) | sign)


def test_e4m3_encode_keeps_negative_zero_and_saturates():
    got = oracle.e4m3_encode(np.array([0.0, -0.0, 448.0, -448.0, 460.0, 1e9], np.float32))
    assert list(got) == [0x00, 0x80, 0x7E, 0xFE, 0x7E, 0x7E]


# ------------------------------------------------------------------ rotation
H128 = scipy.linalg.hadamard(128).astype(np.float64)


def test_hadamard_matches_scipy_sylvester_on_bf16_inputs():
    g = np.random.default_rng(13)
    for scale in (1.0, 1e-3, 37.0):
        x = (g.standard_normal(128) * scale).astype(np.float32)
        xb = (_torch_bf16_bits(x).astype(np.uint32) << 16).view(np.float32)
        ref = (H128 @ xb.astype(np.float64) / np.sqrt(128.0)).astype(np.float32)
        assert np.array_equal(oracle.hadamard128(xb), ref)


def test_hadamard_basis_vectors_and_involution():
    e0 = np.zeros(128, np.float32)
    e0[0] = 1
    assert np.all(oracle.hadamard128(e0) == np.float32(1 / np.sqrt(128)))
    ones = np.ones(128, np.float32)
    y = oracle.hadamard128(ones)
    assert y[0] == np.float32(np.sqrt(128.0)) and np.all(y[1:] == 0)
    g = np.random.default_rng(14)
    x = g.standard_normal(128).astype(np.float32)
    xx = oracle.hadamard128(oracle.hadamard128(x))
    np.testing.assert_allclose(xx, x, rtol=0, atol=4e-7 * np.abs(x).max())
    assert abs(np.linalg.norm(oracle.hadamard128(x)) - np.linalg.norm(x)) < 1e-5 * np.linalg.norm(x)


@pytest.mark.parametrize("r", [1, 2, 64, 37, 127])
def test_hadamard_rows_map_to_basis(r):
    row = H128[r].astype(np.float32)
    y = oracle.hadamard128(row)
    expect = np.zeros(128, np.float32)
    expect[r] = np.float32(np.sqrt(128.0))
    assert np.array_equal(y, expect)
