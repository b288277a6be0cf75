"""Pins of the oracle's number codecs against the formats' own definitions and
against independent library routines (torch's float8_e4m3fn and bfloat16
conversions), plus brute-force nearest-value search.

The formats are the ones the MpFA paper page names ("MpFA: Hardware-Efficient
Train-Free QK4V8 FlashAttention Kernels on Blackwell GPUs", §4.1): NVFP4
elements (E2M1), e4m3 scale factors and FP8 e4m3 for P and V.
"""
import numpy as np
import pytest
import torch

# E2M1 magnitudes by code 0..7 (sign bit 0x8), from the format's definition:
# 1 sign, 2 exponent (bias 1), 1 mantissa bit, subnormal at exponent 0.
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3_torch_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _tie_even_nearest(a, mags):
    """Brute force: index of the nearest magnitude (linear scan), ties to the even index."""
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.argmax(cand, axis=1)
    two = cand.sum(axis=1) > 1
    # a tie is always between two adjacent codes: pick the even one
    idx2 = idx + 1
    pick = np.where(two & (idx % 2 == 1), idx2, idx)
    return np.where(a >= mags[-1], len(mags) - 1, pick)


def _probe_values(mags, lo_exp=-14, hi=None, n_random=20000, seed=0):
    mags = np.asarray(mags, dtype=np.float64)
    mids = (mags[1:] + mags[:-1]) / 2
    base = np.concatenate([mags, mids]).astype(np.float32)
    vals = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))]
    rng = np.random.default_rng(seed)
    top = hi if hi is not None else mags[-1] * 1.2
    vals.append((rng.uniform(0, 1, n_random) * top).astype(np.float32))
    vals.append((np.exp2(rng.uniform(lo_exp, np.log2(top), n_random))).astype(np.float32))
    v = np.concatenate(vals)
    v = v[v >= 0]
    return np.concatenate([v, -v]).astype(np.float32)


def test_e2m1_decode_table(oracle_mod):
    t = oracle_mod.e2m1_table()
    assert list(t[:8]) == E2M1_VALUES
    assert list(-t[8:]) == E2M1_VALUES
    assert np.signbit(t[8]) and not np.signbit(t[0])


def test_e4m3_decode_matches_torch(oracle_mod):
    mine = oracle_mod.e4m3_table()
    ref = _e4m3_torch_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6 and mine[0x38] == 1.0


def test_e4m3_encode_matches_torch_in_range(oracle_mod):
    x = _probe_values(oracle_mod.e4m3_table()[:127], lo_exp=-12, hi=448.0)
    x = x[np.abs(x) <= 448.0]
    mine = oracle_mod.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encode_bruteforce_and_saturation(oracle_mod):
    mags = _e4m3_torch_table()[:127]
    x = _probe_values(mags, lo_exp=-13)
    mine = oracle_mod.e4m3_encode(x.astype(np.float64))
    idx = _tie_even_nearest(np.abs(x).astype(np.float64), mags)
    expect = (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(mine, expect)
    big = oracle_mod.e4m3_encode(np.array([464.0, 500.0, 1e30, -1e30, -449.0]))
    assert list(big) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e2m1_encode_bruteforce(oracle_mod):
    mags = np.array(E2M1_VALUES)
    x = _probe_values(mags, lo_exp=-4)
    mine = oracle_mod.e2m1_encode(x.astype(np.float64))
    idx = _tie_even_nearest(np.abs(x).astype(np.float64), mags)
    expect = (idx | np.where(np.signbit(x), 8, 0)).astype(np.uint8)
    assert np.array_equal(mine, expect)
    # explicit ties: 0.25 -> 0, 0.75 -> 1.0 (code 2), 1.25 -> 1.0 (code 2), 2.5 -> 2 (code 4), 5 -> 4 (code 6)
    assert list(oracle_mod.e2m1_encode(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0]))) == \
        [0, 2, 2, 4, 4, 6, 6, 7, 7]


def test_signed_zero(oracle_mod):
    assert list(oracle_mod.e4m3_encode(np.array([0.0, -0.0, -1e-30, 1e-30]))) == [0x00, 0x80, 0x80, 0x00]
    assert list(oracle_mod.e2m1_encode(np.array([0.0, -0.0, -0.1, 0.1]))) == [0, 8, 8, 0]


def test_bf16_rne_matches_torch(oracle_mod):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-30, 30, 100000))).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with both parities of bit 16
    ties = (rng.integers(0, 2 ** 31, 1000, dtype=np.uint32) & 0x7F7F0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32), np.float32([0.0, -0.0, 1.0, -3.0e38])])
    mine = oracle_mod.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
