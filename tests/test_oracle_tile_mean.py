"""Pins of the oracle's per-query-tile mean mode (the tile-granular reading of
the query smoothing of MpFA §3.2 / §5.1: each query row is centred by the
mean of its own 128-row tile, and the compensation Delta_tile[j] =
Qbar_tile . K~_c[j] enters the scores as a separate term carried in BF16,
like Delta_S, §5.2 / §7.4).

* Tile means: the FP64 mean of each tile's own rows within the fixed-point
  bound (exact on dyadic data), the ragged last tile averaging only the rows
  it has, and order-free inside a tile.
* With identity quantizers the mode is exact attention (the fold restores Q,
  K centring and the LSE row term cancel).
* A lossless case -- centred parts on the NVFP4 grid with zero tile means on
  two channels, tile means of +-10.5 on two other channels that differ from
  tile to tile, keys with a zero sequence mean, lam * S integral -- equals
  exact attention for the full quantized path, so a dropped or misplaced
  tile mean fails it.
* Delta_tile equals the exact rational dot product rounded to fp32 and then
  to bf16, and it is taken against the quantized keys (the unquantized ones
  give other bytes).
* One tile: the query codes equal those of the sequence-mean quantizer.
* A constant key shift leaves the output bit-identical.
"""
import math

import numpy as np
import pytest
import torch

import oracle

from test_oracle_attention import LOSSLESS_SCALE, _lossless_inputs

F32 = np.float32


def _rand(seed, B=1, Hq=2, Hkv=1, N=300, D=128):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, N, D), dtype=F32)
    q[..., 3] += 4.0  # a channel offset the means take out
    k = r.standard_normal((B, Hkv, N, D), dtype=F32)
    k[..., 7] += 3.0
    v = r.standard_normal((B, Hkv, N, D), dtype=F32)
    return q, k, v


def test_tile_means_per_tile_with_ragged_tail():
    q, _, _ = _rand(1, N=300)
    tm = oracle.tile_means(q)
    assert tm.shape == (1, 2, 3, 128)
    for t, (a, b) in enumerate([(0, 128), (128, 256), (256, 300)]):
        ref = q[:, :, a:b].astype(np.float64).mean(axis=2)
        M = np.abs(q[:, :, a:b]).max(axis=2)
        assert np.all(np.abs(tm[:, :, t] - ref) <= 2.0 ** -30 * M * 4 + np.abs(ref) * 2.0 ** -24)
    # dyadic data: exact
    r = np.random.default_rng(2)
    qd = (r.integers(-64, 64, size=(1, 1, 257, 128)) / 8.0).astype(F32)
    tmd = oracle.tile_means(qd)
    for t, (a, b) in enumerate([(0, 128), (128, 256), (256, 257)]):
        np.testing.assert_array_equal(tmd[0, 0, t], (qd[0, 0, a:b].astype(np.float64).mean(axis=0)).astype(F32))


def test_tile_means_order_free_inside_a_tile():
    q, _, _ = _rand(3, N=256)
    perm = np.concatenate([np.random.default_rng(4).permutation(128), 128 + np.arange(128)[::-1]])
    np.testing.assert_array_equal(oracle.tile_means(q), oracle.tile_means(q[:, :, perm]))


@pytest.mark.parametrize("causal", [True, False])
def test_identity_tile_mode_equals_exact(causal):
    q, k, v = _rand(5, B=1, Hq=4, Hkv=2, N=300)
    scale = 1 / math.sqrt(128)
    rows = np.array([[0, h, i] for h in range(4) for i in (0, 1, 127, 128, 200, 299)])
    O, L, _ = oracle.prefill_tile_mean_rows(q, k, v, scale, causal=causal, identity=True, rows=rows,
                                            out_f64=True)
    Oe, Le = oracle.exact_attention(q, k, v, scale, causal=causal, rows=rows)
    assert np.abs(O - Oe).max() < 1e-6 * max(1.0, np.abs(Oe).max())
    assert np.abs(L - Le).max() < 1e-6


def _lossless_tile_inputs(seed, B=1, Hq=2, Hkv=1, N=384):
    rng = np.random.default_rng(seed)
    _, k, v = _lossless_inputs(rng, B, Hq, Hkv, N, nq=N, pm_pairs=True)  # keys: zero sequence mean
    q = np.zeros((B, Hq, N, 128), F32)
    nt = N // 128
    for t in range(nt):
        half = rng.choice([-10.5, 10.5], size=(B, Hq, 64, 2)).astype(F32)
        rows = slice(128 * t, 128 * t + 64)
        q[:, :, rows, 0] = half[..., 0]
        q[:, :, rows, 16] = half[..., 1]
        q[:, :, 128 * t + 64:128 * t + 128, [0, 16]] = -half  # zero tile mean on channels 0, 16
        c = rng.choice([-10.5, 10.5], size=(B, Hq, 2)).astype(F32)
        q[:, :, 128 * t:128 * (t + 1), 32] = c[..., 0:1]  # tile mean +-10.5, centred part 0
        q[:, :, 128 * t:128 * (t + 1), 48] = c[..., 1:2]
    return q, k, v


@pytest.mark.parametrize("causal", [True, False])
def test_lossless_tile_mode_equals_exact(causal):
    q, k, v = _lossless_tile_inputs(7)
    tm = oracle.tile_means(q)
    assert np.all(np.abs(tm[..., [32, 48]]) == 10.5) and np.all(tm[..., [0, 16]] == 0)
    # the tile means differ between tiles, so a wrong tile index changes the scores
    assert np.any(tm[..., 0, [32, 48]] != tm[..., 1, [32, 48]])
    O, L, rows = oracle.prefill_tile_mean_rows(q, k, v, LOSSLESS_SCALE, causal=causal, out_f64=True)
    Oe, Le = oracle.exact_attention(q, k, v, LOSSLESS_SCALE, causal=causal, rows=rows)
    assert np.abs(O - Oe).max() < 1e-12 * max(1.0, np.abs(Oe).max())
    assert np.abs(L - Le).max() < 1e-12


def _fp32_rne(x):
    """The fp32 nearest to the rational x (ties to the even significand)."""
    from fractions import Fraction
    f = np.float32(float(x))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(abs(Fraction(float(c)) - x) for c in cands)
    near = [c for c in cands if abs(Fraction(float(c)) - x) == best]
    if len(near) > 1:
        near = [c for c in near if (int(np.array(c).view(np.uint32)) & 1) == 0]
    return near[0]


def _exact_delta_bits(qbar, kt):
    """bf16(fp32(exact sum)) with the products and the sum in exact rationals."""
    from fractions import Fraction
    qf = [Fraction(float(x)) for x in qbar]
    vals = np.array([_fp32_rne(sum((a * Fraction(float(b)) for a, b in zip(qf, row)), Fraction(0)))
                     for row in kt], dtype=F32)
    return torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_delta_tile_is_the_rounded_exact_dot_with_quantized_keys():
    q, k, _ = _rand(8, Hq=2, Hkv=1, N=200)
    tm = oracle.tile_means(q)
    kq = oracle.quantize_k(k)
    dt = oracle.delta_tile(tm, kq["k_fp4"], kq["k_sf"], kq["k_gscale"])
    assert dt.shape == (1, 2, 2, 200)
    kt = oracle.nvfp4_dequantize(kq["k_fp4"][0, 0], kq["k_sf"][0, 0], kq["k_gscale"])
    for h in range(2):
        for t in range(2):
            np.testing.assert_array_equal(dt[0, h, t], _exact_delta_bits(tm[0, h, t], kt[:60]).tolist()
                                          + list(dt[0, h, t, 60:]))
    # against the unquantized centred keys the bytes differ (a plausible mistake)
    kc = (k[0, 0] - kq["k_mean"][0, 0][None, :]).astype(F32).astype(np.float64)
    wrong = oracle.delta_tile_row(tm[0, 0, 0], kc)
    assert np.mean(wrong != dt[0, 0, 0]) > 0.5
    # and against the sequence mean instead of the tile mean
    wrong2 = oracle.delta_tile_row(oracle.channel_mean(q)[0, 0], kt)
    assert np.mean(wrong2 != dt[0, 0, 0]) > 0.5


def test_delta_tile_enters_the_scores_in_bf16():
    """The mode's output equals the blocked attention of the tile-centred
    operands with the bf16 Delta_tile as the score offset -- and moves when the
    offset is used unrounded (so the rounding is part of what is pinned)."""
    q, k, v = _rand(11, Hq=2, Hkv=1, N=260)
    scale = 1 / math.sqrt(128)
    rows = np.array([[0, h, i] for h in range(2) for i in range(0, 260, 7)])
    O, L, _ = oracle.prefill_tile_mean_rows(q, k, v, scale, rows=rows, out_f64=True)
    tm = oracle.tile_means(q)
    kq = oracle.quantize_k(k)
    vq = oracle.quantize_v(v)
    codes, sf, g = oracle.quantize_q_tiles(q, tm)
    kt = oracle.nvfp4_dequantize(kq["k_fp4"][0, 0], kq["k_sf"][0, 0], kq["k_gscale"])
    vt = oracle.e4m3_table()[vq["v_fp8"][0, 0]]
    moved = 0.0
    for i, (_, h, r) in enumerate(rows):
        t = r // 128
        qop = oracle.nvfp4_dequantize(codes[0, h, r:r + 1], sf[0, h, r:r + 1], g)
        d_bf = oracle.bf16_to_f64(oracle.delta_tile_row(tm[0, h, t], kt))
        d_ex = kt @ tm[0, h, t].astype(np.float64)
        for d, check in ((d_bf, True), (d_ex, False)):
            m, l, acc = oracle.attn_state(qop, np.array([r]), kt, vt, d, 0, 260, scale, True)
            o = acc[0] * float(vq["v_scale"]) / (oracle.P_SCALE * l[0])
            if check:
                np.testing.assert_allclose(o, O[i], rtol=0, atol=1e-12)
            else:
                moved = max(moved, np.abs(o - O[i]).max())
    assert moved > 0.0


def test_one_tile_codes_equal_sequence_mean_codes():
    q, _, _ = _rand(9, N=100)
    tm = oracle.tile_means(q)
    np.testing.assert_array_equal(tm[:, :, 0], oracle.channel_mean(q))
    c1, s1, g1 = oracle.quantize_q_tiles(q, tm)
    c2, s2, g2 = oracle.quantize_q(q, oracle.channel_mean(q))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    assert g1 == g2


def test_constant_key_shift_leaves_output_bit_identical():
    """Exact fp32 steps (dyadic data, power-of-two N): the key mean absorbs the
    shift, and the LSE moves by scale * (Q_i . u) as exact attention's does."""
    r = np.random.default_rng(10)
    N = 256
    q = (r.integers(-32, 32, size=(1, 2, N, 128)) / 8.0).astype(F32)
    k = (r.integers(-32, 32, size=(1, 1, N, 128)) / 8.0).astype(F32)
    v = r.standard_normal((1, 1, N, 128), dtype=F32)
    u = r.integers(-100, 100, 128).astype(F32)
    rows = np.array([[0, h, i] for h in range(2) for i in (0, 100, 129, 255)])
    O1, L1, _ = oracle.prefill_tile_mean_rows(q, k, v, 0.1, rows=rows)
    O2, L2, _ = oracle.prefill_tile_mean_rows(q, (k + u).astype(F32), v, 0.1, rows=rows)
    np.testing.assert_array_equal(O1, O2)
    shift = 0.1 * (q[0][rows[:, 1], rows[:, 2]].astype(np.float64) @ u.astype(np.float64))
    assert np.allclose(L2 - L1, shift, atol=1e-9)
