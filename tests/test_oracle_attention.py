"""Pins of the oracle's attention logic against exact FP64 attention, exact
special cases and softmax invariants (MpFA paper page, "MpFA:
Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on Blackwell GPUs":
§3.2 compensation before masking and max, §4.1 FP32 softmax state and FP8 P,
§5.1 base-2 exponent with folded scale, §5.3 split-KV with log-sum-exp merge).
"""
import math

import numpy as np
import torch
import pytest


def _rand_inputs(rng, B, Hq, Hkv, N, D=128, n_out=8, sigma=2.0, nq=None):
    q = rng.standard_normal((B, Hq, nq or N, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    for h in range(Hkv):
        ch = rng.choice(D, n_out, replace=False)
        k[:, h][..., ch] += rng.normal(0, sigma, n_out).astype(np.float32)
    return q, k, v


# ------------------------------------------------------- identity mode ----
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("smooth", [True, False])
def test_identity_prefill_equals_exact(oracle_mod, causal, smooth):
    rng = np.random.default_rng(10)
    q, k, v = _rand_inputs(rng, 2, 4, 2, 300)
    scale = 1 / math.sqrt(128)
    O, L, rows = oracle_mod.prefill_rows(q, k, v, scale, causal=causal, smooth=smooth, identity=True,
                                         out_f64=True)
    Oe, Le = oracle_mod.exact_attention(q, k, v, scale, causal=causal, rows=rows)
    assert np.abs(O - Oe).max() < 1e-12
    assert np.abs(L - Le).max() < 1e-12


@pytest.mark.parametrize("splits", [1, 3, 8])
@pytest.mark.parametrize("smooth", [True, False])
def test_identity_decode_equals_exact(oracle_mod, splits, smooth):
    rng = np.random.default_rng(11)
    N = 1000
    q, k, v = _rand_inputs(rng, 2, 4, 2, N, nq=1)
    qm = rng.normal(0, 1 / math.sqrt(N), (2, 4, 128)).astype(np.float32)
    scale = 1 / math.sqrt(128)
    O, L = oracle_mod.decode(q, k, v, qm, splits, scale, smooth=smooth, identity=True, out_f64=True)
    Oe, Le = oracle_mod.exact_attention(q, k, v, scale, causal=False)
    assert np.abs(O.reshape(-1, 128) - Oe).max() < 1e-12
    assert np.abs(L.ravel() - Le).max() < 1e-12


def test_decode_partitions_are_whole_blocks(oracle_mod):
    from oracle.pipeline import decode_partitions
    assert decode_partitions(131072, 32) == [(4096 * p, 4096 * (p + 1)) for p in range(32)]
    parts = decode_partitions(1000, 3)  # chunk = 128 * ceil(1000 / 384) = 384
    assert parts == [(0, 384), (384, 768), (768, 1000)]
    parts = decode_partitions(200, 8)  # chunk 128: two non-empty partitions, six empty
    assert parts[:2] == [(0, 128), (128, 200)] and all(p0 == p1 for p0, p1 in parts[2:])


# ------------------------------------------------- lossless special case ----
def _lossless_inputs(rng, B, Hq, Hkv, N, nq=None, pm_pairs=False):
    """Q, K on the NVFP4 grid (global scale 2^-8, block scales 448) and V on the
    E4M3 grid (scale 1), arranged so that lam * S is an integer in [-4, 4] with
    lam = 2 / 18.375: every p = 2^-k is exactly representable after the x448 FP8
    rounding, so the quantized path must equal exact attention."""
    D = 128
    nq = nq or N
    q = np.zeros((B, Hq, nq, D), np.float32)
    q[..., 0::16] = np.where(rng.random((B, Hq, nq, 8)) < 0.5, -10.5, 10.5)
    k = np.zeros((B, Hkv, N, D), np.float32)
    k[..., 1::16] = 10.5
    k[..., 0:64:16] = 1.75 * rng.choice([0.0, 0.5], size=(B, Hkv, N, 4))
    table = oracle_mod_table()
    finite = table[np.isfinite(table)]
    v = rng.choice(finite[np.abs(finite) <= 448], size=(B, Hkv, N, D)).astype(np.float32)
    v[..., 0, 0] = 448.0
    if pm_pairs:  # zero channel means: second half of the tokens negates the first
        h = N // 2
        k[:, :, h:] = -k[:, :, :h]
        v[:, :, h:] = -v[:, :, :h]
        hq = nq // 2
        q[:, :, hq:] = -q[:, :, :hq]
    return q, k, v


def oracle_mod_table():
    import oracle
    return oracle.e4m3_table()


LAM = 2.0 / 18.375
LOSSLESS_SCALE = LAM * math.log(2.0)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("pv", ["fp8", "bf16"])
def test_lossless_prefill_equals_exact(oracle_mod, causal, pv):
    """Operands on the grids and lam * S integral: p = 2^-n is exact in E4M3
    and in bf16 (448 p too: 448 = 7 * 2^6), and V on the E4M3 grid is on the
    bf16 grid, so both P.V precision assignments equal exact attention."""
    rng = np.random.default_rng(12)
    q, k, v = _lossless_inputs(rng, 1, 2, 1, 384)
    O, L, rows = oracle_mod.prefill_rows(q, k, v, LOSSLESS_SCALE, causal=causal, smooth=False,
                                         out_f64=True, pv=pv)
    Oe, Le = oracle_mod.exact_attention(q, k, v, LOSSLESS_SCALE, causal=causal, rows=rows)
    assert np.abs(O - Oe).max() < 1e-12 * max(1.0, np.abs(Oe).max())
    assert np.abs(L - Le).max() < 1e-12


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_lossless_decode_equals_exact(oracle_mod, splits):
    rng = np.random.default_rng(13)
    q, k, v = _lossless_inputs(rng, 2, 4, 2, 700, nq=1)
    O, L = oracle_mod.decode(q, k, v, None, splits, LOSSLESS_SCALE, smooth=False, out_f64=True)
    Oe, Le = oracle_mod.exact_attention(q, k, v, LOSSLESS_SCALE, causal=False)
    assert np.abs(O.reshape(-1, 128) - Oe).max() < 1e-12 * max(1.0, np.abs(Oe).max())
    assert np.abs(L.ravel() - Le).max() < 1e-12


def test_lossless_blocking_invariance(oracle_mod):
    rng = np.random.default_rng(14)
    q, k, v = _lossless_inputs(rng, 1, 1, 1, 512)
    qt, kt, vt = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64)
    pos = np.arange(512)
    res = [oracle_mod.attn_state(qt, pos, kt, vt, None, 0, 512, LOSSLESS_SCALE, True, block=bs)
           for bs in (32, 128, 512)]
    for m, l, acc in res[1:]:
        o0 = res[0][2] / res[0][1][:, None]
        assert np.allclose(acc / l[:, None], o0, rtol=1e-14, atol=1e-14)


def test_lossless_smooth_equals_direct_when_means_vanish(oracle_mod):
    rng = np.random.default_rng(15)
    q, k, v = _lossless_inputs(rng, 1, 2, 1, 256, pm_pairs=True)
    q[..., 16:64:16] = 0.0  # keep lam * S within [-2, 2] so every 448 p stays exact
    Os, Ls, _ = oracle_mod.prefill_rows(q, k, v, LOSSLESS_SCALE, smooth=True, out_f64=True)
    Od, Ld, _ = oracle_mod.prefill_rows(q, k, v, LOSSLESS_SCALE, smooth=False, out_f64=True)
    assert np.array_equal(Os, Od) and np.allclose(Ls, Ld, atol=1e-13)


# ------------------------------------------------------------ invariants ----
def test_unit_values_give_unit_output(oracle_mod):
    rng = np.random.default_rng(16)
    q, k, _ = _rand_inputs(rng, 1, 2, 1, 640)
    v = np.ones_like(k)
    O, _, _ = oracle_mod.prefill_rows(q, k, v, 1 / math.sqrt(128))
    # each p-hat is within one E4M3 rounding (2^-4 relative) of 448 p, subnormal tails aside
    assert np.all(np.abs(O - 1.0) <= 2.0 ** -4 + 5e-3)


def test_causal_row0_is_first_value(oracle_mod):
    rng = np.random.default_rng(17)
    q, k, v = _rand_inputs(rng, 1, 4, 2, 200)
    O, _, rows = oracle_mod.prefill_rows(q, k, v, 1 / math.sqrt(128))
    vq = oracle_mod.quantize_v(v)
    vt = oracle_mod.e4m3_table()[vq["v_fp8"]] * float(vq["v_scale"])
    for r, (b, h, i) in enumerate(rows):
        if i == 0:
            assert np.array_equal(O[r], vt[b, h // 2, 0].astype(np.float32))


def test_identical_keys_give_mean_of_values(oracle_mod):
    rng = np.random.default_rng(18)
    q, k, v = _rand_inputs(rng, 1, 2, 1, 300)
    k[:] = k[:, :, :1]
    for smooth in (True, False):
        O, _, rows = oracle_mod.prefill_rows(q, k, v, 1 / math.sqrt(128), smooth=smooth, out_f64=True)
        vq = oracle_mod.quantize_v(v)
        vt = oracle_mod.e4m3_table()[vq["v_fp8"]] * float(vq["v_scale"])
        for r, (b, h, i) in enumerate(rows):
            assert np.allclose(O[r], vt[b, 0, :i + 1].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_smooth_invariant_to_constant_key_shift(oracle_mod):
    """Adding one vector u to every key leaves O bit-identical in smooth mode when
    all fp32 steps are exact (dyadic data, power-of-two N), and shifts the LSE by
    scale * (Q_i . u), as for exact attention."""
    rng = np.random.default_rng(19)
    N = 256
    q = (rng.integers(-32, 32, (1, 2, N, 128)) / 8.0).astype(np.float32)
    k = (rng.integers(-32, 32, (1, 1, N, 128)) / 8.0).astype(np.float32)
    v = rng.standard_normal((1, 1, N, 128)).astype(np.float32)
    u = rng.integers(-100, 100, 128).astype(np.float32)
    scale = 1 / math.sqrt(128)
    O1, L1, rows = oracle_mod.prefill_rows(q, k, v, scale)
    O2, L2, _ = oracle_mod.prefill_rows(q, k + u, v, scale)
    assert np.array_equal(O1, O2)
    shift = scale * (q[0][rows[:, 1], rows[:, 2]].astype(np.float64) @ u.astype(np.float64))
    assert np.allclose(L2 - L1, shift, atol=1e-9)


def test_decode_state_equals_prefill_row_state(oracle_mod):
    """One partition over keys [0, i] gives the same state bits as prefill row i."""
    rng = np.random.default_rng(20)
    q, k, v = _rand_inputs(rng, 1, 1, 1, 520)
    qt, kt, vt = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64)
    delta = rng.standard_normal(520)
    for i in (0, 127, 128, 300, 519):
        a = oracle_mod.attn_state(qt[i:i + 1], np.array([i]), kt, vt, delta, 0, 520, 0.1, True)
        b = oracle_mod.attn_state(qt[i:i + 1], np.array([-1]), kt, vt, delta, 0, i + 1, 0.1, True)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_smoothing_reduces_error_on_strong_outliers(oracle_mod):
    rng = np.random.default_rng(21)
    q, k, v = _rand_inputs(rng, 1, 2, 1, 512, n_out=8, sigma=8.0)
    scale = 1 / math.sqrt(128)
    Oe, _ = oracle_mod.exact_attention(q, k, v, scale)
    errs = {}
    for smooth in (True, False):
        O, _, _ = oracle_mod.prefill_rows(q, k, v, scale, smooth=smooth)
        errs[smooth] = np.linalg.norm(O - Oe) / np.linalg.norm(Oe)
    assert errs[True] < errs[False]


def test_ambiguity_bound_marks_p_on_an_e4m3_midpoint(oracle_mod):
    """448 p = 432 lies halfway between the E4M3 values 416 and 448: the bound
    is 32 |v| for that key and zero for a key far from a midpoint, and asking
    for it leaves m, l and acc unchanged."""
    lam = 0.1 / math.log(2.0)
    ds = math.log2(432.0 / 448.0) / lam  # 448 * 2^(lam * ds) = 432
    D = 128
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((3, D))
    k[1, 0] = ds
    k[2, 0] = math.log2(300.0 / 448.0) / lam  # 448 p = 300: far from a midpoint (288 | 320)
    v = np.random.default_rng(3).standard_normal((3, D))
    m, l, acc, amb = oracle_mod.attn_state(q, np.array([-1]), k, v, None, 0, 3, 0.1, True, ambiguity=True)
    np.testing.assert_allclose(amb[0], 32.0 * np.abs(v[1]), rtol=0, atol=0)
    m2, l2, acc2 = oracle_mod.attn_state(q, np.array([-1]), k, v, None, 0, 3, 0.1, True)
    assert m[0] == m2[0] and l[0] == l2[0] and np.array_equal(acc, acc2)
    # without P rounding there is nothing to be ambiguous about
    _, _, _, amb0 = oracle_mod.attn_state(q, np.array([-1]), k, v, None, 0, 3, 0.1, False, ambiguity=True)
    assert not amb0.any()


def _two_key_row(oracle_mod, target, p_format, lam_scale=0.1):
    """One query, two keys: key 0 at the row max (448 p = 448), key 1 placed so
    that 448 p = target; V = unit vectors, so acc holds each key's rounded
    448 p in its own channel."""
    lam = lam_scale / math.log(2.0)
    D = 128
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((2, D))
    k[1, 0] = math.log2(target / 448.0) / lam
    v = np.zeros((2, D))
    v[0, 0] = 1.0
    v[1, 1] = 1.0
    return oracle_mod.attn_state(q, np.array([-1]), k, v, None, 0, 2, lam_scale, True, ambiguity=True,
                                 p_format=p_format)


def test_bf16_p_is_one_rounding_of_448p(oracle_mod):
    """The BF16 P.V assignment rounds 448 p to the nearest bf16 (8 significant
    bits, ties to the even significand): values well inside a bf16 interval
    round like torch's conversion, an exact tie goes to the even neighbour,
    and E4M3 would round the same values differently."""
    for target in (300.4, 301.7, 123.45, 3.3, 0.0123):
        _, _, acc, amb = _two_key_row(oracle_mod, target, "bf16")
        want = torch.tensor(target, dtype=torch.float32).to(torch.bfloat16).double().item()
        assert abs(acc[0, 1] - want) <= 1e-9 * want, (target, acc[0, 1], want)
        assert not amb.any()
        _, _, acc8, _ = _two_key_row(oracle_mod, target, "e4m3")
        assert acc8[0, 1] != acc[0, 1]
    # 301 lies halfway between 300 (even significand) and 302
    _, _, acc, amb = _two_key_row(oracle_mod, 301.0, "bf16")
    assert acc[0, 1] == 300.0 and acc[0, 0] == 448.0
    assert amb[0, 1] == 2.0 and amb[0, 0] == 0.0


def test_ambiguity_window_widens_with_the_exp2_error(oracle_mod):
    """A P value 1e-4 (relative) away from an E4M3 midpoint is unambiguous for
    an FP32 exp2 (window 2^-16) and ambiguous for an exp2 with 2^-12 relative
    error."""
    target = 432.0 * (1 + 1e-4)
    _, _, _, amb = _two_key_row(oracle_mod, target, "e4m3")
    assert not amb.any()
    lam_scale = 0.1
    lam = lam_scale / math.log(2.0)
    D = 128
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((2, D))
    k[1, 0] = math.log2(target / 448.0) / lam
    v = np.zeros((2, D))
    v[1, 1] = 1.0
    _, _, _, amb2 = oracle_mod.attn_state(q, np.array([-1]), k, v, None, 0, 2, lam_scale, True,
                                          ambiguity=True, amb_rel=2.0 ** -12)
    assert amb2[0, 1] == 32.0
