"""Pins of the oracle's stage-one steps: order-free channel means, NVFP4 and
FP8 quantizers, the rank-one compensation vector, and the closed-form byte
counts the MpFA paper page states ("MpFA: Hardware-Efficient Train-Free QK4V8
FlashAttention Kernels on Blackwell GPUs", §4.1, §4.2, §5.1, §6, §7.2, §7.4).
"""
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_tie_even(mags, t):
    """Index of the magnitude nearest to t >= 0 (linear scan), ties to the even index,
    saturating at the top."""
    if t >= mags[-1]:
        return len(mags) - 1
    d = np.abs(np.asarray(mags) - t)
    cand = np.flatnonzero(d == d.min())
    return int(cand[0] if len(cand) == 1 or cand[0] % 2 == 0 else cand[1])


def _e4m3_mags():
    codes = torch.arange(127, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------------ means --
def test_mean_exact_for_dyadic(oracle_mod):
    rng = np.random.default_rng(0)
    x = (rng.integers(-4096, 4096, size=(256, 16)) / 8.0).astype(np.float32)
    m = oracle_mod.channel_mean(x)
    exact = x.astype(np.float64).sum(axis=0) / 256.0  # exact: dyadic sum of small integers/8
    assert np.array_equal(m.astype(np.float64), exact)


def test_mean_permutation_invariant_and_accurate(oracle_mod):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((1000, 32)) * np.exp2(rng.uniform(-8, 8, (1, 32)))).astype(np.float32)
    x[:, 3] += 50.0
    m1 = oracle_mod.channel_mean(x)
    m2 = oracle_mod.channel_mean(np.ascontiguousarray(x[rng.permutation(1000)]))
    assert np.array_equal(m1.view(np.uint32), m2.view(np.uint32))
    for d in range(32):
        ref = math.fsum(float(v) for v in x[:, d]) / 1000.0
        M = float(np.abs(x[:, d]).max())
        # fixed-point rounding (<= 2^-31 M per token, averaged) + fp32 rounding of the result
        assert abs(float(m1[d]) - ref) <= 2.0 ** -30 * M + abs(ref) * 2.0 ** -24 + 1e-45


def test_mean_zero_and_constant(oracle_mod):
    z = np.zeros((10, 16), np.float32)
    assert np.all(oracle_mod.channel_mean(z) == 0)
    c = np.full((7, 16), np.float32(0.1))
    assert np.all(oracle_mod.channel_mean(c) == np.float32(0.1))


# ------------------------------------------------------------------ NVFP4 --
def _grid_rows(rng, rows, D, g_exp=-8):
    """Rows whose NVFP4 quantization is exact: global amax 2688 * 2^g_exp, every
    16-block holds one element of magnitude 6 * s * g (s an E4M3 value)."""
    mags = _e4m3_mags()
    g = 2.0 ** g_exp
    x = np.zeros((rows, D))
    for r in range(rows):
        for b in range(D // 16):
            s = mags[rng.integers(40, 127)] if (r, b) != (0, 0) else 448.0
            codes = rng.integers(0, 8, 16)
            vals = E2M1_VALUES[codes] * np.where(rng.random(16) < 0.5, -1, 1)
            vals[rng.integers(16)] = 6.0 * (1 if rng.random() < 0.5 else -1)
            x[r, b * 16:(b + 1) * 16] = vals * s * g
    return x.astype(np.float32)


def test_nvfp4_roundtrip_exact_on_grid(oracle_mod):
    rng = np.random.default_rng(2)
    x = _grid_rows(rng, 64, 128)
    g = oracle_mod.nvfp4_global_scale(oracle_mod.amax(x))
    assert g == np.float32(2.0 ** -8)
    codes, sf = oracle_mod.nvfp4_quantize(x, g)
    back = oracle_mod.nvfp4_dequantize(codes, sf, g)
    assert np.array_equal(back, x.astype(np.float64))


def test_nvfp4_codes_are_nearest(oracle_mod):
    """Scale byte = nearest E4M3 to fp32(a_b / fp32(6 g)); element code = nearest E2M1
    to fp32(x / fp32(s g)) with ties to even; brute force per element."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 128)) * np.exp2(rng.uniform(-3, 3, (200, 1)))).astype(np.float32)
    x[:, 5] += 7.0
    x[7, 16:32] = 0.0
    x[8, 32:48] = -0.0
    g = oracle_mod.nvfp4_global_scale(oracle_mod.amax(x))
    codes, sf = oracle_mod.nvfp4_quantize(x, g)
    mags = _e4m3_mags()
    six_g = np.float32(6.0) * np.float32(g)
    for r in range(0, 200, 7):
        for b in range(8):
            blk = x[r, b * 16:(b + 1) * 16]
            a = np.float32(np.abs(blk).max())
            t = float(np.float32(a / six_g))
            want = _nearest_tie_even(mags, t)
            assert sf[r, b] == want
            s = np.float32(mags[want])
            sg = np.float32(s * np.float32(g))
            for j in range(16):
                byte = codes[r, (b * 16 + j) // 2]
                c = (byte >> 4) if j % 2 else (byte & 15)
                if s == 0:
                    assert c == (8 if np.signbit(blk[j]) else 0)
                    continue
                y = abs(float(np.float32(blk[j] / sg)))
                idx = _nearest_tie_even(E2M1_VALUES, y)
                assert c == idx | (8 if np.signbit(blk[j]) else 0)


def test_nvfp4_packing_low_nibble_first(oracle_mod):
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -0.5, 1.0  # E2M1 codes 7, 0x9, 2 once s * g == 1
    g = np.float32(1.0 / 448.0)
    codes, sf = oracle_mod.nvfp4_quantize(x, g)
    s = oracle_mod.e4m3_table()[sf[0, 0]]
    assert s == 448.0
    assert codes[0, 0] == (7 | (0x9 << 4)) and codes[0, 1] == 2


def test_nvfp4_error_bound(oracle_mod):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((500, 128)).astype(np.float32)
    x[:, [3, 40, 77]] += rng.normal(0, 2, 3).astype(np.float32)
    g = oracle_mod.nvfp4_global_scale(oracle_mod.amax(x))
    codes, sf = oracle_mod.nvfp4_quantize(x, g)
    back = oracle_mod.nvfp4_dequantize(codes, sf, g)
    s = oracle_mod.e4m3_table()[sf].repeat(16, axis=-1)
    blk_amax = np.abs(x.reshape(500, 8, 16)).max(axis=-1).repeat(16, axis=-1)
    # half of the largest grid step (between 4 and 6) plus the saturation gap above 6 s g
    bound = s * float(g) + np.maximum(0.0, blk_amax - 6.0 * s * float(g)) + 1e-6 * blk_amax
    assert np.all(np.abs(back - x) <= bound)


# -------------------------------------------------------------------- FP8 --
def test_fp8_v_matches_torch_conversion(oracle_mod):
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((300, 128)) * 3).astype(np.float32)
    v[0, 0] = -17.0
    s = oracle_mod.fp8_scale(oracle_mod.amax(v))
    assert s == np.float32(np.float32(17.0) / np.float32(448.0))
    codes = oracle_mod.fp8_quantize(v, s)
    ref = torch.from_numpy((v / s).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())


# ---------------------------------------------------------------- delta_S --
def _bf16_bits_of_f32(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _exact_then_round(qm, kc):
    """bf16(fp32(exact sum of the exact FP64 products)), by math.fsum."""
    exact = np.array([math.fsum(float(a) * float(b) for a, b in zip(qm, row)) for row in kc])
    return _bf16_bits_of_f32(exact.astype(np.float32)), exact


def _fp32_accumulated(qm, kc):
    """A plausible mistake: the dot product accumulated in FP32."""
    out = np.empty(len(kc), dtype=np.float32)
    for j, row in enumerate(kc):
        acc = np.float32(0.0)
        for a, b in zip(qm, row):
            acc = np.float32(acc + np.float32(a) * np.float32(b))
        out[j] = acc
    return _bf16_bits_of_f32(out)


def _direct_to_bf16(x):
    """Another plausible mistake: the FP64 sum rounded to bf16 in one step
    (round to 8 significant bits, ties to even), skipping the fp32 rounding."""
    out = np.empty(len(x), dtype=np.uint16)
    for j, v in enumerate(x):
        if v == 0.0:
            out[j] = 0x8000 if math.copysign(1.0, v) < 0 else 0
            continue
        _, e = math.frexp(v)
        r = round(math.ldexp(v, 8 - e)) * 2.0 ** (e - 8)  # Python round: ties to even
        out[j] = _bf16_bits_of_f32(np.float32(r))
    return out


def test_delta_s_bit_exact_against_exact_sum(oracle_mod):
    """Delta_S = bf16(fp32(sum_d Qbar_d K_c[j, d])) with the sum in FP64 over
    ascending d (products of two fp32 values are exact in FP64).  On inputs
    whose partial sums stay inside FP64's 53 bits -- all of these -- that is
    the exact sum rounded once to fp32 and once to bf16, so the oracle must
    equal math.fsum's exact sum rounded that way, byte for byte."""
    rng = np.random.default_rng(6)
    kc = (rng.standard_normal((2000, 128)) * 2).astype(np.float32)
    qm = (rng.standard_normal(128) * 0.1).astype(np.float32)
    ref, exact = _exact_then_round(qm, kc)
    assert np.array_equal(oracle_mod.delta_s(qm, kc), ref)
    got = oracle_mod.bf16_to_f64(ref)
    rel = np.abs(got - exact) / np.maximum(np.abs(exact), 1e-30)
    assert np.all(rel <= 2.0 ** -8)  # the page's bound for BF16 carriage of delta_S (§7.4)


def test_delta_s_crafted_rounding_rows(oracle_mod):
    """Rows on which the two plausible mistakes give other bytes:
    - catastrophic cancellation: 2^24 + 1 - 2^24 is 0 in FP32 accumulation and
      1 in FP64 (and likewise 2^40 + 3 - 2^40);
    - double rounding: 1 + 2^-8 + 2^-30 rounds to fp32 1 + 2^-8, a bf16 tie
      that goes to the even 1.0, while one rounding straight to bf16 gives
      1 + 2^-7.
    The oracle must give the exact-sum bytes on every row, and each mistake
    must differ from them on the rows built against it."""
    D = 128
    qm = np.zeros(D, dtype=np.float32)
    qm[:3] = 1.0
    rows = np.zeros((6, D), dtype=np.float32)
    rows[0, :3] = [2.0 ** 24, 1.0, -2.0 ** 24]            # FP32 accumulation loses the 1
    rows[1, :3] = [2.0 ** 40, 3.0, -2.0 ** 40]            # likewise the 3
    rows[2, :3] = [1.0, 2.0 ** -8, 2.0 ** -30]            # double rounding
    rows[3, :3] = [-1.0, -(2.0 ** -8), -(2.0 ** -30)]     # its mirror
    rows[4, :3] = [3.0, 2.0 ** -7, 2.0 ** -29]           # the same at 3 (bf16 step 2^-6)
    rows[5, :3] = [1.0, -1.0, 0.0]                        # exact zero
    got = oracle_mod.delta_s(qm, rows)
    ref, exact = _exact_then_round(qm, rows)
    assert np.array_equal(got, ref)
    assert got[0] == 0x3F80 and got[1] == 0x4040 and got[2] == 0x3F80 and got[3] == 0xBF80
    assert got[4] == 0x4040 and got[5] == 0x0000
    fp32acc = _fp32_accumulated(qm, rows)
    assert fp32acc[0] != got[0] and fp32acc[1] != got[1]
    direct = _direct_to_bf16(exact)
    assert direct[2] != got[2] and direct[3] != got[3] and direct[4] != got[4]


def test_delta_s_sums_in_ascending_channel_order(oracle_mod):
    """Where FP64 itself rounds, the stated order decides: 2^60 + 1 - 2^60
    summed over ascending d in FP64 is 0 (the exact sum is 1, and summing the
    other way round, 1 first, keeps it too only if the large terms cancel
    first).  The oracle follows the ascending-d FP64 rule that the GPU
    stage one also follows."""
    D = 128
    qm = np.zeros(D, dtype=np.float32)
    qm[:3] = 1.0
    row = np.zeros((1, D), dtype=np.float32)
    row[0, :3] = [2.0 ** 60, 1.0, -2.0 ** 60]
    assert oracle_mod.delta_s(qm, row)[0] == 0x0000
    row[0, :3] = [2.0 ** 60, -2.0 ** 60, 1.0]
    assert oracle_mod.delta_s(qm, row)[0] == 0x3F80


# ---------------------------------------------------- page closed forms --
def test_page_constants():
    with open(GOLDEN) as f:
        c = json.load(f)
    D = 128
    k_bytes = D / 2 + D / 16  # NVFP4 codes + one E4M3 scale per 16 elements
    v_bytes = D  # FP8
    bf16_bytes = 2 * D * 2
    assert abs(bf16_bytes / (k_bytes + v_bytes) - c["kv_bytes_ratio_vs_bf16"]["value"]) < 1e-12
    # delta_S: one bf16 per (q-head, token); GQA 32:8 -> 4 q-heads per kv-head
    G = 4
    frac = G * 2 / (k_bytes + v_bytes + 8)  # of the decode bytes per token per kv-head
    assert abs(G * 2 / (k_bytes + v_bytes) - c["delta_s_kv_traffic_fraction"]["value"]) < 0.005
    assert frac < 0.05
    assert 128 * 128 == c["score_elements_per_block"]["value"]
    assert 2.0 ** -8 == c["bf16_delta_rel_err_bound"]["value"]
