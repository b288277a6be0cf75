"""Pins of the oracle's NVFP4 + NVFP4 precision assignment (MpFA paper page,
"MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
Blackwell GPUs", §3.1 and Fig. 3(a): P quantized to NVFP4 with a scale per 16
elements computed on the softmax path, V in NVFP4 for a block-scaled P.V).

What fixes each part, independently of the oracle's own encoders:
* V blocks run along the keys: every dequantized value is the brute-force
  nearest grid value of its (16-key block, channel) under the brute-force
  nearest E4M3 block scale (a head-dim blocking or a transposed layout picks
  other block maxima and fails);
* P: an identity V makes acc expose 448 p^ key by key; each p^ is the
  brute-force nearest NVFP4 value of fp32(p) in its 16-key group with the
  global scale fp32(1/2688) (masked keys count as zero), and l sums the
  unquantized p;
* the lossless special case: scores with lam * S in {0, -1, -2} (p spans at
  most 4x inside any 16-key group) and V on the NVFP4 grid along the keys
  make both quantizations exact up to the rounding of the two global scales
  (relative 2^-24 each), so the output equals exact attention to 3e-7;
* a key whose scaled p sits on an E2M1 midpoint is reported as ambiguous.
"""
import math

import numpy as np
import pytest

G_P = np.float32(1.0) / np.float32(2688.0)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_positive():
    """All finite non-negative E4M3 magnitudes, by code (0 .. 0x7E), from
    the format's definition (bias 7, subnormals m/8 * 2^-6)."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


E4M3 = _e4m3_positive()


def _nearest(a, table):
    """Index of the nearest table entry to a >= 0 (ties to the even index),
    saturating at the last entry: a plain scan."""
    if a >= table[-1]:
        return len(table) - 1
    d = np.abs(table - a)
    best = np.flatnonzero(d == d.min())
    return int(best[0] if len(best) == 1 else best[best % 2 == 0][0])


def _brute_block(x, g):
    """NVFP4 of 16 fp32 values with global scale g, by nearest-value scans:
    returns the dequantized values (FP64)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).max()
    six_g = np.float32(6.0) * np.float32(g)
    s = E4M3[_nearest(float(np.float32(a / six_g)), E4M3)]
    sg = np.float32(np.float32(s) * np.float32(g))
    if s == 0.0 or sg == 0.0:
        return np.zeros(16)
    out = np.empty(16)
    for i, xi in enumerate(x):
        qv = float(np.float32(np.float32(abs(xi)) / sg))
        out[i] = math.copysign(E2M1[_nearest(qv, E2M1)], xi) * s * float(g)
    return out


# --------------------------------------------------------------------- V ----
def test_v_nvfp4_blocks_run_along_the_keys(oracle_mod):
    rng = np.random.default_rng(30)
    N, D = 50, 128  # three whole 16-key blocks and a ragged one of 2
    v = rng.standard_normal((1, 2, N, D)).astype(np.float32)
    v[0, 1, 7, 5] = 9.0  # the tensor amax
    v[0, 0, 33, 100] = -3.0e-3  # a small block
    v[0, 0, 32:48, 100] *= 1e-3
    vq = oracle_mod.quantize_v_nvfp4(v)
    assert vq["v_fp4"].shape == (1, 2, 4, D, 8) and vq["v_sf"].shape == (1, 2, 4, D)
    g = vq["v_gscale"]
    assert g == np.float32(np.float32(9.0) / np.float32(2688.0))
    for hk in range(2):
        got = oracle_mod.dequantize_v_nvfp4(vq, 0, hk, N)
        pad = np.zeros((64, D), np.float32)
        pad[:N] = v[0, hk]
        for kb in range(4):
            for d in (0, 5, 63, 100, 127):
                want = _brute_block(pad[16 * kb:16 * kb + 16, d], g)
                n = min(16, N - 16 * kb)
                assert np.array_equal(got[16 * kb:16 * kb + n, d], want[:n]), (hk, kb, d)


def test_v_nvfp4_code_nibble_order(oracle_mod):
    """Key 2t of a block in the low nibble of byte t: a single non-zero key
    per block shows up in exactly the nibble the layout says."""
    N, D = 32, 128
    v = np.zeros((1, 1, N, D), np.float32)
    for d in range(D):
        v[0, 0, d % 32, d] = 6.0  # key d % 32 of channel d
    vq = oracle_mod.quantize_v_nvfp4(v)
    for d in range(D):
        key = d % 32
        kb, t = divmod(key, 16)
        byte = vq["v_fp4"][0, 0, kb, d, t // 2]
        assert (byte >> 4 if t % 2 else byte & 15) == 7  # E2M1 code of 6
        assert vq["v_fp4"][0, 0, kb, d].sum() == byte
        assert vq["v_fp4"][0, 0, 1 - kb, d].sum() == 0


# --------------------------------------------------------------------- P ----
def _probe(oracle_mod, scores, lam_scale, row_pos=-1, amb_rel=None):
    """acc of one row with k = 0, scores given as delta and V = identity
    (key j -> channel j): acc[j] = 448 p^_j."""
    n = len(scores)
    D = 128
    q = np.zeros((1, D))
    k = np.zeros((n, D))
    v = np.eye(n, D)
    kw = {} if amb_rel is None else {"amb_rel": amb_rel}
    return oracle_mod.attn_state(q, np.array([row_pos]), k, v, np.asarray(scores, np.float64), 0, n,
                                 lam_scale, ambiguity=True, p_format="nvfp4", **kw)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("row_pos", [-1, 70, 5])
def test_p_nvfp4_is_the_nearest_value_per_16_keys(oracle_mod, seed, row_pos):
    rng = np.random.default_rng(40 + seed)
    scale = 0.09
    s = rng.normal(0, 12.0, 128)
    s[96:112] -= 400.0  # a group whose p underflow to zero
    m, l, acc, amb = _probe(oracle_mod, s, scale, row_pos)
    lam = scale / math.log(2.0)
    vis = np.arange(128) <= (row_pos if row_pos >= 0 else 127)
    mx = s[vis].max()
    p = np.where(vis, np.exp2(lam * (s - mx)), 0.0)
    assert m[0] == mx
    assert abs(l[0] - p.sum()) <= 1e-15 * p.sum()
    for g0 in range(0, 128, 16):
        want = 448.0 * _brute_block(p[g0:g0 + 16].astype(np.float32), G_P)
        assert np.array_equal(acc[0, g0:g0 + 16], want), g0
    assert not acc[0, ~vis].any()


def test_p_nvfp4_two_blocks_rescale_and_accumulate(oracle_mod):
    """Across two KV blocks of 128 keys the first block's p^ are rescaled by
    alpha like the other formats' (acc = alpha acc + ...)."""
    rng = np.random.default_rng(50)
    scale = 0.1
    lam = scale / math.log(2.0)
    s = rng.normal(0, 10.0, 256)
    s[200] = s.max() + 5.0  # the max moves in the second block
    n, D = 256, 128
    q = np.zeros((1, D))
    k = np.zeros((n, D))
    v = np.zeros((n, D))
    v[:, 0] = 1.0
    m, l, acc = oracle_mod.attn_state(q, np.array([-1]), k, v, s, 0, n, scale, p_format="nvfp4")
    m1 = s[:128].max()
    p1 = np.exp2(lam * (s[:128] - m1))
    q1 = sum(_brute_block(p1[g:g + 16].astype(np.float32), G_P).sum() for g in range(0, 128, 16))
    p2 = np.exp2(lam * (s[128:] - s.max()))
    q2 = sum(_brute_block(p2[g:g + 16].astype(np.float32), G_P).sum() for g in range(0, 128, 16))
    alpha = np.exp2(lam * (m1 - s.max()))
    assert abs(acc[0, 0] - 448.0 * (alpha * q1 + q2)) <= 1e-12 * acc[0, 0]
    assert abs(l[0] - (alpha * p1.sum() + p2.sum())) <= 1e-14 * l[0]


def test_p_nvfp4_midpoint_is_ambiguous(oracle_mod):
    """lam = 1 and p = 2^-3 next to a group max of 1: the element quotient is
    6/8 = 0.75, an E2M1 midpoint (exactly, in fp32), so the key is ambiguous
    even with a zero window; moved 1e-6 (relative) off the midpoint it is
    ambiguous within the FP32-exp2 window only.  A quotient of 3 is not."""
    s = np.zeros(16)
    s[3] = -3.0  # p = 1/8
    s[5] = -1.0  # p = 1/2: quotient 3, not near a midpoint
    scale = math.log(2.0)
    for rel in (None, 0.0):
        _, _, acc, amb = _probe(oracle_mod, s, scale, amb_rel=rel)
        assert amb[0, 3] > 0.0 and amb[0, 5] == 0.0 and amb[0, 0] == 0.0
        assert acc[0, 3] == 448.0 * 1.0 * 448.0 * float(G_P)  # the tie goes to the even code (1.0)
    s[3] = -3.0 + 1.5e-6
    _, _, acc, amb = _probe(oracle_mod, s, scale)
    assert amb[0, 3] > 0.0
    _, _, acc0, amb0 = _probe(oracle_mod, s, scale, amb_rel=0.0)
    assert np.array_equal(acc, acc0) and not amb0.any()


# ------------------------------------------------------ lossless case ----
def _lossless_pv4_inputs(rng, N, Hq=2):
    """lam * S in {0, -1, -2} with key 0 at 0 for every row (so the running
    max is 0 from the first block on), Q and K on the NVFP4 grid as in the
    FP8 lossless case, V on the NVFP4 grid along the keys (per 16-key block
    and channel: codes times 2^e with one entry at +-6 2^e)."""
    D = 128
    q = np.full((1, Hq, N, D), 0.0, np.float32)
    q[..., 0::16] = -10.5
    k = np.zeros((1, 1, N, D), np.float32)
    k[..., 1::16] = 10.5
    k[..., 0:32:16] = 1.75 * rng.choice([0.0, 0.5], size=(1, 1, N, 2))
    k[:, :, 0, 0:32:16] = 0.0
    nb = (N + 15) // 16
    e = rng.integers(-3, 1, size=(nb, D))
    codes = rng.choice(E2M1, size=(nb * 16, D)) * rng.choice([-1.0, 1.0], size=(nb * 16, D))
    top = rng.integers(0, 16, size=(nb, D))
    top[-1] %= N - 16 * (nb - 1)  # the block max must be a key that exists
    for kb in range(nb):
        codes[16 * kb + top[kb], np.arange(D)] = 6.0 * rng.choice([-1.0, 1.0], size=D)
    v = (codes * np.repeat(2.0 ** e, 16, axis=0))[:N][None, None].astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("causal", [True, False])
def test_lossless_pv_nvfp4_equals_exact(oracle_mod, causal):
    from test_oracle_attention import LOSSLESS_SCALE
    rng = np.random.default_rng(60)
    q, k, v = _lossless_pv4_inputs(rng, 300)
    O, L, rows = oracle_mod.prefill_rows(q, k, v, LOSSLESS_SCALE, causal=causal, smooth=False,
                                         out_f64=True, pv="nvfp4")
    Oe, Le = oracle_mod.exact_attention(q, k, v, LOSSLESS_SCALE, causal=causal, rows=rows)
    assert np.abs(O - Oe).max() <= 3e-7 * np.abs(Oe).max()
    assert np.abs(L - Le).max() < 1e-12
    # the same inputs through FP8 P.V are not exact (V off the E4M3 grid at
    # this scale), so the comparison above does tell the formats apart
    O8, _, _ = oracle_mod.prefill_rows(q, k, v, LOSSLESS_SCALE, causal=causal, smooth=False,
                                       out_f64=True)
    assert np.abs(O8 - Oe).max() > 1e-3 * np.abs(Oe).max()


def test_p_nvfp4_scale_midpoint_is_ambiguous(oracle_mod):
    """A 16-key group whose largest p puts amax / fp32(6 G_P) next to the
    E4M3 midpoint 432 (between the scales 416 and 448): the group's scale
    decision is ambiguous, and the key that sets it moves with the other
    scale (its code stays 6, its value follows the scale).  The group that
    holds the row maximum (quotient 6, scale 448) is not ambiguous, and with
    a zero window neither is."""
    s = np.full(32, -100.0)  # p ~ 2^-100: zero codes, far from every midpoint
    s[0] = 0.0  # the row max: group 0's p = 1
    s[16] = math.log2(432.0 / 448.0) + 1e-6  # group 1 amax p ~ 432/448, 1e-6 off the midpoint
    scale = math.log(2.0)  # lam = 1
    _, _, acc, amb = _probe(oracle_mod, s, scale)
    assert amb[0, 16] > 0.0
    assert amb[0, 0] == 0.0 and not amb[0, 17:32].any()
    g = float(G_P)
    assert acc[0, 16] in (448.0 * 6 * 416 * g, 448.0 * 6 * 448 * g)
    assert abs(amb[0, 16] - 448.0 * 6 * 32 * g) < 1e-9
    _, _, acc0, amb0 = _probe(oracle_mod, s, scale, amb_rel=0.0)
    assert np.array_equal(acc, acc0) and not amb0.any()
