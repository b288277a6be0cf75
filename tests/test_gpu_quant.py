"""GPU parity of the stage-one quantizers: the bytes and scalars the HIP
kernels write must equal the oracle's bit for bit (means, NVFP4 K codes and
scales, the K global scale, Delta_S, FP8 V codes and scale)."""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _compare_k(mpfa, oracle_mod, k, q=None, q_mean=None, smooth=True, dtype=None):
    import torch
    dtype = dtype or torch.float32
    kd = dev(k, dtype)
    qd = None if q is None else dev(q, dtype)
    qmd = None if q_mean is None else dev(q_mean)
    got = mpfa.quantize_k(kd, q=qd, q_mean=qmd, smooth=smooth, Hq=None if smooth else 0)
    torch.cuda.synchronize()
    ref = oracle_mod.quantize_k(k, q=q, q_mean=q_mean, smooth=smooth)
    assert_bytes_equal("k_fp4", host(got["k_fp4"]), ref["k_fp4"])
    assert_bytes_equal("k_sf", host(got["k_sf"]), ref["k_sf"])
    assert_bytes_equal("k_gscale", host(got["k_gscale"]).view(np.uint32),
                       np.array([ref["k_gscale"]], dtype=np.float32).view(np.uint32))
    if smooth:
        assert_bytes_equal("k_mean", host(got["k_mean"]).view(np.uint32),
                           ref["k_mean"].astype(np.float32).view(np.uint32))
        if q is not None:
            assert_bytes_equal("q_mean", host(got["q_mean"]).view(np.uint32),
                               ref["q_mean"].astype(np.float32).view(np.uint32))
        assert_bytes_equal("delta_s", host(got["delta_s"]), ref["delta_s"])


def test_quantize_k_smooth_small_fp32(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("prefill_1k_2x1")
    say(f"case: quantize_k smooth fp32 {cfg.B}x{cfg.Hq}/{cfg.Hkv}x{cfg.N}")
    _compare_k(mpfa, oracle_mod, synth.full(cfg, "k"), q=synth.full(cfg, "q"))


def test_quantize_k_smooth_fp32_past_the_last_level_cache(mpfa, oracle_mod):
    """fp32 Q and K of 335 MB together, more than the 256 MiB last-level cache:
    the statistics passes take their streaming form (non-temporal loads,
    four rows in flight) on the fp32 path; every byte as the oracle's."""
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("prefill_1k_2x1", B=1, Hq=16, Hkv=4, N=32768)
    say(f"case: quantize_k smooth fp32 {cfg.B}x{cfg.Hq}/{cfg.Hkv}x{cfg.N} (Q + K 335 MB)")
    _compare_k(mpfa, oracle_mod, synth.full(cfg, "k"), q=synth.full(cfg, "q"))


@pytest.mark.parametrize("N", [1, 77, 1000])
def test_quantize_k_smooth_bf16_gqa_ragged(mpfa, oracle_mod, N):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=2, Hq=10, Hkv=2, N=N)
    say(f"case: quantize_k smooth bf16 G=5 N={N}")
    _compare_k(mpfa, oracle_mod, synth.full(cfg, "k"), q=synth.full(cfg, "q"), dtype=torch.bfloat16)


def test_quantize_k_direct_bf16(mpfa, oracle_mod):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("qwen14b_prefill_32k", B=1, Hq=5, Hkv=1, N=1000)
    say("case: quantize_k direct bf16 with spikes")
    _compare_k(mpfa, oracle_mod, synth.full(cfg, "k"), smooth=False, dtype=torch.bfloat16)


def test_quantize_k_frozen_query_means(mpfa, oracle_mod):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_decode_128k", B=2, Hq=8, Hkv=2, N=700)
    say("case: quantize_k with frozen decode query means")
    _compare_k(mpfa, oracle_mod, synth.full(cfg, "k"), q_mean=synth.q_mean(cfg), dtype=torch.bfloat16)


def test_nvfp4_ties_and_signed_zero(mpfa, oracle_mod):
    """Direct-mode K rows built so that the global scale is exactly 1 and the
    block scales are exact: elements land on every E2M1 midpoint (ties to the
    even code), on -0, just above and below midpoints, and in all-zero
    blocks."""
    rng = np.random.default_rng(7)
    D = 128
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    rows = []
    row = np.zeros(D, dtype=np.float32)
    row[0] = 2688.0  # tensor amax -> global scale 2688 / 2688 = 1
    rows.append(row)
    for s in (1.0, 0.5, 2.0, 0.125, 3.0, 0.0078125, 448.0):
        for sign in (1.0, -1.0):
            row = np.zeros(D, dtype=np.float32)
            for blk in range(8):
                x = np.zeros(16, dtype=np.float32)
                x[0] = 6.0 * s  # block amax -> scale code exactly s
                x[1:8] = sign * mids * s
                x[8:15] = sign * np.nextafter(mids, np.float32(10)) * s if blk % 2 else \
                    sign * np.nextafter(mids, np.float32(-10)) * s
                x[15] = -0.0
                row[blk * 16:(blk + 1) * 16] = x
            rows.append(row)
    rows.append(np.zeros(D, dtype=np.float32))
    rows.append(np.full(D, -0.0, dtype=np.float32))
    rows.append((rng.standard_normal(D) * 1e-3).astype(np.float32))
    k = np.stack(rows)[None, None]
    say(f"case: NVFP4 tie rows ({k.shape[2]} rows)")
    _compare_k(mpfa, oracle_mod, k, smooth=False)


def test_e4m3_codec_sweep_through_v(mpfa, oracle_mod):
    """V with amax exactly 448 has scale 1, so its codes are the E4M3 codes of
    the values themselves: sweep every E4M3 midpoint, its neighbours one ulp
    away, the subnormal range and signed zeros."""
    import torch
    table = oracle_mod.e4m3_table()[:0x7F]
    mids = (table[:-1] + table[1:]) / 2
    vals = [np.float32(448.0)]
    for m in mids.astype(np.float32):
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1000))]
    vals += list(table.astype(np.float32))
    vals += list(np.linspace(0, 2 ** -6, 4001, dtype=np.float32))
    vals = np.array(vals, dtype=np.float32)
    vals = np.concatenate([vals, -vals, np.array([0.0, -0.0], dtype=np.float32)])
    pad = (-len(vals)) % 128
    vals = np.concatenate([vals, np.zeros(pad, dtype=np.float32)])
    v = vals.reshape(1, 1, -1, 128)
    say(f"case: E4M3 sweep, {vals.size} values")
    got = mpfa.quantize_v(dev(v))
    torch.cuda.synchronize()
    ref = oracle_mod.quantize_v(v)
    assert host(got["v_scale"])[0] == np.float32(1.0) == ref["v_scale"]
    rows = mpfa.v_tiles_to_rows(host(got["v_fp8"]), v.shape[2])
    assert_bytes_equal("v_fp8", rows, ref["v_fp8"])


@pytest.mark.parametrize("N,dtype", [(1024, "f32"), (77, "bf16"), (1, "bf16")])
def test_quantize_v(mpfa, oracle_mod, N, dtype):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("qwen14b_prefill_32k", B=2, Hq=4, Hkv=2, N=N, dtype=dtype)
    v = synth.full(cfg, "v")
    say(f"case: quantize_v N={N} {dtype}")
    got = mpfa.quantize_v(dev(v, torch.bfloat16 if dtype == "bf16" else torch.float32))
    torch.cuda.synchronize()
    ref = oracle_mod.quantize_v(v)
    assert_bytes_equal("v_scale", host(got["v_scale"]).view(np.uint32),
                       np.array([ref["v_scale"]], dtype=np.float32).view(np.uint32))
    tiled = host(got["v_fp8"])
    assert_bytes_equal("v_fp8", mpfa.v_tiles_to_rows(tiled, N), ref["v_fp8"])
    # positions past N in the last tile are code 0
    full = mpfa.v_tiles_to_rows(tiled, tiled.shape[2] * 32)
    assert (full[:, :, N:, :] == 0).all()


def test_delta_s_crafted_rounding_rows(mpfa, oracle_mod):
    """Delta_S rows built so that an FP32-accumulated dot product (catastrophic
    cancellation), a single rounding of the FP64 sum straight to bf16 (double
    rounding at a bf16 tie) or another summation order would each give other
    bytes; every row also appears negated, so the K mean is exactly zero and
    K_c = K.  The query mean is frozen (an input)."""
    import torch
    D = 128
    base = np.zeros((8, D), dtype=np.float32)
    base[0, :3] = [2.0 ** 24, 1.0, -2.0 ** 24]
    base[1, :3] = [2.0 ** 40, 3.0, -2.0 ** 40]
    base[2, :3] = [1.0, 2.0 ** -8, 2.0 ** -30]
    base[3, :3] = [3.0, 2.0 ** -7, 2.0 ** -29]
    base[4, :3] = [2.0 ** 60, 1.0, -2.0 ** 60]
    base[5, :3] = [2.0 ** 60, -2.0 ** 60, 1.0]
    base[6, :3] = [1.0, -1.0, 0.0]
    base[7, :3] = [-0.75, 2.0 ** -9, -(2.0 ** -33)]
    k = np.concatenate([base, -base])[None, None]
    qm = np.zeros((1, 1, D), dtype=np.float32)
    qm[0, 0, :3] = 1.0
    say(f"case: crafted Delta_S rounding rows ({k.shape[2]} rows)")
    _compare_k(mpfa, oracle_mod, k, q_mean=qm, dtype=torch.float32)
    ref = oracle_mod.quantize_k(k, q_mean=qm)
    assert ref["delta_s"][0, 0, 0] == 0x3F80 and ref["delta_s"][0, 0, 4] == 0x0000
