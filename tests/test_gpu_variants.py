"""GPU parity of the prefill's precision and placement variants (MpFA page
section 3.1, Fig. 3(a): NVFP4 + BF16 P.V; section 7.4 "Compensation
placement": an element-wise add instead of the rank-one MMA; section 5.1: a
polynomial for part of the exponentials) against the oracle:

* element-wise compensation and the rank-one MMA step: the same scores as
  the smoothing oracle (S = Q~ K~^T + Delta_S before the mask and the max);
* polynomial exp2: the smoothing and direct oracles, with the oracle's
  rounding-ambiguity window widened to the polynomial's relative error
  (2^-13 > 7.5e-5), since a P value that close to an E4M3 midpoint may round
  either way;
* bf16 P.V: the oracle with P rounded to bf16 (of 448 p) and V in bf16; the
  bf16 V cache byte for byte;
* NVFP4 P.V: the oracle with P quantized to NVFP4 per 16 keys and V in NVFP4
  along the keys; the NVFP4 V cache (codes, scales, global scale) byte for
  byte.

Output within |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (+ the ambiguity slack),
LSE within 2e-3, on every row of small cases and on sampled rows of the 32K
benchmark inputs."""
import time

import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_bytes_equal, assert_close, dev, host, say, sweep_count

pytestmark = pytest.mark.gpu

POLY_AMB_REL = 2.0 ** -13


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _caches(mpfa, variant, qd, kd, vd, smooth):
    kq = mpfa.quantize_k(kd, q=qd) if smooth else mpfa.quantize_k(kd, smooth=False)
    if variant == "pv_bf16":
        vq = mpfa.pack_v_bf16(vd)
    elif variant == "pv_nvfp4":
        vq = mpfa.quantize_v_nvfp4(vd)
    else:
        vq = mpfa.quantize_v(vd)
    return kq, vq


PV = {"pv_bf16": "bf16", "pv_nvfp4": "nvfp4"}


def _check(mpfa, oracle_mod, cfg, variant, smooth=True, causal=True, edit=None):
    import torch
    from mixed_precision_flashattention_amd import synth
    in_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    if edit is not None:
        q, k, v = edit(q, k, v)
    say(f"case: prefill variant {variant} B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} {cfg.dtype} "
        f"smooth={smooth} causal={causal}{' ' + edit.__name__ if edit is not None else ''}")
    qd, kd, vd = dev(q, in_dtype), dev(k, in_dtype), dev(v, in_dtype)
    kq, vq = _caches(mpfa, variant, qd, kd, vd, smooth)
    out, lse = mpfa.prefill_variant(variant, qd, kq, vq, cfg.scale, causal=causal,
                                    out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    pv = PV.get(variant, "fp8")
    amb_rel = POLY_AMB_REL if variant == "poly_exp2" else None
    if variant == "pv_bf16":
        ref = oracle_mod.quantize_v_bf16(v)
        tiles = host(vq["v_bf16"])  # [B, Hkv, T, 4, 128, 8]
        B, Hkv, T = tiles.shape[:3]
        rows = tiles.transpose(0, 1, 2, 3, 5, 4).reshape(B, Hkv, T * 32, 128)
        assert_bytes_equal("v_bf16", rows[:, :, :cfg.N], ref)
        assert not rows[:, :, cfg.N:].any(), "the bf16 V cache is zero past N"
    if variant == "pv_nvfp4":
        ref = oracle_mod.quantize_v_nvfp4(v)
        assert_bytes_equal("v_fp4", host(vq["v_fp4"]), ref["v_fp4"])
        assert_bytes_equal("v_sf", host(vq["v_sf"]), ref["v_sf"])
        assert_bytes_equal("v_gscale", host(vq["v_gscale"]).view(np.uint32),
                           np.array([ref["v_gscale"]], np.float32).view(np.uint32))
    O, LSE, _, AMB = oracle_mod.prefill_rows(q, k, v, cfg.scale, causal=causal, smooth=smooth,
                                             ambiguity=True, pv=pv, amb_rel=amb_rel)
    assert_close("out", host(out).reshape(-1, 128), O, slack=AMB)
    assert_close("lse", host(lse).reshape(-1), LSE, atol=LSE_ATOL, rtol=0.0)
    return host(out)


@pytest.mark.parametrize("variant", ["rank_one", "elementwise", "poly_exp2", "pv_bf16", "pv_nvfp4"])
def test_variant_small_config(mpfa, oracle_mod, variant):
    from mixed_precision_flashattention_amd import synth
    _check(mpfa, oracle_mod, synth.config("prefill_1k_2x1"), variant)


@pytest.mark.parametrize("variant", ["rank_one", "elementwise", "poly_exp2", "pv_bf16", "pv_nvfp4"])
@pytest.mark.parametrize("N", [1, 129, 300])
def test_variant_gqa5_spikes_ragged(mpfa, oracle_mod, variant, N):
    from mixed_precision_flashattention_amd import synth
    _check(mpfa, oracle_mod, synth.config("qwen14b_prefill_32k", B=2, Hq=10, Hkv=2, N=N), variant)


@pytest.mark.parametrize("variant", ["poly_exp2", "pv_bf16", "pv_nvfp4"])
def test_variant_direct_mode(mpfa, oracle_mod, variant):
    from mixed_precision_flashattention_amd import synth
    _check(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=4, Hkv=2, N=333), variant,
           smooth=False)


@pytest.mark.parametrize("variant", ["rank_one", "elementwise", "pv_bf16", "pv_nvfp4"])
def test_variant_non_causal(mpfa, oracle_mod, variant):
    from mixed_precision_flashattention_amd import synth
    _check(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=2, Hkv=1, N=260), variant,
           causal=False)


def _zero_k(q, k, v):
    return q, np.zeros_like(k), v


def _same_key(q, k, v):
    return q, np.ascontiguousarray(np.broadcast_to(k[:, :, :1, :], k.shape)), v


def _zero_v(q, k, v):
    return q, k, np.zeros_like(v)


def _zero_q(q, k, v):
    return np.zeros_like(q), k, v


def _offset_query(q, k, v):
    """Queries offset by up to +-6 per channel (bf16-exact): the sequence mean
    carries most of Q, so the compensation term Qbar . K_c dominates the
    scores."""
    x = (q + np.linspace(-6.0, 6.0, q.shape[-1], dtype=np.float32)).astype(np.float32)
    u = x.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32), k, v


@pytest.mark.parametrize("edit", [_zero_k, _same_key, _zero_v, _zero_q, _offset_query],
                         ids=lambda f: f.__name__)
@pytest.mark.parametrize("variant", ["rank_one", "elementwise", "pv_bf16", "pv_nvfp4"])
def test_variant_degenerate_inputs(mpfa, oracle_mod, variant, edit):
    """Zero keys or queries (every score equal: P of a whole group at its
    maximum), keys identical along the sequence (centred K zero), zero V
    (a zero V cache, a zero output), and queries carried mostly by their
    sequence mean (the compensation term dominates the scores), through the
    other compensation placements and P.V precisions."""
    from mixed_precision_flashattention_amd import synth
    out = _check(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=4, Hkv=2, N=200),
                 variant, edit=edit)
    if edit is _zero_v:
        assert not np.any(out), "zero V must give a zero output"


@pytest.mark.parametrize("variant", ["elementwise", "rank_one"])
def test_placements_match_the_library_kernel(mpfa, variant):
    """The three placements of the compensation (the score accumulator's
    input, an element-wise add, a rank-one MMA step) compute the same scores;
    their outputs agree far inside the oracle tolerance."""
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=1, Hq=8, Hkv=2, N=1000)
    q, k, v = (dev(synth.full(cfg, t), torch.bfloat16) for t in ("q", "k", "v"))
    say(f"case: {variant} against the library's compensation placement, N1000")
    kq, vq = mpfa.quantize_k(k, q=q), mpfa.quantize_v(v)
    a, _ = mpfa.prefill(q, kq, vq, cfg.scale, out_dtype=torch.float32)
    b, _ = mpfa.prefill_variant(variant, q, kq, vq, cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(f"{variant} vs library", host(b).reshape(-1, 128), host(a).reshape(-1, 128),
                 atol=1e-3, rtol=5e-3)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["rank_one", "elementwise", "poly_exp2", "pv_bf16", "pv_nvfp4"])
def test_variant_fullsize_qwen14b_32k(mpfa, oracle_mod, variant):
    """Each variant on the 32K benchmark inputs, in the launch configuration the
    benchmark times, on synth.sample_rows."""
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("qwen14b_prefill_32k")
    say(f"case: full-size prefill variant {variant} {cfg.name} (benchmark inputs)")
    t0 = time.time()
    x = synth.device_inputs(cfg, "cuda")
    kq, vq = _caches(mpfa, variant, x["q"], x["k"], x["v"], True)
    rows = synth.sample_rows(cfg)
    idx = [torch.from_numpy(rows[:, i]).cuda() for i in range(3)]
    out, lse = mpfa.prefill_variant(variant, x["q"], kq, vq, cfg.scale, causal=True,
                                    out_dtype=torch.float32, with_lse=True)
    got = host(out[idx[0], idx[1], idx[2]])
    got_lse = host(lse[idx[0], idx[1], idx[2]])
    del out, lse, kq, vq
    torch.cuda.synchronize()
    qh, kh, vh = (x[t].float().cpu().numpy() for t in ("q", "k", "v"))
    del x
    torch.cuda.empty_cache()
    say(f"  gpu done ({time.time() - t0:.1f} s); oracle on {len(rows)} sampled rows")
    ops = oracle_mod.Operands(qh, kh, vh, cfg.scale, smooth=True, identity=False,
                              pv=PV.get(variant, "fp8"))
    O, LSE, _, AMB = oracle_mod.prefill_rows(
        qh, kh, vh, cfg.scale, causal=True, smooth=True, rows=rows, ops=ops, ambiguity=True,
        amb_rel=POLY_AMB_REL if variant == "poly_exp2" else None)
    say(f"  oracle done ({time.time() - t0:.1f} s)")
    assert_close("out f32", got, O, slack=AMB)
    assert_close("lse", got_lse, LSE, atol=LSE_ATOL, rtol=0.0)


# ---- seeded random shapes: variant, batch, KV heads, GQA factor, ragged
# length, input dtype, causality and (for the P.V and exp2 variants)
# smoothing drawn from a fixed seed ----
def _variant_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 3, 5, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))
        variant = str(rng.choice(["rank_one", "elementwise", "poly_exp2", "pv_bf16", "pv_nvfp4"]))
        smooth = variant in ("rank_one", "elementwise") or bool(rng.integers(0, 2))
        cases.append(dict(variant=variant, B=int(rng.integers(1, 4)), Hkv=hkv, Hq=hkv * g,
                          N=int(rng.integers(1, 700)), bf16=bool(rng.integers(0, 2)),
                          causal=bool(rng.integers(0, 2)), smooth=smooth))
    return cases


@pytest.mark.parametrize("case", _variant_cases(20261207, sweep_count(8)), ids=lambda c: (
    f"{c['variant']}-B{c['B']}-H{c['Hq']}x{c['Hkv']}-N{c['N']}-{'bf16' if c['bf16'] else 'f32'}-"
    f"{'causal' if c['causal'] else 'full'}-{'smooth' if c['smooth'] else 'direct'}"))
def test_variant_random_shapes(mpfa, oracle_mod, case):
    from mixed_precision_flashattention_amd import synth
    base = "llama8b_prefill_16k" if case["bf16"] else "prefill_1k_2x1"
    cfg = synth.config(base, B=case["B"], Hq=case["Hq"], Hkv=case["Hkv"], N=case["N"])
    _check(mpfa, oracle_mod, cfg, case["variant"], smooth=case["smooth"], causal=case["causal"])
