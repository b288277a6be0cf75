"""GPU parity of the per-query-tile mean prefill (mpfa_prefill_tile_mean)
against the oracle: the tile means and the centred K cache byte for byte,
the output element by element within |gpu - oracle| <= 2e-3 + 1e-2 |oracle|
and the LSE within 2e-3, on every row, over several tiles, ragged tails, GQA
groups and degenerate queries."""
import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_bytes_equal, assert_close, dev, host, say, sweep_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _check_tile(mpfa, oracle_mod, cfg, causal=True, out_bf16=False, edit=None):
    import torch
    from mixed_precision_flashattention_amd import synth
    in_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    if edit is not None:
        q, k, v = edit(q, k, v)
    say(f"case: tile-mean prefill B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} {cfg.dtype} "
        f"causal={causal} out={'bf16' if out_bf16 else 'f32'}{' edited inputs' if edit is not None else ''}")
    qd, kd, vd = dev(q, in_dtype), dev(k, in_dtype), dev(v, in_dtype)
    kq = mpfa.quantize_k(kd)  # centring only
    assert "delta_s" not in kq
    vq = mpfa.quantize_v(vd)
    out, lse, tm = mpfa.prefill_tile_mean(qd, kq, vq, cfg.scale, causal=causal, out_dtype=out_dtype,
                                          with_lse=True)
    torch.cuda.synchronize()
    kref = oracle_mod.quantize_k(k)
    assert_bytes_equal("k_mean", host(kq["k_mean"]).view(np.uint32), kref["k_mean"].view(np.uint32))
    assert_bytes_equal("k_fp4", host(kq["k_fp4"]), kref["k_fp4"])
    assert_bytes_equal("k_sf", host(kq["k_sf"]), kref["k_sf"])
    assert_bytes_equal("tile means", host(tm).view(np.uint32), oracle_mod.tile_means(q).view(np.uint32))
    O, LSE, rows, AMB = oracle_mod.prefill_tile_mean_rows(q, k, v, cfg.scale, causal=causal,
                                                          ambiguity=True)
    extra = 2.0 ** -8 if out_bf16 else 0.0
    assert_close("out", host(out).reshape(-1, 128), O, rtol=1e-2 + extra, slack=AMB)
    assert_close("lse", host(lse).reshape(-1), LSE, atol=LSE_ATOL, rtol=0.0)
    return host(out), O


def test_tile_mean_small_config_full(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_tile(mpfa, oracle_mod, synth.config("prefill_1k_2x1"))


@pytest.mark.parametrize("N", [1, 127, 129, 300])
def test_tile_mean_gqa2_bf16_ragged(mpfa, oracle_mod, N):
    from mixed_precision_flashattention_amd import synth
    _check_tile(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=2, Hq=4, Hkv=2, N=N),
                out_bf16=True)


def test_tile_mean_gqa5_spikes(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_tile(mpfa, oracle_mod, synth.config("qwen14b_prefill_32k", B=1, Hq=10, Hkv=2, N=520))


def test_tile_mean_non_causal(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_tile(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=2, Hkv=1, N=333),
                causal=False)


def test_tile_mean_mha_xcd_mapping(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_tile(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=2, Hq=4, Hkv=4, N=400))


def test_tile_mean_queries_with_large_tile_offsets(mpfa, oracle_mod):
    """Each 128-row tile of Q shifted by its own offset vector (large against
    the spread): the case the per-tile centring is for."""
    from mixed_precision_flashattention_amd import synth

    def edit(q, k, v):
        r = np.random.default_rng(31)
        q = q.copy()
        for t in range(0, q.shape[2], 128):
            q[:, :, t:t + 128] += (6.0 * r.standard_normal((q.shape[0], q.shape[1], 1, 128))).astype(np.float32)
        return q.astype(np.float32), k, v
    _check_tile(mpfa, oracle_mod, synth.config("prefill_1k_2x1", N=600), edit=edit)


def test_tile_mean_degenerate_queries(mpfa, oracle_mod):
    """Q constant inside every tile (the centred queries are all zero, the
    global scale falls back to 1 and only the tile means' column terms remain) and an
    all-zero Q."""
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("prefill_1k_2x1", N=300)

    def const_tiles(q, k, v):
        q = q.copy()
        for t in range(0, q.shape[2], 128):
            q[:, :, t:t + 128] = q[:, :, t:t + 1]
        return q, k, v
    _check_tile(mpfa, oracle_mod, cfg, edit=const_tiles)
    _check_tile(mpfa, oracle_mod, cfg, edit=lambda q, k, v: (np.zeros_like(q), k, v))


def test_tile_mean_with_a_smoothing_cache_is_identical(mpfa, oracle_mod):
    """The K bytes of a smoothing-mode cache are those of the centring-only
    cache, so the tile-mean prefill gives bit-identical results on either."""
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=1, Hq=4, Hkv=1, N=260)
    q, k, v = (dev(synth.full(cfg, t), torch.bfloat16) for t in ("q", "k", "v"))
    say("case: tile-mean prefill on a centring-only and on a smoothing cache, N260")
    vq = mpfa.quantize_v(v)
    o1, l1, _ = mpfa.prefill_tile_mean(q, mpfa.quantize_k(k), vq, cfg.scale, out_dtype=torch.float32,
                                       with_lse=True)
    o2, l2, _ = mpfa.prefill_tile_mean(q, mpfa.quantize_k(k, q=q), vq, cfg.scale,
                                       out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- seeded random shapes: batch, KV heads, GQA factor, ragged length, input
# dtype, causality and output dtype drawn from a fixed seed ----
def _tile_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 3, 5, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))
        cases.append(dict(B=int(rng.integers(1, 4)), Hkv=hkv, Hq=hkv * g, N=int(rng.integers(1, 700)),
                          bf16=bool(rng.integers(0, 2)), causal=bool(rng.integers(0, 2)),
                          out_bf16=bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("case", _tile_cases(20261206, sweep_count(6)), ids=lambda c: (
    f"B{c['B']}-H{c['Hq']}x{c['Hkv']}-N{c['N']}-{'bf16' if c['bf16'] else 'f32'}-"
    f"{'causal' if c['causal'] else 'full'}"))
def test_tile_mean_random_shapes(mpfa, oracle_mod, case):
    from mixed_precision_flashattention_amd import synth
    base = "llama8b_prefill_16k" if case["bf16"] else "prefill_1k_2x1"
    cfg = synth.config(base, B=case["B"], Hq=case["Hq"], Hkv=case["Hkv"], N=case["N"])
    _check_tile(mpfa, oracle_mod, cfg, causal=case["causal"], out_bf16=case["out_bf16"])
