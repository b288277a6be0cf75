"""Parity at the full workload sizes, in the launch configuration the benchmark
times (same shapes, same grid, same caches).

Inputs are the seeded device draws the benchmark itself uses
(``synth.device_inputs``, the same laws as the host generator); the oracle
receives host copies of those inputs, never a GPU result.  The GPU runs every
call at full size.  The oracle recomputes the per-tensor statistics (means,
global scales) over the whole inputs and then checks:

* the quantized caches of sampled heads byte for byte (K codes, K block
  scales, FP8 V, the rank-one vector Delta_S), plus the global scales and all
  the means exactly;
* the attention output on sampled outputs: for prefill, ``synth.sample_rows``
  (every row of the first two and of the last query tile of three query heads
  of the first and last batch entry, plus 256 seeded random rows); for
  decode, every query head of the first and last batch entry plus 32 seeded
  random (batch, query head) pairs.

The output is compared both in the dtype the benchmark writes (bf16, one extra
rounding allowed) and in fp32 together with the log-sum-exp.  Tolerances as in
the small parity tests: |gpu - oracle| <= 2e-3 + 1e-2 |oracle|, LSE within 2e-3.
"""
import time

import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_bytes_equal, assert_close, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

BF16_EXTRA = 2.0 ** -8


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _h(t):
    """Host fp32 / raw copy of a device tensor."""
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().cpu().numpy()
    if t.dtype == torch.int16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _check_caches(mpfa, ops, kq, vq, cfg):
    """Global scales and means exactly; cache bytes of sampled heads."""
    assert_bytes_equal("k_gscale", _h(kq["k_gscale"]).view(np.uint32),
                       np.asarray([ops.kq["k_gscale"]], dtype=np.float32).view(np.uint32))
    assert_bytes_equal("v_scale", _h(vq["v_scale"]).view(np.uint32),
                       np.asarray([ops.vq["v_scale"]], dtype=np.float32).view(np.uint32))
    assert_bytes_equal("k_mean", _h(kq["k_mean"]).view(np.uint32),
                       ops.k_mean.astype(np.float32).view(np.uint32))
    assert_bytes_equal("q_mean", _h(kq["q_mean"]).view(np.uint32),
                       ops.kq["q_mean"].astype(np.float32).view(np.uint32))
    for b in sorted({0, cfg.B - 1}):
        for hk in sorted({0, cfg.Hkv - 1}):
            tag = f"[b={b} kv={hk}]"
            assert_bytes_equal("k_fp4" + tag, _h(kq["k_fp4"][b, hk]), ops.kq["k_fp4"][b, hk])
            assert_bytes_equal("k_sf" + tag, _h(kq["k_sf"][b, hk]), ops.kq["k_sf"][b, hk])
            v_rows = mpfa.v_tiles_to_rows(_h(vq["v_fp8"][b, hk]), cfg.N)
            assert_bytes_equal("v_fp8" + tag, v_rows, ops.vq["v_fp8"][b, hk])
        for h in sorted({0, cfg.G - 1, cfg.Hq - 1}):
            assert_bytes_equal(f"delta_s[b={b} q={h}]", _h(kq["delta_s"][b, h]), ops.kq["delta_s"][b, h])


def _prefill_full(mpfa, oracle_mod, name):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config(name)
    say(f"case: full-size prefill {cfg.name} B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} "
        f"{cfg.dtype} causal smooth (benchmark inputs)")
    t0 = time.time()
    x = synth.device_inputs(cfg, "cuda")
    kq = mpfa.quantize_k(x["k"], q=x["q"])
    vq = mpfa.quantize_v(x["v"])
    rows = synth.sample_rows(cfg)
    idx = [torch.from_numpy(rows[:, i]).cuda() for i in range(3)]
    out, _ = mpfa.prefill(x["q"], kq, vq, cfg.scale, causal=True, out_dtype=torch.bfloat16)
    got_bf16 = _h(out[idx[0], idx[1], idx[2]])
    del out
    out, lse = mpfa.prefill(x["q"], kq, vq, cfg.scale, causal=True, out_dtype=torch.float32,
                            with_lse=True)
    got = _h(out[idx[0], idx[1], idx[2]])
    got_lse = _h(lse[idx[0], idx[1], idx[2]])
    del out, lse
    torch.cuda.synchronize()
    say(f"  gpu calls done ({time.time() - t0:.1f} s); copying inputs to the host")
    qh, kh, vh = _h(x["q"]), _h(x["k"]), _h(x["v"])
    say(f"  oracle statistics and quantization over the whole inputs ({time.time() - t0:.1f} s)")
    ops = oracle_mod.Operands(qh, kh, vh, cfg.scale, smooth=True, identity=False)
    _check_caches(mpfa, ops, kq, vq, cfg)
    del kq, vq, x
    torch.cuda.empty_cache()
    say(f"  oracle attention on {len(rows)} sampled rows ({time.time() - t0:.1f} s)")
    O, LSE, _, AMB = oracle_mod.prefill_rows(qh, kh, vh, cfg.scale, causal=True, smooth=True, rows=rows,
                                             ops=ops, ambiguity=True)
    say(f"  oracle done ({time.time() - t0:.1f} s)")
    assert_close("out bf16", got_bf16, O, rtol=1e-2 + BF16_EXTRA, slack=AMB)
    assert_close("out f32", got, O, slack=AMB)
    assert_close("lse", got_lse, LSE, atol=LSE_ATOL, rtol=0.0)


def test_fullsize_prefill_llama8b_16k(mpfa, oracle_mod):
    _prefill_full(mpfa, oracle_mod, "llama8b_prefill_16k")


def test_fullsize_prefill_qwen14b_32k_spikes(mpfa, oracle_mod):
    _prefill_full(mpfa, oracle_mod, "qwen14b_prefill_32k")


def test_fullsize_prefill_llama8b_128k_lse(mpfa, oracle_mod):
    _prefill_full(mpfa, oracle_mod, "llama8b_prefill_128k_lse")


def test_fullsize_prefill_tile_mean_llama8b_16k(mpfa, oracle_mod):
    """The per-query-tile mean prefill on the 16K benchmark inputs: every tile
    mean and the centred K cache's mean and global scale exactly, sampled
    cache rows byte for byte, output and LSE on the sampled rows."""
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k")
    say(f"case: full-size tile-mean prefill {cfg.name} B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} "
        f"{cfg.dtype} causal (benchmark inputs)")
    t0 = time.time()
    x = synth.device_inputs(cfg, "cuda")
    kq = mpfa.quantize_k(x["k"])
    vq = mpfa.quantize_v(x["v"])
    rows = synth.sample_rows(cfg)
    idx = [torch.from_numpy(rows[:, i]).cuda() for i in range(3)]
    out, _, _ = mpfa.prefill_tile_mean(x["q"], kq, vq, cfg.scale, causal=True, out_dtype=torch.bfloat16)
    got_bf16 = _h(out[idx[0], idx[1], idx[2]])
    del out
    out, lse, tm = mpfa.prefill_tile_mean(x["q"], kq, vq, cfg.scale, causal=True,
                                          out_dtype=torch.float32, with_lse=True)
    got = _h(out[idx[0], idx[1], idx[2]])
    got_lse = _h(lse[idx[0], idx[1], idx[2]])
    got_tm = _h(tm)
    del out, lse, tm
    torch.cuda.synchronize()
    say(f"  gpu calls done ({time.time() - t0:.1f} s); copying inputs to the host")
    qh, kh, vh = _h(x["q"]), _h(x["k"]), _h(x["v"])
    kref = oracle_mod.quantize_k(kh)
    assert_bytes_equal("tile means", got_tm.view(np.uint32), oracle_mod.tile_means(qh).view(np.uint32))
    assert_bytes_equal("k_mean", _h(kq["k_mean"]).view(np.uint32), kref["k_mean"].view(np.uint32))
    assert_bytes_equal("k_gscale", _h(kq["k_gscale"]).view(np.uint32),
                       np.asarray([kref["k_gscale"]], dtype=np.float32).view(np.uint32))
    for hk in sorted({0, cfg.Hkv - 1}):
        assert_bytes_equal(f"k_fp4[kv={hk}]", _h(kq["k_fp4"][0, hk]), kref["k_fp4"][0, hk])
        assert_bytes_equal(f"k_sf[kv={hk}]", _h(kq["k_sf"][0, hk]), kref["k_sf"][0, hk])
    del kq, vq, x
    torch.cuda.empty_cache()
    say(f"  oracle attention on {len(rows)} sampled rows ({time.time() - t0:.1f} s)")
    O, LSE, _, AMB = oracle_mod.prefill_tile_mean_rows(qh, kh, vh, cfg.scale, causal=True, rows=rows,
                                                       ambiguity=True)
    say(f"  oracle done ({time.time() - t0:.1f} s)")
    assert_close("out bf16", got_bf16, O, rtol=1e-2 + BF16_EXTRA, slack=AMB)
    assert_close("out f32", got, O, slack=AMB)
    assert_close("lse", got_lse, LSE, atol=LSE_ATOL, rtol=0.0)


def test_fullsize_decode_llama8b_128k(mpfa, oracle_mod):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_decode_128k")
    say(f"case: full-size decode {cfg.name} B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} "
        f"splits {cfg.num_splits} smooth (benchmark inputs)")
    t0 = time.time()
    x = synth.device_inputs(cfg, "cuda")
    kq = mpfa.quantize_k(x["k"], q_mean=x["q_mean"])
    vq = mpfa.quantize_v(x["v"])
    out, _ = mpfa.decode(x["q"], kq, vq, cfg.scale, cfg.num_splits, out_dtype=torch.bfloat16)
    got_bf16 = _h(out)
    out, lse = mpfa.decode(x["q"], kq, vq, cfg.scale, cfg.num_splits, out_dtype=torch.float32,
                           with_lse=True)
    got, got_lse = _h(out), _h(lse)
    torch.cuda.synchronize()
    say(f"  gpu calls done ({time.time() - t0:.1f} s); copying inputs to the host")
    qh, qmh = _h(x["q"]), _h(x["q_mean"])
    kh, vh = _h(x["k"]), _h(x["v"])
    say(f"  oracle statistics and quantization over the whole inputs ({time.time() - t0:.1f} s)")
    ops = oracle_mod.Operands(qh, kh, vh, cfg.scale, smooth=True, identity=False, q_mean=qmh)
    _check_caches(mpfa, ops, kq, vq, cfg)
    del kq, vq, x
    torch.cuda.empty_cache()
    # every head of the first and last batch entry, plus 32 seeded random pairs
    r = np.random.default_rng(4)
    heads = sorted({(b, h) for b in (0, cfg.B - 1) for h in range(cfg.Hq)}
                   | {(int(r.integers(cfg.B)), int(r.integers(cfg.Hq))) for _ in range(32)})
    say(f"  oracle decode on {len(heads)} (batch, head) pairs ({time.time() - t0:.1f} s)")
    O, LSE = oracle_mod.decode(qh, kh, vh, qmh, cfg.num_splits, cfg.scale, smooth=True, heads=heads,
                               ops=ops)
    say(f"  oracle done ({time.time() - t0:.1f} s)")
    sel = tuple(np.array(heads).T)
    assert_close("out bf16", got_bf16[sel], O, rtol=1e-2 + BF16_EXTRA)
    assert_close("out f32", got[sel], O)
    assert_close("lse", got_lse[sel], LSE, atol=LSE_ATOL, rtol=0.0)
