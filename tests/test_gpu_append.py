"""GPU parity of the decode-time cache write (mpfa_append_kv) against the
oracle: caches byte for byte, then a decode over the appended caches within
the attention tolerance."""
import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_bytes_equal, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _empty_like(kq, vq):
    import torch
    ek = {n: (torch.zeros_like(t) if n in ("k_fp4", "k_sf", "delta_s") else t.clone())
          for n, t in kq.items()}
    ev = {"v_fp8": torch.zeros_like(vq["v_fp8"]), "v_scale": vq["v_scale"].clone()}
    return ek, ev


@pytest.mark.parametrize("smooth", [True, False])
def test_chunked_append_reproduces_bulk_caches(mpfa, oracle_mod, smooth):
    """Chunks of 20 tokens at different positions per batch entry (entry 0
    forward, entry 1 backward), with the statistics the bulk pass froze."""
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=2, Hq=8, Hkv=2, N=310)
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    say(f"case: append chunks B2 Hq8/Hkv2 N310 bf16 smooth={smooth}")
    kd, vd = dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    kq = mpfa.quantize_k(kd, q=dev(q, torch.bfloat16)) if smooth else mpfa.quantize_k(kd, smooth=False)
    vq = mpfa.quantize_v(vd)
    ek, ev = _empty_like(kq, vq)
    T = 20
    starts = list(range(0, cfg.N, T))
    for i in range(len(starts)):
        pos = [starts[i], starts[len(starts) - 1 - i]]
        tt = [min(T, cfg.N - p) for p in pos]
        if tt[0] != tt[1]:  # the ragged last chunk: write it per entry
            for b in range(2):
                kn = kd[b:b + 1, :, pos[b]:pos[b] + tt[b]].contiguous()
                vn = vd[b:b + 1, :, pos[b]:pos[b] + tt[b]].contiguous()
                sub_k = {n: t[b:b + 1] for n, t in ek.items() if n not in ("k_gscale",)}
                sub_k["k_gscale"] = ek["k_gscale"]
                sub_v = {"v_fp8": ev["v_fp8"][b:b + 1], "v_scale": ev["v_scale"]}
                mpfa.append_kv(kn, vn, torch.zeros(1, dtype=torch.int32, device="cuda") + pos[b],
                               sub_k, sub_v)
            continue
        kn = torch.stack([kd[b, :, pos[b]:pos[b] + T] for b in range(2)]).contiguous()
        vn = torch.stack([vd[b, :, pos[b]:pos[b] + T] for b in range(2)]).contiguous()
        mpfa.append_kv(kn, vn, torch.tensor(pos, dtype=torch.int32, device="cuda"), ek, ev)
    torch.cuda.synchronize()
    for n in ("k_fp4", "k_sf") + (("delta_s",) if smooth else ()):
        assert_bytes_equal(n + " vs bulk", host(ek[n]), host(kq[n]))
    assert_bytes_equal("v_fp8 vs bulk", host(ev["v_fp8"]), host(vq["v_fp8"]))
    # and against the oracle's bulk first stage
    okq = oracle_mod.quantize_k(k, q=q) if smooth else oracle_mod.quantize_k(k, smooth=False)
    assert_bytes_equal("k_fp4 vs oracle", host(ek["k_fp4"]), okq["k_fp4"])
    assert_bytes_equal("v_fp8 vs oracle", mpfa.v_tiles_to_rows(host(ev["v_fp8"]), cfg.N),
                       oracle_mod.quantize_v(v)["v_fp8"])


def test_decode_append_then_decode(mpfa, oracle_mod):
    """One new token per request at different lengths, written into a prefix
    cache with frozen statistics; the caches match the oracle's append byte
    for byte and a decode over them matches the oracle's decode of the same
    caches."""
    import torch
    from mixed_precision_flashattention_amd import synth
    B, Hq, Hkv, N0, Ncap = 3, 8, 2, 200, 260
    cfg = synth.config("llama8b_decode_128k", B=B, Hq=Hq, Hkv=Hkv, N=N0, num_splits=3)
    k, v = synth.full(cfg, "k"), synth.full(cfg, "v")
    qm = synth.q_mean(cfg)
    r = np.random.default_rng(11)
    kn = r.standard_normal((B, Hkv, 1, 128)).astype(np.float32) * 1.5
    vn = r.standard_normal((B, Hkv, 1, 128)).astype(np.float32)
    kn = host(dev(kn, torch.bfloat16))  # bf16 values, as the cache inputs
    vn = host(dev(vn, torch.bfloat16))
    pos = np.array([200, 203, 250], dtype=np.int32)
    say("case: decode append B3 Hq8/Hkv2 prefix 200, capacity 260, positions 200/203/250")
    # GPU: prefix caches padded to the capacity, then the append
    kq = mpfa.quantize_k(dev(k, torch.bfloat16), q_mean=dev(qm))
    vq = mpfa.quantize_v(dev(v, torch.bfloat16))
    ck = {"k_fp4": torch.zeros((B, Hkv, Ncap, 64), dtype=torch.uint8, device="cuda"),
          "k_sf": torch.zeros((B, Hkv, Ncap, 8), dtype=torch.uint8, device="cuda"),
          "delta_s": torch.zeros((B, Hq, Ncap), dtype=torch.int16, device="cuda"),
          "k_gscale": kq["k_gscale"], "k_mean": kq["k_mean"], "q_mean": kq["q_mean"]}
    ck["k_fp4"][:, :, :N0] = kq["k_fp4"]
    ck["k_sf"][:, :, :N0] = kq["k_sf"]
    ck["delta_s"][:, :, :N0] = kq["delta_s"]
    nt0 = (N0 + 31) // 32
    cv = {"v_fp8": torch.zeros((B, Hkv, (Ncap + 31) // 32, 2, 128, 16), dtype=torch.uint8, device="cuda"),
          "v_scale": vq["v_scale"]}
    cv["v_fp8"][:, :, :nt0] = vq["v_fp8"]
    mpfa.append_kv(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16),
                   torch.from_numpy(pos).cuda(), ck, cv)
    torch.cuda.synchronize()
    # oracle: the same prefix caches (row layout) and the same append
    okq = oracle_mod.quantize_k(k, q_mean=qm)
    ovq = oracle_mod.quantize_v(v)
    cache = {"k_fp4": np.zeros((B, Hkv, Ncap, 64), np.uint8), "k_sf": np.zeros((B, Hkv, Ncap, 8), np.uint8),
             "delta_s": np.zeros((B, Hq, Ncap), np.uint16), "v_fp8": np.zeros((B, Hkv, Ncap, 128), np.uint8),
             "k_gscale": okq["k_gscale"], "v_scale": ovq["v_scale"]}
    cache["k_fp4"][:, :, :N0] = okq["k_fp4"]
    cache["k_sf"][:, :, :N0] = okq["k_sf"]
    cache["delta_s"][:, :, :N0] = okq["delta_s"]
    cache["v_fp8"][:, :, :N0] = ovq["v_fp8"]
    cache = oracle_mod.append_kv(kn, vn, pos, cache, q_mean=qm, k_mean=okq["k_mean"])
    for n in ("k_fp4", "k_sf", "delta_s"):
        assert_bytes_equal(n, host(ck[n]), cache[n])
    assert_bytes_equal("v_fp8", mpfa.v_tiles_to_rows(host(cv["v_fp8"]), Ncap), cache["v_fp8"])
    # decode over all Ncap positions (rows never written hold zero codes)
    q = synth.full(cfg, "q")
    out, lse = mpfa.decode(dev(q, torch.bfloat16), ck, cv, cfg.scale, 3, out_dtype=torch.float32,
                           with_lse=True)
    torch.cuda.synchronize()
    ops = oracle_mod.Operands.from_cache(q, cache, Ncap, q_mean=qm, k_mean=okq["k_mean"])
    O, LSE = oracle_mod.decode(q, None, None, qm, 3, cfg.scale, smooth=True, ops=ops)
    assert_close("out", host(out).reshape(-1, 128), O.reshape(-1, 128))
    assert_close("lse", host(lse).reshape(-1), LSE.reshape(-1), atol=LSE_ATOL, rtol=0.0)


def test_append_out_of_range_position_writes_nothing(mpfa):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=2, Hq=4, Hkv=2, N=64)
    k, v = synth.full(cfg, "k"), synth.full(cfg, "v")
    say("case: append with positions out of range (-1 and N_cap)")
    kq = mpfa.quantize_k(dev(k, torch.bfloat16), smooth=False)
    vq = mpfa.quantize_v(dev(v, torch.bfloat16))
    before = (host(kq["k_fp4"]).copy(), host(kq["k_sf"]).copy(), host(vq["v_fp8"]).copy())
    kn = torch.ones((2, 2, 1, 128), dtype=torch.bfloat16, device="cuda")
    mpfa.append_kv(kn, kn, torch.tensor([-1, 64], dtype=torch.int32, device="cuda"), kq, vq)
    torch.cuda.synchronize()
    assert_bytes_equal("k_fp4", host(kq["k_fp4"]), before[0])
    assert_bytes_equal("k_sf", host(kq["k_sf"]), before[1])
    assert_bytes_equal("v_fp8", host(vq["v_fp8"]), before[2])
