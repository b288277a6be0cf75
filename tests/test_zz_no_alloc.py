"""GPU test of the allocation-free decode (mpfa_decode_static): called through
the C ABI twice in a row -- the second call smaller, so it runs on the first
call's leftovers in the fixed scratch array -- each output bit-identical to
mpfa_decode's with a caller-owned workspace on the same inputs, and within
the oracle's tolerance of the oracle's decode."""
import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _one(mpfa, oracle_mod, cfg, check_oracle):
    import torch
    from mixed_precision_flashattention_amd import synth
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    qm = synth.q_mean(cfg)
    say(f"case: static-scratch decode B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} "
        f"splits {cfg.num_splits}")
    qd = dev(q, torch.bfloat16)
    kq = mpfa.quantize_k(dev(k, torch.bfloat16), q_mean=dev(qm))
    vq = mpfa.quantize_v(dev(v, torch.bfloat16))
    args = (qd, cfg.Hkv, cfg.N, kq["q_mean"], kq["k_mean"], kq["k_fp4"], kq["k_sf"], kq["k_gscale"],
            vq["v_fp8"], vq["v_scale"], kq["delta_s"], cfg.scale, cfg.num_splits)
    out_s = torch.full((cfg.B, cfg.Hq, 128), float("nan"), dtype=torch.float32, device=qd.device)
    lse_s = torch.full((cfg.B, cfg.Hq), float("nan"), dtype=torch.float32, device=qd.device)
    mpfa.mpfa_decode_static(*args, out_s, lse_s)
    out_w = torch.empty_like(out_s)
    lse_w = torch.empty_like(lse_s)
    ws = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_DECODE, cfg.B, cfg.Hq, cfg.Hkv, cfg.N,
                                               128, cfg.num_splits), dtype=torch.uint8,
                     device=qd.device)
    ws.fill_(0xA5)
    mpfa.mpfa_decode(*args, out_w, lse_w, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w), "static-scratch decode differs from the workspace decode"
    assert torch.equal(lse_s, lse_w)
    if check_oracle:
        O, LSE = oracle_mod.decode(q, k, v, qm, cfg.num_splits, cfg.scale, smooth=True)
        assert_close("out", host(out_s).reshape(-1, 128), O.reshape(-1, 128))
        assert_close("lse", host(lse_s).reshape(-1), LSE.reshape(-1), atol=LSE_ATOL, rtol=0.0)


def test_static_scratch_decode_two_calls_second_smaller(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    big = synth.config("llama8b_decode_128k", B=16, N=4096)  # 16 x 32 heads, 32 splits
    small = synth.config("llama8b_decode_128k", B=2, Hq=8, Hkv=2, N=700, num_splits=3)
    _one(mpfa, oracle_mod, big, check_oracle=False)
    _one(mpfa, oracle_mod, small, check_oracle=True)


def test_static_scratch_decode_rejects_a_workspace_past_its_array(mpfa):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_decode_128k", B=1, N=256)
    q = torch.zeros((64, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    kq = mpfa.quantize_k(torch.zeros((64, 8, 256, 128), dtype=torch.bfloat16, device="cuda"),
                         smooth=False)
    vq = mpfa.quantize_v(torch.zeros((64, 8, 256, 128), dtype=torch.bfloat16, device="cuda"))
    out = torch.empty((64, 32, 128), dtype=torch.float32, device="cuda")
    need = mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_DECODE, 64, 32, 8, 256, 128, 64)
    assert need > mpfa.MPFA_DECODE_STATIC_SCRATCH_BYTES
    with pytest.raises(mpfa.MpfaError) as e:
        mpfa.mpfa_decode_static(q, 8, 256, None, None, kq["k_fp4"], kq["k_sf"], kq["k_gscale"],
                                vq["v_fp8"], vq["v_scale"], None, cfg.scale, 64, out, None)
    assert e.value.status == -3
    torch.cuda.synchronize()
