"""The library's calls captured in a HIP graph: the caller owns every buffer
and the library neither allocates nor synchronizes, so a stage-one pass, a
prefill and a split-KV decode can be recorded once and replayed.  Each
replay must reproduce the eager call's bytes exactly; outputs are cleared
and eager calls run between replays, so a replay that reads stale memory
or depends on state left by an earlier call shows up."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _buffers(mpfa, torch, B, Hq, Hkv, N, P, dev):
    D = 128
    u8, f32 = torch.uint8, torch.float32
    b = {"k_fp4": torch.empty((B, Hkv, N, 64), dtype=u8, device=dev),
         "k_sf": torch.empty((B, Hkv, N, 8), dtype=u8, device=dev),
         "k_gscale": torch.empty(1, dtype=f32, device=dev),
         "k_mean": torch.empty((B, Hkv, D), dtype=f32, device=dev),
         "q_mean": torch.empty((B, Hq, D), dtype=f32, device=dev),
         "delta_s": torch.empty((B, Hq, N), dtype=torch.int16, device=dev),
         "q_amax": torch.empty(1, dtype=torch.float32, device=dev),
         "v_fp8": torch.empty((B, Hkv, (N + 31) // 32, 2, D, 16), dtype=u8, device=dev),
         "v_scale": torch.empty(1, dtype=f32, device=dev),
         "out": torch.empty((B, Hq, N, D), dtype=f32, device=dev),
         "lse": torch.empty((B, Hq, N), dtype=f32, device=dev),
         "dout": torch.empty((B, Hq, D), dtype=f32, device=dev),
         "dlse": torch.empty((B, Hq), dtype=f32, device=dev)}
    ws = lambda op, n_splits=1: torch.empty(  # noqa: E731
        max(mpfa.mpfa_workspace_bytes(op, B, Hq, Hkv, N, D, n_splits), 256), dtype=u8, device=dev)
    b["ws_k"] = ws(mpfa.MPFA_OP_QUANTIZE_K)
    b["ws_v"] = ws(mpfa.MPFA_OP_QUANTIZE_V)
    b["ws_p"] = ws(mpfa.MPFA_OP_PREFILL)
    b["ws_d"] = ws(mpfa.MPFA_OP_DECODE, P)
    return b


def test_graph_replays_equal_eager(mpfa):
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=1, Hq=8, Hkv=2, N=777)
    B, Hq, Hkv, N, P = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, 3
    say(f"case: graph capture of stage one (Q_c amax handed on) + prefill + decode "
        f"B{B} Hq{Hq}/Hkv{Hkv} N{N} {P} splits, bf16 inputs")
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(synth.full(cfg, t)).to(dev).to(torch.bfloat16)
               for t in ("q", "k", "v"))
    qd = q[:, :, -1:, :].contiguous()  # one decode query per head: the last row
    b = _buffers(mpfa, torch, B, Hq, Hkv, N, P, dev)

    def calls():
        mpfa.mpfa_quantize_k_nvfp4_with_q_amax(k, q, b["q_mean"], b["k_mean"], b["k_fp4"],
                                               b["k_sf"], b["k_gscale"], b["delta_s"], b["q_amax"],
                                               b["ws_k"])
        mpfa.mpfa_quantize_v_fp8(v, b["v_fp8"], b["v_scale"], b["ws_v"])
        mpfa.mpfa_prefill_with_q_amax(q, Hkv, b["q_mean"], b["k_mean"], b["k_fp4"], b["k_sf"],
                                      b["k_gscale"], b["v_fp8"], b["v_scale"], b["delta_s"],
                                      b["q_amax"], cfg.scale, True, b["out"], b["lse"], b["ws_p"])
        mpfa.mpfa_decode(qd, Hkv, N, b["q_mean"], b["k_mean"], b["k_fp4"], b["k_sf"],
                         b["k_gscale"], b["v_fp8"], b["v_scale"], b["delta_s"], cfg.scale, P,
                         b["dout"], b["dlse"], b["ws_d"])

    results = ("k_fp4", "k_sf", "k_gscale", "k_mean", "q_mean", "delta_s", "q_amax", "v_fp8",
               "v_scale", "out", "lse", "dout", "dlse")
    calls()
    torch.cuda.synchronize()
    ref = {n: b[n].clone() for n in results}
    assert torch.isfinite(ref["out"]).all() and torch.isfinite(ref["dout"]).all()

    # warm-up on a side stream, then capture (torch's capture stream becomes
    # the current stream, which the binding passes to every call)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for r in range(4):
        for n in results:
            b[n].zero_()
        for n in ("ws_k", "ws_v", "ws_p", "ws_d"):
            b[n].fill_(0xA5)  # workspaces hold garbage between calls
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in results:
            same = torch.equal(b[n], ref[n])
            if not same:
                diff = (b[n].float() - ref[n].float()).abs().max().item()
                say(f"replay {r}: {n} differs from the eager call (max |diff| {diff})")
            assert same, f"replay {r}: {n}"
        say(f"replay {r}: every output identical to the eager call")
        calls()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(b["out"], ref["out"])
