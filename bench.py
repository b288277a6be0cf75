#!/usr/bin/env python3
"""Throughput of the QK4PV8 hot path on one MI355X.

One step = the whole path on one batch of the Llama-3.1-8B-shaped causal
prefill (batch 1, 32 query / 8 KV heads, head_dim 128, 16384 tokens, bf16
inputs with K channel outliers): stage one (channel means, centring, NVFP4
K, Delta_S, FP8 V) followed by the smoothed QK4PV8 prefill.  `value` is the
prefill's algorithmic attention FLOPs (4 * 128 per visible (query, key)
pair) per second of whole step.

Also reported, each timed on its own with HIP events on the launch stream:
the prefill call alone (the dominant kernel, against the mixed FP4/FP8 MFMA
roofline), the direct (unsmoothed) prefill, and the split-KV decode of the
Llama-3.1-8B-shaped 128K cache (batch 16, 32 splits) as KV bytes per second
against HBM bandwidth.  The CPU oracle is timed on a bounded sample of the
prefill workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks
PEAK_FP4 = 10.1e15
PEAK_FP8 = 5.0e15
PEAK_MIXED = 1.0 / (0.5 / PEAK_FP4 + 0.5 / PEAK_FP8)  # half the FLOPs in each contraction
PEAK_HBM = 8.0e12


def prefill_flops(B, Hq, N, causal=True):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * 128 * pairs * B * Hq


def decode_bytes(B, Hq, Hkv, N, smooth=True):
    return B * Hkv * N * (64 + 8 + 128) + (B * Hq * N * 2 if smooth else 0)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_calls(fn, iters, warmup):
    """Average ms per call over `iters` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def cpu_baseline(cfg, target_s=12.0):
    """The oracle's blocked attention on sampled rows of one (batch, query
    head) of the workload, operands quantized and dequantized by the oracle
    beforehand (outside the timing).  Returns (TFLOP/s, threads, sample)."""
    import oracle
    from mixed_precision_flashattention_amd import synth
    q = synth.head(cfg, "q", 0, 0)[None, None]
    k = synth.head(cfg, "k", 0, 0)[None, None]
    v = synth.head(cfg, "v", 0, 0)[None, None]
    t0 = time.perf_counter()
    prep = oracle.pipeline._prepare(q, k, v, cfg.scale, smooth=True, identity=False)
    t_prep = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done_rows, done_flops, spent = 0, 0.0, 0.0
    batch = max(threads, 16)
    while spent < target_s and done_rows < cfg.N:
        rows = np.sort(rng.integers(0, cfg.N, batch)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_state(prep["qt"][0, 0][rows], rows, prep["kt"][0, 0], prep["vt"][0, 0],
                          prep["delta"][0, 0], 0, cfg.N, cfg.scale, True)
        spent += time.perf_counter() - t0
        done_rows += len(rows)
        done_flops += 4.0 * 128 * float((rows + 1).sum())
    sample = (f"{done_rows} random query rows of one (batch, head) of {cfg.name}, oracle block loop "
              f"in FP64 ({spent:.1f} s; operand quantization {t_prep:.1f} s untimed)")
    return done_flops / spent / 1e12, threads, sample


def accuracy_report(mpfa):
    """Error of the GPU output against FP32 exact attention (the oracle's FP64
    reference on the unquantized inputs), with and without smoothing, on the
    small fp32 configuration (1024 tokens, 2/1 heads, 8 outlier channels)."""
    import oracle
    import torch
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("prefill_1k_2x1")
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    ref, _ = oracle.exact_attention(q, k, v, cfg.scale, causal=True)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = {}
    vq = mpfa.quantize_v(vd)
    for smooth in (True, False):
        kq = mpfa.quantize_k(kd, q=qd) if smooth else mpfa.quantize_k(kd, smooth=False)
        o, _ = mpfa.prefill(qd, kq, vq, cfg.scale, causal=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        g = o.cpu().numpy().reshape(-1, 128).astype(np.float64)
        d = g - ref
        out["smooth" if smooth else "direct"] = {
            "max_abs": float(np.abs(d).max()), "mean_abs": float(np.abs(d).mean()),
            "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)),
            "cos": float((g * ref).sum() / (np.linalg.norm(g) * np.linalg.norm(ref)))}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_prefill_16k")
    ap.add_argument("--decode-workload", default="llama8b_decode_128k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixed_precision_flashattention_amd as mpfa
    from mixed_precision_flashattention_amd import synth

    mpfa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config(args.workload)
    B, Hq, Hkv, N, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.D
    log(f"[bench] {torch.cuda.get_device_name(0)} hip {torch.version.hip}; workload {cfg.name}")
    x = synth.device_inputs(cfg, dev)
    q, k, v = x["q"], x["k"], x["v"]

    # preallocated caches, outputs and workspaces: nothing is allocated in the loop
    kq = {"k_fp4": torch.empty((B, Hkv, N, 64), dtype=torch.uint8, device=dev),
          "k_sf": torch.empty((B, Hkv, N, 8), dtype=torch.uint8, device=dev),
          "k_gscale": torch.empty(1, dtype=torch.float32, device=dev),
          "k_mean": torch.empty((B, Hkv, D), dtype=torch.float32, device=dev),
          "q_mean": torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
          "delta_s": torch.empty((B, Hq, N), dtype=torch.int16, device=dev)}
    vq = {"v_fp8": torch.empty((B, Hkv, (N + 31) // 32, D, 32), dtype=torch.uint8, device=dev),
          "v_scale": torch.empty(1, dtype=torch.float32, device=dev)}
    out = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=dev)
    ws_k = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_QUANTIZE_K, B, Hq, Hkv, N),
                       dtype=torch.uint8, device=dev)
    ws_v = torch.empty(256, dtype=torch.uint8, device=dev)
    ws_p = torch.empty(256, dtype=torch.uint8, device=dev)

    def stage1():
        mpfa.mpfa_quantize_k_nvfp4(k, q, kq["q_mean"], kq["k_mean"], kq["k_fp4"], kq["k_sf"],
                                   kq["k_gscale"], kq["delta_s"], ws_k)
        mpfa.mpfa_quantize_v_fp8(v, vq["v_fp8"], vq["v_scale"], ws_v)

    def prefill_call():
        mpfa.mpfa_prefill(q, Hkv, kq["q_mean"], kq["k_mean"], kq["k_fp4"], kq["k_sf"],
                          kq["k_gscale"], vq["v_fp8"], vq["v_scale"], kq["delta_s"], cfg.scale,
                          True, out, None, ws_p)

    def step():
        stage1()
        prefill_call()

    # ---- timed steps (contract: W warmup, then exactly K steps) ----------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    flops = prefill_flops(B, Hq, N)
    value = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms -> {value:.1f} TFLOP/s (whole path)")

    # ---- the dominant kernel, alone --------------------------------------
    stage1()
    ms_prefill = time_calls(prefill_call, args.steps, 2)
    ms_stage1 = time_calls(stage1, args.steps, 1)
    achieved = flops / (ms_prefill * 1e-3) / 1e12
    log(f"[bench] prefill call {ms_prefill:.3f} ms -> {achieved:.1f} TFLOP/s; stage one {ms_stage1:.3f} ms")
    kq_direct = mpfa.quantize_k(k, smooth=False)

    def prefill_direct():
        mpfa.mpfa_prefill(q, Hkv, None, None, kq_direct["k_fp4"], kq_direct["k_sf"],
                          kq_direct["k_gscale"], vq["v_fp8"], vq["v_scale"], None, cfg.scale, True,
                          out, None, ws_p)

    ms_direct = time_calls(prefill_direct, args.steps, 2)
    log(f"[bench] direct prefill {ms_direct:.3f} ms")
    del kq_direct

    result = {
        "metric": "attention TFLOPS (prefill) and KV GB/s (decode) vs MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "nvfp4-qk/fp8-pv/fp32-softmax",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_len": N,
                   "head_dim": D, "causal": True, "smoothing": True, "input_dtype": cfg.dtype,
                   "output_dtype": "bf16",
                   "step": "stage one (means, NVFP4 K, Delta_S, FP8 V) + prefill"},
        "roofline": {"bound": "mfma", "kernel": "mpfa_prefill (Q amax pre-pass + k_prefill)",
                     "achieved": round(achieved, 2), "peak": round(PEAK_MIXED / 1e12, 1),
                     "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_MIXED, 4),
                     "traffic": None,
                     "flops_per_launch": flops, "ms_per_launch": round(ms_prefill, 4)},
        "prefill_ms": round(ms_prefill, 4), "prefill_direct_ms": round(ms_direct, 4),
        "stage_one_ms": round(ms_stage1, 4),
        "compensation_overhead": round(ms_prefill / ms_direct - 1.0, 4),
    }
    del q, k, v, x, kq, vq, out
    torch.cuda.empty_cache()

    # ---- decode -----------------------------------------------------------
    if not args.no_decode:
        dcfg = synth.config(args.decode_workload)
        dx = synth.device_inputs(dcfg, dev)
        dkq = mpfa.quantize_k(dx["k"], q_mean=dx["q_mean"])
        dvq = mpfa.quantize_v(dx["v"])
        del dx["k"], dx["v"]
        torch.cuda.empty_cache()
        dq = dx["q"]
        dout = torch.empty((dcfg.B, dcfg.Hq, D), dtype=torch.bfloat16, device=dev)
        dws = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_DECODE, dcfg.B, dcfg.Hq, dcfg.Hkv,
                                                    dcfg.N, D, dcfg.num_splits),
                          dtype=torch.uint8, device=dev)

        def decode_call(smooth=True):
            mpfa.mpfa_decode(dq, dcfg.Hkv, dcfg.N, dkq["q_mean"] if smooth else None,
                             dkq["k_mean"] if smooth else None, dkq["k_fp4"], dkq["k_sf"],
                             dkq["k_gscale"], dvq["v_fp8"], dvq["v_scale"],
                             dkq["delta_s"] if smooth else None, dcfg.scale, dcfg.num_splits,
                             dout, None, dws)

        ms_dec = time_calls(decode_call, max(args.steps, 10), 3)
        ms_dec_direct = time_calls(lambda: decode_call(False), max(args.steps, 10), 3)
        nbytes = decode_bytes(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.N)
        gbs = nbytes / (ms_dec * 1e-3) / 1e9
        nbytes_d = decode_bytes(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.N, smooth=False)
        gbs_d = nbytes_d / (ms_dec_direct * 1e-3) / 1e9
        log(f"[bench] decode {ms_dec:.3f} ms -> {gbs:.0f} GB/s; direct {ms_dec_direct:.3f} ms -> {gbs_d:.0f} GB/s")
        result["decode"] = {
            "workload": dcfg.name, "batch": dcfg.B, "q_heads": dcfg.Hq, "kv_heads": dcfg.Hkv,
            "kv_len": dcfg.N, "num_splits": dcfg.num_splits, "ms": round(ms_dec, 4),
            "value": round(gbs, 1), "unit": "GB/s", "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": round(gbs * 1e9 / PEAK_HBM, 4), "traffic": None},
            "direct_ms": round(ms_dec_direct, 4), "direct_GBps": round(gbs_d, 1)}
        del dkq, dvq, dq, dout, dws, dx
        torch.cuda.empty_cache()

    if not args.no_accuracy:
        result["accuracy_vs_fp64_exact"] = accuracy_report(mpfa)

    if not args.no_cpu_baseline:
        tf, threads, sample = cpu_baseline(cfg, args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads,
                                  "kind": "oracle", "sample": sample}
        log(f"[bench] cpu oracle {tf * 1e3:.3f} GFLOP/s on {threads} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
