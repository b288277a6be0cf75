#!/usr/bin/env python3
"""Throughput of the QK4PV8 hot path on one MI355X.

One step = the whole path on one batch of the Qwen3-14B-shaped causal
prefill (batch 1, 40 query / 8 KV heads, head_dim 128, 32768 tokens, bf16
inputs with K channel outliers and 0.1% of the entries of Q, K and V scaled
by 20): stage one (channel means, centring, NVFP4 K, Delta_S, FP8 V) followed
by the smoothed QK4PV8 prefill.  `value` is the prefill's algorithmic
attention FLOPs (4 * 128 per visible (query, key) pair) per second of whole
step.

Also reported, each timed on its own with HIP events on the launch stream:
the prefill call alone (the dominant kernel, against the mixed FP4/FP8 MFMA
roofline), the same call with and without the compensation term on one
centred K cache (the compensation overhead), its placement variants, the
prefill with
per-128-row query-tile means (mpfa_prefill_tile_mean), the Llama-3.1-8B-shaped
16K prefill and the 128K two-sequence prefill with LSE, and the split-KV
decode of the Llama-3.1-8B-shaped 128K cache (batch 16, 32 splits) as KV bytes
per second against HBM bandwidth, the same caches as a shuffled pool of
128-token pages (paged decode, full and ragged lengths), and the one-token
cache write.  The error against FP64 exact attention is reported on the small
fp32 case (every row) and on sampled rows of the 16K and 32K workloads, with
and without compensation.  The CPU oracle is timed on a bounded sample of the
32K workload on the host cores.

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
# The NVFP4 score product runs exactly on FP16 MFMA (gfx950's block-scaled FP4
# MFMA takes power-of-two scales per 32 elements, NVFP4 has E4M3 scales per
# 16), P.V on FP8: the peak of that instruction mix, half the FLOPs on each.
PEAK_F16 = 2.5e15
PEAK_F16_FP8 = 1.0 / (0.5 / PEAK_F16 + 0.5 / PEAK_FP8)


# Sources of the kernels one call runs (the call's launch sequence is in
# api.hip, its pre-passes in quant.hip).
KERNEL_SOURCES = {
    "prefill": ["csrc/api.hip", "csrc/prefill.hip", "csrc/quant.hip", "csrc/mpfa_device.hpp",
                "csrc/mpfa_internal.hpp"],
    "decode": ["csrc/api.hip", "csrc/decode.hip", "csrc/quant.hip", "csrc/mpfa_device.hpp",
               "csrc/mpfa_internal.hpp"],
    "quant": ["csrc/quant.hip", "csrc/mpfa_device.hpp", "csrc/mpfa_internal.hpp"],
}


def source_hash(kind):
    """sha256 of the sources a kernel is built from (package-relative paths),
    with comments and whitespace removed, so only a change of code counts."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "mixed_precision_flashattention_amd", rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per call from profiles/traffic.json (rocprofv3 FETCH_SIZE and
    WRITE_SIZE, scaled by the copy-kernel factors), or None when the entry is
    missing or was taken on kernel sources that have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f)["calls"][name]
    except (OSError, KeyError, ValueError):
        return None
    if entry.get("source_sha256") != source_hash(entry["kind"]):
        return None
    return int(entry["bytes_per_call"])


def prefill_flops(B, Hq, N, causal=True):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * 128 * pairs * B * Hq


def decode_bytes(B, Hq, Hkv, N, smooth=True):
    return B * Hkv * N * (64 + 8 + 128) + (B * Hq * N * 2 if smooth else 0)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


WARM_MS = 60.0  # back-to-back work before any timed region


def warm_up(fn, calls, min_ms=WARM_MS, max_calls=200):
    """`calls` untimed calls, then, issued back to back, as many more as fill
    `min_ms` at the rate the first ones ran: after an idle or memory-bound
    stretch the shader clock takes some tens of milliseconds of matrix work
    to settle, and a region timed before that reads slow."""
    import torch
    calls = max(calls, 1)
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    spent = (time.perf_counter() - t0) * 1e3
    if spent < min_ms:
        per_call = max(spent / calls, 1e-3)
        extra = min(max_calls, int(np.ceil((min_ms - spent) / per_call)))
        for _ in range(extra):
            fn()
        torch.cuda.synchronize()
        calls += extra
    return calls


def time_calls(fn, iters, warmup):
    """Average ms per call over `iters` calls, HIP events on the current
    stream, after `warm_up`."""
    import torch
    time_calls.warm_calls = warm_up(fn, warmup)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def median_call_ms(fn, n=20):
    """Median of n single calls, each bracketed by its own HIP events on the
    current stream (after `warm_up`)."""
    import torch
    warm_up(fn, 1)
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(st)
        fn()
        e1.record(st)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def host_env():
    """Shader clock levels as the amdgpu kernel driver lists them (the active one marked),
    the host CPU model and its logical core count."""
    import glob
    import platform
    env = {"cpu_model": platform.processor() or None, "cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    env["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                levels = [ln.strip() for ln in f if ln.strip()]
        except OSError:
            continue
        if levels:
            env["sclk_levels"] = levels
            break
    return env


def valu_ceiling(peaks, achieved):
    """The softmax's vector-ALU ceiling measured by mpfa_peaks (TFLOP/s of
    algorithmic work one softmax wave per SIMD could serve if the matrix
    products were free), as a fraction of the FP4/FP8 roofline, and the
    fraction of it the prefill reaches; None without a peaks run."""
    t = (peaks or {}).get("softmax_valu_tflops")
    if not t:
        return None
    return {"tflops": t, "frac_of_roofline": round(t * 1e12 / PEAK_MIXED, 4),
            "achieved_frac": round(achieved / t, 4),
            "block_ns": peaks.get("softmax_block_ns")}


def schedule_ceiling(peaks, achieved):
    """The ceilings of the prefill's two-group schedule measured by
    mpfa_peaks with its per-block MFMA and softmax instruction mix and random
    operands: "free_operands" with the operands in registers (the floor set
    by the instruction mix and the barriers) and "lds_feed" with the kernel's
    operand traffic (K~, V and the accumulator inputs read from LDS, the next
    blocks brought in by direct loads); TFLOP/s of algorithmic work, cycles
    per body (one 128-key block for all 8 waves), the clock the probe ran
    at, and the fraction of each the prefill reaches; None without a peaks
    run."""
    out = {}
    for key, name in (("pingpong", "free_operands"), ("pingpong_lds", "lds_feed")):
        d = (peaks or {}).get(key)
        if not d:
            return None
        out[name] = {"tflops": d["tflops"], "frac_of_roofline": round(d["tflops"] * 1e12 / PEAK_MIXED, 4),
                     "achieved_frac": round(achieved / d["tflops"], 4),
                     "body_cycles": d.get("body_cycles"), "clock_GHz": d.get("clock_GHz")}
    return out


def measured_peaks():
    """The device's measured ceilings from the standalone probe built beside
    the library (mixed_precision_flashattention_amd/mpfa_peaks): MFMA rates of
    the instructions the kernels use and HBM streaming-read bandwidth.  Run as
    a child process before this process touches the GPU.  None if the probe
    is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "mixed_precision_flashattention_amd", "mpfa_peaks")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except (OSError, subprocess.TimeoutExpired):
        return None
    if r.returncode != 0:
        log(f"[bench] peak probe failed ({r.returncode}): {r.stderr.strip()[-200:]}")
        return None
    try:
        return json.loads(r.stdout.strip().splitlines()[-1])
    except (ValueError, IndexError):
        return None


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
    ops = oracle.Operands(q, k, v, cfg.scale, smooth=True, identity=False)
    kt, vt, delta = ops.k(0, 0), ops.v(0, 0), ops.delta(0, 0)
    t_prep = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done_rows, done_flops, spent = 0, 0.0, 0.0
    batch = max(threads, 16)
    while spent < target_s and done_rows < 16 * cfg.N:
        rows = np.sort(rng.integers(0, cfg.N, batch)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_state(ops.q(0, 0, rows), rows, kt, vt, delta, 0, cfg.N, cfg.scale, True)
        spent += time.perf_counter() - t0
        done_rows += len(rows)
        done_flops += 4.0 * 128 * float((rows + 1).sum())
    sample = (f"{done_rows} random query rows of one (batch, head) of {cfg.name}, oracle block loop "
              f"in FP64 ({spent:.1f} s; operand quantization {t_prep:.1f} s untimed)")
    return done_flops / spent / 1e12, threads, sample


def cpu_plan():
    """The CPU baseline widened (--cpu-plan, a CPU-only run that reports no
    GPU figure): the oracle on every configuration, on the host cores: the
    small prefill and the 128K decode in full; the 16K, 32K and 128K
    prefills on synth.sample_rows with their full-run attention time
    extrapolated by the count of visible (query, key) pairs (labelled as
    such).  Quantizers run on the whole tensors and are timed apart.
    Prints one JSON line."""
    import oracle
    from mixed_precision_flashattention_amd import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    entries = []

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    for name in ("prefill_1k_2x1", "llama8b_prefill_16k", "qwen14b_prefill_32k",
                 "llama8b_prefill_128k_lse"):
        cfg = synth.config(name)
        (q, k, v), t_gen = timed(lambda: tuple(synth.full(cfg, t) for t in ("q", "k", "v")))
        log(f"[cpu-plan] {name}: inputs drawn ({t_gen:.1f} s)")
        ops, t_quant = timed(lambda: oracle.Operands(q, k, v, cfg.scale, smooth=True, identity=False))
        log(f"[cpu-plan] {name}: stage one on the whole tensors {t_quant:.1f} s")
        full_pairs = cfg.B * cfg.Hq * cfg.N * (cfg.N + 1) / 2
        whole = name == "prefill_1k_2x1"
        rows = None if whole else synth.sample_rows(cfg)
        _, t_att = timed(lambda: oracle.prefill_rows(q, k, v, cfg.scale, causal=True, smooth=True,
                                                     rows=rows, ops=ops))
        pairs = full_pairs if whole else float((rows[:, 2] + 1).sum())
        e = {"workload": name, "run": "full" if whole else "sampled rows",
             "rows": int(cfg.B * cfg.Hq * cfg.N) if whole else int(len(rows)),
             "pairs": pairs, "stage_one_s": round(t_quant, 2), "attention_s": round(t_att, 2),
             "attention_TFLOPs": 4.0 * 128 * pairs / t_att / 1e12}
        if not whole:
            e["attention_full_s_extrapolated"] = round(t_att * full_pairs / pairs, 1)
            e["label"] = "extrapolated from the sampled rows by the count of visible pairs"
        log(f"[cpu-plan] {name}: attention {t_att:.1f} s over {pairs:.3g} pairs "
            f"({e['attention_TFLOPs'] * 1e3:.3f} GFLOP/s)")
        entries.append(e)
        del q, k, v, ops

    cfg = synth.config("llama8b_decode_128k")
    (q, k, v), t_gen = timed(lambda: tuple(synth.full(cfg, t) for t in ("q", "k", "v")))
    qm = synth.q_mean(cfg)
    log(f"[cpu-plan] {cfg.name}: inputs drawn ({t_gen:.1f} s)")
    ops, t_quant = timed(lambda: oracle.Operands(q, k, v, cfg.scale, smooth=True, identity=False,
                                                 q_mean=qm))
    log(f"[cpu-plan] {cfg.name}: stage one on the whole tensors {t_quant:.1f} s")
    del k, v
    _, t_att = timed(lambda: oracle.decode(q, None, None, qm, cfg.num_splits, cfg.scale,
                                           smooth=True, ops=ops))
    nbytes = decode_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.N)
    log(f"[cpu-plan] {cfg.name}: decode {t_att:.1f} s")
    entries.append({"workload": cfg.name, "run": "full", "rows": cfg.B * cfg.Hq,
                    "pairs": float(cfg.B * cfg.Hq * cfg.N), "stage_one_s": round(t_quant, 2),
                    "attention_s": round(t_att, 2), "attention_GBps": nbytes / t_att / 1e9,
                    "note": "one query row per call: the oracle's loop over rows runs on one thread"})
    env = host_env()
    print(json.dumps({"cpu_oracle_plan": entries, "threads": threads,
                      "cpu_model": env.get("cpu_model"), "cpu_count": env.get("cpu_count")}),
          flush=True)


def _error_stats(got, ref):
    d = got - ref
    return {"max_abs": float(np.abs(d).max()), "mean_abs": float(np.abs(d).mean()),
            "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)),
            "cos": float((got * ref).sum() / (np.linalg.norm(got) * np.linalg.norm(ref)))}


def _mode_outputs(mpfa, q, k, v, scale):
    """fp32 outputs of the three prefill modes on one set of device inputs:
    smoothing by the sequence means, direct (no smoothing), per-tile means;
    and of the smoothing mode with the other two P.V precision assignments
    (bf16 P and V; NVFP4 P and V)."""
    import torch
    vq = mpfa.quantize_v(v)
    res = {}
    kq = mpfa.quantize_k(k, q=q)
    res["smooth"], _ = mpfa.prefill(q, kq, vq, scale, causal=True, out_dtype=torch.float32)
    res["smooth_pv_bf16"], _ = mpfa.prefill_variant("pv_bf16", q, kq, mpfa.pack_v_bf16(v), scale,
                                                    causal=True, out_dtype=torch.float32)
    res["smooth_pv_nvfp4"], _ = mpfa.prefill_variant("pv_nvfp4", q, kq, mpfa.quantize_v_nvfp4(v),
                                                     scale, causal=True, out_dtype=torch.float32)
    del kq
    kq = mpfa.quantize_k(k, smooth=False)
    res["direct"], _ = mpfa.prefill(q, kq, vq, scale, causal=True, out_dtype=torch.float32)
    del kq
    kq = mpfa.quantize_k(k)
    res["tile_mean"], _, _ = mpfa.prefill_tile_mean(q, kq, vq, scale, causal=True,
                                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    return res


def _exact_rows(q, k, v, scale, rows):
    """Exact causal attention in FP64 on unquantized inputs for chosen query
    rows of one head: softmax over keys 0..i of scale * q_i . k_j, then the
    weighted sum of the V rows.  q [N, D], k / v [N, D]; returns [len(rows), D].
    The accuracy figures measure the quantized path against this."""
    q = np.asarray(q, dtype=np.float64)[rows]
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), k.shape[1]))
    for n, i in enumerate(rows):
        s = scale * (k[:i + 1] @ q[n])
        w = np.exp(s - s.max())
        out[n] = (w @ v[:i + 1]) / w.sum()
    return out


def accuracy_report(mpfa, synth, dev):
    """Error of the GPU output against exact attention (FP64 on the
    unquantized inputs) with smoothing by the sequence means,
    without smoothing, and with per-128-row query-tile means: every row of the
    small fp32 case (1024 tokens, 2/1 heads, 8 outlier channels) and the
    sampled rows of the 16K and 32K workloads (the rows the full-size parity
    tests check), on the benchmark's own device inputs; and the 16K workload
    with ten times stronger key ridges."""
    import torch
    out = {}
    cfg = synth.config("prefill_1k_2x1")
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    every = np.arange(cfg.N)
    ref = np.concatenate([_exact_rows(q[b, h], k[b, h // cfg.G], v[b, h // cfg.G], cfg.scale, every)
                          for b in range(q.shape[0]) for h in range(q.shape[1])])
    res = _mode_outputs(mpfa, *(torch.from_numpy(x).to(dev) for x in (q, k, v)), cfg.scale)
    out[cfg.name] = {"rows": "every row",
                     **{m: _error_stats(o.cpu().numpy().reshape(-1, 128).astype(np.float64), ref)
                        for m, o in res.items()}}
    # the 16K and 32K workloads as specified, and the 16K one with ridges ten
    # times stronger (offsets of sigma 20 on its 5 outlier channels), the
    # regime the method's smoothing is for
    for name, over in (("llama8b_prefill_16k", {}), ("qwen14b_prefill_32k", {}),
                       ("llama8b_prefill_16k", {"koff_sigma": 20.0})):
        cfg = synth.config(name, **over)
        x = synth.device_inputs(cfg, dev)
        res = _mode_outputs(mpfa, x["q"], x["k"], x["v"], cfg.scale)
        rows = synth.sample_rows(cfg)
        refs, gots = [], {m: [] for m in res}
        for b, h in sorted({(int(r[0]), int(r[1])) for r in rows}):
            sel = rows[(rows[:, 0] == b) & (rows[:, 1] == h)][:, 2]
            hk = h // cfg.G
            refs.append(_exact_rows(x["q"][b, h].float().cpu().numpy(),
                                    x["k"][b, hk].float().cpu().numpy(),
                                    x["v"][b, hk].float().cpu().numpy(), cfg.scale, sel))
            idx = torch.from_numpy(sel).to(dev)
            for m, o in res.items():
                gots[m].append(o[b, h].index_select(0, idx).cpu().numpy().astype(np.float64))
        ref = np.concatenate(refs)
        key = name + ("_ridges_sigma20" if over else "")
        out[key] = {"rows": f"{len(ref)} sampled rows (synth.sample_rows)",
                    **{m: _error_stats(np.concatenate(g), ref) for m, g in gots.items()}}
        del x, res
        torch.cuda.empty_cache()
    return out


def measure_prefill(mpfa, synth, dev, name, iters):
    """One workload's prefill call (bf16 output, LSE when the workload asks
    for it) timed with HIP events, against the FP4/FP8 roofline."""
    import torch
    pcfg = synth.config(name)
    px = synth.device_inputs(pcfg, dev)
    pkq = mpfa.quantize_k(px["k"], q=px["q"])
    pvq = mpfa.quantize_v(px["v"])
    del px["k"], px["v"]
    pout = torch.empty(px["q"].shape, dtype=torch.bfloat16, device=dev)
    plse = torch.empty(px["q"].shape[:3], dtype=torch.float32, device=dev) if pcfg.lse else None
    pws = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_PREFILL, pcfg.B, pcfg.Hq, pcfg.Hkv,
                                                pcfg.N), dtype=torch.uint8, device=dev)

    def call():
        mpfa.prefill(px["q"], pkq, pvq, pcfg.scale, causal=True, out=pout, lse=plse,
                     with_lse=pcfg.lse, ws=pws)

    ms = time_calls(call, iters, 1)
    fl = prefill_flops(pcfg.B, pcfg.Hq, pcfg.N)
    ach = fl / (ms * 1e-3) / 1e12
    log(f"[bench] prefill {pcfg.name}: {ms:.3f} ms -> {ach:.1f} TFLOP/s "
        f"({ach * 1e12 / PEAK_MIXED:.3f} of the FP4/FP8 roofline)")
    return {"workload": pcfg.name, "batch": pcfg.B, "q_heads": pcfg.Hq, "kv_heads": pcfg.Hkv,
            "seq_len": pcfg.N, "lse": pcfg.lse, "ms": round(ms, 4), "flops_per_call": fl,
            "roofline": {"bound": "mfma", "achieved": round(ach, 2),
                         "peak": round(PEAK_MIXED / 1e12, 1), "unit": "TFLOP/s",
                         "frac": round(ach * 1e12 / PEAK_MIXED, 4),
                         "traffic": measured_traffic(f"mpfa_prefill {pcfg.name}")},
            "frac_of_fp16_fp8_instruction_peak": round(ach * 1e12 / PEAK_F16_FP8, 4)}


def measure_decode_paged(mpfa, dcfg, dkq, dvq, dq, dout, dws, iters):
    """The decode workload's caches scattered into a shuffled pool of 128-token
    pages: the paged decode at every request's full length (same bytes as the
    contiguous decode) and at ragged lengths (uniform in [N/8, N], seeded)."""
    import torch
    B, Hq, Hkv, N, D = dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.N, 128
    P = mpfa.PAGE_SIZE
    npg = N // P
    g = torch.Generator(device="cpu").manual_seed(7)
    perm = torch.randperm(B * npg, generator=g).to(dq.device)
    pool = {}
    for name, t, shape in (("k_fp4", dkq["k_fp4"], (B, Hkv, npg, P, 64)),
                           ("k_sf", dkq["k_sf"], (B, Hkv, npg, P, 8)),
                           ("v_fp8", dvq["v_fp8"], (B, Hkv, npg, 4, 2, D, 16)),
                           ("delta_s", dkq["delta_s"], (B, Hq, npg, P))):
        x = t.reshape(shape).transpose(1, 2).reshape((B * npg,) + (shape[1],) + shape[3:])
        pool[name] = torch.empty_like(x)
        pool[name][perm] = x
    pool["k_gscale"] = dkq["k_gscale"].reshape(1).repeat(B).contiguous()
    pool["v_scale"] = dvq["v_scale"].reshape(1).repeat(B).contiguous()
    pool["q_mean"], pool["k_mean"] = dkq["q_mean"], dkq["k_mean"]
    table = perm.reshape(B, npg).to(torch.int32).contiguous()
    full = torch.full((B,), N, dtype=torch.int32, device=dq.device)
    ragged_host = torch.randint(N // 8, N + 1, (B,), generator=g, dtype=torch.int32)
    ragged = ragged_host.to(dq.device)

    def call(lens):
        mpfa.decode_paged(dq, pool, table, lens, dcfg.scale, dcfg.num_splits, out=dout, ws=dws)

    ms_full = float(np.median([time_calls(lambda: call(full), iters, 3) for _ in range(3)]))
    ms_rag = float(np.median([time_calls(lambda: call(ragged), iters, 3) for _ in range(3)]))
    per_tok = Hkv * (64 + 8 + 128) + Hq * 2
    by_full = B * N * per_tok
    by_rag = int(ragged_host.sum()) * per_tok
    gbs_full = by_full / (ms_full * 1e-3) / 1e9
    gbs_rag = by_rag / (ms_rag * 1e-3) / 1e9
    log(f"[bench] paged decode {ms_full:.3f} ms -> {gbs_full:.0f} GB/s; ragged lengths "
        f"{ms_rag:.3f} ms -> {gbs_rag:.0f} GB/s")
    del pool, table
    torch.cuda.empty_cache()
    return {"workload": dcfg.name + " in 128-token pages (shuffled)", "ms": round(ms_full, 4),
            "value": round(gbs_full, 1), "unit": "GB/s", "bytes_per_call": by_full,
            "roofline": {"bound": "hbm", "achieved": round(gbs_full, 1), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": round(gbs_full * 1e9 / PEAK_HBM, 4),
                         "traffic": None},
            "ragged": {"lengths": "uniform in [N/8, N], seed 7", "tokens": int(ragged_host.sum()),
                       "ms": round(ms_rag, 4), "GBps": round(gbs_rag, 1)}}


def write_traffic(run_dir, args):
    """profiles/traffic.json from six counter runs of `bench.py --only X`
    (X in prefill, decode, copy; one FETCH_SIZE and one WRITE_SIZE pass each).
    FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by the
    factor that maps the 1 GiB copy's reading to the 1 GiB it moved.  A call's
    bytes are summed over its dispatches (fill, amax pre-pass, main kernel(s)),
    averaged over the three calls."""
    import collections
    import csv

    def load(op, counter):
        path = os.path.join(run_dir, f"pmc_{op}_{counter}", "run_counter_collection.csv")
        vals, names = collections.defaultdict(float), {}
        with open(path) as f:
            for r in csv.DictReader(f):
                i = int(r["Dispatch_Id"])
                vals[i] += float(r["Counter_Value"])
                names[i] = r["Kernel_Name"]
        return vals, names

    def short(name):
        return name.split("(")[0].replace("void ", "").replace("mpfa::", "")

    cf, cn = load("copy", "FETCH_SIZE")
    cw, _ = load("copy", "WRITE_SIZE")
    copies = [i for i, n in cn.items() if "copyBuffer" in n or "copy" in n.lower()][-3:]
    fetch_kib = sum(cf[i] for i in copies) / len(copies)
    write_kib = sum(cw[i] for i in copies) / len(copies)
    moved_kib = (1 << 30) / 1024
    F, W = moved_kib / fetch_kib, moved_kib / write_kib
    out = {"calibration": {"copy_bytes": 1 << 30, "fetch_kib": round(fetch_kib, 1),
                           "write_kib": round(write_kib, 1), "fetch_factor": round(F, 5),
                           "write_factor": round(W, 5)},
           "command": "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv "
                      "-d DIR/pmc_<op>_<counter> -o run -- python bench.py --only <op> "
                      "(op prefill_short: --only prefill --workload llama8b_prefill_16k); "
                      "then python bench.py --write-traffic DIR",
           "calls": {}}
    # dispatches of one call relative to its main kernel: prefill = K
    # expansion and attention (the Q_c amax comes from the first stage);
    # decode = the query amax, split, combine
    # prefill_tile = fill, tile means with the tile-centred Q amax, its fold, K
    # expansion, attention
    calls = [("prefill", "prefill", "k_prefill<1, 0>", (-1, 0),
              f"mpfa_prefill {args.workload}"),
             ("decode", "decode", "k_decode_split<true, false>", (-1, 0, 1),
              f"mpfa_decode {args.decode_workload}")]
    if os.path.isdir(os.path.join(run_dir, "pmc_prefill_short_FETCH_SIZE")):
        calls.append(("prefill_short", "prefill", "k_prefill<1, 0>", (-1, 0),
                      f"mpfa_prefill {args.short_workload}"))
    if os.path.isdir(os.path.join(run_dir, "pmc_prefill_tile_FETCH_SIZE")):
        calls.append(("prefill_tile", "prefill", "k_prefill<2, 0>", (-4, -3, -2, -1, 0),
                      f"mpfa_prefill_tile_mean {args.workload}"))
    for op, kind, main_kernel, offsets, name in calls:
        fv, fn = load(op, "FETCH_SIZE")
        wv, wn = load(op, "WRITE_SIZE")
        parts = {}
        for vals, names, key in ((fv, fn, "fetch_kib"), (wv, wn, "write_kib")):
            mains = sorted(i for i, n in names.items() if main_kernel in n)
            for o in offsets:
                kname = short(names[mains[0] + o])
                avg = sum(vals[i + o] for i in mains) / len(mains)
                parts.setdefault(kname, {})[key] = round(avg, 1)
        for p in parts.values():
            p["bytes"] = int((p["fetch_kib"] * F + p["write_kib"] * W) * 1024)
        out["calls"][name] = {"kind": kind, "source_sha256": source_hash(kind), "kernels": parts,
                              "bytes_per_call": sum(p["bytes"] for p in parts.values())}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def profile_only(args, mpfa, synth, dev):
    """Three calls of one operation for rocprofv3 counter passes: the prefill
    call of the bench workload (smoothed, or with per-tile query means), the
    decode call of the decode workload, or a 1 GiB device-to-device copy (the
    calibration of FETCH_SIZE / WRITE_SIZE)."""
    import torch
    if args.only == "copy":
        a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
    elif args.only == "prefill":
        cfg = synth.config(args.workload)
        x = synth.device_inputs(cfg, dev)
        kq = mpfa.quantize_k(x["k"], q=x["q"])
        vq = mpfa.quantize_v(x["v"])
        out = torch.empty(x["q"].shape, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_PREFILL, cfg.B, cfg.Hq, cfg.Hkv, cfg.N),
                         dtype=torch.uint8, device=dev)
        for _ in range(3):
            mpfa.prefill(x["q"], kq, vq, cfg.scale, causal=True, out=out, ws=ws)
    elif args.only == "prefill_tile":
        cfg = synth.config(args.workload)
        x = synth.device_inputs(cfg, dev)
        kq = mpfa.quantize_k(x["k"])
        vq = mpfa.quantize_v(x["v"])
        out = torch.empty(x["q"].shape, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_PREFILL, cfg.B, cfg.Hq, cfg.Hkv, cfg.N),
                         dtype=torch.uint8, device=dev)
        for _ in range(3):
            mpfa.prefill_tile_mean(x["q"], kq, vq, cfg.scale, causal=True, out=out, ws=ws)
    else:
        cfg = synth.config(args.decode_workload)
        x = synth.device_inputs(cfg, dev)
        kq = mpfa.quantize_k(x["k"], q_mean=x["q_mean"])
        vq = mpfa.quantize_v(x["v"])
        del x["k"], x["v"]
        out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            mpfa.decode(x["q"], kq, vq, cfg.scale, cfg.num_splits, out=out)
    torch.cuda.synchronize()
    log(f"[bench] --only {args.only}: 3 calls done")


# The pages' own figures for this path (NVIDIA B200, MpFA page section 7.2
# "Kernel-level performance" and section 1): context only, another machine.
B200_CONTEXT = {
    "source": "MpFA page, section 7.2 (prefill and decode kernel results) and section 1",
    "prefill_TFLOPS": "1672-1817 (causal, 16K-128K, GQA 32:8)",
    "prefill_speedup_vs_bf16_fa4_geomean": {"gqa_32_8": 1.31, "gqa_40_8": 1.33},
    "decode_TFLOPS_128k": 22.8,
    "decode_speedup_vs_split_kv_bf16_fa4_average": 2.08,
    "compensation_overhead_rank_one": "1.3-2.5% (2.0% geomean, 16K-64K)",
    "compensation_overhead_elementwise": "18.6-22.7% (20.1% geomean)",
}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen14b_prefill_32k")
    ap.add_argument("--decode-workload", default="llama8b_decode_128k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--short-workload", default="llama8b_prefill_16k")
    ap.add_argument("--no-16k", action="store_true")
    ap.add_argument("--lse-workload", default="llama8b_prefill_128k_lse")
    ap.add_argument("--no-128k", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the probe of the measured MFMA and HBM ceilings")
    ap.add_argument("--only", choices=["prefill", "prefill_tile", "decode", "copy"], default=None,
                    help="counter-collection mode: set up, run 3 calls of one operation, exit")
    ap.add_argument("--write-traffic", metavar="DIR", default=None,
                    help="build profiles/traffic.json from the rocprofv3 counter CSVs in DIR "
                         "(pmc_{prefill,decode,copy}_{FETCH_SIZE,WRITE_SIZE}/run_counter_collection.csv)")
    ap.add_argument("--cpu-plan", action="store_true",
                    help="run the CPU oracle on every configuration (full or sampled rows with "
                         "extrapolation) on the host cores, print one JSON line and exit; no GPU")
    args = ap.parse_args()
    if args.cpu_plan:
        cpu_plan()
        return
    if args.write_traffic:
        write_traffic(args.write_traffic, args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    peaks = None
    if not args.only and not args.no_peaks:
        peaks = measured_peaks()  # a child process, before this one touches the GPU
        if peaks:
            log(f"[bench] measured ceilings: MFMA {peaks.get('mfma_tflops')} TFLOP/s, "
                f"softmax VALU {peaks.get('softmax_valu_tflops')} TFLOP/s, "
                f"ping-pong schedule {(peaks.get('pingpong') or {}).get('tflops')} / "
                f"{(peaks.get('pingpong_lds') or {}).get('tflops')} TFLOP/s (free operands / LDS feed), "
                f"read {peaks.get('read_GBps')} GB/s")

    import torch
    import mixed_precision_flashattention_amd as mpfa
    from mixed_precision_flashattention_amd import synth

    mpfa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        profile_only(args, mpfa, synth, dev)
        return
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
          "delta_s": torch.empty((B, Hq, N), dtype=torch.int16, device=dev),
          "q_amax": torch.empty(1, dtype=torch.float32, device=dev)}
    vq = {"v_fp8": torch.empty((B, Hkv, (N + 31) // 32, 2, D, 16), dtype=torch.uint8, device=dev),
          "v_scale": torch.empty(1, dtype=torch.float32, device=dev)}
    out = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=dev)
    ws_k = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_QUANTIZE_K, B, Hq, Hkv, N),
                       dtype=torch.uint8, device=dev)
    ws_v = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_QUANTIZE_V, B, 0, Hkv, N),
                       dtype=torch.uint8, device=dev)
    ws_p = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_PREFILL, B, Hq, Hkv, N),
                       dtype=torch.uint8, device=dev)

    def stage1():
        mpfa.mpfa_quantize_k_nvfp4_with_q_amax(k, q, kq["q_mean"], kq["k_mean"], kq["k_fp4"],
                                               kq["k_sf"], kq["k_gscale"], kq["delta_s"],
                                               kq["q_amax"], ws_k)
        mpfa.mpfa_quantize_v_fp8(v, vq["v_fp8"], vq["v_scale"], ws_v)

    def prefill_call():
        mpfa.mpfa_prefill_with_q_amax(q, Hkv, kq["q_mean"], kq["k_mean"], kq["k_fp4"],
                                      kq["k_sf"], kq["k_gscale"], vq["v_fp8"], vq["v_scale"],
                                      kq["delta_s"], kq["q_amax"], cfg.scale, True, out, None, ws_p)

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
    warm_prefill = time_calls.warm_calls
    ms_prefill_median = median_call_ms(prefill_call)
    ms_stage1 = time_calls(stage1, args.steps, 1)
    achieved = flops / (ms_prefill * 1e-3) / 1e12
    log(f"[bench] prefill call {ms_prefill:.3f} ms -> {achieved:.1f} TFLOP/s "
        f"({achieved * 1e12 / PEAK_MIXED:.4f} of the FP4/FP8 roofline; {args.steps} calls after "
        f"{warm_prefill} untimed); stage one {ms_stage1:.3f} ms")

    # ---- compensation overhead: one centred K cache, the same call with and
    # without the compensation term.  Without Delta_S the centred cache gives
    # Q . K_c = Q_c . K_c + Qbar . K_c, the same scores up to the query
    # quantization, so the softmax does the same work; both calls take their
    # query amax in their own pass.
    def prefill_smooth_own_amax():
        mpfa.mpfa_prefill(q, Hkv, kq["q_mean"], kq["k_mean"], kq["k_fp4"], kq["k_sf"],
                          kq["k_gscale"], vq["v_fp8"], vq["v_scale"], kq["delta_s"], cfg.scale,
                          True, out, None, ws_p)

    def prefill_no_compensation():
        mpfa.mpfa_prefill(q, Hkv, None, None, kq["k_fp4"], kq["k_sf"], kq["k_gscale"],
                          vq["v_fp8"], vq["v_scale"], None, cfg.scale, True, out, None, ws_p)

    ms_pair = {"smooth": [], "no_compensation": []}
    for _ in range(3):  # interleaved, so clock drift hits both alike
        ms_pair["smooth"].append(time_calls(prefill_smooth_own_amax, max(3, args.steps // 2), 1))
        ms_pair["no_compensation"].append(time_calls(prefill_no_compensation,
                                                     max(3, args.steps // 2), 1))
    ms_smooth_own = float(np.median(ms_pair["smooth"]))
    ms_no_comp = float(np.median(ms_pair["no_compensation"]))
    log(f"[bench] same centred cache: with the compensation {ms_smooth_own:.3f} ms, without "
        f"{ms_no_comp:.3f} ms ({ms_smooth_own / ms_no_comp - 1:+.2%})")
    # precision / placement variants (MpFA page section 3.1 Fig. 3(a), 7.4,
    # 5.1) on the same caches, each taking its query amax in its own pass like
    # the smoothing call they are compared with
    var_vq = {"pv_bf16": mpfa.pack_v_bf16(v), "pv_nvfp4": mpfa.quantize_v_nvfp4(v)}
    ws_p4 = torch.empty(mpfa.mpfa_workspace_bytes(mpfa.MPFA_OP_PREFILL_PV_NVFP4, B, Hq, Hkv, N),
                        dtype=torch.uint8, device=dev)
    ms_var = {}
    for name in ("rank_one", "elementwise", "poly_exp2", "pv_bf16", "pv_nvfp4"):
        def var_call(name=name):
            mpfa.prefill_variant(name, q, kq, var_vq.get(name, vq), cfg.scale, causal=True,
                                 out=out, ws=ws_p4 if name == "pv_nvfp4" else ws_p)
        ms_var[name] = time_calls(var_call, max(3, args.steps // 2), 1)
        log(f"[bench] variant {name}: {ms_var[name]:.3f} ms ({ms_var[name] / ms_smooth_own - 1:+.2%} "
            f"against the smoothing call)")
    del var_vq, ws_p4
    torch.cuda.empty_cache()

    # the unsmoothed (direct) prefill on its own uncentred cache
    kq_direct = mpfa.quantize_k(k, smooth=False)

    def prefill_direct():
        mpfa.mpfa_prefill(q, Hkv, None, None, kq_direct["k_fp4"], kq_direct["k_sf"],
                          kq_direct["k_gscale"], vq["v_fp8"], vq["v_scale"], None, cfg.scale, True,
                          out, None, ws_p)

    ms_direct = time_calls(prefill_direct, args.steps, 2)
    log(f"[bench] direct prefill (uncentred cache) {ms_direct:.3f} ms")
    del kq_direct

    # per-query-tile mean mode: a centred K cache (no Delta_S), the tile means
    # and the attention in one call
    kq_tile = mpfa.quantize_k(k)
    tmean = torch.empty((B, Hq, (N + 127) // 128, D), dtype=torch.float32, device=dev)

    def prefill_tile():
        mpfa.mpfa_prefill_tile_mean(q, Hkv, kq_tile["k_mean"], kq_tile["k_fp4"], kq_tile["k_sf"],
                                    kq_tile["k_gscale"], vq["v_fp8"], vq["v_scale"], cfg.scale, True,
                                    out, None, tmean, ws_p)

    ms_tile = time_calls(prefill_tile, args.steps, 2)
    ach_tile = flops / (ms_tile * 1e-3) / 1e12
    log(f"[bench] tile-mean prefill {ms_tile:.3f} ms -> {ach_tile:.1f} TFLOP/s "
        f"({ach_tile * 1e12 / PEAK_MIXED:.4f} of the FP4/FP8 roofline)")
    del kq_tile, tmean

    result = {
        "metric": "attention TFLOPS (prefill) and KV GB/s (decode) vs MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "nvfp4-qk/fp8-pv/fp32-softmax",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_len": N,
                   "head_dim": D, "causal": True, "smoothing": True, "input_dtype": cfg.dtype,
                   "spikes": "0.1% of Q, K, V entries x20", "output_dtype": "bf16",
                   "step": "stage one (means, NVFP4 K, Delta_S, FP8 V) + prefill"},
        "roofline": {"bound": "mfma",
                     "kernel": "mpfa_prefill_with_q_amax (k_expand_k + k_prefill<1, 0>)",
                     "achieved": round(achieved, 2), "peak": round(PEAK_MIXED / 1e12, 1),
                     "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_MIXED, 4),
                     "traffic": measured_traffic(f"mpfa_prefill {cfg.name}"),
                     "flops_per_launch": flops, "ms_per_launch": round(ms_prefill, 4),
                     "frac_of_fp16_fp8_instruction_peak": round(achieved * 1e12 / PEAK_F16_FP8, 4),
                     # the secondary ceiling: one softmax wave per SIMD running
                     # the kernel's per-block softmax mix with free matrix work
                     # (measured by mpfa_peaks on this device)
                     "valu_softmax_ceiling": valu_ceiling(peaks, achieved),
                     # the ceilings of the kernel's schedule and instruction
                     # mix with free operands and with its LDS operand
                     # traffic (mpfa_peaks)
                     "schedule_ceiling": schedule_ceiling(peaks, achieved)},
        "prefill_ms": round(ms_prefill, 4), "prefill_median_ms": round(ms_prefill_median, 4),
        "stage_one_ms": round(ms_stage1, 4),
        "compensation": {
            "cache": "one centred K cache; the call with Delta_S (the score accumulator's "
                     "input) and without it; "
                     "both take the query amax in their own pass",
            "with_ms": round(ms_smooth_own, 4), "without_ms": round(ms_no_comp, 4),
            "overhead": round(ms_smooth_own / ms_no_comp - 1.0, 4),
            "samples_ms": {k_: [round(t, 4) for t in v_] for k_, v_ in ms_pair.items()}},
        "variants": {
            "reference": "the smoothing call with its own query-amax pass "
                         "(compensation.with_ms); same caches",
            **{name: {"ms": round(t, 4), "vs_smoothing": round(t / ms_smooth_own - 1.0, 4)}
               for name, t in ms_var.items()},
            "what": {"rank_one": "Delta_S written into the score accumulator by its own "
                                 "rank-one bf16 MFMA step per tile (MpFA 5.2 MMA placement)",
                     "elementwise": "Delta_S added per score on the VALU (MpFA 7.4 placement)",
                     "poly_exp2": "one exp2 in four by a fitted cubic (MpFA 5.1 split)",
                     "pv_bf16": "P and V in bf16, P.V on bf16 MFMA (MpFA 3.1 NVFP4+BF16)",
                     "pv_nvfp4": "P quantized to NVFP4 per 16 keys on the softmax path, V from "
                                 "an NVFP4 cache (16-key blocks) expanded per call, P.V on f16 "
                                 "MFMA over the exact values (MpFA 3.1 NVFP4+NVFP4)"}},
        "prefill_direct_ms": round(ms_direct, 4),
        "prefill_tile_mean": {"ms": round(ms_tile, 4),
                              "roofline": {"bound": "mfma", "achieved": round(ach_tile, 2),
                                           "peak": round(PEAK_MIXED / 1e12, 1), "unit": "TFLOP/s",
                                           "frac": round(ach_tile * 1e12 / PEAK_MIXED, 4),
                                           "traffic": measured_traffic(
                                               f"mpfa_prefill_tile_mean {cfg.name}")}},
        "b200_context": B200_CONTEXT,
        "env": {"gpu": torch.cuda.get_device_name(0),
                "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
                "hip": torch.version.hip, "torch": torch.__version__, **host_env()},
        # measured on this device by the peak probe (context for the published
        # peaks the roofline fractions use)
        "measured_peaks": peaks,
    }
    del q, k, v, x, kq, vq, out
    torch.cuda.empty_cache()

    # ---- the other prefill workloads: 16K Llama-shaped, and the 128K
    # two-sequence prefill that also writes the LSE ------------------------
    if not args.no_16k:
        result["prefill_16k"] = measure_prefill(mpfa, synth, dev, args.short_workload,
                                                max(3, args.steps))
        torch.cuda.empty_cache()
    if not args.no_128k:
        result["prefill_128k_lse"] = measure_prefill(mpfa, synth, dev, args.lse_workload, 2)
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

        # smoothing and direct calls interleaved over three rounds of 20 calls
        # each (the median round is reported), so that both see the same
        # state of the device
        dec_rounds = {"smooth": [], "direct": []}
        for _ in range(3):
            dec_rounds["smooth"].append(time_calls(decode_call, 20, 3))
            dec_rounds["direct"].append(time_calls(lambda: decode_call(False), 20, 3))
        ms_dec = float(np.median(dec_rounds["smooth"]))
        ms_dec_direct = float(np.median(dec_rounds["direct"]))
        ms_dec_median = median_call_ms(decode_call)
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
                         "unit": "GB/s", "frac": round(gbs * 1e9 / PEAK_HBM, 4),
                         "traffic": measured_traffic("mpfa_decode llama8b_decode_128k")},
            "median_ms": round(ms_dec_median, 4),
            "rounds_ms": {k: [round(x, 4) for x in v] for k, v in dec_rounds.items()},
            "direct_ms": round(ms_dec_direct, 4), "direct_GBps": round(gbs_d, 1),
            # attention FLOPs (4 * 128 per (query head, key)), for context only
            "flops_per_call": 4.0 * D * dcfg.N * dcfg.B * dcfg.Hq,
            "TFLOPs": round(4.0 * D * dcfg.N * dcfg.B * dcfg.Hq / (ms_dec * 1e-3) / 1e12, 2)}
        # decode-time cache write of one new token per request (centring against
        # the frozen means, NVFP4 K / FP8 V with the frozen scales, Delta_S)
        kn = torch.randn((dcfg.B, dcfg.Hkv, 1, D), device=dev).to(torch.bfloat16)
        vn = torch.randn((dcfg.B, dcfg.Hkv, 1, D), device=dev).to(torch.bfloat16)
        pos = torch.full((dcfg.B,), dcfg.N - 1, dtype=torch.int32, device=dev)
        ms_app = time_calls(lambda: mpfa.append_kv(kn, vn, pos, dkq, dvq), max(args.steps, 10), 3)
        log(f"[bench] append of one token per request: {ms_app * 1e3:.1f} us")
        result["decode"]["append_one_token_us"] = round(ms_app * 1e3, 2)
        result["decode_paged"] = measure_decode_paged(mpfa, dcfg, dkq, dvq, dq, dout, dws,
                                                      max(args.steps, 10))
        del dkq, dvq, dq, dout, dws, dx, kn, vn, pos
        torch.cuda.empty_cache()

    if not args.no_accuracy:
        result["accuracy_vs_fp64_exact"] = accuracy_report(mpfa, synth, dev)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        tf, threads, sample = cpu_baseline(cfg, args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads,
                                  "kind": "oracle", "sample": sample}
        log(f"[bench] cpu oracle {tf * 1e3:.3f} GFLOP/s on {threads} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
