"""Seeded synthetic inputs shaped like the attention heads the MpFA paper measures
("MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on Blackwell
GPUs", §7.1: Llama-3.1-8B GQA 32:8 and Qwen3-14B GQA 40:8, head_dim 128).

This module only draws random numbers: it holds none of the method's
arithmetic, so both the GPU path and the CPU oracle can take their inputs
from it.  Every (tensor, batch, head) slice comes from its own PCG64 stream,
so any slice can be regenerated on its own (the large configurations are
checked on sampled heads and rows).

Distributions: Q, K, V ~ N(0, 1) in fp32; K gets a per-channel offset
~ N(0, 4) (sigma 2; ``koff_sigma`` overrides it for the stronger ridges of the
accuracy study) on a few channels per KV head, constant across tokens and
shared by every batch entry (the persistent channel "ridges" of §4.2);
optionally a fraction of entries of Q, K and V is multiplied by a spike
factor.  bf16 configurations round the fp32 draws to bf16 (round to nearest
even, via torch).  Decode draws the frozen query mean Qbar ~ N(0, 1/N_kv) per
(batch, q-head, channel), the law of the mean of N_kv iid N(0, 1) queries.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "koff": 4, "qmean": 5, "sample": 6}


@dataclass(frozen=True)
class Config:
    name: str
    kind: str  # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    N: int  # sequence length (prefill) or KV length (decode)
    D: int = 128
    dtype: str = "bf16"  # input dtype: "bf16" or "f32"
    n_outlier: int = 5  # K outlier channels per KV head
    koff_sigma: float = 2.0  # standard deviation of their offsets
    spike_frac: float = 0.0
    spike_mult: float = 20.0
    num_splits: int = 1
    lse: bool = False
    causal: bool = True
    seed: int = 0
    cid: int = 0  # stream id of the configuration
    smooth: bool = True
    notes: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


CONFIGS = {
    "prefill_1k_2x1": Config("prefill_1k_2x1", "prefill", 1, 2, 1, 1024, dtype="f32", n_outlier=8,
                             cid=1, notes="small causal prefill, fp32 inputs, 8 outlier channels"),
    "llama8b_prefill_16k": Config("llama8b_prefill_16k", "prefill", 1, 32, 8, 16384, cid=2,
                                  notes="Llama-3.1-8B-shaped causal prefill"),
    "qwen14b_prefill_32k": Config("qwen14b_prefill_32k", "prefill", 1, 40, 8, 32768, spike_frac=0.001,
                                  cid=3, notes="Qwen3-14B-shaped causal prefill with x20 spikes"),
    "llama8b_decode_128k": Config("llama8b_decode_128k", "decode", 16, 32, 8, 131072, num_splits=32,
                                  causal=False, cid=4, notes="Llama-3.1-8B-shaped split-KV decode"),
    "llama8b_prefill_128k_lse": Config("llama8b_prefill_128k_lse", "prefill", 2, 32, 8, 131072, lse=True,
                                       cid=5, notes="long causal prefill writing LSE"),
}


def config(name: str, **overrides) -> Config:
    import dataclasses
    return dataclasses.replace(CONFIGS[name], **overrides)


def _rng(cfg: Config, tensor: str, *idx: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, cfg.cid, TENSOR_IDS[tensor], *idx])
    return np.random.Generator(np.random.PCG64(ss))


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def k_outliers(cfg: Config, h: int) -> tuple[np.ndarray, np.ndarray]:
    """(channels, offsets) of KV head h."""
    r = _rng(cfg, "koff", h)
    ch = r.choice(cfg.D, size=cfg.n_outlier, replace=False)
    off = r.normal(0.0, cfg.koff_sigma, size=cfg.n_outlier).astype(np.float32)
    return ch, off


def head(cfg: Config, tensor: str, b: int, h: int, n_tokens: int | None = None) -> np.ndarray:
    """One [tokens, D] slice (fp32 values, bf16-representable for bf16 configs).

    tensor in {"q", "k", "v"}; decode queries have one token."""
    T = n_tokens if n_tokens is not None else (1 if (tensor == "q" and cfg.kind == "decode") else cfg.N)
    r = _rng(cfg, tensor, b, h)
    x = r.standard_normal((T, cfg.D), dtype=np.float32)
    if tensor == "k" and cfg.n_outlier > 0:
        ch, off = k_outliers(cfg, h)
        x[:, ch] += off[None, :]
    if cfg.spike_frac > 0:
        mask = r.random((T, cfg.D)) < cfg.spike_frac
        x[mask] *= np.float32(cfg.spike_mult)
    return _to_dtype(x, cfg.dtype)


def q_mean(cfg: Config) -> np.ndarray:
    """Frozen decode query means [B, Hq, D] ~ N(0, 1/N_kv)."""
    out = np.empty((cfg.B, cfg.Hq, cfg.D), dtype=np.float32)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            out[b, h] = _rng(cfg, "qmean", b, h).normal(0.0, 1.0 / np.sqrt(cfg.N), cfg.D)
    return out


def full(cfg: Config, tensor: str) -> np.ndarray:
    """Whole [B, H, T, D] host tensor (fp32 values).  Use only for sizes that fit."""
    H = cfg.Hq if tensor == "q" else cfg.Hkv
    T = 1 if (tensor == "q" and cfg.kind == "decode") else cfg.N
    out = np.empty((cfg.B, H, T, cfg.D), dtype=np.float32)
    for b in range(cfg.B):
        for h in range(H):
            out[b, h] = head(cfg, tensor, b, h)
    return out


def to_device(cfg: Config, tensor: str, device="cuda"):
    """Device tensor [B, H, T, D] in the configuration's dtype, filled head by head
    so the host never holds more than one head."""
    import torch
    H = cfg.Hq if tensor == "q" else cfg.Hkv
    T = 1 if (tensor == "q" and cfg.kind == "decode") else cfg.N
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty((cfg.B, H, T, cfg.D), dtype=tdt, device=device)
    for b in range(cfg.B):
        for h in range(H):
            out[b, h].copy_(torch.from_numpy(head(cfg, tensor, b, h)).to(tdt))
    return out


def sample_rows(cfg: Config, n_random: int = 256) -> np.ndarray:
    """Deterministic row sample [R, 3] of (b, q-head, position) for large prefill
    configurations: every row of query tiles 0, 1 and the last tile (128 rows each)
    for heads {0, G-1, Hq-1} of batch 0 and the last batch, plus n_random seeded rows."""
    rows = []
    last_tile = (cfg.N - 1) // 128
    for b in sorted({0, cfg.B - 1}):
        for h in sorted({0, cfg.G - 1, cfg.Hq - 1}):
            for t in sorted({0, min(1, last_tile), last_tile}):
                for i in range(t * 128, min((t + 1) * 128, cfg.N)):
                    rows.append((b, h, i))
    r = _rng(cfg, "sample", 0, 0)
    for _ in range(n_random):
        rows.append((int(r.integers(cfg.B)), int(r.integers(cfg.Hq)), int(r.integers(cfg.N))))
    return np.array(sorted(set(rows)), dtype=np.int64)


def device_inputs(cfg: Config, device="cuda", seed: int | None = None):
    """Q, K, V drawn directly on the device (for the throughput runs, whose
    tensors are too large to draw on the host head by head): the same laws as
    ``head`` -- N(0, 1), the same per-KV-head outlier channels and offsets as
    ``k_outliers``, optional spikes -- from a seeded torch generator, rounded
    to the configuration's dtype.  Decode also gets frozen query means.
    Returns a dict of device tensors."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1000003 + cfg.cid if seed is None else seed)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    nq = 1 if cfg.kind == "decode" else cfg.N
    out = {}
    for name, H, T in (("q", cfg.Hq, nq), ("k", cfg.Hkv, cfg.N), ("v", cfg.Hkv, cfg.N)):
        x = torch.empty((cfg.B, H, T, cfg.D), dtype=tdt, device=device)
        for b in range(cfg.B):  # one batch entry at a time bounds the fp32 scratch
            xb = torch.randn((H, T, cfg.D), generator=g, device=device, dtype=torch.float32)
            if name == "k" and cfg.n_outlier > 0:
                for h in range(H):
                    ch, off = k_outliers(cfg, h)
                    xb[h][:, torch.from_numpy(ch).to(device)] += torch.from_numpy(off).to(device)
            if cfg.spike_frac > 0:
                mask = torch.rand(xb.shape, generator=g, device=device) < cfg.spike_frac
                xb[mask] *= cfg.spike_mult
            x[b].copy_(xb.to(tdt))
            del xb
        out[name] = x
    if cfg.kind == "decode":
        out["q_mean"] = torch.randn((cfg.B, cfg.Hq, cfg.D), generator=g, device=device,
                                    dtype=torch.float32) / float(np.sqrt(cfg.N))
    return out
