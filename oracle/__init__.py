"""CPU oracle for the QK4PV8 attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does; the two
share no code, headers, tables or helpers.

Method source: the MpFA paper page, "MpFA: Hardware-Efficient Train-Free QK4V8
FlashAttention Kernels on Blackwell GPUs" (cited as "MpFA §x").  The numeric
core lives in ``mpfa_oracle.c`` (plain C, FP64, built with
``-ffp-contract=off``); this module binds it with ctypes and composes the
steps in the paper's order: sequence statistics and centering, NVFP4
quantization of Q_c and K_c, FP8 quantization of V, the rank-one compensation
vector, then blocked online-softmax attention (prefill) or partitioned
attention with a log-sum-exp merge (decode).

``identity=True`` skips every quantizer and the P rounding and keeps the
centering and compensation in FP64; the result then equals exact attention,
which pins the compensation algebra (see ``exact_attention``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mpfa_oracle.c")
_LIB = os.path.join(_HERE, "libmpfa_oracle.so")
_lib = None

KV_BLOCK = 128  # keys per online-softmax block (MpFA §3.2: M = N = 128 KV block)
P_SCALE = 448.0  # fixed FP8 scale of P (MpFA §5.1: P is bounded, fixed scale)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        sig = {
            "oracle_e2m1_decode": (f64, [i32]),
            "oracle_e4m3_decode": (f64, [i32]),
            "oracle_e2m1_encode": (i32, [f64]),
            "oracle_e4m3_encode": (i32, [f64]),
            "oracle_bf16_rne": (ctypes.c_uint16, [f32]),
            "oracle_channel_mean": (None, [P, i64, i32, P]),
            "oracle_amax": (f32, [P, i64]),
            "oracle_nvfp4_global_scale": (f32, [f32]),
            "oracle_nvfp4_quantize": (None, [P, i64, i32, f32, P, P]),
            "oracle_nvfp4_dequantize": (None, [P, P, i64, i32, f32, P]),
            "oracle_fp8_scale": (f32, [f32]),
            "oracle_fp8_quantize": (None, [P, i64, f32, P]),
            "oracle_delta_s": (None, [P, P, i64, i32, P]),
            "oracle_attn_state": (None, [i32, i32, P, P, P, P, P, i64, i64, i32, f64, i32, f64, P,
                                         P, P, P]),
            "oracle_merge_states": (None, [i32, i32, i32, P, P, P, f64, P, P, P]),
            "oracle_e4m3_encode_array": (None, [P, i64, P]),
            "oracle_e2m1_encode_array": (None, [P, i64, P]),
            "oracle_bf16_rne_array": (None, [P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- codecs --
def e2m1_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.int64)
    return np.array([L.oracle_e2m1_decode(int(x)) for x in c.ravel()]).reshape(c.shape)


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.int64)
    return np.array([L.oracle_e4m3_decode(int(x)) for x in c.ravel()]).reshape(c.shape)


def e4m3_table() -> np.ndarray:
    """FP64 value of each of the 256 E4M3 codes (NaN for 0x7F / 0xFF)."""
    return e4m3_decode(np.arange(256))


def e2m1_table() -> np.ndarray:
    return e2m1_decode(np.arange(16))


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(x), x.size, _p(out))
    return out


def e2m1_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e2m1_encode_array(_p(x), x.size, _p(out))
    return out


def bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(x), x.size, _p(out))
    return out


def bf16_to_f64(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16
    return h.view(np.float32).astype(np.float64)


# ----------------------------------------------------- statistics & codes --
def channel_mean(x: np.ndarray) -> np.ndarray:
    """Order-free fixed-point mean over axis -2 of a [..., T, D] fp32 array."""
    x = np.asarray(x, dtype=np.float32)
    T, D = x.shape[-2], x.shape[-1]
    flat = np.ascontiguousarray(x.reshape(-1, T, D))
    out = np.empty((flat.shape[0], D), dtype=np.float32)
    L = lib()
    for i in range(flat.shape[0]):
        sl = np.ascontiguousarray(flat[i])
        o = np.empty(D, dtype=np.float32)
        L.oracle_channel_mean(_p(sl), T, D, _p(o))
        out[i] = o
    return out.reshape(x.shape[:-2] + (D,))


def amax(x: np.ndarray) -> np.float32:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return np.float32(lib().oracle_amax(_p(x.ravel()), x.size))


def nvfp4_global_scale(a: float) -> np.float32:
    return np.float32(lib().oracle_nvfp4_global_scale(float(np.float32(a))))


def nvfp4_quantize(x: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    """x [..., D] fp32 -> (codes [..., D/2] u8, scales [..., D/16] u8) with global scale g."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    D = x.shape[-1]
    rows = x.size // D
    codes = np.zeros(x.shape[:-1] + (D // 2,), dtype=np.uint8)
    sf = np.zeros(x.shape[:-1] + (D // 16,), dtype=np.uint8)
    lib().oracle_nvfp4_quantize(_p(x), rows, D, float(np.float32(g)), _p(codes), _p(sf))
    return codes, sf


def nvfp4_dequantize(codes: np.ndarray, sf: np.ndarray, g) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    D = codes.shape[-1] * 2
    rows = codes.size // (D // 2)
    out = np.empty(codes.shape[:-1] + (D,), dtype=np.float64)
    lib().oracle_nvfp4_dequantize(_p(codes), _p(sf), rows, D, float(np.float32(g)), _p(out))
    return out


def fp8_scale(a: float) -> np.float32:
    return np.float32(lib().oracle_fp8_scale(float(np.float32(a))))


def fp8_quantize(x: np.ndarray, s) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_fp8_quantize(_p(x), x.size, float(np.float32(s)), _p(out))
    return out


def delta_s(qmean: np.ndarray, kc: np.ndarray) -> np.ndarray:
    """qmean [D] fp32, kc [T, D] fp32 -> bf16 bits [T]."""
    qmean = np.ascontiguousarray(qmean, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.float32)
    T, D = kc.shape
    out = np.empty(T, dtype=np.uint16)
    lib().oracle_delta_s(_p(qmean), _p(kc), T, D, _p(out))
    return out


P_FORMATS = {"none": 0, "e4m3": 1, "bf16": 2, "nvfp4": 3}
AMB_REL = 2.0 ** -16  # how close to a rounding midpoint an FP32 exp2 cannot decide


def attn_state(q, row_pos, k, v, delta, kv_begin, kv_end, scale, quant_p=True, block=KV_BLOCK,
               ambiguity=False, p_format=None, amb_rel=AMB_REL):
    """Blocked online-softmax state of R rows over keys [kv_begin, kv_end).

    q [R, D] f64; row_pos [R] int64 (-1: every key visible); k, v [Nk, D] f64;
    delta [Nk] f64 or None.  P is rounded as p_format says ("e4m3": the
    method's FP8 P with its fixed scale 448; "bf16": bf16 of 448 p, the BF16
    P.V assignment; "nvfp4": NVFP4 of p over 16-key groups with the fixed
    global scale fp32(1/2688), the NVFP4 P.V assignment, acc in units of
    448 p; "none": not rounded); by default quant_p picks "e4m3" or "none".  Returns (m [R], l [R], acc [R, D]) in FP64, and with
    ambiguity=True also amb [R, D]: how far acc may move if the keys whose
    448 p sits within amb_rel (relative) of a rounding midpoint round the
    other way (both roundings are correct for a p computed in FP32, or with
    the relative error amb_rel)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rp = np.ascontiguousarray(row_pos, dtype=np.int64)
    R, D = q.shape
    m = np.empty(R)
    l = np.empty(R)
    acc = np.empty((R, D))
    amb = np.empty((R, D)) if ambiguity else None
    dp = None
    if delta is not None:
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        dp = _p(delta)
    fmt = P_FORMATS[p_format] if p_format is not None else (1 if quant_p else 0)
    lib().oracle_attn_state(D, R, _p(q), _p(rp), _p(k), _p(v), dp, int(kv_begin), int(kv_end),
                            int(block), float(scale), fmt, float(amb_rel), _p(m), _p(l), _p(acc),
                            _p(amb) if ambiguity else None)
    return (m, l, acc, amb) if ambiguity else (m, l, acc)


def merge_states(m, l, acc, scale):
    """m, l [R, P]; acc [R, P, D] -> merged (m [R], l [R], acc [R, D])."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    R, P = m.shape
    D = acc.shape[-1]
    om, ol, oacc = np.empty(R), np.empty(R), np.empty((R, D))
    lib().oracle_merge_states(D, R, P, _p(m), _p(l), _p(acc), float(scale), _p(om), _p(ol), _p(oacc))
    return om, ol, oacc


from .pipeline import (  # noqa: E402  (pipeline uses the bindings above)
    PAGE,
    Q_TILE,
    Operands,
    append_kv,
    append_kv_paged,
    decode,
    decode_paged,
    decode_partitions,
    exact_attention,
    gather_pages,
    prefill_rows,
    prefill_tile_mean_rows,
    quantize_k,
    quantize_q,
    quantize_q_tiles,
    quantize_v,
    quantize_v_bf16,
    quantize_v_nvfp4,
    dequantize_v_nvfp4,
    tile_means,
    delta_tile,
    delta_tile_row,
)

__all__ = [
    "build", "lib", "KV_BLOCK", "P_SCALE",
    "e2m1_decode", "e4m3_decode", "e2m1_table", "e4m3_table", "e2m1_encode", "e4m3_encode",
    "bf16_rne", "bf16_to_f64", "P_FORMATS", "AMB_REL", "channel_mean", "amax", "nvfp4_global_scale", "nvfp4_quantize",
    "nvfp4_dequantize", "fp8_scale", "fp8_quantize", "delta_s", "attn_state", "merge_states",
    "quantize_k", "quantize_v", "quantize_v_bf16", "quantize_v_nvfp4", "dequantize_v_nvfp4",
    "quantize_q", "prefill_rows", "decode", "decode_partitions",
    "exact_attention", "Operands", "append_kv", "PAGE", "gather_pages", "decode_paged",
    "append_kv_paged", "Q_TILE", "tile_means", "quantize_q_tiles", "delta_tile", "delta_tile_row",
    "prefill_tile_mean_rows"
]
