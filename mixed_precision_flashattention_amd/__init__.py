"""Python binding of libmpfa.so, the QK4PV8 attention library for MI355X.

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI declared in ``include/mpfa.h``.  torch supplies device
memory and the current stream.  The functions named like the C entry points
take every buffer from the caller; the short-named helpers allocate the
outputs and workspace with torch and call them.

Importing does not load the library; the first call does, and raises if
``libmpfa.so`` has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmpfa.so")

MPFA_F32 = 0
MPFA_BF16 = 1
MPFA_OP_QUANTIZE_K = 0
MPFA_OP_QUANTIZE_V = 1
MPFA_OP_PREFILL = 2
MPFA_OP_DECODE = 3
MPFA_OP_PREFILL_PV_NVFP4 = 4
MPFA_DECODE_MAX_GROUP = 8
MPFA_DECODE_STATIC_SCRATCH_BYTES = 16777216
HEAD_DIM = 128
V_TILE = 32  # tokens per V tile (two head-dim-major halves of 16 tokens)

EXPORTS = ("mpfa_workspace_bytes", "mpfa_status_string", "mpfa_quantize_k_nvfp4",
           "mpfa_quantize_k_nvfp4_with_q_amax", "mpfa_quantize_v_fp8", "mpfa_append_kv",
           "mpfa_append_kv_paged", "mpfa_prefill", "mpfa_prefill_with_q_amax", "mpfa_decode",
           "mpfa_decode_paged", "mpfa_prefill_tile_mean", "mpfa_prefill_elementwise",
           "mpfa_prefill_poly_exp2", "mpfa_pack_v_bf16", "mpfa_prefill_pv_bf16",
           "mpfa_quantize_v_nvfp4", "mpfa_prefill_pv_nvfp4", "mpfa_decode_static",
           "mpfa_prefill_rank_one")
PAGE_SIZE = 128  # tokens per page of a paged cache

_lib = None


class MpfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status} ({status_string(status)})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmpfa.so (built by ``__graft_entry__.build()``) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.mpfa_workspace_bytes.restype = sz
    L.mpfa_workspace_bytes.argtypes = [i32] * 7
    L.mpfa_status_string.restype = ctypes.c_char_p
    L.mpfa_status_string.argtypes = [i32]
    L.mpfa_quantize_k_nvfp4.restype = i32
    L.mpfa_quantize_k_nvfp4.argtypes = [P, i32, i32, i32, i32, i32, P, i32, i32, P, P, P, P, P, P,
                                        P, sz, P]
    L.mpfa_quantize_k_nvfp4_with_q_amax.restype = i32
    L.mpfa_quantize_k_nvfp4_with_q_amax.argtypes = [P, i32, i32, i32, i32, i32, P, i32, i32, P, P,
                                                    P, P, P, P, P, P, sz, P]
    L.mpfa_quantize_v_fp8.restype = i32
    L.mpfa_quantize_v_fp8.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, sz, P]
    L.mpfa_append_kv.restype = i32
    L.mpfa_append_kv.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, i32, P, P, P, P, P, P, P, P,
                                 P]
    L.mpfa_prefill.restype = i32
    L.mpfa_prefill.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f32, i32,
                               P, i32, P, P, sz, P]
    L.mpfa_prefill_with_q_amax.restype = i32
    L.mpfa_prefill_with_q_amax.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                           P, f32, i32, P, i32, P, P, sz, P]
    for name in ("mpfa_prefill_elementwise", "mpfa_prefill_poly_exp2", "mpfa_prefill_rank_one"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f32,
                                     i32, P, i32, P, P, sz, P]
    L.mpfa_prefill_pv_bf16.restype = i32
    L.mpfa_prefill_pv_bf16.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, f32, i32,
                                       P, i32, P, P, sz, P]
    L.mpfa_pack_v_bf16.restype = i32
    L.mpfa_pack_v_bf16.argtypes = [P, i32, i32, i32, i32, i32, P, P]
    L.mpfa_quantize_v_nvfp4.restype = i32
    L.mpfa_quantize_v_nvfp4.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, sz, P]
    L.mpfa_prefill_pv_nvfp4.restype = i32
    L.mpfa_prefill_pv_nvfp4.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                        f32, i32, P, i32, P, P, sz, P]
    L.mpfa_prefill_tile_mean.restype = i32
    L.mpfa_prefill_tile_mean.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, f32, i32,
                                         P, i32, P, P, P, sz, P]
    L.mpfa_decode.restype = i32
    L.mpfa_decode.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f32, i32,
                              P, i32, P, P, sz, P]
    L.mpfa_decode_static.restype = i32
    L.mpfa_decode_static.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f32,
                                     i32, P, i32, P, P]
    L.mpfa_append_kv_paged.restype = i32
    L.mpfa_append_kv_paged.argtypes = [P, P, i32, i32, i32, i32, P, P, i32, i32, i32, i32, P, P, P,
                                       P, P, P, P, P, P]
    L.mpfa_decode_paged.restype = i32
    L.mpfa_decode_paged.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, i32,
                                    i32, i32, f32, i32, P, i32, P, P, sz, P]
    _lib = L
    return L


def status_string(status: int) -> str:
    return load_library().mpfa_status_string(int(status)).decode()


def mpfa_workspace_bytes(op: int, B: int, Hq: int, Hkv: int, N: int, D: int = HEAD_DIM,
                         num_splits: int = 1) -> int:
    return int(load_library().mpfa_workspace_bytes(op, B, Hq, Hkv, N, D, num_splits))


# ----------------------------------------------------------- marshalling --
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MPFA_F32
    if t.dtype == torch.bfloat16:
        return MPFA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16 expected")


def _check(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _raise(fn: str, status: int):
    if status != 0:
        raise MpfaError(fn, status)


def mpfa_quantize_k_nvfp4(k, q, q_mean, k_mean, k_fp4, k_sf, k_gscale, delta_s, ws, Hq=None,
                          stream=None):
    """C-ABI call: k [B, Hkv, N, 128]; q [B, Hq, N, 128] or None (then q_mean is
    an input); direct mode when k_mean, delta_s (and q_mean) are None."""
    _check(k, q, q_mean, k_mean, k_fp4, k_sf, k_gscale, delta_s, ws)
    B, Hkv, N, D = k.shape
    if Hq is None:
        Hq = q.shape[1] if q is not None else (q_mean.shape[1] if q_mean is not None else 0)
    st = load_library().mpfa_quantize_k_nvfp4(
        _ptr(k), _dtype_code(k), B, Hkv, N, D, _ptr(q), _dtype_code(q) if q is not None else 0,
        Hq, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4), _ptr(k_sf), _ptr(k_gscale), _ptr(delta_s),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_quantize_k_nvfp4", st)


def mpfa_quantize_k_nvfp4_with_q_amax(k, q, q_mean, k_mean, k_fp4, k_sf, k_gscale, delta_s,
                                      q_amax, ws, stream=None):
    """C-ABI call: smoothing mode with q given; also writes q_amax (float32 [1]),
    the Q_c amax that mpfa_prefill_with_q_amax takes for this q."""
    _check(k, q, q_mean, k_mean, k_fp4, k_sf, k_gscale, delta_s, q_amax, ws)
    B, Hkv, N, D = k.shape
    st = load_library().mpfa_quantize_k_nvfp4_with_q_amax(
        _ptr(k), _dtype_code(k), B, Hkv, N, D, _ptr(q), _dtype_code(q), q.shape[1], _ptr(q_mean),
        _ptr(k_mean), _ptr(k_fp4), _ptr(k_sf), _ptr(k_gscale), _ptr(delta_s), _ptr(q_amax),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_quantize_k_nvfp4_with_q_amax", st)


def mpfa_quantize_v_fp8(v, v_fp8, v_scale, ws, stream=None):
    _check(v, v_fp8, v_scale, ws)
    B, Hkv, N, D = v.shape
    st = load_library().mpfa_quantize_v_fp8(_ptr(v), _dtype_code(v), B, Hkv, N, D, _ptr(v_fp8),
                                            _ptr(v_scale), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream))
    _raise("mpfa_quantize_v_fp8", st)


def mpfa_prefill(q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s,
                 softmax_scale, causal, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, out, lse, ws)
    B, Hq, N, D = q.shape
    st = load_library().mpfa_prefill(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s),
        float(softmax_scale), int(bool(causal)), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_prefill", st)


def mpfa_prefill_with_q_amax(q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale,
                             delta_s, q_amax, softmax_scale, causal, out, lse, ws, stream=None):
    """C-ABI call; q_amax: float32 [1], the Q_c amax that
    mpfa_quantize_k_nvfp4_with_q_amax wrote for this same q (no pass over q)."""
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, q_amax, out, lse, ws)
    B, Hq, N, D = q.shape
    st = load_library().mpfa_prefill_with_q_amax(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s), _ptr(q_amax),
        float(softmax_scale), int(bool(causal)), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_prefill_with_q_amax", st)


def _prefill_variant(fn, q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s,
                     softmax_scale, causal, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, out, lse, ws)
    B, Hq, N, D = q.shape
    st = getattr(load_library(), fn)(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s),
        float(softmax_scale), int(bool(causal)), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise(fn, st)


def mpfa_prefill_elementwise(*args, **kw):
    """C-ABI call, the arguments of mpfa_prefill (smoothing mode)."""
    _prefill_variant("mpfa_prefill_elementwise", *args, **kw)


def mpfa_prefill_rank_one(*args, **kw):
    """C-ABI call, the arguments of mpfa_prefill (smoothing mode)."""
    _prefill_variant("mpfa_prefill_rank_one", *args, **kw)


def mpfa_prefill_poly_exp2(*args, **kw):
    """C-ABI call, the arguments of mpfa_prefill."""
    _prefill_variant("mpfa_prefill_poly_exp2", *args, **kw)


def mpfa_pack_v_bf16(v, v_bf16, stream=None):
    _check(v, v_bf16)
    B, Hkv, N, D = v.shape
    st = load_library().mpfa_pack_v_bf16(_ptr(v), _dtype_code(v), B, Hkv, N, D, _ptr(v_bf16),
                                         _stream(stream))
    _raise("mpfa_pack_v_bf16", st)


def mpfa_prefill_pv_bf16(q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_bf16, delta_s,
                         softmax_scale, causal, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_bf16, delta_s, out, lse, ws)
    B, Hq, N, D = q.shape
    st = load_library().mpfa_prefill_pv_bf16(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_bf16), _ptr(delta_s), float(softmax_scale),
        int(bool(causal)), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_prefill_pv_bf16", st)


def mpfa_quantize_v_nvfp4(v, v_fp4, v_sf, v_gscale, ws, stream=None):
    _check(v, v_fp4, v_sf, v_gscale, ws)
    B, Hkv, N, D = v.shape
    st = load_library().mpfa_quantize_v_nvfp4(_ptr(v), _dtype_code(v), B, Hkv, N, D, _ptr(v_fp4),
                                              _ptr(v_sf), _ptr(v_gscale), _ptr(ws),
                                              ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_quantize_v_nvfp4", st)


def mpfa_prefill_pv_nvfp4(q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp4, v_sf, v_gscale,
                          delta_s, softmax_scale, causal, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp4, v_sf, v_gscale, delta_s, out, lse, ws)
    B, Hq, N, D = q.shape
    st = load_library().mpfa_prefill_pv_nvfp4(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp4), _ptr(v_sf), _ptr(v_gscale), _ptr(delta_s),
        float(softmax_scale), int(bool(causal)), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_prefill_pv_nvfp4", st)


def mpfa_prefill_tile_mean(q, Hkv, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, softmax_scale,
                           causal, out, lse, q_tile_mean, ws, stream=None):
    _check(q, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, out, lse, q_tile_mean, ws)
    B, Hq, N, D = q.shape
    st = load_library().mpfa_prefill_tile_mean(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N, D, _ptr(k_mean), _ptr(k_fp4), _ptr(k_sf),
        _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), float(softmax_scale), int(bool(causal)),
        _ptr(out), _dtype_code(out), _ptr(lse), _ptr(q_tile_mean), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_prefill_tile_mean", st)


def mpfa_append_kv(k_new, v_new, pos, q_mean, k_mean, k_gscale, v_scale, k_fp4, k_sf, v_fp8,
                   delta_s, Hq=None, stream=None):
    """k_new, v_new [B, Hkv, T, 128]; pos int32 [B]; caches of capacity
    k_fp4.shape[2] tokens (smoothing iff k_mean is given)."""
    _check(k_new, v_new, pos, q_mean, k_mean, k_gscale, v_scale, k_fp4, k_sf, v_fp8, delta_s)
    import torch
    if pos.dtype != torch.int32:
        raise TypeError("pos must be an int32 tensor")
    B, Hkv, T, D = k_new.shape
    N_cap = k_fp4.shape[2]
    if Hq is None:
        Hq = q_mean.shape[1] if q_mean is not None else 0
    st = load_library().mpfa_append_kv(
        _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, Hkv, T, D, N_cap, _ptr(pos), Hq,
        _ptr(q_mean), _ptr(k_mean), _ptr(k_gscale), _ptr(v_scale), _ptr(k_fp4), _ptr(k_sf),
        _ptr(v_fp8), _ptr(delta_s), _stream(stream))
    _raise("mpfa_append_kv", st)


def mpfa_decode(q, Hkv, N_kv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s,
                softmax_scale, num_splits, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, out, lse, ws)
    B, Hq = q.shape[0], q.shape[1]
    D = q.shape[-1]
    st = load_library().mpfa_decode(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N_kv, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s),
        float(softmax_scale), int(num_splits), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_decode", st)


def mpfa_decode_static(q, Hkv, N_kv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s,
                       softmax_scale, num_splits, out, lse, stream=None):
    """C-ABI call: mpfa_decode without a workspace (the library's fixed
    per-GPU scratch array; nothing is allocated)."""
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, out, lse)
    B, Hq = q.shape[0], q.shape[1]
    D = q.shape[-1]
    st = load_library().mpfa_decode_static(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, N_kv, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4),
        _ptr(k_sf), _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s),
        float(softmax_scale), int(num_splits), _ptr(out), _dtype_code(out), _ptr(lse),
        _stream(stream))
    _raise("mpfa_decode_static", st)


def _int32(*ts):
    import torch
    for t in ts:
        if t.dtype != torch.int32:
            raise TypeError("block tables, lengths and positions must be int32 tensors")


def mpfa_append_kv_paged(k_new, v_new, pos, block_table, q_mean, k_mean, k_gscale, v_scale, k_fp4,
                         k_sf, v_fp8, delta_s, Hq=None, stream=None):
    """k_new, v_new [B, Hkv, 1, 128]; pos, block_table int32 [B], [B, max_pages];
    a page pool k_fp4 [P, Hkv, 128, 64] ... (smoothing iff k_mean is given)."""
    _check(k_new, v_new, pos, block_table, q_mean, k_mean, k_gscale, v_scale, k_fp4, k_sf, v_fp8,
           delta_s)
    _int32(pos, block_table)
    B, Hkv, _, D = k_new.shape
    if Hq is None:
        Hq = q_mean.shape[1] if q_mean is not None else 0
    st = load_library().mpfa_append_kv_paged(
        _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, Hkv, D, _ptr(pos), _ptr(block_table),
        block_table.shape[1], k_fp4.shape[0], PAGE_SIZE, Hq, _ptr(q_mean), _ptr(k_mean),
        _ptr(k_gscale), _ptr(v_scale), _ptr(k_fp4), _ptr(k_sf), _ptr(v_fp8), _ptr(delta_s),
        _stream(stream))
    _raise("mpfa_append_kv_paged", st)


def mpfa_decode_paged(q, Hkv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s,
                      block_table, seq_lens, softmax_scale, num_splits, out, lse, ws, stream=None):
    _check(q, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8, v_scale, delta_s, block_table, seq_lens,
           out, lse, ws)
    _int32(block_table, seq_lens)
    B, Hq = q.shape[0], q.shape[1]
    D = q.shape[-1]
    st = load_library().mpfa_decode_paged(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, D, _ptr(q_mean), _ptr(k_mean), _ptr(k_fp4), _ptr(k_sf),
        _ptr(k_gscale), _ptr(v_fp8), _ptr(v_scale), _ptr(delta_s), _ptr(block_table),
        _ptr(seq_lens), block_table.shape[1], k_fp4.shape[0], PAGE_SIZE, float(softmax_scale),
        int(num_splits), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _raise("mpfa_decode_paged", st)


# ------------------------------------------------------ allocating helpers --
def _workspace(op, B, Hq, Hkv, N, num_splits, device):
    import torch
    n = mpfa_workspace_bytes(op, B, Hq, Hkv, N, HEAD_DIM, num_splits)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def query_identity(q):
    """What identifies one query tensor's contents for the Q_c amax hand-off,
    as a small host int64 tensor: its storage address, in-place version
    counter, device index, dtype code and shape."""
    import torch
    return torch.tensor([q.data_ptr(), q._version, q.device.index or 0, _dtype_code(q), *q.shape],
                        dtype=torch.int64)


def quantize_k(k, q=None, q_mean=None, smooth=True, Hq=None, stream=None):
    """Allocate and fill the NVFP4 K cache.  Returns a dict with k_fp4, k_sf,
    k_gscale and, in smoothing mode, k_mean, q_mean and delta_s (and, with q
    given, q_amax: the Q_c amax that ``prefill`` then takes instead of a pass
    over q, with q_amax_of: the identity of that q, which ``prefill`` checks).
    Smoothing with neither q nor q_mean only centres K (k_mean, no delta_s):
    the cache of ``prefill_tile_mean``."""
    import torch
    B, Hkv, N, D = k.shape
    dev = k.device
    out = {"k_fp4": torch.empty((B, Hkv, N, D // 2), dtype=torch.uint8, device=dev),
           "k_sf": torch.empty((B, Hkv, N, D // 16), dtype=torch.uint8, device=dev),
           "k_gscale": torch.empty(1, dtype=torch.float32, device=dev)}
    if smooth and q is None and q_mean is None:
        out["k_mean"] = torch.empty((B, Hkv, D), dtype=torch.float32, device=dev)
        ws = _workspace(MPFA_OP_QUANTIZE_K, B, 0, Hkv, N, 1, dev)
        mpfa_quantize_k_nvfp4(k, None, None, out["k_mean"], out["k_fp4"], out["k_sf"],
                              out["k_gscale"], None, ws, Hq=0, stream=stream)
    elif smooth:
        if Hq is None:
            Hq = q.shape[1] if q is not None else q_mean.shape[1]
        if q is not None:
            q_mean = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        out.update(k_mean=torch.empty((B, Hkv, D), dtype=torch.float32, device=dev),
                   q_mean=q_mean,
                   delta_s=torch.empty((B, Hq, N), dtype=torch.int16, device=dev))
        ws = _workspace(MPFA_OP_QUANTIZE_K, B, Hq if q is not None else 0, Hkv, N, 1, dev)
        if q is not None:
            out["q_amax"] = torch.empty(1, dtype=torch.float32, device=dev)
            out["q_amax_of"] = query_identity(q)
            mpfa_quantize_k_nvfp4_with_q_amax(k, q, q_mean, out["k_mean"], out["k_fp4"],
                                              out["k_sf"], out["k_gscale"], out["delta_s"],
                                              out["q_amax"], ws, stream=stream)
        else:
            mpfa_quantize_k_nvfp4(k, q, q_mean, out["k_mean"], out["k_fp4"], out["k_sf"],
                                  out["k_gscale"], out["delta_s"], ws, Hq=Hq, stream=stream)
    else:
        ws = _workspace(MPFA_OP_QUANTIZE_K, B, 0, Hkv, N, 1, dev)
        mpfa_quantize_k_nvfp4(k, None, None, None, out["k_fp4"], out["k_sf"], out["k_gscale"],
                              None, ws, Hq=0, stream=stream)
    return out


def quantize_v(v, stream=None):
    """Allocate and fill the FP8 V cache (tiled layout, see mpfa.h)."""
    import torch
    B, Hkv, N, D = v.shape
    n_tiles = (N + V_TILE - 1) // V_TILE
    out = {"v_fp8": torch.empty((B, Hkv, n_tiles, 2, D, V_TILE // 2), dtype=torch.uint8,
                                device=v.device),
           "v_scale": torch.empty(1, dtype=torch.float32, device=v.device)}
    ws = _workspace(MPFA_OP_QUANTIZE_V, B, 0, Hkv, N, 1, v.device)
    mpfa_quantize_v_fp8(v, out["v_fp8"], out["v_scale"], ws, stream=stream)
    return out


def prefill(q, kq, vq, softmax_scale, causal=True, out_dtype=None, with_lse=False, ws=None,
            out=None, lse=None, stream=None):
    """QK4PV8 prefill from the caches returned by quantize_k / quantize_v.
    Smoothing iff kq holds delta_s.  When kq holds the Q_c amax of the q that
    quantize_k saw, the call takes it (mpfa_prefill_with_q_amax, no pass over
    q); that q must be this q, unchanged since: any other q raises ValueError
    (its global scale would be wrong).  Returns (out, lse or None)."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = kq["k_fp4"].shape[1]
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=out_dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(MPFA_OP_PREFILL, B, Hq, Hkv, N, 1, q.device)
    smooth = kq.get("delta_s") is not None
    args = (q, Hkv, kq.get("q_mean") if smooth else None, kq.get("k_mean") if smooth else None,
            kq["k_fp4"], kq["k_sf"], kq["k_gscale"], vq["v_fp8"], vq["v_scale"],
            kq.get("delta_s") if smooth else None)
    if smooth and kq.get("q_amax") is not None:
        ident = kq.get("q_amax_of")
        if ident is None or not torch.equal(ident, query_identity(q)):
            raise ValueError("kq['q_amax'] is the Q_c amax of another query tensor (or of this one "
                             "before an in-place change): quantize_k with this q, or drop q_amax")
        mpfa_prefill_with_q_amax(*args, kq["q_amax"], softmax_scale, causal, out,
                                 lse if with_lse else None, ws, stream=stream)
    else:
        mpfa_prefill(*args, softmax_scale, causal, out, lse if with_lse else None, ws,
                     stream=stream)
    return out, (lse if with_lse else None)


def pack_v_bf16(v, stream=None):
    """Allocate and fill the bf16 V cache of the bf16 P.V variant."""
    import torch
    B, Hkv, N, D = v.shape
    out = torch.empty((B, Hkv, (N + V_TILE - 1) // V_TILE, 4, D, 8), dtype=torch.int16,
                      device=v.device)
    mpfa_pack_v_bf16(v, out, stream=stream)
    return {"v_bf16": out}


def quantize_v_nvfp4(v, stream=None):
    """Allocate and fill the NVFP4 V cache of the NVFP4 P.V variant (16-key
    blocks per channel, see mpfa.h)."""
    import torch
    B, Hkv, N, D = v.shape
    nb = (N + 15) // 16
    out = {"v_fp4": torch.empty((B, Hkv, nb, D, 8), dtype=torch.uint8, device=v.device),
           "v_sf": torch.empty((B, Hkv, nb, D), dtype=torch.uint8, device=v.device),
           "v_gscale": torch.empty(1, dtype=torch.float32, device=v.device)}
    ws = _workspace(MPFA_OP_QUANTIZE_V, B, 0, Hkv, N, 1, v.device)
    mpfa_quantize_v_nvfp4(v, out["v_fp4"], out["v_sf"], out["v_gscale"], ws, stream=stream)
    return out


def prefill_variant(variant, q, kq, vq, softmax_scale, causal=True, out_dtype=None, with_lse=False,
                    ws=None, out=None, lse=None, stream=None):
    """One of the prefill's precision / placement variants on the caches of
    quantize_k (smoothing iff kq holds delta_s): "elementwise" (Delta_S added
    per score on the vector ALUs; smoothing only), "rank_one" (Delta_S by a
    rank-one bf16 matrix step; smoothing only), "poly_exp2" (one exponential
    in four by a cubic), "pv_bf16" (vq from pack_v_bf16: bf16 P and V),
    "pv_nvfp4" (vq from quantize_v_nvfp4: NVFP4 P and V).  The query amax is
    taken in the call's own pass.  Returns (out, lse or None)."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = kq["k_fp4"].shape[1]
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=out_dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if ws is None:
        op = MPFA_OP_PREFILL_PV_NVFP4 if variant == "pv_nvfp4" else MPFA_OP_PREFILL
        ws = _workspace(op, B, Hq, Hkv, N, 1, q.device)
    smooth = kq.get("delta_s") is not None
    common = (q, Hkv, kq.get("q_mean") if smooth else None, kq.get("k_mean") if smooth else None,
              kq["k_fp4"], kq["k_sf"], kq["k_gscale"])
    tail = (softmax_scale, causal, out, lse if with_lse else None, ws)
    if variant == "pv_bf16":
        mpfa_prefill_pv_bf16(*common, vq["v_bf16"], kq.get("delta_s") if smooth else None, *tail,
                             stream=stream)
    elif variant == "pv_nvfp4":
        mpfa_prefill_pv_nvfp4(*common, vq["v_fp4"], vq["v_sf"], vq["v_gscale"],
                              kq.get("delta_s") if smooth else None, *tail, stream=stream)
    elif variant in ("elementwise", "poly_exp2", "rank_one"):
        _prefill_variant(f"mpfa_prefill_{variant}", *common, vq["v_fp8"], vq["v_scale"],
                         kq.get("delta_s") if smooth else None, *tail, stream=stream)
    else:
        raise ValueError(f"unknown variant {variant!r}")
    return out, (lse if with_lse else None)


def prefill_tile_mean(q, kq, vq, softmax_scale, causal=True, out_dtype=None, with_lse=False,
                      ws=None, out=None, lse=None, q_tile_mean=None, stream=None):
    """Prefill with the queries smoothed per 128-row tile; kq must hold a
    centred K cache (``quantize_k(k)`` with neither q nor q_mean, or a
    smoothing-mode cache).  Returns (out, lse or None, q_tile_mean)."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = kq["k_fp4"].shape[1]
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=out_dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if q_tile_mean is None:
        q_tile_mean = torch.empty((B, Hq, (N + 127) // 128, D), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(MPFA_OP_PREFILL, B, Hq, Hkv, N, 1, q.device)
    mpfa_prefill_tile_mean(q, Hkv, kq["k_mean"], kq["k_fp4"], kq["k_sf"], kq["k_gscale"],
                           vq["v_fp8"], vq["v_scale"], softmax_scale, causal, out,
                           lse if with_lse else None, q_tile_mean, ws, stream=stream)
    return out, (lse if with_lse else None), q_tile_mean


def decode(q, kq, vq, softmax_scale, num_splits, out_dtype=None, with_lse=False, ws=None, out=None,
           lse=None, stream=None):
    """Split-KV decode; q [B, Hq, 1, 128].  Returns (out [B, Hq, 128], lse or None)."""
    import torch
    B, Hq = q.shape[0], q.shape[1]
    Hkv, N = kq["k_fp4"].shape[1], kq["k_fp4"].shape[2]
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(MPFA_OP_DECODE, B, Hq, Hkv, N, num_splits, q.device)
    smooth = kq.get("delta_s") is not None
    mpfa_decode(q, Hkv, N, kq.get("q_mean") if smooth else None, kq.get("k_mean") if smooth else None,
                kq["k_fp4"], kq["k_sf"], kq["k_gscale"], vq["v_fp8"], vq["v_scale"],
                kq.get("delta_s") if smooth else None, softmax_scale, num_splits, out,
                lse if with_lse else None, ws, stream=stream)
    return out, (lse if with_lse else None)


def append_kv(k_new, v_new, pos, kq, vq, stream=None):
    """Write new tokens into the caches returned by quantize_k / quantize_v
    (capacity = their length) at positions pos[b] + t, with their frozen
    means and scales; smoothing iff kq holds delta_s."""
    smooth = "delta_s" in kq
    mpfa_append_kv(k_new, v_new, pos, kq.get("q_mean") if smooth else None,
                   kq.get("k_mean") if smooth else None, kq["k_gscale"], vq["v_scale"],
                   kq["k_fp4"], kq["k_sf"], vq["v_fp8"], kq.get("delta_s") if smooth else None,
                   stream=stream)


def decode_paged(q, pool, block_table, seq_lens, softmax_scale, num_splits, out_dtype=None,
                 with_lse=False, ws=None, out=None, lse=None, stream=None):
    """Split-KV decode over a paged cache.  pool: k_fp4 [P, Hkv, 128, 64],
    k_sf [P, Hkv, 128, 8], v_fp8 [P, Hkv, 4, 2, 128, 16], per-request k_gscale
    and v_scale [B] and, in smoothing mode, delta_s [P, Hq, 128], q_mean
    [B, Hq, 128], k_mean [B, Hkv, 128].  Returns (out [B, Hq, 128], lse or None)."""
    import torch
    B, Hq = q.shape[0], q.shape[1]
    Hkv = pool["k_fp4"].shape[1]
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(MPFA_OP_DECODE, B, Hq, Hkv, 1, num_splits, q.device)
    smooth = pool.get("delta_s") is not None
    mpfa_decode_paged(q, Hkv, pool.get("q_mean") if smooth else None,
                      pool.get("k_mean") if smooth else None, pool["k_fp4"], pool["k_sf"],
                      pool["k_gscale"], pool["v_fp8"], pool["v_scale"],
                      pool.get("delta_s") if smooth else None, block_table, seq_lens, softmax_scale,
                      num_splits, out, lse if with_lse else None, ws, stream=stream)
    return out, (lse if with_lse else None)


def append_kv_paged(k_new, v_new, pos, pool, block_table, stream=None):
    """Write one new token per request into a paged cache (pool as in
    decode_paged) at positions pos[b], with each request's frozen means and
    scales; smoothing iff the pool holds delta_s."""
    smooth = pool.get("delta_s") is not None
    mpfa_append_kv_paged(k_new, v_new, pos, block_table, pool.get("q_mean") if smooth else None,
                         pool.get("k_mean") if smooth else None, pool["k_gscale"], pool["v_scale"],
                         pool["k_fp4"], pool["k_sf"], pool["v_fp8"],
                         pool.get("delta_s") if smooth else None, stream=stream)


def v_tiles_to_rows(v_fp8_tiled, N: int):
    """Host-side layout helper: tiled V codes [..., T, 2, 128, 16] (token t,
    channel d at [t / 32][(t % 32) / 16][d][t % 16]) -> [..., N, 128] (a pure
    permutation of bytes, used to compare caches element by element)."""
    x = v_fp8_tiled
    lead = x.shape[:-4]
    T = x.shape[-4]
    x = x.reshape(*lead, T, 2, HEAD_DIM, V_TILE // 2).swapaxes(-1, -2)
    x = x.reshape(*lead, T * V_TILE, HEAD_DIM)
    return x[..., :N, :]
