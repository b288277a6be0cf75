"""CPU checks of the C-ABI library: it loads, exports every function that
include/mpfa.h declares, sizes workspaces, and rejects invalid arguments
before launching anything (every call here fails validation, so no HIP
work is ever enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpfa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpfa_\w+)\s*\(", text)))


def header_define(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    import mixed_precision_flashattention_amd as mpfa
    if not os.path.exists(mpfa.LIB_PATH):
        from mixed_precision_flashattention_amd import _build
        _build.build()
    return mpfa.load_library()


def test_header_declares_the_four_entry_points():
    fns = header_functions()
    for name in ("mpfa_quantize_k_nvfp4", "mpfa_quantize_v_fp8", "mpfa_prefill", "mpfa_decode",
                 "mpfa_workspace_bytes", "mpfa_status_string"):
        assert name in fns


# The boundary's four calls and two helpers, argument for argument (types and
# order) as the scope table of the build states them.
CONTRACT = {
    "mpfa_workspace_bytes": ("size_t", "int op, int B, int Hq, int Hkv, int N, int D, int num_splits"),
    "mpfa_status_string": ("const char*", "int status"),
    "mpfa_quantize_k_nvfp4": (
        "int", "const void* k, int k_dtype, int B, int Hkv, int N, int D, const void* q_or_null, "
        "int q_dtype, int Hq, float* q_mean, float* k_mean, uint8_t* k_fp4, uint8_t* k_sf, "
        "float* k_gscale, uint16_t* delta_s, void* ws, size_t ws_bytes, void* stream"),
    "mpfa_quantize_v_fp8": (
        "int", "const void* v, int v_dtype, int B, int Hkv, int N, int D, uint8_t* v_fp8, "
        "float* v_scale, void* ws, size_t ws_bytes, void* stream"),
    "mpfa_prefill": (
        "int", "const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D, "
        "const float* q_mean, const float* k_mean, const uint8_t* k_fp4, const uint8_t* k_sf, "
        "const float* k_gscale, const uint8_t* v_fp8, const float* v_scale, "
        "const uint16_t* delta_s, float softmax_scale, int causal, void* out, int out_dtype, "
        "float* lse_or_null, void* ws, size_t ws_bytes, void* stream"),
    # "the same operand list" as the prefill, with N_kv and num_splits
    "mpfa_decode": (
        "int", "const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D, "
        "const float* q_mean, const float* k_mean, const uint8_t* k_fp4, const uint8_t* k_sf, "
        "const float* k_gscale, const uint8_t* v_fp8, const float* v_scale, "
        "const uint16_t* delta_s, float softmax_scale, int num_splits, void* out, int out_dtype, "
        "float* lse, void* ws, size_t ws_bytes, void* stream"),
}


def _declaration(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"([\w\s\*]+?)\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    ret = " ".join(m.group(1).split()).replace(" *", "*")
    args = ", ".join(" ".join(a.split()).replace(" *", "*") for a in m.group(2).split(","))
    return ret.split("\n")[-1].strip(), args


@pytest.mark.parametrize("name", sorted(CONTRACT))
def test_boundary_prototypes_verbatim(name):
    ret, args = _declaration(name)
    want_ret, want_args = CONTRACT[name]
    assert ret.endswith(want_ret), (name, ret)
    assert args == want_args, (name, args)


def test_library_exports_every_declared_symbol(lib):
    import mixed_precision_flashattention_amd as mpfa
    out = subprocess.run(["nm", "-D", "--defined-only", mpfa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(mpfa_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(mpfa.EXPORTS) == set(header_functions())


def test_constants_match_header():
    import mixed_precision_flashattention_amd as mpfa
    for name in ("MPFA_F32", "MPFA_BF16", "MPFA_OP_QUANTIZE_K", "MPFA_OP_QUANTIZE_V",
                 "MPFA_OP_PREFILL", "MPFA_OP_DECODE", "MPFA_OP_PREFILL_PV_NVFP4",
                 "MPFA_DECODE_MAX_GROUP",
                 "MPFA_DECODE_STATIC_SCRATCH_BYTES"):
        assert getattr(mpfa, name) == header_define(name), name


def test_status_strings(lib):
    assert lib.mpfa_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4):
        assert lib.mpfa_status_string(code) != b"unknown status"
    assert lib.mpfa_status_string(7) == b"unknown status"


def test_workspace_sizes(lib):
    ws = lib.mpfa_workspace_bytes
    # decode: the amax slots (64 x 128 B) + m, l [B*Hq*P] + acc [B*Hq*P*128]
    # floats, 256-aligned
    AMAX = 64 * 128
    B, Hq, Hkv, N, P = 16, 32, 8, 131072, 32
    n = ws(3, B, Hq, Hkv, N, 128, P)
    assert n % 256 == 0
    assert n >= AMAX + B * Hq * P * (2 + 128) * 4
    assert n < AMAX + B * Hq * P * (2 + 128) * 4 + 4 * 256
    # quantize_k with a query tensor needs the query statistics too
    assert ws(0, 1, 32, 8, 1024, 128, 1) > ws(0, 1, 0, 8, 1024, 128, 1)
    assert ws(1, 1, 0, 8, 1024, 128, 1) == AMAX
    # prefill: the Q amax slots + K expanded to FP16 block images (32 KB per
    # (batch, KV head, 128-key block))
    assert ws(2, 1, 32, 8, 1024, 128, 1) == AMAX + 8 * 8 * 32768
    assert ws(2, 2, 32, 8, 1001, 128, 1) == AMAX + 2 * 8 * 8 * 32768
    assert ws(2, 1, 4, 1, 1, 128, 1) == AMAX + 32768
    # NVFP4 P.V: also the FP16 image of V, 8 KB per (batch, KV head, 32-key tile)
    assert ws(4, 1, 32, 8, 1024, 128, 1) == ws(2, 1, 32, 8, 1024, 128, 1) + 8 * 32 * 8192
    assert ws(4, 2, 32, 8, 1001, 128, 1) == ws(2, 2, 32, 8, 1001, 128, 1) + 2 * 8 * 32 * 8192
    assert ws(4, 1, 4, 1, 1, 128, 1) == AMAX + 32768 + 8192
    assert ws(9, 1, 32, 8, 1024, 128, 1) == 0
    assert ws(3, 1, 32, 8, 1024, 128, 0) == 0
    assert ws(0, 0, 32, 8, 1024, 128, 1) == 0


class _Fake:
    """16-byte aligned host buffers standing in for device pointers: every call
    below fails validation before anything would dereference them."""

    def __init__(self):
        self.buf = ctypes.create_string_buffer(4096 + 16)
        base = ctypes.addressof(self.buf)
        self.p = ctypes.c_void_p((base + 15) // 16 * 16)
        self.mis = ctypes.c_void_p(self.p.value + 4)


def _prefill(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, scale=0.088, causal=1,
             out=f.p, out_dtype=1, lse=None, ws=f.p, ws_bytes=256, stream=None)
    a.update(kw)
    return lib.mpfa_prefill(*a.values())


def _prefill_qa(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, q_amax=f.p, scale=0.088,
             causal=1, out=f.p, out_dtype=1, lse=None, ws=f.p, ws_bytes=256, stream=None)
    a.update(kw)
    return lib.mpfa_prefill_with_q_amax(*a.values())


def test_prefill_with_q_amax_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, WS = -1, -3
    assert _prefill_qa(lib, f, q_amax=None) == INVALID
    assert _prefill_qa(lib, f, q_amax=f.mis) == INVALID
    assert _prefill_qa(lib, f, delta_s=None) == INVALID  # direct mode has no first-stage amax
    assert _prefill_qa(lib, f, delta_s=None, q_mean=None, k_mean=None) == INVALID
    assert _prefill_qa(lib, f, ws_bytes=16) == WS  # otherwise validated as mpfa_prefill


def _decode(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, scale=0.088, splits=2,
             out=f.p, out_dtype=1, lse=None, ws=f.p, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.mpfa_decode(*a.values())


def test_prefill_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP, WS = -1, -2, -3
    assert _prefill(lib, f, D=64) == UNSUP
    assert _prefill(lib, f, q_dtype=5) == UNSUP
    assert _prefill(lib, f, out_dtype=2) == UNSUP
    assert _prefill(lib, f, Hq=3) == INVALID  # Hq % Hkv != 0
    assert _prefill(lib, f, N=0) == INVALID
    assert _prefill(lib, f, B=0) == INVALID
    assert _prefill(lib, f, q=None) == INVALID
    assert _prefill(lib, f, k_fp4=f.mis) == INVALID
    assert _prefill(lib, f, q_mean=None) == INVALID  # smoothing needs the means
    assert _prefill(lib, f, scale=0.0) == INVALID
    assert _prefill(lib, f, scale=float("nan")) == INVALID
    assert _prefill(lib, f, ws_bytes=16) == WS


@pytest.mark.parametrize("name", ["mpfa_prefill_elementwise", "mpfa_prefill_rank_one"])
def test_compensation_placements_reject_bad_arguments(lib, name):
    """The placement variants need a Delta_S; otherwise validated as
    mpfa_prefill (their argument list is its own)."""
    f = _Fake()
    INVALID, WS = -1, -3
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, scale=0.088, causal=1,
             out=f.p, out_dtype=1, lse=None, ws=f.p, ws_bytes=256, stream=None)
    fn = getattr(lib, name)
    assert fn(*dict(a, delta_s=None, q_mean=None, k_mean=None).values()) == INVALID
    assert fn(*dict(a, Hq=3).values()) == INVALID
    assert fn(*dict(a, ws_bytes=16).values()) == WS


def _prefill_tile(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, k_mean=f.p, k_fp4=f.p, k_sf=f.p,
             k_gscale=f.p, v_fp8=f.p, v_scale=f.p, scale=0.088, causal=1, out=f.p, out_dtype=1,
             lse=None, q_tile_mean=f.p, ws=f.p, ws_bytes=256, stream=None)
    a.update(kw)
    return lib.mpfa_prefill_tile_mean(*a.values())


def test_prefill_tile_mean_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP, WS = -1, -2, -3
    assert _prefill_tile(lib, f, D=64) == UNSUP
    assert _prefill_tile(lib, f, q_dtype=5) == UNSUP
    assert _prefill_tile(lib, f, Hq=3) == INVALID
    assert _prefill_tile(lib, f, k_mean=None) == INVALID  # K must be cached centred
    assert _prefill_tile(lib, f, q_tile_mean=None) == INVALID
    assert _prefill_tile(lib, f, q_tile_mean=f.mis) == INVALID
    assert _prefill_tile(lib, f, scale=-1.0) == INVALID
    assert _prefill_tile(lib, f, ws_bytes=16) == WS  # the workspace of mpfa_prefill


def test_decode_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP, WS = -1, -2, -3
    assert _decode(lib, f, Hq=18) == UNSUP  # group of 9 query heads
    assert _decode(lib, f, splits=0) == INVALID
    assert _decode(lib, f, Hq=4, Hkv=3) == INVALID
    assert _decode(lib, f, ws_bytes=256) == WS
    assert _decode(lib, f, out=None) == INVALID
    assert _decode(lib, f, D=256) == UNSUP


def test_quantizers_reject_bad_arguments(lib):
    f = _Fake()
    qk = lib.mpfa_quantize_k_nvfp4
    # (k, k_dtype, B, Hkv, N, D, q, q_dtype, Hq, q_mean, k_mean, k_fp4, k_sf, k_gscale, delta_s, ws, ws_bytes, stream)
    # centring only (k_mean without delta_s) takes no query tensor
    assert qk(f.p, 1, 1, 2, 64, 128, f.p, 1, 4, None, f.p, f.p, f.p, f.p, None, f.p, 1 << 20, None) == -1
    assert qk(f.p, 1, 1, 2, 64, 128, None, 0, 0, None, f.mis, f.p, f.p, f.p, None, f.p, 1 << 20, None) == -1
    assert qk(f.p, 1, 1, 2, 64, 128, None, 0, 4, None, f.p, f.p, f.p, f.p, f.p, f.p, 1 << 20, None) == -1
    assert qk(f.p, 1, 1, 2, 64, 128, None, 0, 3, f.p, f.p, f.p, f.p, f.p, f.p, f.p, 1 << 20, None) == -1
    assert qk(f.p, 3, 1, 2, 64, 128, None, 0, 0, None, None, f.p, f.p, f.p, None, f.p, 1 << 20, None) == -2
    assert qk(f.mis, 1, 1, 2, 64, 128, None, 0, 0, None, None, f.p, f.p, f.p, None, f.p, 1 << 20, None) == -1
    assert qk(f.p, 1, 1, 2, 64, 128, None, 0, 0, None, None, f.p, f.p, f.p, None, f.p, 8, None) == -3
    qa = lib.mpfa_quantize_k_nvfp4_with_q_amax
    # (... delta_s, q_amax, ws, ws_bytes, stream): smoothing with q only, q_amax required
    assert qa(f.p, 1, 1, 2, 64, 128, None, 0, 4, f.p, f.p, f.p, f.p, f.p, f.p, f.p, f.p, 1 << 20, None) == -1
    assert qa(f.p, 1, 1, 2, 64, 128, f.p, 1, 4, f.p, f.p, f.p, f.p, f.p, None, f.p, f.p, 1 << 20, None) == -1
    assert qa(f.p, 1, 1, 2, 64, 128, f.p, 1, 4, f.p, f.p, f.p, f.p, f.p, f.p, None, f.p, 1 << 20, None) == -1
    assert qa(f.p, 1, 1, 2, 64, 128, f.p, 1, 4, f.p, f.p, f.p, f.p, f.p, f.p, f.mis, f.p, 1 << 20, None) == -1
    assert qa(f.p, 1, 1, 2, 64, 128, f.p, 1, 4, f.p, f.p, f.p, f.p, f.p, f.p, f.p, f.p, 8, None) == -3
    qv = lib.mpfa_quantize_v_fp8
    assert qv(f.p, 1, 1, 2, 64, 64, f.p, f.p, f.p, 256, None) == -2
    assert qv(f.p, 1, 1, 2, 64, 128, None, f.p, f.p, 256, None) == -1
    assert qv(f.p, 1, 1, 2, 64, 128, f.p, f.p, f.p, 8, None) == -3


def test_nvfp4_pv_entry_points_reject_bad_arguments(lib):
    f = _Fake()
    qv = lib.mpfa_quantize_v_nvfp4
    # (v, v_dtype, B, Hkv, N, D, v_fp4, v_sf, v_gscale, ws, ws_bytes, stream)
    assert qv(f.p, 1, 1, 2, 64, 64, f.p, f.p, f.p, f.p, 1 << 16, None) == -2
    assert qv(f.p, 3, 1, 2, 64, 128, f.p, f.p, f.p, f.p, 1 << 16, None) == -2
    assert qv(f.p, 1, 1, 2, 64, 128, f.p, None, f.p, f.p, 1 << 16, None) == -1
    assert qv(f.p, 1, 1, 2, 64, 128, f.p, f.mis, f.p, f.p, 1 << 16, None) == -1
    assert qv(f.p, 1, 1, 2, 0, 128, f.p, f.p, f.p, f.p, 1 << 16, None) == -1
    assert qv(f.p, 1, 1, 2, 64, 128, f.p, f.p, f.p, f.p, 8, None) == -3
    pv = lib.mpfa_prefill_pv_nvfp4

    def call(**kw):
        a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p,
                 k_fp4=f.p, k_sf=f.p, k_gscale=f.p, v_fp4=f.p, v_sf=f.p, v_gscale=f.p, delta_s=f.p,
                 scale=0.088, causal=1, out=f.p, out_dtype=1, lse=None, ws=f.p, ws_bytes=256,
                 stream=None)
        a.update(kw)
        return pv(*a.values())
    assert call(v_sf=None) == -1
    assert call(v_gscale=None) == -1
    assert call(v_sf=f.mis) == -1
    assert call(D=64) == -2
    assert call(Hq=3) == -1
    # the workspace must hold the V image too: the plain prefill's size is short
    need = lib.mpfa_workspace_bytes(2, 1, 4, 2, 256, 128, 1)
    assert call(ws_bytes=need) == -3


def _append(lib, f, **kw):
    a = dict(k_new=f.p, v_new=f.p, dtype=1, B=2, Hkv=2, T=1, D=128, N_cap=64, pos=f.p, Hq=4,
             q_mean=f.p, k_mean=f.p, k_gscale=f.p, v_scale=f.p, k_fp4=f.p, k_sf=f.p, v_fp8=f.p,
             delta_s=f.p, stream=None)
    a.update(kw)
    return lib.mpfa_append_kv(*a.values())


def test_append_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP = -1, -2
    assert _append(lib, f, T=0) == INVALID
    assert _append(lib, f, T=65) == INVALID  # more tokens than the cache holds
    assert _append(lib, f, pos=None) == INVALID
    assert _append(lib, f, k_gscale=None) == INVALID
    assert _append(lib, f, k_fp4=f.mis) == INVALID
    assert _append(lib, f, q_mean=None) == INVALID  # smoothing needs both means
    assert _append(lib, f, delta_s=None) == INVALID
    assert _append(lib, f, k_mean=None, q_mean=None) == INVALID  # delta_s without the means
    assert _append(lib, f, Hq=3) == INVALID
    assert _append(lib, f, D=64) == UNSUP
    assert _append(lib, f, dtype=7) == UNSUP
    assert _append(lib, f, Hq=2 * 121) == UNSUP  # a group of 121 query heads


def _append_paged(lib, f, **kw):
    a = dict(k_new=f.p, v_new=f.p, dtype=1, B=2, Hkv=2, D=128, pos=f.p, table=f.p, max_pages=4,
             num_pages=8, page_size=128, Hq=4, q_mean=f.p, k_mean=f.p, k_gscale=f.p, v_scale=f.p,
             k_fp4=f.p, k_sf=f.p, v_fp8=f.p, delta_s=f.p, stream=None)
    a.update(kw)
    return lib.mpfa_append_kv_paged(*a.values())


def test_paged_append_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP = -1, -2
    assert _append_paged(lib, f, page_size=64) == UNSUP
    assert _append_paged(lib, f, max_pages=0) == INVALID
    assert _append_paged(lib, f, num_pages=0) == INVALID
    assert _append_paged(lib, f, max_pages=1 << 24) == INVALID  # 128 max_pages overflows int32
    assert _append_paged(lib, f, table=None) == INVALID
    assert _append_paged(lib, f, pos=None) == INVALID
    assert _append_paged(lib, f, k_sf=f.mis) == INVALID
    assert _append_paged(lib, f, delta_s=None) == INVALID
    assert _append_paged(lib, f, k_mean=None, q_mean=None) == INVALID
    assert _append_paged(lib, f, Hq=3) == INVALID
    assert _append_paged(lib, f, D=64) == UNSUP


def _decode_paged(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=2, Hq=8, Hkv=2, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, table=f.p, lens=f.p,
             max_pages=4, num_pages=8, page_size=128, scale=0.1, splits=4, out=f.p, out_dtype=1,
             lse=None, ws=f.p, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.mpfa_decode_paged(*a.values())


def test_paged_decode_rejects_bad_arguments(lib):
    f = _Fake()
    INVALID, UNSUP, WS = -1, -2, -3
    assert _decode_paged(lib, f, page_size=256) == UNSUP
    assert _decode_paged(lib, f, Hq=18) == UNSUP
    assert _decode_paged(lib, f, splits=0) == INVALID
    assert _decode_paged(lib, f, max_pages=0) == INVALID
    assert _decode_paged(lib, f, num_pages=0) == INVALID
    assert _decode_paged(lib, f, max_pages=(1 << 24) - 1, splits=1 << 20) == INVALID
    assert _decode_paged(lib, f, table=None) == INVALID
    assert _decode_paged(lib, f, lens=None) == INVALID
    assert _decode_paged(lib, f, k_gscale=None) == INVALID
    assert _decode_paged(lib, f, q_mean=None) == INVALID
    assert _decode_paged(lib, f, ws_bytes=256) == WS
    assert _decode_paged(lib, f, scale=0.0) == INVALID
    assert _decode_paged(lib, f, D=64) == UNSUP


def _decode_static(lib, f, **kw):
    a = dict(q=f.p, q_dtype=1, B=1, Hq=4, Hkv=2, N=256, D=128, q_mean=f.p, k_mean=f.p, k_fp4=f.p,
             k_sf=f.p, k_gscale=f.p, v_fp8=f.p, v_scale=f.p, delta_s=f.p, scale=0.088, splits=2,
             out=f.p, out_dtype=1, lse=None, stream=None)
    a.update(kw)
    return lib.mpfa_decode_static(*a.values())


def test_decode_static_rejects_bad_arguments_and_sizes_past_its_array(lib):
    """Validation runs before the scratch array is looked up: these calls fail
    on the host (nothing is enqueued, no GPU is touched)."""
    f = _Fake()
    INVALID, UNSUP, WS = -1, -2, -3
    assert _decode_static(lib, f, Hq=18) == UNSUP
    assert _decode_static(lib, f, splits=0) == INVALID
    assert _decode_static(lib, f, out=None) == INVALID
    assert _decode_static(lib, f, k_fp4=f.mis) == INVALID
    cap = header_define("MPFA_DECODE_STATIC_SCRATCH_BYTES")
    ws = lib.mpfa_workspace_bytes
    # the largest batch whose workspace fits, and one past it
    B = 1
    while ws(3, B + 1, 32, 8, 1024, 128, 32) <= cap:
        B += 1
    assert ws(3, B, 32, 8, 1024, 128, 32) <= cap < ws(3, B + 1, 32, 8, 1024, 128, 32)
    assert _decode_static(lib, f, B=B + 1, Hq=32, Hkv=8, splits=32) == WS
    assert B >= 16  # the 128K decode workload (batch 16, 32 query heads, 32 splits) fits
