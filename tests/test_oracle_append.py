"""Pins of the oracle's decode-time cache write (MpFA §6 "Online quantization":
the new token is centred against the frozen per-request means and written
with the cache's frozen scales, its compensation entries in the same pass).

* Appending a sequence chunk by chunk, in any order, with the statistics the
  bulk first stage froze reproduces the bulk caches byte for byte: quantization
  is per token row once the means and the per-tensor scales are fixed.
* Values beyond the frozen range saturate to the largest codes.
* A decode built from the caches equals the decode of the raw inputs.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


def _inputs(seed, B=2, Hq=4, Hkv=2, N=150, D=128):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, N, D), dtype=F32)
    k = r.standard_normal((B, Hkv, N, D), dtype=F32)
    k[:, :, :, 5] += 3.0  # a channel ridge, so the means matter
    v = r.standard_normal((B, Hkv, N, D), dtype=F32)
    return q, k, v


def _empty_cache(B, Hq, Hkv, N, D, kq, vq, smooth):
    cache = {"k_fp4": np.zeros((B, Hkv, N, D // 2), np.uint8),
             "k_sf": np.zeros((B, Hkv, N, D // 16), np.uint8),
             "k_gscale": kq["k_gscale"],
             "v_fp8": np.zeros((B, Hkv, N, D), np.uint8),
             "v_scale": vq["v_scale"]}
    if smooth:
        cache["delta_s"] = np.zeros((B, Hq, N), np.uint16)
    return cache


@pytest.mark.parametrize("smooth", [True, False])
def test_chunked_append_equals_bulk_quantization(smooth):
    q, k, v = _inputs(1)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    kq = oracle.quantize_k(k, q=q) if smooth else oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    cache = _empty_cache(B, Hq, Hkv, N, D, kq, vq, smooth)
    # chunks of one common length T per call, batch entries at different
    # positions: entry 0 walks forward, entry 1 backward
    T = 10
    starts = list(range(0, N, T))
    for i in range(len(starts)):
        pos = np.array([starts[i], starts[len(starts) - 1 - i]])
        kn = np.stack([k[b, :, pos[b]:pos[b] + T] for b in range(B)])
        vn = np.stack([v[b, :, pos[b]:pos[b] + T] for b in range(B)])
        cache = oracle.append_kv(kn, vn, pos, cache,
                                 q_mean=kq["q_mean"] if smooth else None,
                                 k_mean=kq["k_mean"] if smooth else None)
    for name in ("k_fp4", "k_sf"):
        np.testing.assert_array_equal(cache[name], kq[name])
    np.testing.assert_array_equal(cache["v_fp8"], vq["v_fp8"])
    if smooth:
        np.testing.assert_array_equal(cache["delta_s"], kq["delta_s"])


def test_append_saturates_beyond_the_frozen_range():
    q, k, v = _inputs(2, B=1, Hq=2, Hkv=1, N=64)
    kq = oracle.quantize_k(k, q=q)
    vq = oracle.quantize_v(v)
    cache = _empty_cache(1, 2, 1, 65, 128, kq, vq, True)
    big = np.full((1, 1, 1, 128), 1e4, dtype=F32)
    big[..., 1::2] *= -1
    out = oracle.append_kv(big, big, np.array([64]), cache, q_mean=kq["q_mean"], k_mean=kq["k_mean"])
    codes = out["k_fp4"][0, 0, 64]
    lo, hi = codes & 0xF, codes >> 4
    # element 2t (low nibble) positive, 2t+1 negative; all at the largest magnitude (code 7)
    assert np.all(lo == 0x7) and np.all(hi == 0xF)
    assert np.all(out["k_sf"][0, 0, 64] == 0x7E)  # block scale saturates at 448
    row = out["v_fp8"][0, 0, 64]
    assert np.all(row[0::2] == 0x7E) and np.all(row[1::2] == 0xFE)
    # rows that were not appended are untouched
    np.testing.assert_array_equal(out["k_fp4"][0, 0, :64], 0)


@pytest.mark.parametrize("smooth", [True, False])
def test_decode_from_cache_equals_decode_of_raw_inputs(smooth):
    q, k, v = _inputs(3, B=2, Hq=4, Hkv=2, N=300)
    qd = q[:, :, :1]
    r = np.random.default_rng(7)
    qm = (r.standard_normal((2, 4, 128)) / np.sqrt(300)).astype(F32)
    O, L = oracle.decode(qd, k, v, qm if smooth else None, 3, 1 / np.sqrt(128), smooth=smooth)
    kq = oracle.quantize_k(k, q_mean=qm) if smooth else oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    cache = {**{n: kq[n] for n in ("k_fp4", "k_sf", "k_gscale")}, **vq}
    if smooth:
        cache["delta_s"] = kq["delta_s"]
    ops = oracle.Operands.from_cache(qd, cache, 300, q_mean=qm, k_mean=kq.get("k_mean"))
    O2, L2 = oracle.decode(qd, None, None, qm if smooth else None, 3, 1 / np.sqrt(128),
                           smooth=smooth, ops=ops)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
