"""Pins of the oracle's paged-cache decode and cache write (MpFA §5.3 and §6
"Serving system": fixed-size pages, the Delta_S side cache indexed by the
same physical pages, a constant number of KV partitions).

* A pool whose pages are a permutation of a contiguous cache's 128-token
  blocks decodes exactly like the contiguous cache (same bytes, same scales,
  same call-level Q quantization).
* With ragged per-request lengths, the lossless special case (every
  quantizer exact, lam * S integral) equals FP64 exact attention over each
  request's own keys, for several partition counts.
* Writing the tokens one at a time into pages with the statistics the bulk
  first stage froze reproduces the bulk cache's bytes in every page.
* A request with no positions returns O = 0 and LSE = -inf; a length past
  the block table's capacity is clamped to it.
"""
import math

import numpy as np
import pytest

import oracle

from test_oracle_attention import LOSSLESS_SCALE, _lossless_inputs

F32 = np.float32
PAGE = oracle.PAGE


def _inputs(seed, B=3, Hq=8, Hkv=2, N=300, D=128):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, 1, D), dtype=F32)
    k = r.standard_normal((B, Hkv, N, D), dtype=F32)
    k[:, :, :, 7] += 2.5
    v = r.standard_normal((B, Hkv, N, D), dtype=F32)
    qm = (r.standard_normal((B, Hq, D)) / math.sqrt(N)).astype(F32)
    return q, k, v, qm


def _to_pool(cache, B, rng, extra=3):
    """Scatter a contiguous cache [B, H, N, ...] into a shuffled page pool.
    Returns (pool, block_table); unused pages hold random bytes."""
    N = cache["k_fp4"].shape[2]
    npg = -(-N // PAGE)
    perm = rng.permutation(B * npg + extra)
    table = perm[:B * npg].reshape(B, npg).astype(np.int32)
    P = B * npg + extra
    pool = {}
    for name in ("k_fp4", "k_sf", "v_fp8", "delta_s"):
        if cache.get(name) is None:
            continue
        a = np.asarray(cache[name])
        shape = (P, a.shape[1], PAGE) + a.shape[3:]
        out = rng.integers(0, 256, size=shape).astype(a.dtype)
        for b in range(B):
            for i in range(npg):
                blk = a[b, :, i * PAGE:(i + 1) * PAGE]
                out[table[b, i], :, :blk.shape[1]] = blk
        pool[name] = out
    return pool, table


@pytest.mark.parametrize("smooth", [True, False])
def test_shuffled_pages_decode_like_the_contiguous_cache(smooth):
    q, k, v, qm = _inputs(1)
    B, Hq, _, D = q.shape
    N = k.shape[2]
    kq = oracle.quantize_k(k, q_mean=qm) if smooth else oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    cache = {"k_fp4": kq["k_fp4"], "k_sf": kq["k_sf"], "v_fp8": vq["v_fp8"],
             "delta_s": kq.get("delta_s") if smooth else None,
             "k_gscale": kq["k_gscale"], "v_scale": vq["v_scale"]}
    rng = np.random.default_rng(5)
    pool, table = _to_pool(cache, B, rng)
    pool["k_gscale"] = np.full(B, kq["k_gscale"], F32)
    pool["v_scale"] = np.full(B, vq["v_scale"], F32)
    km = kq.get("k_mean") if smooth else None
    for splits in (1, 3, 8):
        O, L = oracle.decode_paged(q, pool, table, np.full(B, N), qm if smooth else None, km, splits,
                                   1 / math.sqrt(D))
        ops = oracle.Operands.from_cache(q, cache, N, q_mean=qm if smooth else None, k_mean=km)
        Oc, Lc = oracle.decode(q, None, None, qm if smooth else None, splits, 1 / math.sqrt(D),
                               smooth=smooth, ops=ops)
        np.testing.assert_array_equal(O, Oc)
        np.testing.assert_array_equal(L, Lc)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_ragged_lengths_lossless_equal_exact_attention(splits):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, Nmax = 4, 4, 2, 520
    q, k, v = _lossless_inputs(rng, B, Hq, Hkv, Nmax, nq=1)
    lens = np.array([1, 200, 385, 520])
    kq = oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    cache = {"k_fp4": kq["k_fp4"], "k_sf": kq["k_sf"], "v_fp8": vq["v_fp8"]}
    pool, table = _to_pool(cache, B, rng)
    pool["k_gscale"] = np.full(B, kq["k_gscale"], F32)
    pool["v_scale"] = np.full(B, vq["v_scale"], F32)
    O, L = oracle.decode_paged(q, pool, table, lens, None, None, splits, LOSSLESS_SCALE, out_f64=True)
    for b in range(B):
        n = lens[b]
        Oe, Le = oracle.exact_attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], LOSSLESS_SCALE,
                                        causal=False)
        assert np.abs(O[b] - Oe.reshape(Hq, 128)).max() < 1e-12 * max(1.0, np.abs(Oe).max())
        assert np.abs(L[b] - Le.ravel()).max() < 1e-12


@pytest.mark.parametrize("smooth", [True, False])
def test_token_by_token_page_writes_reproduce_the_bulk_cache(smooth):
    q, k, v, qm = _inputs(2, B=2, Hq=4, Hkv=2, N=260)
    B, Hq = q.shape[:2]
    Hkv, N = k.shape[1], k.shape[2]
    kq = oracle.quantize_k(k, q_mean=qm) if smooth else oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    npg = -(-N // PAGE)
    rng = np.random.default_rng(9)
    table = rng.permutation(B * npg).reshape(B, npg).astype(np.int32)
    P = B * npg
    pool = {"k_fp4": np.zeros((P, Hkv, PAGE, 64), np.uint8), "k_sf": np.zeros((P, Hkv, PAGE, 8), np.uint8),
            "v_fp8": np.zeros((P, Hkv, PAGE, 128), np.uint8),
            "k_gscale": np.full(B, kq["k_gscale"], F32), "v_scale": np.full(B, vq["v_scale"], F32)}
    if smooth:
        pool["delta_s"] = np.zeros((P, Hq, PAGE), np.uint16)
    km = kq["k_mean"] if smooth else None
    for t in range(N):
        pool = oracle.append_kv_paged(k[:, :, t:t + 1], v[:, :, t:t + 1], np.full(B, t), pool, table,
                                      q_mean=qm if smooth else None, k_mean=km)
    names = ("k_fp4", "k_sf", "v_fp8") + (("delta_s",) if smooth else ())
    bulk = {"k_fp4": kq["k_fp4"], "k_sf": kq["k_sf"], "v_fp8": vq["v_fp8"],
            "delta_s": kq.get("delta_s")}
    for b in range(B):
        g = oracle.gather_pages(pool, table, b, N)
        for name in names:
            np.testing.assert_array_equal(g[name][0], bulk[name][b], err_msg=name)
    # positions outside the table (and pages outside the pool) write nothing
    before = {n: pool[n].copy() for n in names}
    bad = np.array([-1, npg * PAGE])
    pool2 = oracle.append_kv_paged(k[:, :, :1] * 0 + 5, v[:, :, :1] * 0 + 5, bad, pool, table,
                                   q_mean=qm if smooth else None, k_mean=km)
    table_bad = table.copy()
    table_bad[:, 0] = P + 4
    pool3 = oracle.append_kv_paged(k[:, :, :1] * 0 + 5, v[:, :, :1] * 0 + 5, np.zeros(B), pool, table_bad,
                                   q_mean=qm if smooth else None, k_mean=km)
    for n in names:
        np.testing.assert_array_equal(pool2[n], before[n])
        np.testing.assert_array_equal(pool3[n], before[n])


def test_empty_and_over_long_requests():
    q, k, v, qm = _inputs(3, B=3, Hq=4, Hkv=2, N=256)
    kq = oracle.quantize_k(k, smooth=False)
    vq = oracle.quantize_v(v)
    cache = {"k_fp4": kq["k_fp4"], "k_sf": kq["k_sf"], "v_fp8": vq["v_fp8"]}
    rng = np.random.default_rng(4)
    pool, table = _to_pool(cache, 3, rng)
    pool["k_gscale"] = np.full(3, kq["k_gscale"], F32)
    pool["v_scale"] = np.full(3, vq["v_scale"], F32)
    O, L = oracle.decode_paged(q, pool, table, np.array([0, 256, 100000]), None, None, 2, 0.1)
    assert np.all(O[0] == 0) and np.all(L[0] == -np.inf)
    np.testing.assert_array_equal(O[2], oracle.decode_paged(q, pool, table, np.array([0, 256, 256]),
                                                            None, None, 2, 0.1)[0][2])
    assert np.all(np.isfinite(O[1:])) and np.all(np.isfinite(L[1:]))
