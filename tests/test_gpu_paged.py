"""GPU parity of the paged-cache decode and cache write (mpfa_decode_paged,
mpfa_append_kv_paged) against the oracle's decode_paged / append_kv_paged,
through the C ABI.  Pools are shuffled pages; unused pages and the slots past
each request's length hold random bytes (FP8 NaN codes included), which the
kernels must never let into a result."""
import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_bytes_equal, assert_close, dev, host, say, sweep_count

pytestmark = pytest.mark.gpu
PAGE = 128


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _empty_pool(B, Hq, Hkv, num_pages, smooth, seed, fill="random"):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)

    def u8(*shape):
        if fill == "zeros":
            return torch.zeros(shape, dtype=torch.uint8, device="cuda")
        return torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)

    pool = {"k_fp4": u8(num_pages, Hkv, PAGE, 64), "k_sf": u8(num_pages, Hkv, PAGE, 8),
            "v_fp8": u8(num_pages, Hkv, 4, 2, 128, 16)}
    if smooth:
        pool["delta_s"] = u8(num_pages, Hq, PAGE, 2).view(torch.int16).reshape(num_pages, Hq, PAGE)
    return pool


def _fill_request(pool, b, table, kq, vq, n):
    """Scatter request b's contiguous caches (batch size 1, length n) into its pages."""
    for i in range(-(-n // PAGE)):
        pg = int(table[b, i])
        lo, hi = i * PAGE, min((i + 1) * PAGE, n)
        pool["k_fp4"][pg, :, :hi - lo] = kq["k_fp4"][0, :, lo:hi]
        pool["k_sf"][pg, :, :hi - lo] = kq["k_sf"][0, :, lo:hi]
        nt = -(-(hi - lo) // 32)
        pool["v_fp8"][pg, :, :nt] = vq["v_fp8"][0, :, 4 * i:4 * i + nt]
        if "delta_s" in pool:
            pool["delta_s"][pg, :, :hi - lo] = kq["delta_s"][0, :, lo:hi]


def _host_pool(mpfa, pool, B):
    h = {"k_fp4": host(pool["k_fp4"]), "k_sf": host(pool["k_sf"]),
         "v_fp8": mpfa.v_tiles_to_rows(host(pool["v_fp8"]), PAGE),
         "k_gscale": host(pool["k_gscale"]), "v_scale": host(pool["v_scale"])}
    if "delta_s" in pool:
        h["delta_s"] = host(pool["delta_s"])
    return h


def _ragged_setup(mpfa, smooth, lens, B, Hq, Hkv, max_pages, seed, extra_pages=3, cap_data=None):
    """Per-request first stage on random data (each request its own scales and
    means), scattered into a shuffled pool.  Returns (pool, table, q, qm_host)."""
    import torch
    from mixed_precision_flashattention_amd import synth
    rng = np.random.default_rng(seed)
    npgs = [-(-(cap_data or max(n, 0)) // PAGE) for n in lens]
    used = sum(npgs)
    num_pages = used + extra_pages
    perm = rng.permutation(num_pages)
    free = perm[used:]  # pages no request's data is in
    table = np.zeros((B, max_pages), np.int32)
    k = 0
    for b, npg in enumerate(npgs):
        table[b, :npg] = perm[k:k + npg]
        table[b, npg:] = free[rng.integers(0, len(free), max_pages - npg)]
        k += npg
    pool = _empty_pool(B, Hq, Hkv, num_pages, smooth, seed)
    kg, vs, qms, kms = [], [], [], []
    for b, n in enumerate(lens):
        n_data = cap_data or n
        if n_data <= 0:
            kg.append(torch.ones(1, device="cuda"))
            vs.append(torch.ones(1, device="cuda"))
            qms.append(torch.zeros((1, Hq, 128), device="cuda"))
            kms.append(torch.zeros((1, Hkv, 128), device="cuda"))
            continue
        cfg = synth.config("llama8b_decode_128k", B=1, Hq=Hq, Hkv=Hkv, N=n_data, num_splits=2)
        kk = dev(synth.full(cfg, "k") * (1.0 + 0.5 * b), torch.bfloat16)
        vv = dev(synth.full(cfg, "v") * (1.0 + 0.25 * b), torch.bfloat16)
        qm = dev(synth.q_mean(cfg))
        kq = mpfa.quantize_k(kk, q_mean=qm) if smooth else mpfa.quantize_k(kk, smooth=False)
        vq = mpfa.quantize_v(vv)
        _fill_request(pool, b, table, kq, vq, n_data)
        kg.append(kq["k_gscale"].reshape(1))
        vs.append(vq["v_scale"].reshape(1))
        qms.append(kq["q_mean"] if smooth else torch.zeros((1, Hq, 128), device="cuda"))
        kms.append(kq["k_mean"] if smooth else torch.zeros((1, Hkv, 128), device="cuda"))
    pool["k_gscale"] = torch.cat(kg).contiguous()
    pool["v_scale"] = torch.cat(vs).contiguous()
    if smooth:
        pool["q_mean"] = torch.cat(qms).contiguous()
        pool["k_mean"] = torch.cat(kms).contiguous()
    q = rng.standard_normal((B, Hq, 1, 128)).astype(np.float32)
    q = host(dev(q, torch.bfloat16))
    return pool, table, q


def _oracle_paged(mpfa, oracle_mod, pool, table, q, lens, splits, scale, heads=None):
    smooth = "delta_s" in pool
    return oracle_mod.decode_paged(q, _host_pool(mpfa, pool, len(lens)), table, np.asarray(lens),
                                   host(pool["q_mean"]) if smooth else None,
                                   host(pool["k_mean"]) if smooth else None, splits, scale,
                                   heads=heads)


@pytest.mark.parametrize("smooth", [True, False])
def test_paged_decode_ragged_lengths(mpfa, oracle_mod, smooth):
    import torch
    B, Hq, Hkv, splits = 4, 8, 2, 3
    lens = [1, 130, 300, 517]
    say(f"case: paged decode B{B} Hq{Hq}/Hkv{Hkv} lengths {lens} splits {splits} smooth={smooth}")
    pool, table, q = _ragged_setup(mpfa, smooth, lens, B, Hq, Hkv, 5, seed=31)
    out, lse = mpfa.decode_paged(dev(q, torch.bfloat16), pool, dev(table), dev(np.array(lens, np.int32)),
                                 0.0883883, splits, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    O, L = _oracle_paged(mpfa, oracle_mod, pool, table, q, lens, splits, 0.0883883)
    assert_close("out", host(out).reshape(-1, 128), O.reshape(-1, 128))
    assert_close("lse", host(lse).ravel(), L.ravel(), atol=LSE_ATOL, rtol=0.0)


@pytest.mark.parametrize("smooth", [True, False])
def test_paged_decode_bitwise_equals_contiguous(mpfa, smooth):
    """The same caches laid out as shuffled pages give the same bits as the
    contiguous decode (only the addressing differs)."""
    import torch
    from mixed_precision_flashattention_amd import synth
    B, Hq, Hkv, N, splits = 2, 8, 2, 300, 3
    say(f"case: paged vs contiguous B{B} N{N} smooth={smooth}")
    cfg = synth.config("llama8b_decode_128k", B=B, Hq=Hq, Hkv=Hkv, N=N, num_splits=splits)
    k, v = dev(synth.full(cfg, "k"), torch.bfloat16), dev(synth.full(cfg, "v"), torch.bfloat16)
    q = dev(synth.full(cfg, "q"), torch.bfloat16)
    kq = mpfa.quantize_k(k, q_mean=dev(synth.q_mean(cfg))) if smooth else mpfa.quantize_k(k, smooth=False)
    vq = mpfa.quantize_v(v)
    out_c, lse_c = mpfa.decode(q, kq, vq, cfg.scale, splits, out_dtype=torch.float32, with_lse=True)
    npg = -(-N // PAGE)
    rng = np.random.default_rng(3)
    num_pages = B * npg + 2
    perm = rng.permutation(num_pages)
    table = perm[:B * npg].reshape(B, npg).astype(np.int32)
    pool = _empty_pool(B, Hq, Hkv, num_pages, smooth, seed=4)
    for b in range(B):
        one_k = {n: t[b:b + 1] for n, t in kq.items() if n in ("k_fp4", "k_sf", "delta_s")}
        _fill_request(pool, b, table, one_k, {"v_fp8": vq["v_fp8"][b:b + 1]}, N)
    pool["k_gscale"] = kq["k_gscale"].reshape(1).repeat(B).contiguous()
    pool["v_scale"] = vq["v_scale"].reshape(1).repeat(B).contiguous()
    if smooth:
        pool["q_mean"], pool["k_mean"] = kq["q_mean"], kq["k_mean"]
    out_p, lse_p = mpfa.decode_paged(q, pool, dev(table), dev(np.full(B, N, np.int32)), cfg.scale, splits,
                                     out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    assert_bytes_equal("out bits", host(out_p).view(np.uint32), host(out_c).view(np.uint32))
    assert_bytes_equal("lse bits", host(lse_p).view(np.uint32), host(lse_c).view(np.uint32))


@pytest.mark.parametrize("smooth", [True, False])
def test_paged_append_then_decode(mpfa, oracle_mod, smooth):
    import torch
    B, Hq, Hkv, splits = 3, 8, 2, 2
    prefix = [5, 127, 256]  # the new tokens land mid-page, at a page's end and on a fresh page
    say(f"case: paged append at {prefix} then decode, smooth={smooth}")
    pool, table, q = _ragged_setup(mpfa, smooth, prefix, B, Hq, Hkv, 3, seed=41)
    # request 2's token opens its third page, which the table points at a free page
    before = _host_pool(mpfa, pool, B)
    r = np.random.default_rng(5)
    kn = host(dev(r.standard_normal((B, Hkv, 1, 128)).astype(np.float32) * 1.5, torch.bfloat16))
    vn = host(dev(r.standard_normal((B, Hkv, 1, 128)).astype(np.float32), torch.bfloat16))
    pos = np.array(prefix, np.int32)
    mpfa.append_kv_paged(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), dev(pos), pool, dev(table))
    torch.cuda.synchronize()
    ref = oracle_mod.append_kv_paged(kn, vn, pos, before, table,
                                     q_mean=host(pool["q_mean"]) if smooth else None,
                                     k_mean=host(pool["k_mean"]) if smooth else None)
    got = _host_pool(mpfa, pool, B)
    for n in ("k_fp4", "k_sf", "v_fp8") + (("delta_s",) if smooth else ()):
        assert_bytes_equal(n, got[n], ref[n])
    lens = [p + 1 for p in prefix]
    out, lse = mpfa.decode_paged(dev(q, torch.bfloat16), pool, dev(table), dev(np.array(lens, np.int32)),
                                 0.0883883, splits, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    O, L = _oracle_paged(mpfa, oracle_mod, pool, table, q, lens, splits, 0.0883883)
    assert_close("out", host(out).reshape(-1, 128), O.reshape(-1, 128))
    assert_close("lse", host(lse).ravel(), L.ravel(), atol=LSE_ATOL, rtol=0.0)
    # positions outside the table and page indices outside the pool write nothing
    snap = {n: t.clone() for n, t in pool.items() if n in ("k_fp4", "k_sf", "v_fp8", "delta_s")}
    bad_table = table.copy()
    bad_table[:, 0] = pool["k_fp4"].shape[0] + 7
    mpfa.append_kv_paged(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16),
                         dev(np.array([-1, 3 * PAGE, 0], np.int32)), pool, dev(table))
    mpfa.append_kv_paged(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), dev(np.zeros(B, np.int32)),
                         pool, dev(bad_table))
    torch.cuda.synchronize()
    # only request 2's in-range write (position 0: page table[2, 0]) may change anything
    for n, t in snap.items():
        a, b0 = host(pool[n]), host(t)
        changed = set(np.nonzero((a != b0).reshape(a.shape[0], -1).any(axis=1))[0])
        assert changed <= {int(table[2, 0])}, (n, changed)


def test_paged_decode_empty_and_over_long_requests(mpfa, oracle_mod):
    import torch
    B, Hq, Hkv, splits, max_pages = 3, 4, 1, 2, 3
    say("case: paged decode with lengths 0, 200 and past the table's capacity")
    pool, table, q = _ragged_setup(mpfa, True, [0, 200, 10 ** 6], B, Hq, Hkv, max_pages, seed=51,
                                   cap_data=max_pages * PAGE)
    lens = np.array([0, 200, 10 ** 6], np.int32)
    out, lse = mpfa.decode_paged(dev(q, torch.bfloat16), pool, dev(table), dev(lens), 0.1, splits,
                                 out_dtype=torch.float32, with_lse=True)
    out_cap, lse_cap = mpfa.decode_paged(dev(q, torch.bfloat16), pool, dev(table),
                                         dev(np.array([0, 200, max_pages * PAGE], np.int32)), 0.1, splits,
                                         out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    o, l = host(out), host(lse)
    assert np.all(o[0] == 0.0) and np.all(l[0] == -np.inf)
    assert_bytes_equal("clamped length", o[2].view(np.uint32), host(out_cap)[2].view(np.uint32))
    O, L = _oracle_paged(mpfa, oracle_mod, pool, table, q, lens, splits, 0.1)
    assert_close("out", o[1:].reshape(-1, 128), O[1:].reshape(-1, 128))
    assert_close("lse", l[1:].ravel(), L[1:].ravel(), atol=LSE_ATOL, rtol=0.0)


# ---- seeded random pools: request count, heads, GQA factor, ragged and empty
# lengths, partitions and spare table slots drawn from a fixed seed ----
def _paged_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))
        lens = [int(x) for x in rng.integers(0, 1500, B)]
        if rng.integers(0, 3) == 0:
            lens[int(rng.integers(0, B))] = 0
        cases.append(dict(B=B, Hkv=hkv, Hq=hkv * g, lens=lens, splits=int(rng.choice([1, 2, 3, 8, 32])),
                          smooth=bool(rng.integers(0, 2)), extra=int(rng.integers(0, 3)), seed=500 + i))
    return cases


@pytest.mark.parametrize("case", _paged_cases(20261205, sweep_count(8)), ids=lambda c: (
    f"B{c['B']}-H{c['Hq']}x{c['Hkv']}-splits{c['splits']}-{'smooth' if c['smooth'] else 'direct'}"))
def test_paged_decode_random_pools(mpfa, oracle_mod, case):
    import torch
    B, Hq, Hkv, lens, splits = case["B"], case["Hq"], case["Hkv"], case["lens"], case["splits"]
    max_pages = max(-(-max(lens) // PAGE), 1) + case["extra"]
    say(f"case: paged decode B{B} Hq{Hq}/Hkv{Hkv} lengths {lens} splits {splits} "
        f"smooth={case['smooth']} table width {max_pages}")
    pool, table, q = _ragged_setup(mpfa, case["smooth"], lens, B, Hq, Hkv, max_pages, seed=case["seed"])
    out, lse = mpfa.decode_paged(dev(q, torch.bfloat16), pool, dev(table), dev(np.array(lens, np.int32)),
                                 0.0883883, splits, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    O, L = _oracle_paged(mpfa, oracle_mod, pool, table, q, lens, splits, 0.0883883)
    assert_close("out", host(out).reshape(-1, 128), O.reshape(-1, 128))
    got, ref = host(lse).ravel(), L.ravel()
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), "empty requests give LSE = -inf, the others a finite one"
    if finite.any():
        assert_close("lse", got[finite], ref[finite], atol=LSE_ATOL, rtol=0.0)
