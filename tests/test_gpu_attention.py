"""GPU parity of QK4PV8 prefill and split-KV decode against the oracle, element
by element: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| on the FP32 output, LSE
within 2e-3.  Sizes span several tiles and ragged tails."""
import numpy as np
import pytest

from gpu_util import LSE_ATOL, assert_close, dev, host, say, sweep_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpfa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_flashattention_amd as m
    m.load_library()
    return m


def _run_prefill(mpfa, q, k, v, scale, causal, smooth, in_dtype, out_dtype, with_lse=True):
    import torch
    qd, kd, vd = dev(q, in_dtype), dev(k, in_dtype), dev(v, in_dtype)
    if smooth:
        kq = mpfa.quantize_k(kd, q=qd)
    else:
        kq = mpfa.quantize_k(kd, smooth=False)
    vq = mpfa.quantize_v(vd)
    out, lse = mpfa.prefill(qd, kq, vq, scale, causal=causal, out_dtype=out_dtype, with_lse=with_lse)
    torch.cuda.synchronize()
    return host(out), (host(lse) if with_lse else None)


def _check_prefill(mpfa, oracle_mod, cfg, causal=True, smooth=True, out_bf16=False, edit=None):
    """Prefill of the configuration's inputs (``edit`` may replace q, k, v)
    against the oracle, every row."""
    import torch
    from mixed_precision_flashattention_amd import synth
    in_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    q, k, v = (synth.full(cfg, t) for t in ("q", "k", "v"))
    if edit is not None:
        q, k, v = edit(q, k, v)
    say(f"case: prefill B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} {cfg.dtype} causal={causal} "
        f"smooth={smooth} out={'bf16' if out_bf16 else 'f32'}"
        f"{' edited inputs' if edit is not None else ''}")
    out, lse = _run_prefill(mpfa, q, k, v, cfg.scale, causal, smooth, in_dtype, out_dtype)
    O, LSE, rows, AMB = oracle_mod.prefill_rows(q, k, v, cfg.scale, causal=causal, smooth=smooth,
                                                ambiguity=True)
    # bf16 output adds one rounding (relative 2^-9) on top of the tolerance
    extra = 2.0 ** -8 if out_bf16 else 0.0
    assert_close("out", out.reshape(-1, 128), O, rtol=1e-2 + extra, slack=AMB)
    assert_close("lse", lse.reshape(-1), LSE, atol=LSE_ATOL, rtol=0.0)
    return out, O


def test_prefill_small_config_full_smooth(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("prefill_1k_2x1"))


def test_prefill_small_config_full_direct(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("prefill_1k_2x1"), smooth=False)


@pytest.mark.parametrize("N", [1, 127, 129, 300])
def test_prefill_gqa2_bf16_ragged(mpfa, oracle_mod, N):
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=2, Hq=4, Hkv=2, N=N),
                   out_bf16=True)


def test_prefill_gqa5_spikes(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("qwen14b_prefill_32k", B=1, Hq=10, Hkv=2, N=520))


@pytest.mark.parametrize("smooth", [True, False])
def test_prefill_non_causal(mpfa, oracle_mod, smooth):
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=2, Hkv=1, N=333),
                   causal=False, smooth=smooth)


def _check_decode(mpfa, oracle_mod, cfg, smooth=True, with_lse=True, edit=None):
    """Split-KV decode of the configuration's inputs (``edit`` may replace
    q, k, v) against the oracle, every (batch, head)."""
    import torch
    from mixed_precision_flashattention_amd import synth
    q, k, v = synth.full(cfg, "q"), synth.full(cfg, "k"), synth.full(cfg, "v")
    if edit is not None:
        q, k, v = edit(q, k, v)
    qm = synth.q_mean(cfg)
    say(f"case: decode B{cfg.B} Hq{cfg.Hq}/Hkv{cfg.Hkv} N{cfg.N} splits{cfg.num_splits} smooth={smooth}"
        f"{' edited inputs' if edit is not None else ''}")
    kd = dev(k, torch.bfloat16)
    kq = mpfa.quantize_k(kd, q_mean=dev(qm)) if smooth else mpfa.quantize_k(kd, smooth=False)
    vq = mpfa.quantize_v(dev(v, torch.bfloat16))
    out, lse = mpfa.decode(dev(q, torch.bfloat16), kq, vq, cfg.scale, cfg.num_splits,
                           out_dtype=torch.float32, with_lse=with_lse)
    torch.cuda.synchronize()
    O, LSE = oracle_mod.decode(q, k, v, qm if smooth else None, cfg.num_splits, cfg.scale, smooth=smooth)
    assert_close("out", host(out).reshape(-1, 128), O.reshape(-1, 128))
    if with_lse:
        assert_close("lse", host(lse).reshape(-1), LSE.reshape(-1), atol=LSE_ATOL, rtol=0.0)
    return host(out), O


@pytest.mark.parametrize("N,splits", [(1000, 3), (4096, 8), (1, 4), (300, 32), (129, 1)])
def test_decode_gqa4(mpfa, oracle_mod, N, splits):
    from mixed_precision_flashattention_amd import synth
    _check_decode(mpfa, oracle_mod,
                  synth.config("llama8b_decode_128k", B=2, Hq=8, Hkv=2, N=N, num_splits=splits))


def test_decode_gqa5_direct(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_decode(mpfa, oracle_mod,
                  synth.config("llama8b_decode_128k", B=1, Hq=10, Hkv=2, N=2000, num_splits=5),
                  smooth=False)


@pytest.mark.parametrize("smooth", [True, False])
def test_prefill_mha_xcd_mapping(mpfa, oracle_mod, smooth):
    """Hq = Hkv (no grouping) with B * Hkv = 8, the XCD-aware workgroup order
    (KV heads dealt to the 8 XCDs), two 256-row units with a ragged tail."""
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=2, Hq=4, Hkv=4, N=400),
                   smooth=smooth)


def test_prefill_gqa2_xcd_mapping_bf16_out(mpfa, oracle_mod):
    """Eight KV heads of two query heads each (XCD-aware order), bf16 output."""
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=1, Hq=16, Hkv=8, N=300),
                   out_bf16=True)


@pytest.mark.parametrize("B", [64, 66])
def test_prefill_query_amax_at_and_past_2048_heads(mpfa, oracle_mod, B):
    """The prefill call's Q_c amax pass leaves one maximum per workgroup (at
    most 2048, folded by the K expansion); B * Hq = 2048 query heads is the
    largest case it covers (one workgroup per head) and 2112 takes the
    slotted-atomic pass instead.  Short ragged sequences."""
    from mixed_precision_flashattention_amd import synth
    _check_prefill(mpfa, oracle_mod, synth.config("llama8b_prefill_16k", B=B, Hq=32, Hkv=8, N=20))


@pytest.mark.parametrize("smooth", [True, False])
def test_decode_mha(mpfa, oracle_mod, smooth):
    """Hq = Hkv: one real row per score tile."""
    from mixed_precision_flashattention_amd import synth
    _check_decode(mpfa, oracle_mod,
                  synth.config("llama8b_decode_128k", B=3, Hq=2, Hkv=2, N=515, num_splits=4),
                  smooth=smooth)


def test_decode_gqa8(mpfa, oracle_mod):
    from mixed_precision_flashattention_amd import synth
    _check_decode(mpfa, oracle_mod,
                  synth.config("llama8b_decode_128k", B=1, Hq=16, Hkv=2, N=777, num_splits=2))


@pytest.mark.parametrize("Hq,N,splits", [(10, 2048, 4), (12, 1000, 3), (16, 1024, 2)])
def test_decode_groups_past_four_whole_delta_rows(mpfa, oracle_mod, Hq, N, splits):
    """Smoothing with GQA groups of 5, 6 and 8 and N a multiple of 8: the
    group's Delta_S rows of every full block are read as 16-byte pieces, two
    per lane when the group has more than four rows (1000 = 7 x 128 + 104
    also ends in a partial block, read entry by entry)."""
    from mixed_precision_flashattention_amd import synth
    _check_decode(mpfa, oracle_mod,
                  synth.config("llama8b_decode_128k", B=2, Hq=Hq, Hkv=2, N=N, num_splits=splits))


# ---- degenerate inputs: a global amax or a centered tensor that is exactly 0 --
def _zero_k(q, k, v):
    return q, np.zeros_like(k), v


def _same_key(q, k, v):
    """Every token of a KV head carries the same key: centered K is (nearly) 0."""
    return q, np.ascontiguousarray(np.broadcast_to(k[:, :, :1, :], k.shape)), v


def _zero_v(q, k, v):
    return q, k, np.zeros_like(v)


def _zero_q(q, k, v):
    return np.zeros_like(q), k, v


def _offset_query(q, k, v):
    """Queries offset by up to +-6 per channel (bf16-exact): the sequence mean
    carries most of Q, so the compensation term Qbar . K_c dominates the
    scores."""
    x = (q + np.linspace(-6.0, 6.0, q.shape[-1], dtype=np.float32)).astype(np.float32)
    u = x.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32), k, v


@pytest.mark.parametrize("edit", [_zero_k, _same_key, _zero_v, _zero_q, _offset_query],
                         ids=lambda f: f.__name__)
@pytest.mark.parametrize("smooth", [True, False])
def test_prefill_degenerate_inputs(mpfa, oracle_mod, edit, smooth):
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_prefill_16k", B=1, Hq=4, Hkv=2, N=200)
    out, O = _check_prefill(mpfa, oracle_mod, cfg, smooth=smooth, edit=edit)
    if edit is _zero_v:
        assert not np.any(out), "zero V must give a zero output"


@pytest.mark.parametrize("edit", [_zero_k, _same_key, _zero_v, _zero_q], ids=lambda f: f.__name__)
def test_decode_degenerate_inputs(mpfa, oracle_mod, edit):
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_decode_128k", B=2, Hq=8, Hkv=2, N=700, num_splits=4)
    out, O = _check_decode(mpfa, oracle_mod, cfg, edit=edit)
    if edit is _zero_v:
        assert not np.any(out), "zero V must give a zero output"


def test_prefill_takes_the_first_stage_query_amax(mpfa, oracle_mod):
    """The Q_c amax written by the first stage (from its channel ranges and
    means) is max |fp32(Q - q_mean)| exactly, and a prefill given it returns
    the bytes of one that takes the amax in its own pass."""
    import torch
    torch.manual_seed(11)
    B, Hq, Hkv, N = 2, 8, 2, 777
    say(f"case: first-stage Q amax, B={B} Hq={Hq} Hkv={Hkv} N={N}")
    q = (torch.randn(B, Hq, N, 128) * 2.0 + torch.randn(1, 1, 1, 128)).to(torch.bfloat16).cuda()
    q[1, 3, 100, 7] = 40.0  # one spike sets the amax
    k = torch.randn(B, Hkv, N, 128).to(torch.bfloat16).cuda()
    v = torch.randn(B, Hkv, N, 128).to(torch.bfloat16).cuda()
    kq = mpfa.quantize_k(k, q=q)
    vq = mpfa.quantize_v(v)
    torch.cuda.synchronize()
    want = (q.float() - kq["q_mean"][:, :, None, :]).abs().max()
    assert kq["q_amax"].item() == want.item()
    scale = 128 ** -0.5
    out_a, lse_a = mpfa.prefill(q, kq, vq, scale, causal=True, with_lse=True)
    kq_no = {key: val for key, val in kq.items() if key not in ("q_amax", "q_amax_of")}
    out_b, lse_b = mpfa.prefill(q, kq_no, vq, scale, causal=True, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(lse_a, lse_b)
    # the hand-off is tied to the q it was computed from: another q (or the
    # same q changed in place) is refused instead of getting a wrong scale
    q2 = q.clone()
    with pytest.raises(ValueError):
        mpfa.prefill(q2, kq, vq, scale, causal=True)
    q.mul_(2.0)
    with pytest.raises(ValueError):
        mpfa.prefill(q, kq, vq, scale, causal=True)


# ---- seeded random shapes: combinations the cases above do not pin down ----
def _sweep_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 3, 5, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))
        cases.append(dict(B=int(rng.integers(1, 4)), Hkv=hkv, Hq=hkv * g,
                          N=int(rng.integers(1, 700)), bf16=bool(rng.integers(0, 2)),
                          causal=bool(rng.integers(0, 2)), smooth=bool(rng.integers(0, 2)),
                          out_bf16=bool(rng.integers(0, 2)), splits=int(rng.choice([1, 2, 3, 7, 16]))))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(20261203, sweep_count(12)), ids=lambda c: (
    f"B{c['B']}-H{c['Hq']}x{c['Hkv']}-N{c['N']}-{'bf16' if c['bf16'] else 'f32'}-"
    f"{'causal' if c['causal'] else 'full'}-{'smooth' if c['smooth'] else 'direct'}"))
def test_prefill_random_shapes(mpfa, oracle_mod, case):
    """Batch, KV heads (odd counts take the plain heaviest-first order), GQA
    factor, length (ragged), input dtype, causality, smoothing and output
    dtype drawn from a fixed seed; every row against the oracle."""
    from mixed_precision_flashattention_amd import synth
    base = "llama8b_prefill_16k" if case["bf16"] else "prefill_1k_2x1"
    cfg = synth.config(base, B=case["B"], Hq=case["Hq"], Hkv=case["Hkv"], N=case["N"])
    _check_prefill(mpfa, oracle_mod, cfg, causal=case["causal"], smooth=case["smooth"],
                   out_bf16=case["out_bf16"])


@pytest.mark.parametrize("case", _sweep_cases(20261204, sweep_count(8)), ids=lambda c: (
    f"B{c['B']}-H{c['Hq']}x{c['Hkv']}-N{c['N']}-splits{c['splits']}-"
    f"{'smooth' if c['smooth'] else 'direct'}"))
def test_decode_random_shapes(mpfa, oracle_mod, case):
    """The same draw for decode: batch, heads, cached length, partitions."""
    from mixed_precision_flashattention_amd import synth
    cfg = synth.config("llama8b_decode_128k", B=case["B"], Hq=case["Hq"], Hkv=case["Hkv"],
                       N=case["N"], num_splits=case["splits"])
    _check_decode(mpfa, oracle_mod, cfg, smooth=case["smooth"])
