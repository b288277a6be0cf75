"""Oracle pipeline: the method's steps composed in the paper's order.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything here works
on host numpy arrays in the logical layouts:

  q [B, Hq, N, D], k / v [B, Hkv, N, D] fp32 (bf16 inputs are widened exactly)
  k codes [B, Hkv, N, D/2] u8 (element 2t in the low nibble), k scales
  [B, Hkv, N, D/16] u8, v codes [B, Hkv, N, D] u8, delta_s [B, Hq, N] bf16 bits.

Query head h reads KV head h // (Hq / Hkv) (contiguous GQA groups).
Source: MpFA paper page ("MpFA: Hardware-Efficient Train-Free QK4V8
FlashAttention Kernels on Blackwell GPUs"), §4-§5; where the page is silent
the reading taken is stated in the docstring of the step that takes it.
"""
from __future__ import annotations

import numpy as np

from . import (KV_BLOCK, P_SCALE, amax, attn_state, bf16_rne, bf16_to_f64, channel_mean, delta_s,
               e4m3_table, fp8_quantize, fp8_scale, merge_states, nvfp4_dequantize,
               nvfp4_global_scale, nvfp4_quantize)

F32 = np.float32
F64 = np.float64


# ------------------------------------------------------------ stage one --
def quantize_k(k, q=None, q_mean=None, smooth=True):
    """Stage one for K (MpFA §5.1 first stage, §6 "Online quantization").

    smooth: K_c = fp32(K - Kbar) with Kbar the per-(b, kv-head) channel mean;
    Qbar is the per-(b, q-head) mean of ``q`` when given, else ``q_mean``
    (frozen means, as in decode); delta_s[b, h, j] = bf16(Qbar[b, h] . K_c[b, h//G, j]).
    With neither ``q`` nor ``q_mean`` only K is centred (no delta_s): the
    cache of the per-query-tile mean mode, which computes its compensation in
    the attention stage.
    direct: K_c = K, no means and no delta_s.
    Then NVFP4 with a global scale from the amax of the whole K_c tensor."""
    k = np.asarray(k, dtype=F32)
    B, Hkv, N, D = k.shape
    out = {}
    if smooth:
        k_mean = channel_mean(k)
        kc = (k - k_mean[:, :, None, :]).astype(F32)
        out.update(k_mean=k_mean)
        if q is not None:
            q_mean = channel_mean(np.asarray(q, dtype=F32))
        if q_mean is not None:
            q_mean = np.asarray(q_mean, dtype=F32)
            Hq = q_mean.shape[1]
            G = Hq // Hkv
            ds = np.empty((B, Hq, N), dtype=np.uint16)
            for b in range(B):
                for h in range(Hq):
                    ds[b, h] = delta_s(q_mean[b, h], kc[b, h // G])
            out.update(q_mean=q_mean, delta_s=ds)
    else:
        kc = k
    g = nvfp4_global_scale(amax(kc))
    codes, sf = nvfp4_quantize(kc, g)
    out.update(k_fp4=codes, k_sf=sf, k_gscale=np.float32(g))
    return out


def quantize_v(v):
    """FP8 E4M3 with one FP32 scale per tensor (MpFA §4.2; V is not centered)."""
    v = np.asarray(v, dtype=F32)
    s = fp8_scale(amax(v))
    return {"v_fp8": fp8_quantize(v, s), "v_scale": np.float32(s)}


def quantize_v_bf16(v):
    """V rounded to bf16 (nearest even), the V operand of the BF16 P.V
    precision assignment (MpFA §3.1, Fig. 3(a): NVFP4 Q.K^T with BF16 P.V).
    Returns bf16 bits [..., D] (uint16)."""
    return bf16_rne(np.asarray(v, dtype=F32))


def quantize_v_nvfp4(v):
    """NVFP4 V for the NVFP4 + NVFP4 precision assignment (MpFA §3.1,
    Fig. 3(a)): the P.V contraction runs over the keys, so V's 16-element
    blocks run along the keys, per channel.  Reading: the O3 steps of
    ``quantize_k`` (global scale from the amax of the whole V tensor, E4M3
    scale per block, E2M1 codes) applied to the rows of V transposed per
    (batch, KV head), keys past N padded with zeros (they change no block
    amax).  Returns v_fp4 [B, Hkv, ceil(N/16), D, 8] u8 (byte t of (block kb,
    channel d) holds keys 16 kb + 2t in the low nibble and 16 kb + 2t + 1 in
    the high one), v_sf [B, Hkv, ceil(N/16), D] u8 and v_gscale."""
    v = np.asarray(v, dtype=F32)
    B, Hkv, N, D = v.shape
    nb = (N + 15) // 16
    g = nvfp4_global_scale(amax(v))
    vp = np.zeros((B, Hkv, nb * 16, D), dtype=F32)
    vp[:, :, :N] = v
    vt = np.ascontiguousarray(vp.transpose(0, 1, 3, 2))  # [B, Hkv, D, keys]
    codes, sf = nvfp4_quantize(vt, g)  # [B, Hkv, D, nb * 8], [B, Hkv, D, nb]
    v_fp4 = np.ascontiguousarray(codes.reshape(B, Hkv, D, nb, 8).transpose(0, 1, 3, 2, 4))
    v_sf = np.ascontiguousarray(sf.transpose(0, 1, 3, 2))
    return {"v_fp4": v_fp4, "v_sf": v_sf, "v_gscale": np.float32(g)}


def dequantize_v_nvfp4(vq, b, hk, n):
    """The dequantized NVFP4 V of (b, KV head hk), keys 0 .. n-1: [n, D] FP64."""
    codes = vq["v_fp4"][b, hk]  # [nb, D, 8]
    sf = vq["v_sf"][b, hk]      # [nb, D]
    nb, D = sf.shape
    rows_c = np.ascontiguousarray(codes.transpose(1, 0, 2).reshape(D, nb * 8))
    rows_s = np.ascontiguousarray(sf.T)
    return nvfp4_dequantize(rows_c, rows_s, vq["v_gscale"]).T[:n]


def quantize_q(q, q_mean=None):
    """NVFP4 of Q_c = fp32(Q - Qbar) (direct mode: Q_c = Q), global scale from the
    amax of the whole Q_c tensor of the call.  Returns (codes, scales, g)."""
    q = np.asarray(q, dtype=F32)
    qc = q if q_mean is None else (q - np.asarray(q_mean, dtype=F32)[..., None, :]).astype(F32)
    g = nvfp4_global_scale(amax(qc))
    codes, sf = nvfp4_quantize(qc, g)
    return codes, sf, np.float32(g)


def append_kv(k_new, v_new, pos, cache, q_mean=None, k_mean=None):
    """Decode-time cache write (MpFA §6 "Online quantization"): the new tokens
    are centred against the frozen per-request means and quantized with the
    cache's frozen scales; in smoothing mode their compensation entries are
    computed in the same pass.

    Reading: the per-tensor global scales of the K and V caches are frozen with
    the means (the pages freeze the statistics for the sequence lifetime and
    re-quantizing the whole cache per token is not an option), so values out
    of their range saturate in the encoders.

    k_new, v_new [B, Hkv, T, D]; token t of batch entry b goes to position
    pos[b] + t.  cache: dict with k_fp4 [B, Hkv, Ncap, D/2], k_sf
    [B, Hkv, Ncap, D/16], k_gscale, v_fp8 [B, Hkv, Ncap, D] (row layout),
    v_scale and, in smoothing mode, delta_s [B, Hq, Ncap] (smoothing iff
    k_mean is given; q_mean [B, Hq, D] then too).  Returns an updated copy."""
    k_new = np.asarray(k_new, dtype=F32)
    v_new = np.asarray(v_new, dtype=F32)
    B, Hkv, T, D = k_new.shape
    out = {name: (np.array(a, copy=True) if isinstance(a, np.ndarray) else a)
           for name, a in cache.items()}
    smooth = k_mean is not None
    if smooth:
        k_mean = np.asarray(k_mean, dtype=F32)
        q_mean = np.asarray(q_mean, dtype=F32)
        Hq = q_mean.shape[1]
        G = Hq // Hkv
    g = np.float32(cache["k_gscale"])
    s = np.float32(cache["v_scale"])
    for b in range(B):
        rows = slice(int(pos[b]), int(pos[b]) + T)
        for hk in range(Hkv):
            kc = (k_new[b, hk] - k_mean[b, hk][None, :]).astype(F32) if smooth else k_new[b, hk]
            codes, sf = nvfp4_quantize(kc, g)
            out["k_fp4"][b, hk, rows] = codes
            out["k_sf"][b, hk, rows] = sf
            out["v_fp8"][b, hk, rows] = fp8_quantize(v_new[b, hk], s)
            if smooth:
                for h in range(hk * G, (hk + 1) * G):
                    out["delta_s"][b, h, rows] = delta_s(q_mean[b, h], kc)
    return out


def _finalize(m, l, acc, s_v, scale, lse_offset, out_f64=False):
    o = acc * float(s_v) / (P_SCALE * l[:, None])
    if not out_f64:
        o = o.astype(F32)
    lse = scale * m + np.log(l)
    if lse_offset is not None:
        lse = lse + lse_offset
    return o, lse


class Operands:
    """The operands of the attention stage, FP64, one head at a time.

    Quantized mode keeps the codes of the whole call (the global scales are
    per-tensor, so they always see every head) and dequantizes a head when it
    is asked for; identity mode widens the inputs.  Fields: s_v, quant_p,
    k_mean (smooth) and the per-head accessors q(b, h, pos), k(b, hk),
    v(b, hk), delta(b, h) (None in direct mode)."""

    def __init__(self, q, k, v, scale, smooth, identity, q_mean=None, pv="fp8"):
        """pv: the P.V precision: "fp8" (the method: E4M3 P with the fixed
        scale 448, FP8 V with a per-tensor scale), "bf16" (P rounded to
        bf16, V in bf16: the NVFP4 + BF16 assignment of MpFA §3.1) or
        "nvfp4" (P and V in NVFP4 over 16-key blocks: the NVFP4 + NVFP4
        assignment of MpFA §3.1)."""
        q = np.asarray(q, dtype=F32)
        k = np.asarray(k, dtype=F32)
        v = np.asarray(v, dtype=F32)
        B, Hq = q.shape[:2]
        Hkv = k.shape[1]
        self.G = Hq // Hkv
        self.n_kv = k.shape[2]
        self.smooth = smooth
        self.identity = identity
        self._q, self._k, self._v = q, k, v
        self.k_mean = None
        self._delta = None
        self.pv = pv
        self.p_format = "none" if identity else {"bf16": "bf16", "nvfp4": "nvfp4"}.get(pv, "e4m3")
        if identity:
            if smooth:
                self.k_mean = channel_mean(k)
                if q_mean is None:
                    q_mean = channel_mean(q)
                self._qm = np.asarray(q_mean, dtype=F64)
            self.s_v, self.quant_p = 1.0, False
            return
        if smooth:
            kq = quantize_k(k, q=q if q_mean is None else None, q_mean=q_mean, smooth=True)
            qcodes, qsf, gq = quantize_q(q, kq["q_mean"])
            self.k_mean = kq["k_mean"]
            self._delta = kq["delta_s"]
        else:
            kq = quantize_k(k, smooth=False)
            qcodes, qsf, gq = quantize_q(q, None)
        if pv == "bf16":
            vq = {"v_bf16": quantize_v_bf16(v)}
            self.s_v = 1.0
        elif pv == "nvfp4":
            vq = quantize_v_nvfp4(v)
            self.s_v = 1.0
        else:
            vq = quantize_v(v)
            self.s_v = float(vq["v_scale"])
        self.kq, self.vq = kq, vq
        self.q_codes, self.q_sf, self.q_gscale = qcodes, qsf, gq
        self.quant_p = True
        self._table = e4m3_table()

    @classmethod
    def from_cache(cls, q, cache, n_kv, q_mean=None, k_mean=None):
        """Operands of a decode over the first n_kv positions of existing
        caches (as written by quantize_k / quantize_v / append_kv): the
        cache codes and their frozen scales are used as they are; Q is
        quantized per call as in __init__ (centred by q_mean in smoothing
        mode, which is on iff cache holds delta_s)."""
        self = cls.__new__(cls)
        q = np.asarray(q, dtype=F32)
        self.smooth = "delta_s" in cache and cache["delta_s"] is not None
        self.identity = False
        self.G = q.shape[1] // cache["k_fp4"].shape[1]
        self.n_kv = n_kv
        self._q = q
        self.kq = {"k_fp4": cache["k_fp4"][:, :, :n_kv], "k_sf": cache["k_sf"][:, :, :n_kv],
                   "k_gscale": np.float32(cache["k_gscale"])}
        self.vq = {"v_fp8": cache["v_fp8"][:, :, :n_kv], "v_scale": np.float32(cache["v_scale"])}
        if self.smooth:
            self.k_mean = np.asarray(k_mean, dtype=F32)
            self._delta = cache["delta_s"][:, :, :n_kv]
            self.q_codes, self.q_sf, self.q_gscale = quantize_q(q, q_mean)
        else:
            self.k_mean = None
            self._delta = None
            self.q_codes, self.q_sf, self.q_gscale = quantize_q(q, None)
        self.s_v = float(self.vq["v_scale"])
        self.quant_p = True
        self.pv, self.p_format = "fp8", "e4m3"
        self._table = e4m3_table()
        return self

    def q(self, b, h, pos):
        if self.identity:
            x = self._q[b, h][pos].astype(F64)
            return x - self._qm[b, h][None, :] if self.smooth else x
        return nvfp4_dequantize(self.q_codes[b, h][pos], self.q_sf[b, h][pos], self.q_gscale)

    def k(self, b, hk):
        if self.identity:
            x = self._k[b, hk].astype(F64)
            return x - self.k_mean[b, hk].astype(F64)[None, :] if self.smooth else x
        return nvfp4_dequantize(self.kq["k_fp4"][b, hk], self.kq["k_sf"][b, hk], self.kq["k_gscale"])

    def v(self, b, hk):
        if self.identity:
            return self._v[b, hk].astype(F64)
        if self.pv == "bf16":
            return bf16_to_f64(self.vq["v_bf16"][b, hk])
        if self.pv == "nvfp4":
            return dequantize_v_nvfp4(self.vq, b, hk, self.n_kv)
        return self._table[self.vq["v_fp8"][b, hk]]

    def delta(self, b, h):
        """Compensation vector of (b, q-head h): the stored bf16 values, or in
        identity mode the FP64 product of the centered keys with Qbar."""
        if not self.smooth:
            return None
        if self.identity:
            return self.k(b, h // self.G) @ self._qm[b, h]
        return bf16_to_f64(self._delta[b, h])


def prefill_rows(q, k, v, scale, causal=True, smooth=True, identity=False, rows=None, out_f64=False,
                 ops=None, ambiguity=False, pv="fp8", amb_rel=None):
    """Causal (or full) prefill, MpFA §5.1 second stage, for the selected rows.

    pv="bf16" gives the NVFP4 + BF16 precision assignment (P and V in bf16,
    MpFA §3.1) and pv="nvfp4" the NVFP4 + NVFP4 one (P and V in NVFP4 over
    16-key blocks) instead of the method's FP8 P.V.  amb_rel: the width of the
    rounding-ambiguity window of AMB (default: an FP32 exp2's, 2^-16).

    rows: None (every row) or an int array [R, 3] of (b, q-head, position).
    ops: an Operands already built from the same q, k, v and mode (else built here).
    Returns (O [R, D] fp32, LSE [R] f64, rows) -- O = acc * s_V / (448 l), LSE in
    natural log with the smoothing row offset scale * (Q_i . Kbar) added back;
    with ambiguity=True also AMB [R, D], the most O may move when the P^
    roundings that sit on an E4M3 midpoint (see ``attn_state``) go the other
    way."""
    q = np.asarray(q, dtype=F32)
    B, Hq, N, D = q.shape
    if ops is None:
        ops = Operands(q, k, v, scale, smooth, identity, pv=pv)
    G = ops.G
    amb_kw = {} if amb_rel is None else {"amb_rel": amb_rel}
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(N), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), D), dtype=F64 if out_f64 else F32)
    LSE = np.empty(len(rows))
    AMB = np.zeros((len(rows), D))
    for b in range(B):
        for hk in range(q.shape[1] // G):
            kt = vt = None
            for h in range(hk * G, (hk + 1) * G):
                sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
                if len(sel) == 0:
                    continue
                if kt is None:
                    kt, vt = ops.k(b, hk), ops.v(b, hk)
                pos = rows[sel, 2]
                row_pos = pos if causal else np.full(len(sel), -1, dtype=np.int64)
                m, l, acc, amb = attn_state(ops.q(b, h, pos), row_pos, kt, vt, ops.delta(b, h), 0, N,
                                            scale, ops.quant_p, ambiguity=True,
                                            p_format=ops.p_format, **amb_kw)
                off = None
                if smooth:
                    off = scale * (q[b, h][pos].astype(F64) @ ops.k_mean[b, hk].astype(F64))
                o, lse = _finalize(m, l, acc, ops.s_v, scale, off, out_f64)
                O[sel] = o
                LSE[sel] = lse
                AMB[sel] = amb * ops.s_v / (P_SCALE * l[:, None])
    return (O, LSE, rows, AMB) if ambiguity else (O, LSE, rows)


# --------------------------------------------- per-query-tile mean mode --
Q_TILE = KV_BLOCK  # query rows per mean in the per-tile mode


def tile_means(q, tile=Q_TILE):
    """Channel means of Q per (b, q-head, tile of ``tile`` consecutive rows),
    by the same order-free fixed-point rule as the sequence means; the last
    tile averages only the rows it has.  q [B, H, N, D] -> [B, H, ceil(N/tile), D] fp32.

    Reading: the per-tile mode centres each query row by the mean of its own
    128-row tile instead of the sequence mean (the paper smooths Q by a mean
    over the queries, MpFA §3.2, §5.1; the tile is the query tile of the
    attention stage)."""
    q = np.asarray(q, dtype=F32)
    B, H, N, D = q.shape
    nt = -(-N // tile)
    out = np.empty((B, H, nt, D), dtype=F32)
    for t in range(nt):
        out[:, :, t] = channel_mean(np.ascontiguousarray(q[:, :, t * tile:(t + 1) * tile]))
    return out


def quantize_q_tiles(q, tm, tile=Q_TILE):
    """NVFP4 of Q_c = fp32(Q - Qbar_tile(row)), one global scale from the amax
    of the whole tile-centred tensor.  Returns (codes, scales, g)."""
    q = np.asarray(q, dtype=F32)
    N = q.shape[2]
    rep = np.repeat(np.asarray(tm, dtype=F32), tile, axis=2)[:, :, :N]
    qc = (q - rep).astype(F32)
    g = nvfp4_global_scale(amax(qc))
    codes, sf = nvfp4_quantize(qc, g)
    return codes, sf, np.float32(g)


def delta_tile(tm, k_codes, k_sf, k_gscale):
    """The compensation term of the per-tile mode, one bf16 value per
    (b, q-head, query tile, key):

        Delta_tile[b, h, t, j] = bf16_rne(fp32(sum_d Qbar_tile[b, h, t, d] * K~_c[b, h//G, j, d]))

    with K~_c the dequantized centred key (code value x block scale x global
    scale) and the sum in FP64 over ascending d (the products of an fp32 mean
    and a 30-bit key are exact in FP64 but for the last bit).

    Reading: the tile's mean Qbar_tile enters the scores as its own column
    term Qbar_tile . K~_c[j], the same rank-one form and the same BF16
    carriage as Delta_S (MpFA §5.2: the compensation is one BF16 matrix
    product written into S before the main product accumulates; §7.4: only
    the compensation term is carried in BF16).  The centred keys it multiplies
    are the quantized ones, since this mode computes the term in the attention
    stage, where only the quantized cache exists.
    tm [B, Hq, T, D] fp32; k_codes [B, Hkv, N, D/2], k_sf [B, Hkv, N, D/16].
    Returns [B, Hq, T, N] uint16 (bf16 bits)."""
    tm = np.asarray(tm, dtype=F32)
    B, Hq, T, D = tm.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    N = k_codes.shape[2]
    out = np.empty((B, Hq, T, N), dtype=np.uint16)
    for b in range(B):
        for hk in range(Hkv):
            kt = nvfp4_dequantize(k_codes[b, hk], k_sf[b, hk], k_gscale)  # [N, D] f64, exact
            for h in range(hk * G, (hk + 1) * G):
                for t in range(T):
                    out[b, h, t] = delta_tile_row(tm[b, h, t], kt)
    return out


def delta_tile_row(qbar, kt):
    """One row of ``delta_tile``: qbar [D] fp32, kt [N, D] the dequantized
    centred keys (FP64) -> [N] bf16 bits; FP64 sum over ascending d, then
    fp32, then bf16 (round to nearest even each time)."""
    qbar = np.asarray(qbar, dtype=F32)
    acc = np.zeros(kt.shape[0])
    for d in range(kt.shape[1]):
        acc = acc + float(qbar[d]) * kt[:, d]
    return bf16_rne(acc.astype(F32))


def prefill_tile_mean_rows(q, k, v, scale, causal=True, identity=False, rows=None, out_f64=False,
                           ambiguity=False):
    """Prefill in the per-query-tile mean mode for the selected rows.

    K is centred by its sequence mean Kbar and quantized as in smoothing mode
    (without delta_s); Q by the mean of each row's 128-row tile
    (``tile_means``, ``quantize_q_tiles``); the scores are
    S_ij = Q~_c,i . K~_c,j + Delta_tile[tile(i), j] (``delta_tile``), FP64,
    before the mask and the running max; the rest is the prefill of
    ``prefill_rows``.  The LSE adds back the row term scale * (Q_i . Kbar),
    as in smoothing mode (Q_i . K_j = Q_c,i . K_c,j + Qbar_tile . K_c,j +
    Q_i . Kbar, the last term constant along the row).
    identity: no quantizer (Q_c and K_c in FP64, the column term
    Qbar_tile . K_c[j] unrounded, P not rounded).  Returns (O, LSE, rows),
    plus AMB as in ``prefill_rows`` with ambiguity=True."""
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    v = np.asarray(v, dtype=F32)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tm = tile_means(q)
    k_mean = channel_mean(k)
    rep = np.repeat(tm, Q_TILE, axis=2)[:, :, :N]
    if identity:
        qop = (q - rep).astype(F32).astype(F64)
        kdeq = lambda b, hk: (k[b, hk] - k_mean[b, hk][None, :]).astype(F32).astype(F64)
        vdeq = lambda b, hk: v[b, hk].astype(F64)
        dtile = lambda b, h, t: kdeq(b, h // G) @ tm[b, h, t].astype(F64)
        s_v, quant_p = 1.0, False
    else:
        kq = quantize_k(k)
        vq = quantize_v(v)
        codes, sf, g = quantize_q_tiles(q, tm)
        qop = nvfp4_dequantize(codes, sf, g)
        kdeq = lambda b, hk: nvfp4_dequantize(kq["k_fp4"][b, hk], kq["k_sf"][b, hk], kq["k_gscale"])
        dtile = lambda b, h, t: bf16_to_f64(delta_tile_row(tm[b, h, t], kdeq(b, h // G)))
        table = e4m3_table()
        vdeq = lambda b, hk: table[vq["v_fp8"][b, hk]]
        s_v, quant_p = float(vq["v_scale"]), True
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(N), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), D), dtype=F64 if out_f64 else F32)
    LSE = np.empty(len(rows))
    AMB = np.zeros((len(rows), D))
    for b in range(B):
        for hk in range(Hkv):
            kt = vt = None
            for h in range(hk * G, (hk + 1) * G):
                for t in range(-(-N // Q_TILE)):
                    sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h) &
                                     (rows[:, 2] // Q_TILE == t))[0]
                    if len(sel) == 0:
                        continue
                    if kt is None:
                        kt, vt = kdeq(b, hk), vdeq(b, hk)
                    pos = rows[sel, 2]
                    row_pos = pos if causal else np.full(len(sel), -1, dtype=np.int64)
                    m, l, acc, amb = attn_state(np.ascontiguousarray(qop[b, h][pos]), row_pos, kt, vt,
                                                dtile(b, h, t), 0, N, scale, quant_p, ambiguity=True)
                    off = scale * (q[b, h][pos].astype(F64) @ k_mean[b, hk].astype(F64))
                    o, lse = _finalize(m, l, acc, s_v, scale, off, out_f64)
                    O[sel] = o
                    LSE[sel] = lse
                    AMB[sel] = amb * s_v / (P_SCALE * l[:, None])
    return (O, LSE, rows, AMB) if ambiguity else (O, LSE, rows)


def decode_partitions(n_kv: int, num_splits: int, block: int = KV_BLOCK):
    """KV partitions of decode (MpFA §5.3: fixed chunks of whole 128-token blocks).

    Reading: chunk = block * ceil(n_kv / (block * num_splits)); partition p covers
    [p*chunk, min((p+1)*chunk, n_kv)) and may be empty."""
    chunk = block * -(-n_kv // (block * num_splits))
    return [(min(p * chunk, n_kv), min((p + 1) * chunk, n_kv)) for p in range(num_splits)]


def decode(q, k, v, q_mean, num_splits, scale, smooth=True, identity=False, out_f64=False, heads=None,
           ops=None):
    """Split-KV decode (MpFA §5.3): one query token per (batch, q-head), every key
    visible, per-partition online-softmax states merged by log-sum-exp.

    q [B, Hq, D] or [B, Hq, 1, D]; q_mean [B, Hq, D] frozen means (smooth mode).
    heads: None (every (b, q-head)) or a list of (b, q-head) pairs.
    ops: an Operands already built from the same inputs and mode (else built here).
    Returns (O, LSE): [B, Hq, D] fp32 and [B, Hq] f64, or [len(heads), D] and
    [len(heads)] for a head list."""
    q = np.asarray(q, dtype=F32)
    if q.ndim == 3:
        q = q[:, :, None, :]
    B, Hq, _, D = q.shape
    N = ops.n_kv if (ops is not None and k is None) else np.asarray(k).shape[2]
    if ops is None:
        ops = Operands(q, k, v, scale, smooth, identity, q_mean=q_mean if smooth else None)
    G = ops.G
    parts = decode_partitions(N, num_splits)
    sel = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else [tuple(x) for x in heads]
    O = np.empty((len(sel), D), dtype=F64 if out_f64 else F32)
    LSE = np.empty(len(sel))
    cache = {}
    for i, (b, h) in enumerate(sel):
        hk = h // G
        if (b, hk) not in cache:
            cache.clear()
            cache[(b, hk)] = (ops.k(b, hk), ops.v(b, hk))
        kt, vt = cache[(b, hk)]
        qt = ops.q(b, h, np.array([0]))
        delta = ops.delta(b, h)
        ms, ls, accs = [], [], []
        for (p0, p1) in parts:
            if p1 <= p0:
                ms.append(-np.inf)
                ls.append(0.0)
                accs.append(np.zeros(D))
                continue
            m, l, acc = attn_state(qt, np.array([-1]), kt, vt, delta, p0, p1, scale, ops.quant_p)
            ms.append(m[0])
            ls.append(l[0])
            accs.append(acc[0])
        m, l, acc = merge_states(np.array([ms]), np.array([ls]), np.array([accs]), scale)
        off = None
        if smooth:
            off = np.array([scale * (q[b, h, 0].astype(F64) @ ops.k_mean[b, hk].astype(F64))])
        o, lse = _finalize(m, l, acc, ops.s_v, scale, off, out_f64)
        O[i] = o[0]
        LSE[i] = lse[0]
    if heads is None:
        return O.reshape(B, Hq, D), LSE.reshape(B, Hq)
    return O, LSE


# ------------------------------------------------------------ paged cache --
PAGE = KV_BLOCK  # tokens per cache page


def gather_pages(pool, block_table, b, n):
    """Request b's first n positions of a paged cache, as a contiguous cache
    with batch size 1 (the layout quantize_k / quantize_v / append_kv use).

    pool: k_fp4 [P, Hkv, PAGE, D/2], k_sf [P, Hkv, PAGE, D/16], v_fp8 [P, Hkv,
    PAGE, D] (row layout), optionally delta_s [P, Hq, PAGE], and the
    per-request frozen scales k_gscale [B], v_scale [B].  Logical page i of
    request b is physical page block_table[b, i] (MpFA §6 "Serving system":
    the compensation side cache follows the same physical page indices)."""
    npg = -(-n // PAGE)
    pages = np.asarray(block_table[b, :npg], dtype=np.int64)

    def rows(a):  # [npg, H, PAGE, ...] -> [1, H, npg * PAGE, ...][:, :, :n]
        x = np.asarray(a)[pages]
        x = np.moveaxis(x, 0, 1)
        x = x.reshape((x.shape[0], npg * PAGE) + x.shape[3:])
        return x[None, :, :n]

    cache = {"k_fp4": rows(pool["k_fp4"]), "k_sf": rows(pool["k_sf"]), "v_fp8": rows(pool["v_fp8"]),
             "k_gscale": np.float32(pool["k_gscale"][b]), "v_scale": np.float32(pool["v_scale"][b])}
    if pool.get("delta_s") is not None:
        cache["delta_s"] = rows(pool["delta_s"])
    return cache


def decode_paged(q, pool, block_table, seq_lens, q_mean, k_mean, num_splits, scale, out_f64=False,
                 heads=None):
    """Split-KV decode over a paged cache with per-request lengths (MpFA §5.3;
    §6 "Serving system": fixed-size pages, a constant number of KV
    partitions, the Delta_S side cache indexed by the same pages).

    q [B, Hq, D] (or [B, Hq, 1, D]); smoothing iff pool holds delta_s (then
    q_mean [B, Hq, D] and k_mean [B, Hkv, D] are the frozen per-request means).
    Readings: Q is quantized once over the whole query tensor of the call, as
    in decode(); request b sees its first seq_lens[b] positions, clamped to
    the capacity of its block-table row, cut into num_splits partitions of
    its own (decode_partitions of its length); the K and V scales are the
    request's own frozen scales.  A request with no positions returns O = 0
    and LSE = -inf.  heads: None (every (b, q-head)) or a list of (b, q-head)
    pairs to compute (the others are left at O = 0, LSE = -inf).
    Returns (O [B, Hq, D], LSE [B, Hq])."""
    q = np.asarray(q, dtype=F32)
    if q.ndim == 3:
        q = q[:, :, None, :]
    B, Hq, _, D = q.shape
    smooth = pool.get("delta_s") is not None
    qm = np.asarray(q_mean, dtype=F32) if smooth else None
    codes, sf, g = quantize_q(q, qm)
    cap = block_table.shape[1] * PAGE
    O = np.zeros((B, Hq, D), dtype=F64 if out_f64 else F32)
    LSE = np.full((B, Hq), -np.inf)
    want = None if heads is None else {}
    if heads is not None:
        for b, h in heads:
            want.setdefault(int(b), []).append(int(h))
    for b in range(B):
        n = int(min(max(int(seq_lens[b]), 0), cap))
        if n == 0 or (want is not None and b not in want):
            continue
        cache = gather_pages(pool, block_table, b, n)
        ops = Operands.from_cache(q[b:b + 1], cache, n, q_mean=qm[b:b + 1] if smooth else None,
                                  k_mean=np.asarray(k_mean)[b:b + 1] if smooth else None)
        ops.q_codes, ops.q_sf, ops.q_gscale = codes[b:b + 1], sf[b:b + 1], g
        if want is None:
            o, lse = decode(q[b:b + 1], None, None, ops.k_mean, num_splits, scale, smooth=smooth,
                            out_f64=out_f64, ops=ops)
            O[b], LSE[b] = o[0], lse[0]
        else:
            hs = want[b]
            o, lse = decode(q[b:b + 1], None, None, ops.k_mean, num_splits, scale, smooth=smooth,
                            out_f64=out_f64, ops=ops, heads=[(0, h) for h in hs])
            O[b, hs], LSE[b, hs] = o, lse
    return O, LSE


def append_kv_paged(k_new, v_new, pos, pool, block_table, q_mean=None, k_mean=None):
    """Decode-time write of one new token per request into a paged cache (MpFA
    §6 "Online quantization" and "Serving system"): the token of request b
    goes to position pos[b], i.e. slot pos[b] % PAGE of physical page
    block_table[b, pos[b] // PAGE], quantized as in append_kv with the
    request's own frozen scales and means.  A request whose position is
    outside its block-table row, or whose page index is outside the pool,
    writes nothing.  k_new, v_new [B, Hkv, 1, D].  Returns an updated copy."""
    k_new = np.asarray(k_new, dtype=F32)
    v_new = np.asarray(v_new, dtype=F32)
    B = k_new.shape[0]
    out = {name: (np.array(a, copy=True) if isinstance(a, np.ndarray) else a) for name, a in pool.items()}
    smooth = k_mean is not None
    n_pages = out["k_fp4"].shape[0]
    for b in range(B):
        p = int(pos[b])
        if p < 0 or p >= block_table.shape[1] * PAGE:
            continue
        pg = int(block_table[b, p // PAGE])
        if pg < 0 or pg >= n_pages:
            continue
        page = {"k_fp4": out["k_fp4"][pg][None], "k_sf": out["k_sf"][pg][None],
                "v_fp8": out["v_fp8"][pg][None], "k_gscale": out["k_gscale"][b],
                "v_scale": out["v_scale"][b]}
        if smooth:
            page["delta_s"] = out["delta_s"][pg][None]
        page = append_kv(k_new[b:b + 1], v_new[b:b + 1], [p % PAGE], page,
                         q_mean=np.asarray(q_mean)[b:b + 1] if smooth else None,
                         k_mean=np.asarray(k_mean)[b:b + 1] if smooth else None)
        for name in ("k_fp4", "k_sf", "v_fp8") + (("delta_s",) if smooth else ()):
            out[name][pg] = page[name][0]
    return out


def exact_attention(q, k, v, scale, causal=True, rows=None):
    """FP64 softmax(scale * Q K^T + mask) V and its natural-log LSE on the
    unquantized inputs (report-only error reference)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    B, Hq, Nq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Nq), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), D))
    LSE = np.empty(len(rows))
    for b in range(B):
        for h in range(Hq):
            sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
            if len(sel) == 0:
                continue
            pos = rows[sel, 2]
            s = scale * (q[b, h][pos] @ k[b, h // G].T)
            if causal:
                s = np.where(np.arange(N)[None, :] <= pos[:, None], s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            den = e.sum(axis=1, keepdims=True)
            O[sel] = (e @ v[b, h // G]) / den
            LSE[sel] = (mx + np.log(den))[:, 0]
    return O, LSE
