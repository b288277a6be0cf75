// Causal / full QK4PV8 prefill for gfx950 (paper "MpFA: ...", section 5.1
// "second stage", section 5.2 "MMA Compensation", section 4.1).
//
// Work unit: one (batch, query head, 128-row query tile); 4 waves of 32 rows.
// Per 128-key block:
//   * the workgroup expands the NVFP4 K block into exact FP16 operands
//     (code value x E4M3 block scale) in LDS and copies the FP8 V tiles and
//     the block's Delta_S into LDS;
//   * each wave computes S^T (keys x its 32 queries) on MFMA: first a bf16
//     step that writes Delta_S * (1 / (gQ gK)) into the accumulator (the
//     rank-one term of section 5.2, no element-wise add on the softmax
//     path), then 8 f16 steps accumulating Q~ K~^T over the head dimension;
//   * softmax in the S^T layout: each lane owns one query and 64 of the 128
//     keys, so the row max is in-lane plus one exchange with lane ^ 32; the
//     global scales and the softmax scale are one constant in the exp2
//     argument (section 5.1), and 448 (the fixed P scale) is added in the
//     exponent;
//   * P is rounded to E4M3 by the hardware converter and fed straight from
//     registers as the B operand of the FP8 P.V MFMA; the key order of the
//     score tiles is permuted so that each lane's P bytes are 32 consecutive
//     keys, matching the head-dim-major V tiles.
#include "mpfa_internal.hpp"

namespace mpfa {

constexpr int kQTile = 128;
constexpr int kKStride = 272;  // bytes per LDS row of K~ (128 f16 + 16 bytes of padding)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(PrefillParams p) {
  __shared__ __align__(16) uint8_t smem_k[kQTile * kKStride];  // K~ block (Q~ in the prologue)
  __shared__ __align__(16) uint8_t smem_v[4 * kD * 32];        // 4 V tiles [d][32 tokens]
  __shared__ uint16_t smem_delta[kBlk];

  const int N = p.N;
  const int nbh = p.B * p.Hq;
  const int wid = blockIdx.x;
  const int tile = p.n_qtiles - 1 - wid / nbh;  // heaviest (last) query tiles first
  const int bh = wid % nbh;
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / p.G;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int row0 = tile * kQTile;
  const bool smooth = p.delta_s != nullptr;

  const float gQ = nvfp4_global_scale(__uint_as_float(*p.q_amax));
  const float gK = *p.k_gscale;
  const float sV = *p.v_scale;
  const float gg = gQ * gK;
  const float lam = p.scale * kLog2e * gg;  // exp2 constant per unit of the MFMA score
  // Delta_S enters the MFMA score in units of 1 / (gQ gK), written as the
  // sum of three bf16 parts (exact to fp32 precision).
  const float cinv = 1.0f / gg;
  const uint32_t c_hi = bf16_rne(cinv);
  const float r1 = cinv - __uint_as_float(c_hi << 16);
  const uint32_t c_mid = bf16_rne(r1);
  const uint32_t c_lo = bf16_rne(r1 - __uint_as_float(c_mid << 16));

  // ---- prologue: NVFP4 of the query tile, expanded to FP16 in LDS --------
  float* lse_part = reinterpret_cast<float*>(smem_v);  // [128 rows][8 blocks]
  for (int u = tid; u < kQTile * 8; u += 256) {
    const int r = u >> 3, blk = u & 7;
    const int qrow = row0 + r;
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float part = 0.0f;
    if (qrow < N) {
      float x[16];
      const int64_t off = ((int64_t)bh * N + qrow) * kD + blk * 16;
      load16(p.q, off, p.q_bf16, x);
      if (smooth) {
        const float* mu = p.q_mean + (int64_t)bh * kD + blk * 16;
        const float* km = p.k_mean + ((int64_t)b * p.Hkv + hk) * kD + blk * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          part = fmaf(x[j], km[j], part);
          x[j] = x[j] - mu[j];
        }
      }
      uint32_t c[16];
      const uint32_t sc = nvfp4_block(x, gQ, c);
      const float s = e4m3_value_pos(sc);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x2 v2 = {(_Float16)(e2m1_value(c[2 * j]) * s),
                          (_Float16)(e2m1_value(c[2 * j + 1]) * s)};
        packed[j] = __builtin_bit_cast(uint32_t, v2);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(smem_k + r * kKStride + blk * 32);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    lse_part[r * 8 + blk] = part;
  }
  __syncthreads();

  // B operand of the score MFMA (Q~^T): query row 32*wave + col, head-dim
  // slots 64*h + 8*kc .. +7 for step kc (the K~ reads use the same slots).
  const int qr = 32 * wave + col;
  i32x4 qf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qf[kc] = *reinterpret_cast<const i32x4*>(smem_k + qr * kKStride + (64 * h + 8 * kc) * 2);
  float lse_off = 0.0f;
  if (p.lse && smooth) {
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) lse_off += lse_part[qr * 8 + blk];
    lse_off *= p.scale;
  }
  // Constant B operand of the rank-one step: slots 0..2 of lane half 0 hold
  // the three bf16 parts of 1 / (gQ gK); everything else is zero.
  const i32x4 dB = {h == 0 ? (int)(c_hi | (c_mid << 16)) : 0, h == 0 ? (int)c_lo : 0, 0, 0};

  const int my_row = row0 + qr;
  const int nblk_all = (N + kBlk - 1) / kBlk;
  const int nblk = p.causal ? min(tile + 1, nblk_all) : nblk_all;
  const int ntiles32 = (N + 31) / 32;
  const int64_t kvh = (int64_t)b * p.Hkv + hk;
  const uint8_t* kbase = p.k_fp4 + kvh * N * 64;
  const uint8_t* sbase = p.k_sf + kvh * N * 8;
  const uint8_t* vbase = p.v_fp8 + kvh * ntiles32 * (kD * 32);
  const uint16_t* dbase = smooth ? p.delta_s + (int64_t)bh * N : nullptr;

  // A-row rho of score tile t holds key 64*(t/2) + 32*hp + 16*(t%2) + vp of
  // the block (hp, vp from rho below); the MFMA output register v of lane
  // half h then holds key 64*(t/2) + 32*h + 16*(t%2) + v.
  const int hp = (col >> 2) & 1, vp = ((col >> 3) << 2) | (col & 3);

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};

  // Per-thread share of a block's loads: K codes of (key, head-dim half),
  // 4 x 16 bytes of the V tiles, one Delta_S entry.  Block j+1 is fetched
  // into registers while block j is computed.
  const int ld_key = tid >> 1, ld_half = tid & 1;
  uint4 kc0 = make_uint4(0, 0, 0, 0), kc1 = kc0;
  uint32_t ksc = 0;
  uint4 vv[4];
  uint32_t dd = 0;
  auto load_block = [&](int jb) {
    const int kb0 = jb * kBlk;
    const int gk = kb0 + ld_key;
    kc0 = make_uint4(0, 0, 0, 0);
    kc1 = kc0;
    ksc = 0;
    if (gk < N) {
      const uint4* src = reinterpret_cast<const uint4*>(kbase + (int64_t)gk * 64 + 32 * ld_half);
      kc0 = src[0];
      kc1 = src[1];
      ksc = *reinterpret_cast<const uint32_t*>(sbase + (int64_t)gk * 8 + 4 * ld_half);
    }
    const int tt0 = kb0 / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int tt = idx >> 8;
      vv[i] = make_uint4(0, 0, 0, 0);
      if (tt0 + tt < ntiles32)
        vv[i] = reinterpret_cast<const uint4*>(vbase + (int64_t)(tt0 + tt) * (kD * 32))[idx & 255];
    }
    if (smooth && tid < kBlk) dd = (kb0 + tid < N) ? dbase[kb0 + tid] : 0u;
  };
  load_block(0);

  for (int j = 0; j < nblk; ++j) {
    const int k0 = j * kBlk;
    __syncthreads();  // every wave is done with the previous block's LDS tiles
    {
      const uint32_t w[8] = {kc0.x, kc0.y, kc0.z, kc0.w, kc1.x, kc1.y, kc1.z, kc1.w};
      uint8_t* dst = smem_k + ld_key * kKStride + ld_half * 128;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t e[4];
        expand_fp4x8(w[i], e4m3_scale_f16x2((ksc >> (8 * (i >> 1))) & 0xFFu), e);
        *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(e[0], e[1], e[2], e[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(smem_v)[tid + 256 * i] = vv[i];
      if (smooth && tid < kBlk) smem_delta[tid] = (uint16_t)dd;
    }
    __syncthreads();
    if (j + 1 < nblk) load_block(j + 1);

    // ---- scores S^T: 4 tiles of 32 keys x 32 queries --------------------
    f32x16 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 64 * (t >> 1) + 32 * hp + 16 * (t & 1) + vp;
      f32x16 acc = f32x16{};
      if (smooth) {
        const uint32_t dv = smem_delta[key];
        const i32x4 dA = {h == 0 ? (int)(dv | (dv << 16)) : 0, h == 0 ? (int)dv : 0, 0, 0};
        acc = mfma32_bf16(dA, dB, acc);
      }
      const uint8_t* krow = smem_k + key * kKStride + 128 * h;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        acc = mfma32_f16(*reinterpret_cast<const i32x4*>(krow + 16 * kc), qf[kc], acc);
      s[t] = acc;
    }

    // ---- mask (diagonal or ragged block only) and online softmax --------
    const bool need_mask = (p.causal && k0 + kBlk > row0) || (k0 + kBlk > N);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + 64 * (t >> 1) + 32 * h + 16 * (t & 1) + v;
          const bool vis = key < N && (!p.causal || key <= my_row);
          if (!vis) s[t][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(lam * (m_run - m_new));
    const float nb = kLog2_448 - lam * m_new;
    m_run = m_new;

    float lsum = 0.0f;
    i32x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = 2 * c + (k >> 2), v0 = 4 * (k & 3);
        const float e0 = fast_exp2(fmaf(s[t][v0], lam, nb));
        const float e1 = fast_exp2(fmaf(s[t][v0 + 1], lam, nb));
        const float e2 = fast_exp2(fmaf(s[t][v0 + 2], lam, nb));
        const float e3 = fast_exp2(fmaf(s[t][v0 + 3], lam, nb));
        lsum += (e0 + e1) + (e2 + e3);
        uint32_t wd = cvt_fp8x2<false>(e0, e1, 0u);
        wd = cvt_fp8x2<true>(e2, e3, wd);
        pb[c][k] = (int)wd;
      }
    }
    l_run = fmaf(alpha, l_run, lsum);

    // ---- O^T = alpha O^T + V^T P^T on FP8 MFMA --------------------------
    if (!__all(alpha == 1.0f)) {  // a row max moved somewhere in this wave
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i32x8 va = *reinterpret_cast<const i32x8*>(smem_v + (2 * c + h) * (kD * 32) +
                                                        (32 * dt + col) * 32);
        o[dt] = mfma32_fp8(va, pb[c], o[dt]);
      }
    }
  }

  // ---- epilogue -----------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_row < N) {
    const float inv = sV / l_tot;
    const int64_t obase = ((int64_t)bh * N + my_row) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        const float a0 = o[dt][4 * g] * inv, a1 = o[dt][4 * g + 1] * inv;
        const float a2 = o[dt][4 * g + 2] * inv, a3 = o[dt][4 * g + 3] * inv;
        if (p.out_bf16) {
          uint2 w;
          w.x = bf16_rne(a0) | (bf16_rne(a1) << 16);
          w.y = bf16_rne(a2) | (bf16_rne(a3) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + obase + d0) = w;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + obase + d0) =
              make_float4(a0, a1, a2, a3);
        }
      }
    if (p.lse && h == 0)
      p.lse[(int64_t)bh * N + my_row] =
          kLn2 * (lam * m_run + log2f(l_tot)) - kLn2 * kLog2_448 + lse_off;
  }
}

void launch_prefill(const PrefillParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((int64_t)p.n_qtiles * p.B * p.Hq);
  hipLaunchKernelGGL(k_prefill, dim3(grid), dim3(256), 0, st, p);
}

}  // namespace mpfa
