// Causal / full QK4PV8 prefill for gfx950 (paper "MpFA: ...", section 5.1
// "second stage", section 5.2 "MMA Compensation", section 4.1).
//
// Work unit: one (batch, query head, 128-row query tile); 4 waves of 32 rows;
// two workgroups share a CU (<= 256 VGPRs per wave), so one workgroup's
// softmax overlaps the other's matrix products.  Per 128-key block:
//   * the workgroup expands the NVFP4 K block into exact FP16 operands
//     (code value x E4M3 block scale) in LDS and copies the FP8 V tiles and
//     the block's Delta_S into LDS; the global loads of block j+1 are issued
//     before block j is computed;
//   * each wave computes S^T (keys x its 32 queries) on MFMA: with
//     smoothing, a first bf16 step writes Delta_S * (1 / (gQ gK)) into the
//     accumulator (the rank-one term of section 5.2 -- no element-wise add on
//     the softmax path), then 8 f16 steps accumulate Q~ K~^T over the head
//     dimension, the four 32-key tiles interleaved so no step waits on the
//     previous one;
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
constexpr int kQStride = 272;  // bytes per LDS row of the prologue's Q~ (128 f16 + padding)
// K~ in LDS: 256-byte rows whose 16 chunks of 16 bytes are permuted by key:
// chunk c of key k sits at c ^ kswz(k).  A 16-lane pass of an operand read
// touches keys {0-3, 32-35, 4-7, 36-39} + base of one chunk column, and
// kswz gives those keys 16 distinct chunk slots, so no two lanes of a pass
// share a bank; the expansion writes (keys 0-7, both halves) spread too.
__device__ __forceinline__ int kswz(int k) { return (k & 7) | (((k >> 5) & 1) << 3); }
// V in LDS: [4 tiles][2 halves][128 channels][16 bytes]: each lane's two
// 16-byte reads are then contiguous across lanes (no bank conflicts).
constexpr int kVTileBytes = kD * 32;

template <bool SMOOTH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(
    PrefillParams p) {
  __shared__ __align__(16) uint8_t smem_k[kQTile * kQStride];  // K~ block (Q~ in the prologue)
  __shared__ __align__(16) uint8_t smem_v[4 * kVTileBytes];    // V block
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

  const float gQ = nvfp4_global_scale(__uint_as_float(*p.q_amax));
  const float gK = *p.k_gscale;
  const float sV = *p.v_scale;
  const float gg = gQ * gK;
  const float lam = p.scale * kLog2e * gg;  // exp2 constant per unit of the MFMA score

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
      if (SMOOTH) {
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
    uint4* dst = reinterpret_cast<uint4*>(smem_k + r * kQStride + blk * 32);
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
    qf[kc] = *reinterpret_cast<const i32x4*>(smem_k + qr * kQStride + (64 * h + 8 * kc) * 2);
  float lse_off = 0.0f;
  if (SMOOTH && p.lse) {
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) lse_off += lse_part[qr * 8 + blk];
    lse_off *= p.scale;
  }
  // Constant B operand of the rank-one step: slots 0..2 of lane half 0 hold
  // 1 / (gQ gK) as the sum of three bf16 parts (exact to fp32 precision);
  // the A operand repeats Delta_S[key] in the same slots.
  i32x4 dB = {0, 0, 0, 0};
  if (SMOOTH) {
    const float cinv = 1.0f / gg;
    const uint32_t c_hi = bf16_rne(cinv);
    const float r1 = cinv - __uint_as_float(c_hi << 16);
    const uint32_t c_mid = bf16_rne(r1);
    const uint32_t c_lo = bf16_rne(r1 - __uint_as_float(c_mid << 16));
    dB = i32x4{h == 0 ? (int)(c_hi | (c_mid << 16)) : 0, h == 0 ? (int)c_lo : 0, 0, 0};
  }

  const int my_row = row0 + qr;
  const int nblk_all = (N + kBlk - 1) / kBlk;
  const int nblk = p.causal ? min(tile + 1, nblk_all) : nblk_all;
  const int ntiles32 = (N + 31) / 32;
  const int64_t kvh = (int64_t)b * p.Hkv + hk;
  const uint8_t* kbase = p.k_fp4 + kvh * N * 64;
  const uint8_t* sbase = p.k_sf + kvh * N * 8;
  const uint8_t* vbase = p.v_fp8 + kvh * ntiles32 * kVTileBytes;
  const uint16_t* dbase = SMOOTH ? p.delta_s + (int64_t)bh * N : nullptr;

  // A-row rho of score tile t holds key 64*(t/2) + 32*hp + 16*(t%2) + vp of
  // the block (hp, vp from rho below); the MFMA output register v of lane
  // half h then holds key 64*(t/2) + 32*h + 16*(t%2) + v.
  const int hp = (col >> 2) & 1, vp = ((col >> 3) << 2) | (col & 3);
  int koff[4], ksw[4];
  const uint8_t* krow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    koff[t] = 64 * (t >> 1) + 32 * hp + 16 * (t & 1) + vp;
    ksw[t] = kswz(koff[t]);
    krow[t] = smem_k + koff[t] * 256;
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};

  // Per-thread share of a block's loads: K codes of (key, head-dim half),
  // 16 bytes of each of the 4 V tiles, one Delta_S entry.  Indices past the end
  // are clamped to the last token: those keys are masked out of the block,
  // so the (finite) values read there never reach the result.
  const int ld_key = tid >> 1, ld_half = tid & 1;
  // V: thread tid moves 16-byte unit (channel tid % 128, half tid / 128) of
  // each tile, global unit 2 * channel + half, so its LDS stores are
  // contiguous across lanes.
  const int vsrc = 2 * (tid & 127) + (tid >> 7);
  uint4 kc0, kc1, vv0, vv1, vv2, vv3;
  uint32_t ksc, dd = 0;
#define MPFA_PREFILL_LOAD(JB)                                                                 \
  do {                                                                                        \
    const int kb0 = (JB) * kBlk;                                                              \
    const int gk = min(kb0 + ld_key, N - 1);                                                  \
    const uint4* src = reinterpret_cast<const uint4*>(kbase + (int64_t)gk * 64 + 32 * ld_half); \
    kc0 = src[0];                                                                             \
    kc1 = src[1];                                                                             \
    ksc = *reinterpret_cast<const uint32_t*>(sbase + (int64_t)gk * 8 + 4 * ld_half);          \
    const int tt0 = kb0 / 32;                                                                 \
    vv0 = reinterpret_cast<const uint4*>(vbase + (int64_t)min(tt0 + 0, ntiles32 - 1) * kVTileBytes)[vsrc]; \
    vv1 = reinterpret_cast<const uint4*>(vbase + (int64_t)min(tt0 + 1, ntiles32 - 1) * kVTileBytes)[vsrc]; \
    vv2 = reinterpret_cast<const uint4*>(vbase + (int64_t)min(tt0 + 2, ntiles32 - 1) * kVTileBytes)[vsrc]; \
    vv3 = reinterpret_cast<const uint4*>(vbase + (int64_t)min(tt0 + 3, ntiles32 - 1) * kVTileBytes)[vsrc]; \
    if (SMOOTH && tid < kBlk) dd = dbase[min(kb0 + tid, N - 1)];                              \
  } while (0)
  MPFA_PREFILL_LOAD(0);

  for (int j = 0; j < nblk; ++j) {
    const int k0 = j * kBlk;
    __syncthreads();  // every wave is done with the previous block's LDS tiles
    {
      const uint32_t w[8] = {kc0.x, kc0.y, kc0.z, kc0.w, kc1.x, kc1.y, kc1.z, kc1.w};
      uint8_t* dst = smem_k + ld_key * 256;
      const int sw = kswz(ld_key);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t e[4];
        expand_fp4x8(w[i], e4m3_scale_f16x2((ksc >> (8 * (i >> 1))) & 0xFFu), e);
        *reinterpret_cast<uint4*>(dst + 16 * ((8 * ld_half + i) ^ sw)) =
            make_uint4(e[0], e[1], e[2], e[3]);
      }
      const int voff = tid * 16;  // = half * 2048 + channel * 16
      *reinterpret_cast<uint4*>(smem_v + 0 * kVTileBytes + voff) = vv0;
      *reinterpret_cast<uint4*>(smem_v + 1 * kVTileBytes + voff) = vv1;
      *reinterpret_cast<uint4*>(smem_v + 2 * kVTileBytes + voff) = vv2;
      *reinterpret_cast<uint4*>(smem_v + 3 * kVTileBytes + voff) = vv3;
      if (SMOOTH && tid < kBlk) smem_delta[tid] = (uint16_t)dd;
    }
    __syncthreads();
    if (j + 1 < nblk) MPFA_PREFILL_LOAD(j + 1);

    // ---- scores S^T: 4 tiles of 32 keys x 32 queries --------------------
    f32x16 s[4];
    if (SMOOTH) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t dv = smem_delta[koff[t]];
        const i32x4 dA = {h == 0 ? (int)(dv | (dv << 16)) : 0, h == 0 ? (int)dv : 0, 0, 0};
        s[t] = mfma32_bf16(dA, dB, f32x16{});
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        s[t] = mfma32_f16(*reinterpret_cast<const i32x4*>(krow[t] + 16 * ((8 * h) ^ ksw[t])),
                          qf[0], f32x16{});
    }
#pragma unroll
    for (int kc = SMOOTH ? 0 : 1; kc < 8; ++kc)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        s[t] = mfma32_f16(
            *reinterpret_cast<const i32x4*>(krow[t] + 16 * ((8 * h + kc) ^ ksw[t])), qf[kc], s[t]);

    // ---- mask (diagonal or ragged block only) and online softmax --------
    const bool need_mask = (p.causal && k0 + kBlk > row0) || (k0 + kBlk > N);
    if (need_mask) {
      const int lim = p.causal ? min(my_row, N - 1) : N - 1;  // last visible key
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + 64 * (t >> 1) + 32 * h + 16 * (t & 1) + v;
          s[t][v] = key <= lim ? s[t][v] : -INFINITY;
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
    for (int c = 0; c < 2; ++c) {
      const uint8_t* vt = smem_v + (2 * c + h) * kVTileBytes + col * 16;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(vt + dt * 512);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(vt + kD * 16 + dt * 512);
        const i32x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma32_fp8(va, pb[c], o[dt]);
      }
    }
  }

  // ---- epilogue -----------------------------------------------------------
  // An MFMA reads its operands from all 64 lanes whatever the execution mask,
  // while loads honour it; so nothing that feeds the accumulators may be moved
  // into a branch on the row.  Every lane normalises, only the stores of rows
  // past the end are skipped.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = sV / l_tot;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] *= inv;
  const bool row_ok = my_row < N;
  const int64_t obase = ((int64_t)bh * N + min(my_row, N - 1)) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * dt + 8 * g + 4 * h;
      const float a0 = o[dt][4 * g], a1 = o[dt][4 * g + 1];
      const float a2 = o[dt][4 * g + 2], a3 = o[dt][4 * g + 3];
      if (p.out_bf16) {
        uint2 w;
        w.x = bf16_rne(a0) | (bf16_rne(a1) << 16);
        w.y = bf16_rne(a2) | (bf16_rne(a3) << 16);
        if (row_ok) *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + obase + d0) = w;
      } else if (row_ok) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + obase + d0) =
            make_float4(a0, a1, a2, a3);
      }
    }
  if (p.lse && h == 0 && row_ok)
    p.lse[(int64_t)bh * N + my_row] =
        kLn2 * (lam * m_run + log2f(l_tot)) - kLn2 * kLog2_448 + lse_off;
}

#undef MPFA_PREFILL_LOAD

void launch_prefill(const PrefillParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((int64_t)p.n_qtiles * p.B * p.Hq);
  if (p.delta_s)
    hipLaunchKernelGGL(k_prefill<true>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(k_prefill<false>, dim3(grid), dim3(256), 0, st, p);
}

}  // namespace mpfa
