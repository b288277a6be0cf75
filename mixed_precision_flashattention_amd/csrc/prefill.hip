// Causal / full QK4PV8 prefill for gfx950 (paper "MpFA: ...", section 5.1
// "second stage", section 5.2 "MMA Compensation", section 4.1).
//
// A pre-pass expands the NVFP4 K cache once per call into exact FP16
// operands K~ = E2M1 code value x E4M3 block scale (at most 6 significant
// bits, range [2^-10, 2688]: exact in FP16; the per-tensor global scale stays
// out and is folded into the exp2 constant).
//
// Work unit: one (batch, query head, 256-row query tile) per workgroup of 8
// waves, one workgroup per CU.  The waves form two row groups of 4 (rows
// 0-127 and 128-255, 32 rows per wave), and each SIMD holds one wave of each
// group.  The groups alternate between workgroup barriers: one runs its
// matrix products while the other runs its softmax, so the matrix cores and
// the vector ALUs of a SIMD work at the same time.  Per 128-key block:
//   * K~ block images and the FP8 V tiles reach LDS by direct global->LDS
//     loads (no registers, no VALU address work), double-buffered and issued
//     one block ahead; Delta_S goes through the registers of the first 128
//     threads, which store it to LDS as Delta_S * (1 / (gQ gK)) in fp32;
//   * each wave computes S^T (keys x its 32 queries) on MFMA: with
//     smoothing, the score accumulators start at Delta_S * (1 / (gQ gK)),
//     read from LDS as the first MFMA's accumulator input (section 5.2's
//     compensation inside the matrix product -- no element-wise add on the
//     softmax path and no matrix step of its own), then 8 f16 steps
//     accumulate Q~ K~^T over the head dimension, the four 32-key tiles
//     interleaved so no step waits on the previous one; Q~ stays in
//     registers for the whole loop;
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

constexpr int kUnitRows = 256;  // query rows per workgroup (two groups of 128)
constexpr int kRowBytes = 256;  // one Q~ row in LDS: 128 f16
// K~ block image (32 KB per 128 keys, the same bytes in the workspace and in
// LDS): 16 chunk columns of 2 KB, one per 8 head-dim elements; chunk c of
// key k sits at c * 2048 + 16 k.  An operand read of head-dim step kc is
// then a per-lane base plus the immediate kc * 2048 (no address arithmetic
// per read), and a direct load is a contiguous 1 KB copy.  The lanes of an
// operand read touch keys {0-3, 32-35, 4-7, 36-39, ...} + base of one
// column: with keys in consecutive 16-byte slots that read is free of bank
// conflicts on gfx950 (measured with the bank-conflict counter on this very
// address pattern; moving keys 32-63 by 8 slots made every read a 2-way
// conflict).
constexpr int kKChunkBytes = kBlk * 16;
constexpr int kKBlockBytes = kBlk * kRowBytes;
// V in LDS: [4 tiles][2 halves][128 channels][16 bytes]: each lane's two
// 16-byte reads are then contiguous across lanes (no bank conflicts).
constexpr int kVTileBytes = kD * 32;
constexpr int kVBlockBytes = 4 * kVTileBytes;
// bf16 V (the bf16 P.V variant): 32-token tiles of 8 KB, 32 KB per block.
constexpr int kVBf16TileBytes = kD * 32 * 2;
constexpr int kVBf16BlockBytes = 4 * kVBf16TileBytes;

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds_addr + 16 i (lds_addr wave-uniform).  Written as inline assembly so the
// compiler's wait-count pass does not treat every later LDS read as
// dependent on it; the kernel waits for these loads itself before the
// barrier that publishes a block.
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory");
}
// The same with a uniform 64-bit base in SGPRs and a non-negative 32-bit
// per-lane offset (the scalar-base form adds the offset zero-extended).
__device__ __forceinline__ void lds_load16_s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void wait_direct_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Wave w's share of K~ block image kimg when NW waves load it: 1 KB pieces
// 32/NW w .. 32/NW (w+1) - 1, each a contiguous copy (lane i moves bytes
// 16 i .. 16 i + 15 of the piece).
template <int NW>
__device__ __forceinline__ void issue_k_block(const uint8_t* kimg, uint32_t dst, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int piece = (32 / NW) * w + i;
    lds_load16_s(kimg + piece * 1024, 16 * lane, dst + piece * 1024);
  }
}

// Wave w's share of V block k0 when NW waves load it: 1 KB pieces
// 16/NW w .. 16/NW (w+1) - 1, each a contiguous copy (the cache's 32-token
// tiles have the layout the P.V operands are read with: [half][channel][16
// tokens]); tiles past the cache are clamped to its last tile (their keys
// are masked).
template <int NW>
__device__ __forceinline__ void issue_v_block(const uint8_t* vbase, int ntiles32, int k0,
                                              uint32_t dst, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int piece = (16 / NW) * w + i;
    const int t = piece >> 2;
    const int tt = min(k0 / 32 + t, ntiles32 - 1);
    lds_load16_s(vbase + (int64_t)tt * kVTileBytes + (piece & 3) * 1024, 16 * lane,
                 dst + piece * 1024);
  }
}

// The same for a bf16 V block (32 KB: 4 tiles of 8 KB, 1 KB pieces), wave w
// moving pieces 32/NW w .. 32/NW (w+1) - 1; tiles past the cache are clamped
// to its last tile (their keys are masked).
template <int NW>
__device__ __forceinline__ void issue_v_block_bf16(const uint8_t* vbase, int ntiles32, int k0,
                                                   uint32_t dst, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int piece = (32 / NW) * w + i;
    const int t = piece >> 3, part = piece & 7;
    const int tt = min(k0 / 32 + t, ntiles32 - 1);
    lds_load16(vbase + (int64_t)tt * kVBf16TileBytes + part * 1024 + 16 * lane,
               dst + t * kVBf16TileBytes + part * 1024);
  }
}

// Workgroup -> (256-row query unit, batch, query head).  Workgroups are dealt
// to the 8 XCDs round-robin; when the KV heads split evenly, XCD x takes KV
// heads x, x + 8, ... with all their query heads and units, so one L2 serves
// each KV head, and inside an XCD the heaviest (last) units go first
// (longest-processing-time order, paper section 5.1).  Otherwise the order
// is the plain LPT one over all heads.
__device__ __forceinline__ void prefill_unit(const PrefillParams& p, int wid, int& unit, int& b,
                                             int& hq) {
  const int nkv = p.B * p.Hkv;
  if ((nkv & 7) == 0) {
    const int x = wid & 7, slot = wid >> 3;
    const int per_unit = (nkv >> 3) * p.G;
    unit = p.n_units - 1 - slot / per_unit;
    const int r = slot % per_unit;
    const int g = x + 8 * (r / p.G);
    b = g / p.Hkv;
    hq = (g % p.Hkv) * p.G + r % p.G;
  } else {
    const int nbh = p.B * p.Hq;
    unit = p.n_units - 1 - wid / nbh;
    const int bh = wid % nbh;
    b = bh / p.Hq;
    hq = bh % p.Hq;
  }
}

// Scores S^T of one 128-key block: 4 tiles of 32 keys x the wave's 32 queries.
// The K~ operands of head-dim step kc + 1 are read from LDS while the four
// MFMAs of step kc run (the scheduling barriers keep the reads that early),
// so the matrix core does not wait on LDS latency.  COMP selects how the
// compensation column term enters the accumulator before the products:
//   0: not at all (direct mode);
//   1: a rank-one bf16 MFMA step, A = the bf16 term of each key (comp: bf16
//      per key), B = 1/(gQ gK) in three bf16 parts (dB);
//   2: as the first product's accumulator input (comp: term x 1/(gQ gK) in
//      fp32 per key): lane half h's output register v of tile t is key
//      64(t/2) + 32h + 16(t%2) + v, so a tile's inputs are four 16-byte
//      reads of consecutive keys, the same for every lane of the half.
template <int COMP, bool BF16>
__device__ __forceinline__ void score_block(f32x16 (&s)[4], const uint8_t* kblk,
                                            const void* comp, const int (&koff)[4],
                                            const int (&kbase)[4], const i32x4 (&qf)[8],
                                            const i32x4& dB, int h) {
  const uint8_t* at[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) at[t] = kblk + kbase[t];
  i32x4 a[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a[0][t] = *reinterpret_cast<const i32x4*>(at[t]);
  if constexpr (COMP == 1) {
    const uint16_t* dblk = static_cast<const uint16_t*>(comp);
    uint32_t dv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dv[t] = dblk[koff[t]];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x4 dA = {h == 0 ? (int)(dv[t] | (dv[t] << 16)) : 0, h == 0 ? (int)dv[t] : 0, 0, 0};
      s[t] = mfma32_bf16(dA, dB, f32x16{});
    }
  } else if constexpr (COMP == 2) {
    const float* dsc = static_cast<const float*>(comp) + 32 * h;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4* src = reinterpret_cast<const f32x4*>(dsc + 64 * (t >> 1) + 16 * (t & 1));
      const f32x4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
      s[t] = f32x16{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                    c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
    }
  }
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    if (kc + 1 < 8) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[(kc + 1) & 1][t] = *reinterpret_cast<const i32x4*>(at[t] + (kc + 1) * kKChunkBytes);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x16 c = (COMP != 0 || kc > 0) ? s[t] : f32x16{};
      s[t] = BF16 ? mfma32_bf16(a[kc & 1][t], qf[kc], c) : mfma32_f16(a[kc & 1][t], qf[kc], c);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Precision / placement variants of the smoothing-mode kernel (the paper's
// section 3.1 and 7.4 comparisons, built as separate kernels; the library's
// calls use kVarNone):
//   kVarElementwise: Delta_S * 1/(gQ gK) added to each score on the VALU at
//     the start of the softmax, instead of entering the score accumulator;
//   kVarRankOne: the term written into the score accumulator by a rank-one
//     bf16 MFMA step per tile (A = Delta_S per key, B = 1/(gQ gK) in three
//     bf16 parts) instead of read from LDS as its input;
//   kVarPolyExp2: one exponential in four evaluated by a cubic on the FMA
//     path instead of the hardware exp2 (the split the paper's B200 kernel
//     uses to relieve its transcendental unit);
//   kVarPvBf16: P rounded to bf16 and V from a bf16 cache, P.V on bf16 MFMA
//     (the NVFP4 + BF16 precision assignment);
//   kVarPvNvfp4: P quantized to NVFP4 per 16 keys on the softmax path (amax,
//     E4M3 scale, correctly rounded quotients, E2M1 codes; global scale
//     fp32(1/2688)) and V from an NVFP4 cache with 16-key blocks, both
//     expanded to exact FP16 values (code x block scale) so that P.V runs
//     on f16 MFMA (the NVFP4 + NVFP4 precision assignment: gfx950's
//     block-scaled FP4 MFMA takes power-of-two scales per 32 elements, not
//     E4M3 scales per 16).
// P of one block as the B operands of the P.V products: E4M3, 32 keys per
// 32x32x64 operand (64 bytes per lane), or bf16 for the bf16 variant, 8 keys
// per 32x32x16 operand (128 bytes per lane): w[t][u] holds keys 8u .. 8u + 7
// of the lane's 16 keys of score tile t.
template <int VAR>
struct PRegs {
  i32x8 w[2];
};
template <>
struct PRegs<kVarPvBf16> {
  i32x4 w[4][2];
};
template <>
struct PRegs<kVarPvNvfp4> {  // the same layout, FP16 values
  i32x4 w[4][2];
};

// 2^x for the FMA path of kVarPolyExp2: x = r + f with r = rint(x), f in
// [-1/2, 1/2]; 2^f by a cubic whose coefficients are a minimax fit of the
// relative error on that interval (Lawson-weighted least squares on 20001
// points; largest relative error 7.5e-5 evaluated in fp32 Horner form), then
// scaled by 2^r.  Arguments below -126 are clamped (the result underflows to
// zero in every P format anyway).
__device__ __forceinline__ float poly_exp2(float x) {
  constexpr float c0 = 0x1.fff694p-1f, c1 = 0x1.62f31ap-1f, c2 = 0x1.f0ddccp-3f, c3 = 0x1.c3f6a6p-5f;
  x = fmaxf(x, -126.0f);
  const float r = __builtin_rintf(x);
  const float f = x - r;
  const float p = fmaf(fmaf(fmaf(c3, f, c2), f, c1), f, c0);
  return __builtin_ldexpf(p, (int)r);
}

// Two fp32 -> two bf16 (round to nearest even) in one word, low half first.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// bf16 V in LDS (kVarPvBf16): [4 tiles of 32 keys][4 groups of 8 keys]
// [128 channels][8 keys] bf16 -- the same bytes as the bf16 V cache's tiles,
// so a block is one contiguous 32 KB copy; a lane's operand is the 8 keys of
// one channel (16 bytes), consecutive lanes read consecutive 16-byte slots.
__device__ __forceinline__ i32x4 v_operand_bf16(const uint8_t* vblk, int i, int h, int col) {
  const int ku = i >> 2, dt = i & 3, t = ku >> 1, u = ku & 1;
  return *reinterpret_cast<const i32x4*>(vblk + (2 * (t >> 1) + h) * kVBf16TileBytes +
                                         (2 * (t & 1) + u) * (kD * 16) + (32 * dt + col) * 16);
}
// O^T += V^T P^T for one block on bf16 (or, F16, f16) MFMA (32 MFMAs: 8 key
// steps of 16 x 4 head-dim tiles); the V operand of MFMA i + 1 is read while
// MFMA i runs.  The k slots of a step are keys 8u .. 8u + 7 of tile t in lane
// half 0 and the same offsets 32 keys on in lane half 1, matching the P
// operand's keys.
template <bool F16>
__device__ __forceinline__ void pv_block_16(f32x16 (&o)[4], const uint8_t* vblk,
                                            const i32x4 (&w)[4][2], int h, int col) {
  i32x4 va[2];
  va[0] = v_operand_bf16(vblk, 0, h, col);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i + 1 < 32) va[(i + 1) & 1] = v_operand_bf16(vblk, i + 1, h, col);
    __builtin_amdgcn_sched_barrier(0);
    const int ku = i >> 2;
    o[i & 3] = F16 ? mfma32_f16(va[i & 1], w[ku >> 1][ku & 1], o[i & 3])
                   : mfma32_bf16(va[i & 1], w[ku >> 1][ku & 1], o[i & 3]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P^T for one block on the FP8 MFMA (8 MFMAs: key half c, head-dim
// tile dt); the V operand of MFMA i + 1 is read while MFMA i runs.
__device__ __forceinline__ i32x8 v_operand(const uint8_t* vblk, int i, int h, int col) {
  const int c = i >> 2, dt = i & 3;
  const uint8_t* vt = vblk + (2 * c + h) * kVTileBytes + col * 16 + dt * 512;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(vt);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(vt + kD * 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int VAR>
__device__ __forceinline__ void pv_block(f32x16 (&o)[4], const uint8_t* vblk, const PRegs<VAR>& pr,
                                         int h, int col) {
  if constexpr (VAR == kVarPvBf16 || VAR == kVarPvNvfp4) {
    pv_block_16<VAR == kVarPvNvfp4>(o, vblk, pr.w, h, col);
  } else {
    i32x8 va[2];
    va[0] = v_operand(vblk, 0, h, col);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 1 < 8) va[(i + 1) & 1] = v_operand(vblk, i + 1, h, col);
      __builtin_amdgcn_sched_barrier(0);
      o[i & 3] = mfma32_fp8(va[i & 1], pr.w[i >> 2], o[i & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Reductions over the lane pair (l, l ^ 32) by one register swap of the lane
// halves: afterwards the first register holds the low lane's value and the
// second the high lane's, in both lanes, so both get the same result.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Mask, online softmax and E4M3 rounding of P for one block; rescales the
// output accumulators when a row max moved.  kVarElementwise first adds
// Delta_S * cinv to every score (dblk: the block's Delta_S entries), the
// other variants change the exponential or P's format.
template <int VAR>
__device__ __forceinline__ void softmax_block(f32x16 (&s)[4], f32x16 (&o)[4], PRegs<VAR>& pr,
                                              float& m_run, float& l_run, float lam, bool mask,
                                              int k0, int lim, int h, const uint16_t* dblk,
                                              float cinv) {
  if constexpr (VAR == kVarElementwise) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // the lane's 16 consecutive keys of tile t: 32 bytes
      const i32x4* dp = reinterpret_cast<const i32x4*>(dblk + 64 * (t >> 1) + 32 * h + 16 * (t & 1));
      const i32x4 d0 = dp[0], d1 = dp[1];
      const uint32_t dw[8] = {(uint32_t)d0[0], (uint32_t)d0[1], (uint32_t)d0[2], (uint32_t)d0[3],
                              (uint32_t)d1[0], (uint32_t)d1[1], (uint32_t)d1[2], (uint32_t)d1[3]};
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float dv = __uint_as_float((v & 1) ? (dw[v >> 1] & 0xFFFF0000u) : (dw[v >> 1] << 16));
        s[t][v] = fmaf(dv, cinv, s[t][v]);
      }
    }
  }
  if (mask) {
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
  mx = max_halves(mx);
  const float m_new = fmaxf(m_run, mx);
  const float alpha = fast_exp2(lam * (m_run - m_new));
  m_run = m_new;
  if constexpr (VAR == kVarPvNvfp4) {
    // p itself (no 448 in the exponent): each 16-key score tile row is one
    // NVFP4 group of P, quantized as the query blocks are and expanded to
    // FP16 code value x block scale for the f16 P.V MFMA
    const float nb = -lam * m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float e[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(s[t][v], lam, nb));
#pragma unroll
      for (int v = 0; v < 16; v += 4) lsum += (e[v] + e[v + 1]) + (e[v + 2] + e[v + 3]);
      uint32_t w[2], pk[8];
      const uint32_t sc = nvfp4_block_packed(e, kNvfp4PScale, w);
      const f16x2 s2 = e4m3_scale_f16x2(sc);
      expand_fp4x8(w[0], s2, pk);
      expand_fp4x8(w[1], s2, pk + 4);
      pr.w[t][0] = i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
      pr.w[t][1] = i32x4{(int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
    }
    l_run = fmaf(alpha, l_run, lsum);
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    return;
  }
  const float nb = kLog2_448 - lam * m_new;

  float lsum;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = 2 * c + (k >> 2), v0 = 4 * (k & 3);
      const float e0 = fast_exp2(fmaf(s[t][v0], lam, nb));
      const float e1 = fast_exp2(fmaf(s[t][v0 + 1], lam, nb));
      const float e2 = fast_exp2(fmaf(s[t][v0 + 2], lam, nb));
      const float e3 = VAR == kVarPolyExp2 ? poly_exp2(fmaf(s[t][v0 + 3], lam, nb))
                                           : fast_exp2(fmaf(s[t][v0 + 3], lam, nb));
      const float part = (e0 + e1) + (e2 + e3);
      lsum = (c == 0 && k == 0) ? part : lsum + part;
      if constexpr (VAR == kVarPvBf16) {
        const int u = (k & 3) >> 1, wi = 2 * (k & 1);
        pr.w[t][u][wi] = (int)cvt_bf16x2(e0, e1);
        pr.w[t][u][wi + 1] = (int)cvt_bf16x2(e2, e3);
      } else {
        // The low half is written first and the high half second, so the
        // register's old content does not matter; e0, which dies here, lets
        // the compiler convert in place (a constant 0, or a value still live
        // such as part, costs a move per word).
        uint32_t wd = cvt_fp8x2<false>(e0, e1, __float_as_uint(e0));
        wd = cvt_fp8x2<true>(e2, e3, wd);
        pr.w[c][k] = (int)wd;
      }
    }
  }
  l_run = fmaf(alpha, l_run, lsum);
  if (!__all(alpha == 1.0f)) {  // a row max moved somewhere in this wave
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
  }
}

// Per-tile mode: Delta_tile of the 32 keys of score tile t of a K~ block for
// this wave's query tile, rounded to bf16, as the score accumulator's input
// fp32(Delta_tile * cinv) per key in dst[key].  A = the
// tile mean split exactly into three bf16 parts (rows 0, 1, 2 of the A
// operand; the other rows zero), B = the K~ operands of tile t, the same
// registers the score product uses as its A operand (an A operand read as B
// is the transposed tile), so D row r, column c = part r . K~[key of c];
// rows 0-2 land in registers 0-2 of lanes 0-31.  The three partial products
// are exact in FP32 (8 x 6 significant bits); they are summed in FP32, scaled
// by the K global scale and rounded once to bf16.
__device__ __forceinline__ float tile_delta_input(float d, float gK, float cinv) {
  return __uint_as_float(bf16_rne(d * gK) << 16) * cinv;
}
__device__ __forceinline__ void tile_delta(const uint8_t* kblk, const uint8_t* qop, int kbase_t,
                                           int koff_t, float gK, float cinv, int lane, float* dst) {
  const uint8_t* at = kblk + kbase_t;
  const bool data = (lane & 31) < 3;
  // lane (r, h) reads the 8 parts of row r for the head-dim slots of half h
  const uint8_t* qa = qop + ((lane >> 5) * 3 + (lane & 31)) * 16;
  f32x16 d = f32x16{};
  i32x4 b[2], a[2];
  b[0] = *reinterpret_cast<const i32x4*>(at);
  a[0] = data ? *reinterpret_cast<const i32x4*>(qa) : i32x4{0, 0, 0, 0};
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    if (kc + 1 < 8) {
      b[(kc + 1) & 1] = *reinterpret_cast<const i32x4*>(at + (kc + 1) * kKChunkBytes);
      a[(kc + 1) & 1] = data ? *reinterpret_cast<const i32x4*>(qa + (kc + 1) * 96) : i32x4{0, 0, 0, 0};
    }
    d = mfma32_bf16(a[kc & 1], b[kc & 1], d);
  }
  if (lane < 32) dst[koff_t] = tile_delta_input((d[0] + d[1]) + d[2], gK, cinv);
}

// The same for both row groups' query tiles in one product: rows 0-2 of the
// A operand hold group 0's tile mean parts and rows 4-6 group 1's, so D rows
// 0-2 land in registers 0-2 of lanes 0-31 and rows 4-6 in registers 0-2 of
// lanes 32-63 (each lane half then holds its group's three partial products
// for the key of its column, summed and rounded exactly as above).
__device__ __forceinline__ void tile_delta_pair(const uint8_t* kblk, const uint8_t* qop,
                                                int kbase_t, int koff_t, float gK, float cinv,
                                                int lane, float* dst0, float* dst1) {
  const uint8_t* at = kblk + kbase_t;
  const int r = lane & 31, g = r >> 2, part = r & 3;
  const bool data = r < 7 && part < 3;
  // lane (r, h) reads the 8 parts of row r for the head-dim slots of half h
  // (lanes of the zero rows keep a base inside the array)
  const uint8_t* qa = qop + (data ? g * 768 + part * 16 : 0) + (lane >> 5) * 48;
  f32x16 d = f32x16{};
  i32x4 b[2], a[2];
  b[0] = *reinterpret_cast<const i32x4*>(at);
  a[0] = data ? *reinterpret_cast<const i32x4*>(qa) : i32x4{0, 0, 0, 0};
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    if (kc + 1 < 8) {
      b[(kc + 1) & 1] = *reinterpret_cast<const i32x4*>(at + (kc + 1) * kKChunkBytes);
      a[(kc + 1) & 1] = data ? *reinterpret_cast<const i32x4*>(qa + (kc + 1) * 96) : i32x4{0, 0, 0, 0};
    }
    d = mfma32_bf16(a[kc & 1], b[kc & 1], d);
  }
  (lane < 32 ? dst0 : dst1)[koff_t] = tile_delta_input((d[0] + d[1]) + d[2], gK, cinv);
}

// Work unit: 256 query rows of one (batch, head) in two groups of 4 waves
// (rows 0-127 and 128-255); each SIMD holds one wave of each group.  The
// groups take turns: between two workgroup barriers one group runs its
// matrix products (P.V of block j-1, then the scores of block j) while the
// other runs the softmax of its previous block, so the matrix cores and the
// vector ALUs of every SIMD are busy at the same time.  Both groups read
// the same K~ / V / Delta_S blocks from LDS (double-buffered, loaded two
// steps ahead by all 8 waves).
// MODE 0: direct; 1: smoothing by the sequence means, Delta_S entering the
// score accumulator; 2: per-tile means: the column term Delta_tile[j] =
// Qbar_tile . K~_c[j] is computed here, one block ahead, and enters the
// score accumulator the same way (BF16 K~ images and query operands, K~
// blocks triple-buffered so the next block is resident while the current
// one is scored).
template <int MODE, int VAR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(
    PrefillParams p) {
  constexpr bool SMOOTH = MODE == 1, TILE = MODE == 2;
  // The compensation term (Delta_S, or Delta_tile in the per-tile mode) times
  // 1/(gQ gK) is the score accumulator's input (section 5.2's compensation
  // inside the matrix product, without an MMA step of its own); kVarRankOne
  // writes it by a rank-one bf16 MMA step, kVarElementwise adds it in the
  // softmax.
  constexpr bool RANK1 = SMOOTH && VAR == kVarRankOne;
  constexpr bool CINIT = (SMOOTH && VAR != kVarElementwise && !RANK1) || TILE;
  constexpr bool DELTA16 = SMOOTH && !CINIT;  // bf16 Delta_S in LDS
  constexpr int COMP = CINIT ? 2 : (RANK1 ? 1 : 0);
  constexpr bool PV16 = VAR == kVarPvBf16 || VAR == kVarPvNvfp4;  // 16-bit V blocks
  constexpr int NKB = TILE ? 3 : 2;       // K~ block buffers
  __shared__ __align__(16) uint8_t smem_k[NKB][kBlk * kRowBytes];  // K~ blocks
  __shared__ __align__(16) uint8_t smem_v[2][PV16 ? kVBf16BlockBytes : kVBlockBytes];  // V blocks
  // bf16 Delta_S of the rank-one and element-wise variants, [buffer][key]
  __shared__ __align__(16) uint16_t smem_delta[2][DELTA16 ? kBlk : 1];
  // the accumulator input term x 1/(gQ gK) in fp32: smoothing [buffer][0][key],
  // per-tile mode [buffer][row group][key]
  __shared__ __align__(16) float smem_comp[CINIT ? 2 : 1][TILE ? 2 : 1][CINIT ? kBlk : 4];
  // per-tile mode: the tile means' bf16 parts as score-operand rows,
  // [row group][kc][lane half][part][8 bf16]
  __shared__ __align__(16) uint8_t smem_qop[TILE ? 2 * 8 * 2 * 3 * 16 : 16];

  const int N = p.N;
  int unit, b, hq;
  prefill_unit(p, blockIdx.x, unit, b, hq);
  const int bh = b * p.Hq + hq, hk = hq / p.G;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int grp = wave >> 2;                                   // row group
  const int h = lane >> 5, col = lane & 31;
  const int row0 = unit * kUnitRows;

  const float gQ = nvfp4_global_scale(__uint_as_float(*p.q_amax));
  const int n_qtiles = (N + kBlk - 1) / kBlk;  // query tiles of the per-tile means
  const float gK = *p.k_gscale;
  // a bf16 V cache is unscaled; NVFP4 P.V: the two global scales
  const float sV = VAR == kVarPvNvfp4 ? kNvfp4PScale * *p.v_scale : (PV16 ? 1.0f : *p.v_scale);
  const float gg = gQ * gK;
  const float lam = p.scale * kLog2e * gg;  // exp2 constant per unit of the MFMA score

  const int nblk_all = (N + kBlk - 1) / kBlk;
  const int64_t kvh = (int64_t)b * p.Hkv + hk;
  const uint8_t* kimg = p.k_f16 + kvh * nblk_all * kKBlockBytes;
  const uint32_t lds_k0 = lds_addr(smem_k[0]), lds_k1 = lds_addr(smem_k[1]);
  // The first K~ block goes out before the queries are quantized, so its
  // load latency overlaps the prologue.
  issue_k_block<8>(kimg, lds_k0, wave, lane);
  if (TILE && nblk_all > 1) issue_k_block<8>(kimg + kKBlockBytes, lds_k1, wave, lane);

  // ---- prologue: NVFP4 of the queries, expanded to FP16 in registers -----
  // Each lane holds, as the B operand of the score MFMA (Q~^T), query row
  // 32*wave + col at head-dim slots 64*h + 8*kc .. +7 for step kc, i.e. the
  // 16-element blocks 4h .. 4h+3 of its row: it quantizes exactly those (no
  // LDS staging, no barrier).
  const int qr = 32 * wave + col;
  const int qrow = row0 + qr;
  i32x4 qf[8];
  float part_sum = 0.0f;  // this lane's half of Q_i . Kbar (the LSE row term)
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int blk = 4 * h + bi;
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float part = 0.0f;
    if (qrow < N) {
      float x[16];
      const int64_t off = ((int64_t)bh * N + qrow) * kD + blk * 16;
      load16(p.q, off, p.q_bf16, x);
      if (SMOOTH || TILE) {
        const float* mu = SMOOTH ? p.q_mean + (int64_t)bh * kD + blk * 16
                                 : p.q_tile_mean + ((int64_t)bh * n_qtiles + (qrow >> 7)) * kD + blk * 16;
        const float* km = p.k_mean + ((int64_t)b * p.Hkv + hk) * kD + blk * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          part = fmaf(x[j], km[j], part);
          x[j] = x[j] - mu[j];
        }
      }
      uint32_t w[2];
      const uint32_t sc = nvfp4_block_packed(x, gQ, w);
      if (TILE) {
        // code value x block scale in BF16 (exact: at most 6 significant bits)
        const float sc_v = e4m3_value_pos(sc);
        expand_fp4x8_bf16(w[0], sc_v, packed);
        expand_fp4x8_bf16(w[1], sc_v, packed + 4);
      } else {
        // code value x block scale in FP16 (exact) by the hardware conversion
        const f16x2 s2 = e4m3_scale_f16x2(sc);
        expand_fp4x8(w[0], s2, packed);
        expand_fp4x8(w[1], s2, packed + 4);
      }
    }
    qf[2 * bi] = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    qf[2 * bi + 1] = i32x4{(int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]};
    part_sum += part;
  }
  float lse_off = 0.0f;
  if ((SMOOTH || TILE) && p.lse) lse_off = p.scale * sum_halves(part_sum);
  // Constant B operand of the rank-one step: slots 0..2 of lane half 0 hold
  // 1 / (gQ gK) as the sum of three bf16 parts (exact to fp32 precision);
  // the A operand repeats Delta_S[key] in the same slots.
  const float cinv = 1.0f / gg;  // score units per unit of Delta
  i32x4 dB = {0, 0, 0, 0};
  if (RANK1) {
    const uint32_t c_hi = bf16_rne(cinv);
    const float r1 = cinv - __uint_as_float(c_hi << 16);
    const uint32_t c_mid = bf16_rne(r1);
    const uint32_t c_lo = bf16_rne(r1 - __uint_as_float(c_mid << 16));
    dB = i32x4{h == 0 ? (int)(c_hi | (c_mid << 16)) : 0, h == 0 ? (int)c_lo : 0, 0, 0};
  }

  const int my_row = row0 + qr;
  const int grow0 = row0 + 128 * grp;  // first row of this wave's group
  // blocks per group (0 for a group past the end), and the loop length
  const int n_a = p.causal ? min(2 * unit + 1, nblk_all) : nblk_all;
  const int n_b = row0 + 128 < N ? (p.causal ? min(2 * unit + 2, nblk_all) : nblk_all) : 0;
  const int n_own = grp ? n_b : n_a;
  const int n_max = max(n_a, n_b);
  const int lim = p.causal ? min(my_row, N - 1) : N - 1;  // last visible key of this row
  const int ntiles32 = (N + 31) / 32;
  const uint8_t* vbase = PV16 ? reinterpret_cast<const uint8_t*>(p.v_bf16) + kvh * ntiles32 * kVBf16TileBytes
                              : p.v_fp8 + kvh * ntiles32 * kVTileBytes;
  const uint16_t* dbase = SMOOTH ? p.delta_s + (int64_t)bh * N : nullptr;
  const uint32_t lds_v0 = lds_addr(smem_v[0]), lds_v1 = lds_addr(smem_v[1]);

  // A-row rho of score tile t holds key 64*(t/2) + 32*hp + 16*(t%2) + vp of
  // the block (hp, vp from rho below); the MFMA output register v of lane
  // half h then holds key 64*(t/2) + 32*h + 16*(t%2) + v.
  const int hp = (col >> 2) & 1, vp = ((col >> 3) << 2) | (col & 3);
  int koff[4], kbase[4];  // A-row key of tile t; its chunk 8 h in the block image
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    koff[t] = 64 * (t >> 1) + 32 * hp + 16 * (t & 1) + vp;
    kbase[t] = 8 * h * kKChunkBytes + 16 * koff[t];
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4], s[4];
  PRegs<VAR> pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};

  uint32_t dd = 0;
  if (SMOOTH && tid < kBlk) dd = dbase[min(tid, N - 1)];

  // Per-tile mode: the means of the unit's two query tiles (2 unit, 2 unit + 1;
  // one per row group) as exact bf16 parts, laid out as the rows of the A
  // operand of tile_delta: entry (g, kc, half, part, i) holds part `part` of
  // Qbar[dim 64 half + 8 kc + i] of tile 2 unit + g (the head-dim order of the
  // score operands).  Then Delta_tile(0) for each group's tile; K~(0) and K~(1)
  // are resident after the barrier.
  const uint8_t* qop_g = smem_qop + (TILE ? grp * 768 : 0);
  if (TILE) {
    uint16_t* qop16 = reinterpret_cast<uint16_t*>(smem_qop);
    for (int e = tid; e < 2 * 8 * 2 * 3 * 8; e += 512) {
      const int i = e & 7, part = (e >> 3) % 3, rest = (e >> 3) / 3;
      const int half = rest & 1, kc = (rest >> 1) & 7, g = rest >> 4;
      const int tile = 2 * unit + g;
      const float x = tile < n_qtiles
                          ? p.q_tile_mean[((int64_t)bh * n_qtiles + tile) * kD + 64 * half + 8 * kc + i]
                          : 0.0f;
      const uint32_t hi = bf16_rne(x);
      const float r1 = x - __uint_as_float(hi << 16);  // exact
      const uint32_t mid = bf16_rne(r1);
      const uint32_t lo = bf16_rne(r1 - __uint_as_float(mid << 16));  // both exact
      qop16[e] = (uint16_t)(part == 0 ? hi : (part == 1 ? mid : lo));
    }
    wait_direct_loads();
    __syncthreads();
    if (n_own > 0)
      tile_delta(smem_k[0], qop_g, kbase[wave & 3], koff[wave & 3], gK, cinv, lane,
                 smem_comp[0][grp]);
  }

  // Steps alternate between the groups: in body j, group 0 runs its matrix
  // phase (P.V of block j-1, scores of block j) in the first step and the
  // softmax of block j in the second; group 1 runs the softmax of block j-1
  // first and its matrix phase second.  The loads of K~(j+1), Delta_S(j+1)
  // and V(j) (their buffers were last read in body j-1) are split between
  // the groups so that neither softmax phase pays for issuing them: group 0
  // issues its half after its matrix phase, group 1 its half at the start of
  // its own; the barrier that opens body j+1 publishes them.  Both loops
  // pass the same barriers.  In the per-tile mode K~ runs one block further ahead (K~(j+2)
  // is issued in body j, into the buffer of K~(j-1)), and in body j the
  // matrix phase of group j % 2 also computes Delta_tile(j+1) of both groups'
  // tiles for key tile (wave & 3) from the resident K~(j+1) (one product for
  // both, the groups taking turns); the next opening barrier publishes it,
  // and its buffers were last read by the scores of block j-1.
#define MPFA_STEP_OPEN(J)                                                                    \
  do {                                                                                       \
    wait_direct_loads(); /* this wave's loads of the previous body have landed */            \
    if (SMOOTH && CINIT && tid < kBlk)                                                       \
      smem_comp[(J) & 1][0][tid] = __uint_as_float(dd << 16) * cinv;                         \
    if (DELTA16 && tid < kBlk) smem_delta[(J) & 1][tid] = (uint16_t)dd;                      \
    __syncthreads();                                                                         \
  } while (0)
#define MPFA_ISSUE(J)                                                                        \
  do {                                                                                       \
    const int jk = (J) + (TILE ? 2 : 1); /* the K~ block loaded in this body */              \
    if (jk < n_max) {                                                                        \
      issue_k_block<8>(kimg + (int64_t)jk * kKBlockBytes, lds_addr(smem_k[jk % NKB]), wave,   \
                       lane);                                                                \
      if (SMOOTH && tid < kBlk) dd = dbase[min(((J) + 1) * kBlk + tid, N - 1)];              \
    }                                                                                        \
    if ((J) < n_max) {                                                                       \
      if (PV16)                                                                              \
        issue_v_block_bf16<8>(vbase, ntiles32, (J) * kBlk, ((J) & 1) ? lds_v1 : lds_v0, wave, \
                              lane);                                                         \
      else                                                                                   \
        issue_v_block<8>(vbase, ntiles32, (J) * kBlk, ((J) & 1) ? lds_v1 : lds_v0, wave, lane); \
    }                                                                                        \
  } while (0)
#define MPFA_MATRIX(J)                                                                       \
  do {                                                                                       \
    if ((J) >= 1 && (J) <= n_own) pv_block<VAR>(o, smem_v[((J) - 1) & 1], pb, h, col);      \
    if ((J) < n_own) {                                                                       \
      score_block<COMP, TILE>(s, smem_k[(J) % NKB],                                          \
                              CINIT ? (const void*)smem_comp[(J) & 1][TILE ? grp : 0]        \
                                    : (const void*)smem_delta[(J) & 1],                      \
                              koff, kbase, qf, dB, h);                                       \
    } else {                                                                                 \
      /* defining s on this path too keeps the old scores from being live */                 \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) s[t] = f32x16{};                         \
    }                                                                                        \
    /* the groups take turns computing Delta_tile(J+1) for both tiles */                    \
    if (TILE && ((J) & 1) == grp && (J) + 1 < n_max)                                         \
      tile_delta_pair(smem_k[((J) + 1) % NKB], smem_qop, kbase[wave & 3], koff[wave & 3], gK,  \
                      cinv, lane, smem_comp[((J) + 1) & 1][0],                               \
                      smem_comp[((J) + 1) & 1][TILE ? 1 : 0]);                               \
  } while (0)
#define MPFA_SOFTMAX(J)                                                                      \
  do {                                                                                       \
    if ((J) >= 0 && (J) < n_own) {                                                           \
      const int k0 = (J) * kBlk;                                                             \
      const bool mask = (p.causal && k0 + kBlk > grow0) || (k0 + kBlk > N);                 \
      softmax_block<VAR>(s, o, pb, m_run, l_run, lam, mask, k0, lim, h,                      \
                         &smem_delta[(J) & 1][0], cinv);                                     \
    } else {                                                                                 \
      pb = PRegs<VAR>{}; /* as for s: keeps old P from being live */                         \
    }                                                                                        \
  } while (0)
  if (grp == 0) {
    for (int j = 0; j <= n_max; ++j) {
      MPFA_STEP_OPEN(j);
      MPFA_MATRIX(j);
      MPFA_ISSUE(j);
      __syncthreads();
      MPFA_SOFTMAX(j);
    }
  } else {
    for (int j = 0; j <= n_max; ++j) {
      MPFA_STEP_OPEN(j);
      MPFA_SOFTMAX(j - 1);
      __syncthreads();
      MPFA_ISSUE(j);
      MPFA_MATRIX(j);
    }
  }
#undef MPFA_STEP_OPEN
#undef MPFA_ISSUE
#undef MPFA_MATRIX
#undef MPFA_SOFTMAX

  // ---- epilogue -----------------------------------------------------------
  // An MFMA reads its operands from all 64 lanes whatever the execution mask,
  // while loads honour it; so nothing that feeds the accumulators may be moved
  // into a branch on the row.  Every lane normalises, only the stores of rows
  // past the end are skipped.
  const float l_tot = sum_halves(l_run);
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
        kLn2 * (lam * m_run + log2f(l_tot)) - (VAR == kVarPvNvfp4 ? 0.0f : kLn2 * kLog2_448) +
        lse_off;
}

// K~ = E2M1 code value x E4M3 block scale in FP16, written as block images
// (one 32 KB image per (batch, KV head, 128-key block), layout above); keys
// past N in the last block are zero.  Thread g = image * 128 + slot expands
// the whole key in that slot: it reads the key's 64 code bytes and 8 scale
// bytes in one piece and writes its 16 chunks, so consecutive threads read
// consecutive rows and write consecutive 16-byte slots of each chunk column.
// With partials non-NULL, block 0 first folds the n_partials per-workgroup
// maxima of the query amax pass into amax_out[0] (the word the attention
// kernel reads), so that pass needs neither a cleared buffer nor a fold
// launch of its own.
template <bool BF16>
__global__ __launch_bounds__(256) void k_expand_k(const uint4* __restrict__ codes,
                                                  const uint2* __restrict__ sf, int N, int nkb,
                                                  int64_t n_threads, uint4* __restrict__ out,
                                                  const float* __restrict__ partials,
                                                  int n_partials, uint32_t* __restrict__ amax_out) {
  if (partials && blockIdx.x == 0) {  // uniform across the block
    __shared__ float red[4];
    float m = 0.0f;
    for (int i = threadIdx.x; i < n_partials; i += 256) m = fmaxf(m, partials[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();  // also orders every read of partials before the store below
    if (threadIdx.x == 0) amax_out[0] = __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  }
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n_threads) return;
  const int slot = (int)(g & (kBlk - 1));
  const int64_t img = g >> 7;  // bhk * nkb + kb
  const int64_t bhk = img / nkb;
  const int key = (int)(img - bhk * nkb) * kBlk + slot;
  uint4* dst = out + img * (kKBlockBytes / 16) + slot;
  if (key >= N) {
#pragma unroll
    for (int c = 0; c < 16; ++c) dst[c * kBlk] = make_uint4(0, 0, 0, 0);
    return;
  }
  const int64_t row = bhk * N + key;
  const uint2 sc = sf[row];
  const uint32_t scw[2] = {sc.x, sc.y};
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {  // 16 code bytes = blocks 2 q4 and 2 q4 + 1
    const uint4 w = codes[row * 4 + q4];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int e = 2 * q4 + half;
      const uint32_t scode = (scw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
      uint32_t v[8];
      if (BF16) {
        const float sf = e4m3_value_pos(scode & 0x7Fu);
        expand_fp4x8_bf16(ww[2 * half], sf, v);
        expand_fp4x8_bf16(ww[2 * half + 1], sf, v + 4);
      } else {
        const f16x2 s2 = e4m3_scale_f16x2(scode);
        expand_fp4x8(ww[2 * half], s2, v);
        expand_fp4x8(ww[2 * half + 1], s2, v + 4);
      }
      dst[(2 * e) * kBlk] = make_uint4(v[0], v[1], v[2], v[3]);
      dst[(2 * e + 1) * kBlk] = make_uint4(v[4], v[5], v[6], v[7]);
    }
  }
}

void launch_expand_k(const uint8_t* k_fp4, const uint8_t* k_sf, int64_t bhk, int N,
                     uint8_t* k_img, hipStream_t st, bool bf16, const float* partials,
                     int n_partials, uint32_t* amax_out) {
  const int nkb = (N + kBlk - 1) / kBlk;
  const int64_t n_threads = bhk * nkb * kBlk;
  const dim3 grid((unsigned)((n_threads + 255) / 256));
  const auto* codes = reinterpret_cast<const uint4*>(k_fp4);
  const auto* sf = reinterpret_cast<const uint2*>(k_sf);
  auto* out = reinterpret_cast<uint4*>(k_img);
  if (bf16)
    hipLaunchKernelGGL(k_expand_k<true>, grid, dim3(256), 0, st, codes, sf, N, nkb, n_threads, out,
                       partials, n_partials, amax_out);
  else
    hipLaunchKernelGGL(k_expand_k<false>, grid, dim3(256), 0, st, codes, sf, N, nkb, n_threads, out,
                       partials, n_partials, amax_out);
}

// bf16 V cache of the bf16 P.V variant (layout in mpfa_internal.hpp): thread g
// writes the 16 bytes of (tile, group of 8 tokens, channel d): the bf16 (round
// to nearest even) of those 8 tokens' element d, zero past N; consecutive
// threads take consecutive channels, so the reads of each token are coalesced.
__global__ __launch_bounds__(256) void k_pack_v_bf16(const void* __restrict__ v, int is_bf16, int N,
                                                     int ntiles, int64_t n_threads,
                                                     uint4* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n_threads) return;
  const int d = (int)(g & (kD - 1));
  const int64_t r = g >> 7;  // (bh * ntiles + tile) * 4 + group
  const int grp = (int)(r & 3);
  const int64_t tb = r >> 2;
  const int64_t bh = tb / ntiles;
  const int t0 = (int)(tb - bh * ntiles) * 32 + grp * 8;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ta = t0 + 2 * i, tb2 = ta + 1;
    const float a = ta < N ? load_elem(v, (bh * N + ta) * kD + d, is_bf16) : 0.0f;
    const float b = tb2 < N ? load_elem(v, (bh * N + tb2) * kD + d, is_bf16) : 0.0f;
    w[i] = bf16_rne(a) | (bf16_rne(b) << 16);
  }
  out[g] = make_uint4(w[0], w[1], w[2], w[3]);
}

void launch_pack_v_bf16(const void* v, int is_bf16, int BH, int N, uint16_t* out, hipStream_t st) {
  const int ntiles = (N + 31) / 32;
  const int64_t n_threads = (int64_t)BH * ntiles * 4 * kD;
  hipLaunchKernelGGL(k_pack_v_bf16, dim3((unsigned)((n_threads + 255) / 256)), dim3(256), 0, st, v,
                     is_bf16, N, ntiles, n_threads, reinterpret_cast<uint4*>(out));
}

// FP16 image of the NVFP4 V cache (NVFP4 P.V variant), the bf16 V cache's
// layout: thread g writes the 16 bytes of (tile, group of 8 keys, channel d),
// the group's 8 codes (one word of the channel's 16-key block) times the
// block scale by the hardware FP4 -> FP16 conversion and one packed multiply;
// zero past the last 16-key block.
__global__ __launch_bounds__(256) void k_expand_v_nvfp4(const uint2* __restrict__ codes,
                                                        const uint8_t* __restrict__ sf, int nb16,
                                                        int ntiles, int64_t n_threads,
                                                        uint4* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n_threads) return;
  const int d = (int)(g & (kD - 1));
  const int64_t r = g >> 7;  // (bh * ntiles + tile) * 4 + group
  const int grp = (int)(r & 3);
  const int64_t tb = r >> 2;
  const int64_t bh = tb / ntiles;
  const int t0 = (int)(tb - bh * ntiles) * 32 + grp * 8;
  const int kb = t0 >> 4;
  uint32_t w4[4] = {0u, 0u, 0u, 0u};
  if (kb < nb16) {
    const int64_t o = (bh * nb16 + kb) * kD + d;
    const uint2 c = codes[o];
    expand_fp4x8((t0 & 8) ? c.y : c.x, e4m3_scale_f16x2(sf[o]), w4);
  }
  out[g] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

void launch_expand_v_nvfp4(const uint8_t* codes, const uint8_t* sf, int BH, int N, uint16_t* out,
                           hipStream_t st) {
  const int ntiles = (N + 31) / 32, nb16 = (N + 15) / 16;
  const int64_t n_threads = (int64_t)BH * ntiles * 4 * kD;
  hipLaunchKernelGGL(k_expand_v_nvfp4, dim3((unsigned)((n_threads + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint2*>(codes), sf, nb16, ntiles, n_threads,
                     reinterpret_cast<uint4*>(out));
}

void launch_prefill(const PrefillParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((int64_t)p.n_units * p.B * p.Hq);
  const dim3 g(grid), b(512);
  if (p.q_tile_mean) {
    hipLaunchKernelGGL((k_prefill<2, kVarNone>), g, b, 0, st, p);
  } else if (p.delta_s) {
    switch (p.variant) {
      case kVarElementwise: hipLaunchKernelGGL((k_prefill<1, kVarElementwise>), g, b, 0, st, p); break;
      case kVarPolyExp2: hipLaunchKernelGGL((k_prefill<1, kVarPolyExp2>), g, b, 0, st, p); break;
      case kVarPvBf16: hipLaunchKernelGGL((k_prefill<1, kVarPvBf16>), g, b, 0, st, p); break;
      case kVarPvNvfp4: hipLaunchKernelGGL((k_prefill<1, kVarPvNvfp4>), g, b, 0, st, p); break;
      case kVarRankOne: hipLaunchKernelGGL((k_prefill<1, kVarRankOne>), g, b, 0, st, p); break;
      default: hipLaunchKernelGGL((k_prefill<1, kVarNone>), g, b, 0, st, p); break;
    }
  } else {
    switch (p.variant) {
      case kVarPolyExp2: hipLaunchKernelGGL((k_prefill<0, kVarPolyExp2>), g, b, 0, st, p); break;
      case kVarPvBf16: hipLaunchKernelGGL((k_prefill<0, kVarPvBf16>), g, b, 0, st, p); break;
      case kVarPvNvfp4: hipLaunchKernelGGL((k_prefill<0, kVarPvNvfp4>), g, b, 0, st, p); break;
      default: hipLaunchKernelGGL((k_prefill<0, kVarNone>), g, b, 0, st, p); break;
    }
  }
}

}  // namespace mpfa
