// Device helpers of the QK4PV8 kernels for gfx950: number-format codecs,
// FP4 -> FP16 operand expansion, MFMA wrappers and small wave utilities.
//
// Formats (paper "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention
// Kernels on Blackwell GPUs", section 4.1 and section 6 "Online
// quantization"): NVFP4 = E2M1 elements with one E4M3 scale per 16 elements
// plus an FP32 per-tensor scale; FP8 = OCP E4M3 ("FN": bias 7, largest
// finite 448, no infinities).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpfa {

constexpr int kD = 128;        // head dimension
constexpr int kBlk = 128;      // keys per online-softmax block
constexpr float kNvfp4Range = 2688.0f;  // 6 * 448: largest E2M1 x E4M3 product
constexpr float kE4M3Max = 448.0f;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------- loading ----
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int is_bf16) {
  if (is_bf16) {
    uint32_t h = reinterpret_cast<const uint16_t*>(p)[i];
    return __uint_as_float(h << 16);
  }
  return reinterpret_cast<const float*>(p)[i];
}

// 16 consecutive elements (16-element aligned) of an fp32 or bf16 tensor.
__device__ __forceinline__ void load16(const void* p, int64_t i, int is_bf16, float* x) {
  if (is_bf16) {
    const uint4* s = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    uint4 a = s[0], b = s[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4* s = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 v = s[j];
      x[4 * j] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------- codecs --
// E2M1 code of x: nearest of the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6},
// ties to the even code, saturating at 6, sign bit (bit 3) copied from x so
// that -0 and negatives rounding to zero keep their sign.  Below 1 the code
// is rint(2|x|) (0, 1 or 2 = the value 1.0; 0.25 and 0.75 go to the even
// codes 0 and 2).  From 1 on, the magnitude codes are the fp32 pattern
// rounded to one mantissa bit: with the mantissa rounded half to even at
// bit 22, (bits >> 22) - 252 is 2 for 1.0, 3 for 1.5, ... 7 for 6.0 (and
// above 7 for what saturates).  Rounding the fp32 mantissa to nearest even
// is the tie rule of the code, because every E2M1 value from 1 on has a
// one-bit mantissa.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  const uint32_t small = (uint32_t)__builtin_rintf(a * 2.0f);
  uint32_t u = __float_as_uint(a);
  u += 0x1FFFFFu + ((u >> 22) & 1u);
  const uint32_t big = min((u >> 22) - 252u, 7u);
  const uint32_t c = a < 1.0f ? small : big;
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Value of an E2M1 code (4 bits).  The normal and the subnormal forms are
// both computed and one is selected (no branch); the sign bit is copied, so
// code 8 gives -0.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float normal = __uint_as_float(((e + 126u) << 23) | (m << 22));
  const float sub = 0.5f * (float)m;
  const float v = e ? normal : sub;
  return __uint_as_float(__float_as_uint(v) | ((c & 8u) << 28));
}

// E4M3 code of a magnitude a >= 0 (finite): round to nearest, ties to the
// even code, saturate at 448 (code 0x7E); never the NaN code.  The normal
// and the subnormal encodings are both computed and one is selected (no
// branch); each is used only in its own range.
__device__ __forceinline__ uint32_t e4m3_encode_mag(float a) {
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the fp32 mantissa to 3 bits, half to even
  const uint32_t normal = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  // below 2^-6: subnormal step 2^-9; rint rounds half to even (8 -> code 0x08 = 2^-6)
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t c = a < 0.015625f ? sub : normal;
  return a >= 448.0f ? 0x7Eu : c;
}

__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  return e4m3_encode_mag(fabsf(x)) | ((__float_as_uint(x) >> 24) & 0x80u);
}

// Value of a non-negative E4M3 code below 0x7F (both forms computed, one
// selected).
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0.001953125f;
  return e ? normal : sub;
}

// bf16 bits of a finite fp32, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// NVFP4 global scale from a tensor amax (the reading: amax / (6 * 448)).
__device__ __forceinline__ float nvfp4_global_scale(float amax) {
  return amax > 0.0f ? amax / kNvfp4Range : 1.0f;
}

// ------------------------------------------ block divisor, RN quotients --
// The 16 elements of an NVFP4 block share one divisor d = s * g, and the
// E2M1 decision is taken on the correctly rounded fp32 quotient x / d.  Here
// the reciprocal is rounded once per block (r = RN(1/d), by IEEE division)
// and each quotient is q0 = x * r followed by two residual corrections
// q <- q + (x - q d) r, each residual exact through the FMA.  The first
// correction makes q faithful, the second rounds it correctly (Markstein's
// theorem on division with a correctly rounded reciprocal, P. Markstein,
// IBM J. Res. Dev. 34(1), 1990).  The divisor is first brought into
// [2^-64, 2^64] by a power-of-two factor applied to both operands (exact),
// so that r stays normal and, for every quotient of magnitude >= 1/8, no
// residual underflows; smaller quotients round to a zero code either way
// and keep their sign by construction.  Six VALU operations per element
// instead of the eleven of the general division, with no branch.
struct BlockDivisor {
  float k, d, r;
};
// d > 0 and finite; zero = true (a zero scale) makes every quotient +-0
__device__ __forceinline__ BlockDivisor block_divisor(float d, bool zero) {
  BlockDivisor v;
  v.k = d < 0x1p-64f ? 0x1p64f : (d > 0x1p64f ? 0x1p-64f : 1.0f);
  v.d = zero ? 1.0f : d * v.k;
  v.r = zero ? 0.0f : 1.0f / v.d;
  return v;
}
__device__ __forceinline__ float block_quotient(const BlockDivisor& v, float x) {
  const float xs = x * v.k;
  const float q0 = xs * v.r;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, v.d, xs), v.r, q0);
  const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, v.d, xs), v.r, q1);
  return __uint_as_float((__float_as_uint(q2) & 0x7FFFFFFFu) | (__float_as_uint(x) & 0x80000000u));
}

// Quantize one 16-element block with global scale g: returns the E4M3 scale
// code and writes the 16 E2M1 codes (one per entry, low 4 bits).
__device__ __forceinline__ uint32_t nvfp4_block(const float* x, float g, uint32_t* codes) {
  float ab = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) ab = fmaxf(ab, fabsf(x[j]));
  const float six_g = 6.0f * g;
  const uint32_t sc = e4m3_encode_mag(ab / six_g);
  const float s = e4m3_value_pos(sc);
  const float sg = s * g;
  const bool zero = (s == 0.0f) || (sg == 0.0f);
  const BlockDivisor dv = block_divisor(sg, zero);  // a zero scale: signed zero codes
#pragma unroll
  for (int j = 0; j < 16; ++j) codes[j] = e2m1_encode(block_quotient(dv, x[j]));
  return sc;
}

// nvfp4_block with the codes packed two per byte (element 2t in the low
// nibble of byte t, w[0] = elements 0-7, w[1] = 8-15) by the hardware
// FP32 -> E2M1 conversion (v_cvt_scalef32_pk_fp4_f32 at unit scale).  Its
// rounding is that of e2m1_encode -- nearest, ties to the even code,
// saturating at 6, sign kept -- checked on gfx950 for every fp32 value
// within 64 ulps of each E2M1 midpoint and grid point (both signs), for +-0,
// tiny and huge values and a million random ones (csrc/fp4_check.hip, run by
// the GPU tests).  The quotients are
// the same correctly rounded ones (block_quotient); a zero scale converts +-0.
__device__ __forceinline__ uint32_t nvfp4_block_packed(const float* x, float g, uint32_t (&w)[2]) {
  float ab = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) ab = fmaxf(ab, fabsf(x[j]));
  const float six_g = 6.0f * g;
  const uint32_t sc = e4m3_encode_mag(ab / six_g);
  const float s = e4m3_value_pos(sc);
  const float sg = s * g;
  const bool zero = (s == 0.0f) || (sg == 0.0f);
  const BlockDivisor dv = block_divisor(sg, zero);
  float q[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) q[j] = block_quotient(dv, x[j]);
  uint32_t w0 = 0u, w1 = 0u;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[0], q[1], 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[2], q[3], 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[4], q[5], 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[6], q[7], 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[8], q[9], 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[10], q[11], 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[12], q[13], 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[14], q[15], 1.0f, 3);
  w[0] = w0;
  w[1] = w1;
  return sc;
}

// ------------------------------------------------ FP4 -> FP16 expansion --
// Expand the 8 E2M1 codes of one 32-bit word (element 2t in the low nibble
// of byte t) into 8 FP16 values code_value * s, packed two per word in
// element order.  Every product of an E2M1 magnitude and an E4M3 scale has
// at most 6 significant bits and lies in [2^-10, 2688], so it is exact in
// FP16 and the MFMA sees exactly the dequantized operand (up to the global
// scale, which is applied in the exponent).
//
// v_cvt_scalef32_pk_f16_fp4 decodes one byte (two codes, low nibble first)
// and applies only the exponent of its scale operand, so it is used with
// scale 1 and the E4M3 scale is applied by one packed FP16 multiply.
__device__ __forceinline__ void expand_fp4x8(uint32_t w, f16x2 s2, uint32_t* out) {
  const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  out[0] = __builtin_bit_cast(uint32_t, a0 * s2);
  out[1] = __builtin_bit_cast(uint32_t, a1 * s2);
  out[2] = __builtin_bit_cast(uint32_t, a2 * s2);
  out[3] = __builtin_bit_cast(uint32_t, a3 * s2);
}

// The same eight codes as BF16 (the products are exact there too): pairs of
// elements 2i (low half) and 2i + 1 (high half) of the word's byte i.
__device__ __forceinline__ void expand_fp4x8_bf16(uint32_t w, float s, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = e2m1_value((w >> (8 * i)) & 15u) * s;
    const float hi = e2m1_value((w >> (8 * i + 4)) & 15u) * s;
    out[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
}

__device__ __forceinline__ f16x2 e4m3_scale_f16x2(uint32_t code) {
  const _Float16 h = (_Float16)e4m3_value_pos(code & 0x7Fu);
  return f16x2{h, h};
}

// ------------------------------------------------------------------ MFMA --
__device__ __forceinline__ f32x16 mfma32_f16(const i32x4& a, const i32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_bf16(const i32x4& a, const i32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// FP8 E4M3 x FP8 E4M3, 32x32x64, without block scales: with both scale
// arguments 0 the compiler emits the unscaled v_mfma_f32_32x32x64_f8f6f4,
// whose products equal the scaled form's at unit scales (E8M0 127) bit for
// bit (the prefill's outputs are identical either way) and which issues a
// little cheaper beside the softmax.
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP8 E4M3 x FP8 E4M3, 16x16x128, without block scales (as above).
__device__ __forceinline__ f32x4 mfma16_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two fp32 -> two E4M3 bytes into the low (HI = false) or high half of `old`
// (hardware conversion, round to nearest even).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ atomics -----
// Non-negative floats order like their bit patterns.
__device__ __forceinline__ void atomic_max_nonneg(uint32_t* p, float v) {
  atomicMax(p, __float_as_uint(v));
}

// Any non-NaN float as an unsigned key in the same order (sign bit flipped
// for non-negative values, all bits for negative ones); a cleared word is
// below every key.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace mpfa
