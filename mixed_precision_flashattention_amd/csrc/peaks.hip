// Measured ceilings of the MI355X that the roofline fractions are quoted
// against: streaming-read bandwidth of HBM (plain and non-temporal 16-byte
// loads over the 128K decode workload's 3.49 GB), the issue rate of the
// MFMA instructions the kernels use (32x32x16 f16 and bf16, 32x32x64 FP8
// and FP4 with unit block scales), the vector-ALU ceiling of the prefill's
// softmax, and the ceilings of the prefill's two-group schedule with its
// instruction mix, without and with its LDS operand traffic.  A standalone program, not part of the library: it
// prints one JSON object.
//
// MFMA probe: every wave runs kIters rounds of 8 independent MFMAs (eight
// accumulators, so no instruction waits on the previous one) on operands
// derived from its lane id; the accumulators are summed and stored so
// nothing is dead.  FLOP = waves x kIters x 8 x 2 M N K.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) { return (uint32_t)(uintptr_t)p; }

constexpr int kIters = 2048;
constexpr int kAcc = 8;

enum Op { F16 = 0, BF16 = 1, FP8 = 2, FP4 = 3 };

template <int OP>
__device__ __forceinline__ f32x16 mma(const i32x8& a, const i32x8& b, const f32x16& c) {
  if constexpr (OP == F16) {
    const i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a4),
                                                  __builtin_bit_cast(f16x8, b4), c, 0, 0, 0);
  } else if constexpr (OP == BF16) {
    const i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                   __builtin_bit_cast(bf16x8, b4), c, 0, 0, 0);
  } else if constexpr (OP == FP8) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  } else {  // E2M1 operands (format code 4): the low four words of each operand
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, 127, 0, 127);
  }
}

template <int OP>
__global__ __launch_bounds__(256) void k_mfma(float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // small finite operands in every format (E4M3 / E2M1 / f16 / bf16 codes
  // chosen from the lane id; the values themselves do not matter)
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((lane + i) & 0x03030303);
    b[i] = 0x30303030 ^ ((lane * 3 + i) & 0x01010101);
  }
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x16{};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = mma<OP>(a, b, acc[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Softmax VALU ceiling: one wave per SIMD (one 4-wave workgroup per CU,
// held alone there by its LDS allocation) runs the prefill's per-block
// softmax instruction mix on the 64 scores a lane owns in the S^T layout
// (128 keys x 32 queries per wave): the row max (in-lane chain and one
// lane-half exchange), the correction factor, exp2 of the scaled and
// shifted scores, the row sum of the unrounded p and the E4M3 conversion of
// P, kSmIters blocks in a row with the scores made opaque each time.  The
// running max does not move after the first block, so the output rescale is
// skipped as in most blocks of the kernel.  Each (block, wave) serves
// 4 x 128 x 128 x 32 FLOP of the prefill's algorithmic work, which gives
// the rate the softmax alone could sustain with free matrix products.
constexpr int kSmIters = 4096;
constexpr double kSmFlopPerBlockWave = 4.0 * 128 * 128 * 32;

__global__ __launch_bounds__(256) void k_softmax(float* __restrict__ out, float lam) {
  const int lane = threadIdx.x & 63;
  float s[64], o[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    s[i] = 0.01f * (float)((lane * 7 + i * 13) & 63);
    o[i] = 1.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  uint32_t pacc = 0u;
  for (int it = 0; it < kSmIters; ++it) {
#pragma unroll
    for (int i = 0; i < 64; ++i) asm volatile("" : "+v"(s[i]));
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 64; ++i) mx = fmaxf(mx, s[i]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false,
                                                    false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(lam * (m_run - m_new));
    const float nb = 8.80735492f - lam * m_new;  // log2(448) - lam m
    m_run = m_new;
    float lsum = 0.0f;
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[4 * k], lam, nb));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[4 * k + 1], lam, nb));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(s[4 * k + 2], lam, nb));
      const float e3 = __builtin_amdgcn_exp2f(fmaf(s[4 * k + 3], lam, nb));
      lsum += (e0 + e1) + (e2 + e3);
      uint32_t wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, __float_as_uint(e0), false);
      w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
    }
    l_run = fmaf(alpha, l_run, lsum);
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int i = 0; i < 64; ++i) o[i] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(w[k]));
    pacc ^= w[0] ^ w[15];
  }
  float t = l_run + (float)(pacc & 1u);
#pragma unroll
  for (int i = 0; i < 64; ++i) t += o[i];
  out[blockIdx.x * 256 + threadIdx.x] = t;
}

// Ping-pong ceilings: the prefill's schedule with its instruction mix.  One
// 8-wave workgroup per CU (held alone by its LDS allocation), two groups of 4
// waves, each SIMD holding one wave of each; per body, between two workgroup
// barriers, one group runs the matrix phase of a block (8 FP8 32x32x64 P.V
// MFMAs, then 32 f16 32x32x16 score MFMAs in four interleaved accumulator
// chains) while the other runs the softmax mix of k_softmax on the scores of
// its previous matrix phase, then the roles swap.  Operands are random
// (finite f16 and E4M3 values), so the chip draws the power, and runs the
// clock, of real data.  Two forms:
//   FEED false: operands from registers -- no LDS reads, loads, mask or
//     rescale: the floor set by the instruction mix and the barriers;
//   FEED true: the kernel's operand traffic -- K~ operands read from LDS one
//     head-dim step ahead, V operands and the score accumulators' inputs
//     from LDS, and each body's next K~ block (32 KB) and a V block (16 KB)
//     brought in by direct global->LDS loads split between the groups and
//     waited for at the barrier that opens the next body (from a 12 MB
//     region per XCD, as a KV head's K~ image and V cache are).
// Each wave stamps the shader-clock counter around its loop, so the ceiling
// is also reported in cycles per body.
constexpr int kPpIters = 1024;
constexpr int kPpRegion = 256 * 49152;  // 256 blocks of K~ (32 KB) + V (16 KB)

__device__ __forceinline__ uint32_t pp_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
// two random f16 values with |x| in [1/4, 1), random signs
__device__ __forceinline__ uint32_t pp_f16x2(uint32_t r) {
  const uint32_t a = (r & 0x83ffu) | (0x3400u + ((r >> 10) & 0x1u) * 0x0400u);
  const uint32_t b = ((r >> 16) & 0x83ffu) | (0x3400u + ((r >> 26) & 0x1u) * 0x0400u);
  return a | (b << 16);
}
// four random E4M3 values, |x| < 1, no NaN code
__device__ __forceinline__ uint32_t pp_e4m3x4(uint32_t r) { return r & 0xb7b7b7b7u; }

__device__ __forceinline__ void pp_lds_load16(const void* base_in, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)base_in;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const void* base = (const void*)(uintptr_t)((hi << 32) | lo);
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

__device__ __forceinline__ f32x16 pp_f16(const i32x4& a, const i32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 pp_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// kbase[t]: this lane's K~ operand slot of score tile t in a block image
// (chunk column 8 h, the permuted key order of the prefill)
template <bool FEED>
__device__ __forceinline__ void pp_matrix(f32x16 (&s)[4], f32x16 (&o)[4], i32x4 (&ka)[4],
                                          const i32x4 (&qf)[8], const i32x8 (&pb)[2],
                                          const uint8_t* kblk, const uint8_t* vblk,
                                          const float* cblk, const int (&kbase)[4], int h, int col) {
  if constexpr (FEED) {
    i32x8 va[2];
    auto vop = [&](int i) {
      const uint8_t* vt = vblk + (2 * (i >> 2) + h) * 4096 + col * 16 + (i & 3) * 512;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(vt);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(vt + 2048);
      return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    va[0] = vop(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 1 < 8) va[(i + 1) & 1] = vop(i + 1);
      __builtin_amdgcn_sched_barrier(0);
      o[i & 3] = pp_fp8(va[i & 1], pb[i >> 2], o[i & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
    i32x4 a[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[0][t] = *reinterpret_cast<const i32x4*>(kblk + kbase[t]);
    const float* dsc = cblk + 32 * h;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4* src = reinterpret_cast<const f32x4*>(dsc + 64 * (t >> 1) + 16 * (t & 1));
      const f32x4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
      s[t] = f32x16{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                    c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
    }
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      if (kc + 1 < 8) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          a[(kc + 1) & 1][t] = *reinterpret_cast<const i32x4*>(kblk + kbase[t] + (kc + 1) * 2048);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = pp_f16(a[kc & 1][t], qf[kc], s[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // opaque K operands keep the score products in the loop (the P operands
    // change every body anyway); the V operands reuse their bits
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(ka[t]));
    const i32x8 va[2] = {
        i32x8{ka[0][0], ka[0][1], ka[0][2], ka[0][3], ka[1][0], ka[1][1], ka[1][2], ka[1][3]},
        i32x8{ka[2][0], ka[2][1], ka[2][2], ka[2][3], ka[3][0], ka[3][1], ka[3][2], ka[3][3]}};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i & 3] = pp_fp8(va[i & 1], pb[i >> 2], o[i & 3]);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = pp_f16(ka[t], qf[kc], kc ? s[t] : f32x16{});
  }
}

__device__ __forceinline__ void pp_softmax(const f32x16 (&s)[4], f32x16 (&o)[4], i32x8 (&pb)[2],
                                           float& m_run, float& l_run, float lam) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false,
                                                  false);
  mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(lam * (m_run - m_new));
  const float nb = 8.80735492f - lam * m_new;  // log2(448) - lam m
  m_run = m_new;
  float lsum = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int t = k >> 2, v0 = 4 * (k & 3);
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[t][v0], lam, nb));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[t][v0 + 1], lam, nb));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(s[t][v0 + 2], lam, nb));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(s[t][v0 + 3], lam, nb));
    lsum += (e0 + e1) + (e2 + e3);
    uint32_t wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, __float_as_uint(e0), false);
    pb[k >> 3][k & 7] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
  }
  l_run = fmaf(alpha, l_run, lsum);
  if (!__all(alpha == 1.0f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
  }
}

template <bool FEED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_pingpong(
    const uint8_t* __restrict__ src, float* __restrict__ out, uint64_t* __restrict__ cycles,
    float lam) {
  __shared__ __align__(16) uint8_t smem_k[2][32768];
  __shared__ __align__(16) uint8_t smem_v[2][16384];
  __shared__ __align__(16) float smem_c[2][128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), grp = wave >> 2;
  const int h = lane >> 5, col = lane & 31;
  const int hp = (col >> 2) & 1, vp = ((col >> 3) << 2) | (col & 3);
  int kbase[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    kbase[t] = 8 * h * 2048 + 16 * (64 * (t >> 1) + 32 * hp + 16 * (t & 1) + vp);
  for (int i = tid; i < 2 * 32768 / 4; i += 512)
    reinterpret_cast<uint32_t*>(smem_k)[i] = pp_f16x2(pp_hash(i * 7919u + blockIdx.x));
  for (int i = tid; i < 2 * 16384 / 4; i += 512)
    reinterpret_cast<uint32_t*>(smem_v)[i] = pp_e4m3x4(pp_hash(i * 104729u + blockIdx.x));
  if (tid < 256) reinterpret_cast<float*>(smem_c)[tid] = 0.5f;
  __syncthreads();
  i32x4 ka[4], qf[8];
  i32x8 pb[2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) ka[t][e] = (int)pp_f16x2(pp_hash(tid * 131u + t * 17u + e));
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      qf[k][e] = (int)(pp_f16x2(pp_hash(tid * 977u + k * 31u + e + 5u)) & 0xbbffbbffu);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[i][j] = 0;
  f32x16 s[4], o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = f32x16{};
    o[t] = f32x16{};
  }
  float m_run = -INFINITY, l_run = 0.0f;
  const uint8_t* region = src + (int64_t)(blockIdx.x & 7) * kPpRegion;
  // this wave's share of the next K~ block and of a V block (1 KB pieces)
  auto issue = [&](int j) {
    const uint8_t* blk = region + (int64_t)((j + blockIdx.x) & 255) * 49152;
    const int b = (j + 1) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pp_lds_load16(blk + (4 * wave + i) * 1024, 16 * lane, lds_addr_of(smem_k[b]) + (4 * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pp_lds_load16(blk + 32768 + (2 * wave + i) * 1024, 16 * lane,
                    lds_addr_of(smem_v[b]) + (2 * wave + i) * 1024);
  };
  // the scheduling fences keep each phase between its two barriers (register
  // work could otherwise be moved across them)
#define PP_BARRIER()                      \
  do {                                    \
    __builtin_amdgcn_sched_barrier(0);    \
    __syncthreads();                      \
    __builtin_amdgcn_sched_barrier(0);    \
  } while (0)
  auto open = [&](int j) {
    if (FEED) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (tid < 128) smem_c[j & 1][tid] = 0.25f + l_run * 1e-30f;
    }
    PP_BARRIER();
  };
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (grp == 0) {
    for (int j = 0; j < kPpIters; ++j) {
      open(j);
      pp_matrix<FEED>(s, o, ka, qf, pb, smem_k[j & 1], smem_v[j & 1], smem_c[j & 1], kbase, h, col);
      if (FEED) issue(j);
      PP_BARRIER();
      pp_softmax(s, o, pb, m_run, l_run, lam);
    }
  } else {
    for (int j = 0; j < kPpIters; ++j) {
      open(j);
      pp_softmax(s, o, pb, m_run, l_run, lam);
      PP_BARRIER();
      if (FEED) issue(j);
      pp_matrix<FEED>(s, o, ka, qf, pb, smem_k[j & 1], smem_v[j & 1], smem_c[j & 1], kbase, h, col);
    }
  }
#undef PP_BARRIER
  if (FEED) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
  float t = l_run;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += o[i][e];
  out[blockIdx.x * 512 + tid] = t;
}

template <bool NT>
__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ a, int64_t n,
                                              uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n; i += 8 * stride) {  // every index < n
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = NT ? __builtin_nontemporal_load(a + i + u * stride) : a[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 x = a[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

#define CHECK(x)                                                          \
  do {                                                                    \
    if ((x) != hipSuccess) {                                              \
      fprintf(stderr, "HIP error %s at line %d\n", #x, __LINE__);         \
      return 1;                                                           \
    }                                                                     \
  } while (0)

template <typename F>
static int time_ms(F launch, int reps, float* ms) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int w = 0; w < 2; ++w) launch();
  CHECK(hipEventRecord(e0, 0));
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipGetLastError());
  CHECK(hipEventElapsedTime(ms, e0, e1));
  *ms /= reps;
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  printf("{\"device\": \"%s\", \"compute_units\": %d", prop.gcnArchName, cus);

  // ---- MFMA issue rates: 32 waves per CU in 256-thread blocks; one wave per
  // SIMD is resident at a time (eight 16-register accumulators plus operands),
  // so the grid runs in eight rounds
  const int blocks = cus * 2 * 4;  // 256-thread blocks = 4 waves each
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
  const char* names[4] = {"f16_32x32x16", "bf16_32x32x16", "fp8_32x32x64", "fp4_32x32x64"};
  const double mnk2[4] = {2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 64,
                          2.0 * 32 * 32 * 64};
  // warm-up: ~20 launches of MFMA work so the clocks have ramped before the
  // first measurement
  for (int w = 0; w < 20; ++w) hipLaunchKernelGGL(k_mfma<F16>, dim3(blocks), dim3(256), 0, 0, out);
  CHECK(hipDeviceSynchronize());
  printf(", \"mfma_tflops\": {");
  for (int op = 0; op < 4; ++op) {
    float ms = 0.0f;
    int rc = 0;
    switch (op) {
      case F16: rc = time_ms([&] { hipLaunchKernelGGL(k_mfma<F16>, dim3(blocks), dim3(256), 0, 0, out); }, 5, &ms); break;
      case BF16: rc = time_ms([&] { hipLaunchKernelGGL(k_mfma<BF16>, dim3(blocks), dim3(256), 0, 0, out); }, 5, &ms); break;
      case FP8: rc = time_ms([&] { hipLaunchKernelGGL(k_mfma<FP8>, dim3(blocks), dim3(256), 0, 0, out); }, 5, &ms); break;
      default: rc = time_ms([&] { hipLaunchKernelGGL(k_mfma<FP4>, dim3(blocks), dim3(256), 0, 0, out); }, 5, &ms); break;
    }
    if (rc) return rc;
    const double flop = (double)blocks * 4 * kIters * kAcc * mnk2[op];
    printf("%s\"%s\": %.1f", op ? ", " : "", names[op], flop / (ms * 1e-3) / 1e12);
  }
  printf("}");

  // ---- softmax VALU ceiling: one workgroup per CU (its 96 KB of LDS keep a
  // second one out), one wave per SIMD
  {
    const size_t lds = 96 * 1024;
    CHECK(hipFuncSetAttribute((const void*)k_softmax, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds));
    float ms = 0.0f;
    if (time_ms([&] { hipLaunchKernelGGL(k_softmax, dim3(cus), dim3(256), lds, 0, out, 0.0127f); }, 5,
                &ms))
      return 1;
    const double flop = (double)cus * 4 * kSmIters * kSmFlopPerBlockWave;
    printf(", \"softmax_valu_tflops\": %.1f, \"softmax_block_ns\": %.1f", flop / (ms * 1e-3) / 1e12,
           ms * 1e6 / kSmIters);
  }
  CHECK(hipFree(out));

  // ---- ping-pong ceilings: one 8-wave workgroup per CU, every wave serves
  // one (block, wave) pair per body; cycles from the waves' own stamps
  {
    uint8_t* src = nullptr;
    float* pout = nullptr;
    uint64_t* cyc = nullptr;
    CHECK(hipMalloc(&src, (size_t)8 * kPpRegion));
    CHECK(hipMemset(src, 0x38, (size_t)8 * kPpRegion));
    CHECK(hipMalloc(&pout, (size_t)cus * 512 * sizeof(float)));
    CHECK(hipMalloc(&cyc, (size_t)cus * sizeof(uint64_t)));
    uint64_t* hc = new uint64_t[cus];
    for (int feed = 0; feed < 2; ++feed) {
      float ms = 0.0f;
      int rc = feed ? time_ms([&] { hipLaunchKernelGGL(k_pingpong<true>, dim3(cus), dim3(512), 0, 0, src, pout, cyc, 0.0127f); }, 5, &ms)
                    : time_ms([&] { hipLaunchKernelGGL(k_pingpong<false>, dim3(cus), dim3(512), 0, 0, src, pout, cyc, 0.0127f); }, 5, &ms);
      if (rc) return rc;
      CHECK(hipMemcpy(hc, cyc, (size_t)cus * sizeof(uint64_t), hipMemcpyDeviceToHost));
      double c = 0.0;
      for (int i = 0; i < cus; ++i) c += (double)hc[i];
      c /= (double)cus * kPpIters;
      const double body_ns = ms * 1e6 / kPpIters;
      const double flop = (double)cus * 8 * kPpIters * kSmFlopPerBlockWave;
      printf(", \"%s\": {\"tflops\": %.1f, \"body_ns\": %.1f, \"body_cycles\": %.0f, \"clock_GHz\": %.2f}",
             feed ? "pingpong_lds" : "pingpong", flop / (ms * 1e-3) / 1e12, body_ns, c, c / body_ns);
    }
    delete[] hc;
    CHECK(hipFree(src));
    CHECK(hipFree(pout));
    CHECK(hipFree(cyc));
  }

  // ---- streaming read over 3,489,660,928 bytes
  const int64_t bytes = 3489660928LL;
  const int64_t n = bytes / 16;
  u32x4* a = nullptr;
  uint32_t* sink = nullptr;
  const int rgrid = 16384;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMalloc(&sink, (size_t)rgrid * 256 * sizeof(uint32_t)));
  float ms_plain = 0.0f, ms_nt = 0.0f;
  if (time_ms([&] { hipLaunchKernelGGL(k_read<false>, dim3(rgrid), dim3(256), 0, 0, a, n, sink); }, 10,
              &ms_plain))
    return 1;
  if (time_ms([&] { hipLaunchKernelGGL(k_read<true>, dim3(rgrid), dim3(256), 0, 0, a, n, sink); }, 10,
              &ms_nt))
    return 1;
  printf(", \"read_GBps\": {\"plain\": %.1f, \"nontemporal\": %.1f, \"bytes\": %lld}",
         bytes / (ms_plain * 1e-3) / 1e9, bytes / (ms_nt * 1e-3) / 1e9, (long long)bytes);
  CHECK(hipFree(a));
  CHECK(hipFree(sink));
  printf("}\n");
  return 0;
}
