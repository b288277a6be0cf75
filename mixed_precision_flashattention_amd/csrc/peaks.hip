// Measured ceilings of the MI355X that the roofline fractions are quoted
// against: streaming-read bandwidth of HBM (plain and non-temporal 16-byte
// loads over the 128K decode workload's 3.49 GB), the issue rate of the
// MFMA instructions the kernels use (32x32x16 f16 and bf16, 32x32x64 FP8
// and FP4 with unit block scales), and the vector-ALU ceiling of the
// prefill's softmax.  A standalone program, not part of the library: it
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
