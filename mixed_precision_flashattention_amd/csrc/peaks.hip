// Measured ceilings of the MI355X that the roofline fractions are quoted
// against: streaming-read bandwidth of HBM (plain and non-temporal 16-byte
// loads over the 128K decode workload's 3.49 GB) and the issue rate of the
// MFMA instructions the kernels use (32x32x16 f16 and bf16, 32x32x64 FP8
// and FP4 with unit block scales).  A standalone program, not part of the
// library: it prints one JSON object.
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
