// Check of the hardware FP32 -> E2M1 conversion the NVFP4 quantizers use
// (v_cvt_scalef32_pk_fp4_f32 at unit scale) against the library's E2M1
// encoder (nearest, ties to the even code, saturating at 6, sign kept): every
// fp32 value within 64 ulps of each E2M1 midpoint and grid point and of a few
// values past the range, both signs, +-0, tiny, huge and denormal values, and
// a million seeded random values in [-8, 8].
//
// Second check: the NVFP4 quantizers' per-block quotients (block_divisor /
// block_quotient: a reciprocal rounded once per block and two FMA residual
// corrections) against IEEE division x / d, for d = every positive E4M3
// value times global scales from 2^-120 to 2^120 and x placed within 4 ulps
// of d times every E2M1 midpoint and grid point, plus seeded random
// quotients in [1/8, 8].  Quotients of magnitude >= 1/8 must be bit-equal
// and every sign must match (smaller ones give a zero code either way).
//
// A standalone program built beside the library; prints one JSON object
// with the mismatch counts and exits non-zero on any mismatch.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mpfa_device.hpp"

using namespace mpfa;

__global__ void k_check(const float* __restrict__ in, int n, uint32_t* __restrict__ bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = in[i];
  const float b = in[(i + 1) % n];  // a second value in the high nibble
  const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
  const uint32_t sw = e2m1_encode(a) | (e2m1_encode(b) << 4);
  if (hw != sw) atomicAdd(bad, 1u);
}

__global__ void k_check_quotient(const float2* __restrict__ xd, int n, uint32_t* __restrict__ bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = xd[i].x, d = xd[i].y;
  const float want = x / d;
  const float got = block_quotient(block_divisor(d, false), x);
  const bool sign_ok = (__float_as_uint(want) >> 31) == (__float_as_uint(got) >> 31);
  const bool big = fabsf(want) >= 0.125f || fabsf(got) >= 0.125f;
  if (!sign_ok || (big && __float_as_uint(want) != __float_as_uint(got))) atomicAdd(bad, 1u);
}

static float bump(float x, int k) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += (uint32_t)k;
  float y;
  memcpy(&y, &u, 4);
  return y;
}

int main() {
  std::vector<float> v;
  const float pts[] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 0.5f,  1.0f,   1.5f,
                       2.0f,  3.0f,  4.0f,  6.0f,  6.5f, 7.0f, 8.0f, 0.125f, 0.375f};
  for (float p : pts)
    for (int k = -64; k <= 64; ++k) {
      v.push_back(bump(p, k));
      v.push_back(-bump(p, k));
    }
  const float extra[] = {0.0f,   -0.0f,  1e-30f, -1e-30f, 1e-40f,  -1e-40f, 0.1f,   0.2f,
                         100.0f, -100.0f, 1e30f, -1e30f,  3.4e38f, -3.4e38f, 12.0f, 24.0f};
  for (float e : extra) v.push_back(e);
  uint32_t state = 12345u;  // xorshift32, seeded
  for (int i = 0; i < 1000000; ++i) {
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    v.push_back(((float)(state >> 8) / 16777216.0f - 0.5f) * 16.0f);
  }
  const int n = (int)v.size();
  float* din = nullptr;
  uint32_t* dbad = nullptr;
  if (hipMalloc(&din, (size_t)n * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&dbad, sizeof(uint32_t)) != hipSuccess) return 2;
  if (hipMemcpy(din, v.data(), (size_t)n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return 2;
  if (hipMemset(dbad, 0, sizeof(uint32_t)) != hipSuccess) return 2;
  hipLaunchKernelGGL(k_check, dim3((n + 255) / 256), dim3(256), 0, 0, din, n, dbad);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  uint32_t bad = 0;
  if (hipMemcpy(&bad, dbad, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return 2;
  (void)hipFree(din);

  // ---- per-block quotients
  std::vector<float> scales = {1.0f, 0x1.37p-120f, 0x1.9p-64f, 0x1.fffffep-65f, 0x1.0p64f,
                               0x1.000002p64f, 0x1.d3p+120f, 3.1e-4f};
  for (int i = 0; i < 56; ++i) {  // seeded scales, exponents 2^-120 .. 2^120
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    const float m = 1.0f + (float)(state >> 9) / 8388608.0f;
    scales.push_back(ldexpf(m, (int)(state % 241u) - 120));
  }
  std::vector<float2> xd;
  for (int c = 1; c < 127; ++c) {  // every positive finite E4M3 value
    const int e = c >> 3, mt = c & 7;
    const float sv = e ? ldexpf(1.0f + mt / 8.0f, e - 7) : ldexpf(mt / 8.0f, -6);
    for (float g : scales) {
      const float d = sv * g;
      if (!(d > 0.0f) || d > 3.0e38f) continue;
      for (float t : pts)
        for (int k = -4; k <= 4; ++k) {
          const float x = bump(t * d, k);
          if (!(fabsf(x) < 3.0e38f)) continue;
          xd.push_back(make_float2(x, d));
          xd.push_back(make_float2(-x, d));
        }
      for (int r = 0; r < 8; ++r) {
        state ^= state << 13;
        state ^= state >> 17;
        state ^= state << 5;
        const float q = ldexpf(1.0f + (float)(state >> 9) / 8388608.0f, (int)(state % 6u) - 3);
        const float x = q * d;
        if (fabsf(x) < 3.0e38f) xd.push_back(make_float2((state & 1u) ? -x : x, d));
      }
    }
  }
  const int nq = (int)xd.size();
  float2* dxd = nullptr;
  if (hipMalloc(&dxd, (size_t)nq * sizeof(float2)) != hipSuccess) return 2;
  if (hipMemcpy(dxd, xd.data(), (size_t)nq * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) return 2;
  if (hipMemset(dbad, 0, sizeof(uint32_t)) != hipSuccess) return 2;
  hipLaunchKernelGGL(k_check_quotient, dim3((nq + 255) / 256), dim3(256), 0, 0, dxd, nq, dbad);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  uint32_t qbad = 0;
  if (hipMemcpy(&qbad, dbad, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return 2;
  (void)hipFree(dxd);
  (void)hipFree(dbad);
  printf("{\"values\": %d, \"mismatches\": %u, \"quotients\": %d, \"quotient_mismatches\": %u}\n", n,
         bad, nq, qbad);
  return bad == 0 && qbad == 0 ? 0 : 1;
}
