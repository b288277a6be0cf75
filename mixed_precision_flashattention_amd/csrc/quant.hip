// Stage-one kernels: sequence statistics, NVFP4 K, the compensation vector
// Delta_S and FP8 V (paper "MpFA: ...", section 5.1 "first stage" and
// section 6 "Online quantization").  These passes are HBM-bound streaming
// kernels; their outputs are defined bit for bit (see mpfa.h), so every
// rounding below is the one the header states.
#include "mpfa_internal.hpp"

namespace mpfa {

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Per (b, h, d): max over tokens of |x|.  Block: 256 threads = 2 token rows
// x 128 channels; grid (token chunks, B*H).
constexpr int kStatRows = 256;

__global__ void k_channel_absmax(const void* __restrict__ x, int is_bf16, int N,
                                 uint32_t* __restrict__ out) {
  const int d = threadIdx.x & 127;
  const int64_t bh = blockIdx.y;
  const int r_begin = blockIdx.x * kStatRows;
  const int r_end = min(N, r_begin + kStatRows);
  float m = 0.0f;
  for (int r = r_begin + (threadIdx.x >> 7); r < r_end; r += 2)
    m = fmaxf(m, fabsf(load_elem(x, (bh * N + r) * kD + d, is_bf16)));
  atomic_max_nonneg(out + bh * kD + d, m);
}

// Per (b, h, d): 64-bit fixed-point sum of x at unit 2^(E-30), where the
// channel amax M lies in [2^(E-1), 2^E).  Each term is rounded to the
// nearest integer (half to even) in FP64, where the scaling is exact; the
// integer sum is exact, so the result does not depend on order.
__global__ void k_channel_fixsum(const void* __restrict__ x, int is_bf16, int N,
                                 const uint32_t* __restrict__ absmax,
                                 unsigned long long* __restrict__ sums) {
  const int d = threadIdx.x & 127;
  const int64_t bh = blockIdx.y;
  const float M = __uint_as_float(absmax[bh * kD + d]);
  if (M == 0.0f) return;
  int E;
  frexpf(M, &E);
  const double unit_inv = ldexp(1.0, 30 - E);
  const int r_begin = blockIdx.x * kStatRows;
  const int r_end = min(N, r_begin + kStatRows);
  long long s = 0;
  for (int r = r_begin + (threadIdx.x >> 7); r < r_end; r += 2) {
    const double y = (double)load_elem(x, (bh * N + r) * kD + d, is_bf16) * unit_inv;
    s += (long long)__builtin_rint(y);
  }
  atomicAdd(sums + bh * kD + d, (unsigned long long)s);
}

// mean = fp32( (double)S / (double)N * 2^(E-30) ), each FP64 op rounded once.
__global__ void k_mean_finalize(const uint32_t* __restrict__ absmax,
                                const unsigned long long* __restrict__ sums, int N, int n,
                                float* __restrict__ mean) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float M = __uint_as_float(absmax[i]);
  if (M == 0.0f) {
    mean[i] = 0.0f;
    return;
  }
  int E;
  frexpf(M, &E);
  const double s = (double)(long long)sums[i];
  const double m = (s / (double)N) * ldexp(1.0, E - 30);
  mean[i] = (float)m;
}

// max |fp32(x - mean[bh, d])| over a whole [BH, N, 128] tensor (mean may be
// NULL).  Grid (row chunks, BH): each thread takes 16-element groups of one
// (batch, head) slice; one atomic per wave.
constexpr int kAmaxGroups = 4096;  // 16-element groups per block (512 rows)

__global__ void k_centered_amax(const void* __restrict__ x, int is_bf16, int N,
                                const float* __restrict__ mean, uint32_t* __restrict__ out) {
  const int64_t bh = blockIdx.y;
  const int64_t n_groups = (int64_t)N * 8;
  const int64_t g_begin = (int64_t)blockIdx.x * kAmaxGroups;
  const int64_t g_end = min(n_groups, g_begin + kAmaxGroups);
  const int d0 = (threadIdx.x & 7) * 16;  // blockDim is a multiple of 8
  float mu[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) mu[j] = mean ? mean[bh * kD + d0 + j] : 0.0f;
  float m = 0.0f;
  for (int64_t gi = g_begin + threadIdx.x; gi < g_end; gi += blockDim.x) {
    float v[16];
    load16(x, (bh * n_groups + gi) * 16, is_bf16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j] - mu[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(out, m);
}

// NVFP4 codes and scales of K_c = fp32(K - k_mean) (k_mean NULL: K_c = K).
// One thread per (token row, 16-element block).
__global__ void k_quantize_k(const void* __restrict__ k, int is_bf16, int64_t n_groups, int N,
                             const float* __restrict__ k_mean,
                             const uint32_t* __restrict__ amax, float* __restrict__ gscale_out,
                             uint8_t* __restrict__ codes, uint8_t* __restrict__ sf) {
  const float g = nvfp4_global_scale(__uint_as_float(*amax));
  const int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gi == 0) *gscale_out = g;
  if (gi >= n_groups) return;
  float v[16];
  load16(k, gi * 16, is_bf16, v);
  if (k_mean) {
    const float* mu = k_mean + (gi / 8 / N) * kD + (int)(gi & 7) * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] - mu[j];
  }
  uint32_t c[16];
  const uint32_t sc = nvfp4_block(v, g, c);
  uint2 packed;
  packed.x = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) |
             (c[6] << 24) | (c[7] << 28);
  packed.y = c[8] | (c[9] << 4) | (c[10] << 8) | (c[11] << 12) | (c[12] << 16) | (c[13] << 20) |
             (c[14] << 24) | (c[15] << 28);
  reinterpret_cast<uint2*>(codes)[gi] = packed;
  sf[gi] = (uint8_t)sc;
}

// Delta_S[b, hk*G + g, t] = bf16(fp32(sum_d q_mean[b, hk*G+g, d] * K_c[b, hk, t, d])),
// the sum in FP64 over ascending d (each product is exact in FP64, so a
// fused multiply-add rounds exactly like an add of the product).
// One thread per (b, hk, token) and group of up to 8 query heads.
__global__ void k_delta_s(const void* __restrict__ k, int is_bf16, int Hkv, int G, int N,
                          const float* __restrict__ k_mean, const float* __restrict__ q_mean,
                          uint16_t* __restrict__ delta) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int bhk = blockIdx.y;       // b * Hkv + hk
  const int g0 = blockIdx.z * 8;
  if (t >= N) return;
  const int ng = min(8, G - g0);
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int64_t hq0 = (int64_t)b * Hkv * G + (int64_t)hk * G + g0;
  const float* km = k_mean + (int64_t)bhk * kD;
  const float* qm = q_mean + hq0 * kD;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t row = ((int64_t)bhk * N + t) * kD;
  for (int d0 = 0; d0 < kD; d0 += 16) {
    float v[16];
    load16(k, row + d0, is_bf16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double kc = (double)(v[j] - km[d0 + j]);
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g < ng) acc[g] = __builtin_fma((double)qm[g * kD + d0 + j], kc, acc[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < 8; ++g)
    if (g < ng) delta[(hq0 + g) * N + t] = (uint16_t)bf16_rne((float)acc[g]);
}

// FP8 E4M3 V in 32-token tiles, head-dim major inside a tile.  Block: 128
// threads (one per channel) x one tile; positions past N are written as 0.
__global__ void k_quantize_v(const void* __restrict__ v, int is_bf16, int N, int n_tiles,
                             const uint32_t* __restrict__ amax, float* __restrict__ vscale_out,
                             uint8_t* __restrict__ out) {
  const float A = __uint_as_float(*amax);
  const float s = A > 0.0f ? A / kE4M3Max : 1.0f;
  const int d = threadIdx.x;
  const int tile = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (tile == 0 && bh == 0 && d == 0) *vscale_out = s;
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int t = tile * 32 + j * 4 + b;
      uint32_t c = 0;
      if (t < N) c = e4m3_encode(load_elem(v, (bh * N + t) * kD + d, is_bf16) / s);
      word |= c << (8 * b);
    }
    w[j] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(out + ((bh * n_tiles + tile) * kD + d) * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// ------------------------------------------------------------- launchers --
static inline unsigned grid_for(int64_t n, int block, unsigned cap) {
  int64_t g = (n + block - 1) / block;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256, 4096)), dim3(256), 0, st, p, n, v);
}

void launch_channel_mean(const void* x, int is_bf16, int BH, int N, uint32_t* absmax,
                         unsigned long long* sums, float* mean, hipStream_t st) {
  dim3 grid((N + kStatRows - 1) / kStatRows, BH);
  hipLaunchKernelGGL(k_channel_absmax, grid, dim3(256), 0, st, x, is_bf16, N, absmax);
  hipLaunchKernelGGL(k_channel_fixsum, grid, dim3(256), 0, st, x, is_bf16, N,
                     (const uint32_t*)absmax, sums);
  const int n = BH * kD;
  hipLaunchKernelGGL(k_mean_finalize, dim3((n + 255) / 256), dim3(256), 0, st,
                     (const uint32_t*)absmax, (const unsigned long long*)sums, N, n, mean);
}

void launch_centered_amax(const void* x, int is_bf16, int BH, int N, const float* mean,
                          uint32_t* out, hipStream_t st) {
  const int64_t n_groups = (int64_t)N * (kD / 16);
  dim3 grid((unsigned)((n_groups + kAmaxGroups - 1) / kAmaxGroups), BH);
  hipLaunchKernelGGL(k_centered_amax, grid, dim3(256), 0, st, x, is_bf16, N, mean, out);
}

void launch_quantize_k_codes(const void* k, int is_bf16, int BH, int N, const float* k_mean,
                             const uint32_t* amax, float* gscale, uint8_t* codes, uint8_t* sf,
                             hipStream_t st) {
  const int64_t n_groups = (int64_t)BH * N * (kD / 16);
  hipLaunchKernelGGL(k_quantize_k, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, st, k,
                     is_bf16, n_groups, N, k_mean, amax, gscale, codes, sf);
}

void launch_delta_s(const void* k, int is_bf16, int B, int Hkv, int G, int N, const float* k_mean,
                    const float* q_mean, uint16_t* delta, hipStream_t st) {
  dim3 grid((N + 127) / 128, B * Hkv, (G + 7) / 8);
  hipLaunchKernelGGL(k_delta_s, grid, dim3(128), 0, st, k, is_bf16, Hkv, G, N, k_mean, q_mean,
                     delta);
}

void launch_quantize_v_codes(const void* v, int is_bf16, int BH, int N, const uint32_t* amax,
                             float* vscale, uint8_t* out, hipStream_t st) {
  const int n_tiles = (N + 31) / 32;
  hipLaunchKernelGGL(k_quantize_v, dim3(n_tiles, BH), dim3(128), 0, st, v, is_bf16, N, n_tiles,
                     amax, vscale, out);
}

}  // namespace mpfa
