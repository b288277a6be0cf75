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

// Per-channel statistics over the tokens of each (batch, head) slice.  Grid
// (row chunks, BH) with about 2048 blocks in all; block = 16 row lanes x 16
// channel groups of 8 channels; each thread keeps 8 channel accumulators over
// rows rl, rl + 16, ... of its chunk (four 16-byte loads in flight), the
// block reduces its 16 row lanes in LDS and then updates the 128 channel
// totals with one atomic each.
// The same with non-temporal loads, for the statistics passes that stream a
// whole tensor once each (nothing they read is reused from the cache).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8_stream(const void* p, int64_t i, int is_bf16, float* x) {
  if (is_bf16) {
    const u32x4_nt a = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_nt*>(reinterpret_cast<const uint16_t*>(p) + i));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(a[j] << 16);
      x[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
    }
  } else {
    const f32x4_nt* s = reinterpret_cast<const f32x4_nt*>(reinterpret_cast<const float*>(p) + i);
    const f32x4_nt a = __builtin_nontemporal_load(s), b = __builtin_nontemporal_load(s + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  }
}

__device__ __forceinline__ void load8(const void* p, int64_t i, int is_bf16, float* x) {
  if (is_bf16) {
    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4* s = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 a = s[0], b = s[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

constexpr int kStatBlocks = 2048;  // target number of blocks per statistics pass
// The two statistics passes read the same tensors one after the other.  When
// they fit in the device's last-level cache (256 MiB on MI355X) the second
// pass finds them there, and each thread keeps 8 rows of loads in flight
// over blocks of whole 128-row steps; when they do not, nothing is reused,
// and the loads are non-temporal with 4 rows in flight (each choice the
// faster one in measurements at 16K and 32K tokens).
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;

// The sequence-mean passes take one or two [BH, N, 128] tensors of the same
// N (K and Q) in one launch: blocks [0, nblk0) cover tensor 0 and the rest
// tensor 1, each as gx row blocks (fastest) times BH heads.  Every result is
// an order-free reduction, so the split of the grid does not change a bit.
struct StatJobs {
  const void* x[2];
  int is_bf16[2], BH[2], rows[2], gx[2];
  uint32_t* range[2];  // [2][BH * 128]: ordered keys of max x, then of max -x
  unsigned long long* sums[2];
  float* mean[2];
  uint32_t* extent[2];  // NULL, or max |fp32(x - mean)| over the tensor
  int nblk0, N;
};
struct StatBlock {
  const void* x;
  int is_bf16, rows, r_begin;
  int64_t bh, nch;
  uint32_t* range;
  unsigned long long* sums;
};
__device__ __forceinline__ StatBlock stat_block(const StatJobs& J) {
  int f = blockIdx.x;
  const int t = f >= J.nblk0;
  if (t) f -= J.nblk0;
  StatBlock b;
  const int gx = t ? J.gx[1] : J.gx[0];
  b.x = t ? J.x[1] : J.x[0];
  b.is_bf16 = t ? J.is_bf16[1] : J.is_bf16[0];
  b.rows = t ? J.rows[1] : J.rows[0];
  b.range = t ? J.range[1] : J.range[0];
  b.nch = (int64_t)(t ? J.BH[1] : J.BH[0]) * kD;
  b.sums = t ? J.sums[1] : J.sums[0];
  b.bh = f / gx;
  b.r_begin = (f % gx) * b.rows;
  return b;
}

// max |x| of channel i from its range: max(max x, max -x)
__device__ __forceinline__ float range_absmax(const uint32_t* range, int64_t nch, int64_t i) {
  return fmaxf(ordered_value(range[i]), ordered_value(range[nch + i]));
}

// Per (b, h, d): max over tokens of x and of -x (the channel's range).
template <bool STREAM, int ROWS>
__global__ __launch_bounds__(256) void k_channel_absmax(StatJobs J) {
  __shared__ float red[2][16][kD];
  const StatBlock sb = stat_block(J);
  const void* x = sb.x;
  const int is_bf16 = sb.is_bf16, N = J.N;
  uint32_t* __restrict__ out = sb.range;
  const int64_t bh = sb.bh;
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int rows_per_block = sb.rows;
  const int r_begin = sb.r_begin;
  const int r_end = min(N, r_begin + rows_per_block);
  float hi[8], lo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) hi[j] = lo[j] = -INFINITY;
  for (int r = r_begin + rl; r < r_end; r += 16 * ROWS) {
    float v[ROWS][8];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      const int64_t i = (bh * N + min(r + 16 * k, r_end - 1)) * kD + 8 * cg;
      if (STREAM) load8_stream(x, i, is_bf16, v[k]); else load8(x, i, is_bf16, v[k]);
    }
#pragma unroll
    for (int k = 0; k < ROWS; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // repeats are harmless
        hi[j] = fmaxf(hi[j], v[k][j]);
        lo[j] = fmaxf(lo[j], -v[k][j]);
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    red[0][rl][8 * cg + j] = hi[j];
    red[1][rl][8 * cg + j] = lo[j];
  }
  __syncthreads();
  if (threadIdx.x < 2 * kD) {
    const int side = threadIdx.x >> 7, c = threadIdx.x & (kD - 1);
    float t = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) t = fmaxf(t, red[side][i][c]);
    atomicMax(out + side * sb.nch + bh * kD + c, ordered_key(t));
  }
}

// RNE(x * 2^shift) as an integer, for |x * 2^shift| < 2^30 (see above).
__device__ __forceinline__ long long fixed_point_term(float x, int shift) {
  return (long long)(int)__builtin_rintf(__builtin_ldexpf(x, shift));
}

// Per (b, h, d): 64-bit fixed-point sum of x at unit 2^(E-30), where the
// channel amax M lies in [2^(E-1), 2^E).  Each term is x scaled by
// 2^(30-E) and rounded to the nearest integer (half to even); the integer
// sum is exact, so the result does not depend on order.  The scaled value
// has magnitude below 2^30, so the FP32 ldexp is exact wherever the result
// can round to a nonzero integer, the FP32 round-to-nearest-even gives the
// same integer as in FP64, and it fits an int32.
template <bool STREAM, int ROWS>
__global__ __launch_bounds__(256) void k_channel_fixsum(StatJobs J) {
  __shared__ long long red[16][kD];
  const StatBlock sb = stat_block(J);
  const void* x = sb.x;
  const int is_bf16 = sb.is_bf16, N = J.N;
  const uint32_t* __restrict__ range = sb.range;
  unsigned long long* __restrict__ sums = sb.sums;
  const int64_t bh = sb.bh;
  const int rows_per_block = sb.rows;
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  int shift[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float M = range_absmax(range, sb.nch, bh * kD + 8 * cg + j);
    int E = 0;
    if (M != 0.0f) frexpf(M, &E);
    shift[j] = 30 - E;  // an all-zero channel scales zeros: it sums to 0
  }
  const int r_begin = sb.r_begin;
  const int r_end = min(N, r_begin + rows_per_block);
  long long acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r_begin + rl; r < r_end; r += 16 * ROWS) {
    float v[ROWS][8];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      const int64_t i = (bh * N + min(r + 16 * k, r_end - 1)) * kD + 8 * cg;
      if (STREAM) load8_stream(x, i, is_bf16, v[k]); else load8(x, i, is_bf16, v[k]);
    }
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      if (r + 16 * k < r_end) {  // every row counted exactly once
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += fixed_point_term(v[k][j], shift[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rl][8 * cg + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < kD) {
    long long t = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += red[i][threadIdx.x];
    atomicAdd(sums + bh * kD + threadIdx.x, (unsigned long long)t);
  }
}

// mean = fp32( (double)S / (double)N * 2^(E-30) ), each FP64 op rounded once.
// Thread i < n0 = BH[0] * 128 finalizes tensor 0's channel i, the rest tensor
// 1's (n0 is a multiple of 128, so no wave spans both).  With extent[t]
// non-NULL (a cleared word) it also takes the tensor's centred amax
// max |fp32(x - mean)| from the ranges: fp32 subtraction is monotone in x
// and x - m rounds to the negation of m - x, so over a channel it is
// max(fp32(max x - m), fp32(m + max -x)), the value a pass over x would
// find; one atomic per wave.
__global__ __launch_bounds__(256) void k_mean_finalize(StatJobs J, int n0, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = i < n;
  const int t = i >= n0;
  if (t) i -= n0;
  const uint32_t* __restrict__ range = t ? J.range[1] : J.range[0];
  const unsigned long long* __restrict__ sums = t ? J.sums[1] : J.sums[0];
  float* __restrict__ mean = t ? J.mean[1] : J.mean[0];
  uint32_t* extent = t ? J.extent[1] : J.extent[0];
  const int64_t nch = (int64_t)(t ? J.BH[1] : J.BH[0]) * kD;
  const int N = J.N;
  float e = 0.0f;
  if (valid) {
    const float hi = ordered_value(range[i]), lo = ordered_value(range[nch + i]);
    const float M = fmaxf(hi, lo);
    float mu = 0.0f;
    if (M != 0.0f) {
      int E;
      frexpf(M, &E);
      const double s = (double)(long long)sums[i];
      mu = (float)((s / (double)N) * ldexp(1.0, E - 30));
    }
    mean[i] = mu;
    const float a = fmaxf(hi - mu, mu + lo);
    e = a > 0.0f ? a : 0.0f;
  }
  if (extent) {  // uniform over the wave
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e = fmaxf(e, __shfl_xor(e, o));
    if ((threadIdx.x & 63) == 0) atomic_max_nonneg(extent, e);
  }
}

// Channel means of each 128-row tile of a [BH, N, 128] tensor by the rule of
// the sequence means above (amax M of the channel over the tile's rows, terms
// rounded to integers at unit 2^(E-30), an exact integer sum, one FP64
// division by the tile's row count).  One block per (tile, bh); thread
// (rl, cg) holds rows rl, rl + 16, ... of the tile for channels 8 cg .. +7,
// so both passes read the rows once.  mean: [BH, ceil(N/128), 128].
// With amax non-NULL the block also takes max |fp32(x - tile mean)| over its
// rows (the rows are still in registers) and adds it to the slotted amax of
// the tile-centred tensor (out[slot * kAmaxSlotWords], cleared beforehand,
// folded afterwards), so no second pass over x is needed for it.
__global__ __launch_bounds__(256) void k_tile_mean(const void* __restrict__ x, int is_bf16, int N,
                                                   float* __restrict__ mean,
                                                   uint32_t* __restrict__ amax) {
  __shared__ float fred[16][kD];
  __shared__ long long ired[16][kD];
  __shared__ float cmax[kD];
  __shared__ float cmean[kD];
  __shared__ float ared[4];
  const int64_t bh = blockIdx.y;
  const int t = blockIdx.x;
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int r0 = t * kBlk, n = min(N - r0, kBlk);
  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + min(rl + 16 * i, n - 1);  // a repeated row is not summed below
    load8(x, (bh * N + r) * kD + 8 * cg, is_bf16, v[i]);
  }
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m[j] = fmaxf(m[j], fabsf(v[i][j]));
    fred[rl][8 * cg + j] = m[j];
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fred[i][threadIdx.x]);
    cmax[threadIdx.x] = a;
  }
  __syncthreads();
  long long acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float M = cmax[8 * cg + j];
    int E = 0;
    if (M != 0.0f) frexpf(M, &E);
    acc[j] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (rl + 16 * i < n) acc[j] += fixed_point_term(v[i][j], 30 - E);
    ired[rl][8 * cg + j] = acc[j];
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    long long S = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) S += ired[i][threadIdx.x];
    const float M = cmax[threadIdx.x];
    float out = 0.0f;
    if (M != 0.0f) {
      int E;
      frexpf(M, &E);
      out = (float)(((double)S / (double)n) * ldexp(1.0, E - 30));
    }
    mean[(bh * gridDim.x + t) * kD + threadIdx.x] = out;
    cmean[threadIdx.x] = out;
  }
  if (!amax) return;  // uniform across the block
  __syncthreads();
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float mu = cmean[8 * cg + j];
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i][j] - mu));  // a repeated row adds nothing
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((threadIdx.x & 63) == 0) ared[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int slot = (blockIdx.x + blockIdx.y * gridDim.x) % kAmaxSlots;
    atomic_max_nonneg(amax + slot * kAmaxSlotWords,
                      fmaxf(fmaxf(ared[0], ared[1]), fmaxf(ared[2], ared[3])));
  }
}

// max |fp32(x - mean[bh, d])| over a whole [BH, N, 128] tensor (mean may be
// NULL).  Same grid and thread layout as the channel statistics; each thread
// keeps one running max, the block reduces it (wave shuffles, then LDS) and
// issues a single atomic.  With partials non-NULL the block instead stores
// its maximum in partials[block] (no atomic, nothing to clear beforehand);
// a later kernel folds them.
__global__ __launch_bounds__(256) void k_centered_amax(const void* __restrict__ x, int is_bf16,
                                                       int N, int rows_per_block,
                                                       const float* __restrict__ mean,
                                                       uint32_t* __restrict__ out,
                                                       float* __restrict__ partials) {
  __shared__ float red[4];
  const int64_t bh = blockIdx.y;
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = mean ? mean[bh * kD + 8 * cg + j] : 0.0f;
  const int r_begin = blockIdx.x * rows_per_block;
  const int r_end = min(N, r_begin + rows_per_block);
  float m = 0.0f;
  for (int r = r_begin + rl; r < r_end; r += 128) {
    float v[8][8];
#pragma unroll
    for (int k = 0; k < 8; ++k)  // a repeated row does not change the max
      load8(x, (bh * N + min(r + 16 * k, r_end - 1)) * kD + 8 * cg, is_bf16, v[k]);
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[k][j] - mu[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (partials) {
      partials[blockIdx.x + blockIdx.y * gridDim.x] = bm;
    } else {
      const int slot = (blockIdx.x + blockIdx.y * gridDim.x) % kAmaxSlots;
      atomic_max_nonneg(out + slot * kAmaxSlotWords, bm);
    }
  }
}

// max |fp32(x - mean[r, d])| over the rows of a [rows, 128] tensor (the
// decode queries: one row per head, mean may be NULL), as kRowsAmaxSlots
// partial maxima: workgroup i reduces rows i R .. i R + R - 1 (R =
// ceil(rows / kRowsAmaxSlots)) and stores its maximum in out[i] (0 when it
// has no rows).  Every slot is written, so nothing needs clearing first, and
// there is no atomic and no fold kernel: a consumer takes the max of the
// slots itself (one wave, one load per lane).
__global__ __launch_bounds__(256) void k_rows_amax(const void* __restrict__ x, int is_bf16,
                                                  int rows, const float* __restrict__ mean,
                                                  float* __restrict__ out) {
  __shared__ float red[4];
  const int R = (rows + kRowsAmaxSlots - 1) / kRowsAmaxSlots;
  const int r0 = min(rows, (int)blockIdx.x * R), r1 = min(rows, r0 + R);
  const int64_t g0 = (int64_t)r0 * (kD / 8), g1 = (int64_t)r1 * (kD / 8);  // groups of 8
  float m = 0.0f;
  for (int64_t g = g0 + threadIdx.x; g < g1; g += 4 * 256) {
    float v[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k)  // a repeated group does not change the max
      load8(x, min(g + 256 * k, g1 - 1) * 8, is_bf16, v[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t e = min(g + 256 * k, g1 - 1) * 8;  // channel e % 128 of row e / 128
      float mu[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mu[j] = mean ? mean[e + j] : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[k][j] - mu[j]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// n per-workgroup maxima (non-negative) folded into out[0] as fp32 bits; one
// block, every read before the barrier, so out may alias partials.
__global__ __launch_bounds__(256) void k_partials_fold(const float* partials, int n,
                                                       uint32_t* out) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, partials[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

// The slots of a reduced amax folded into its first word (one wave).
__global__ __launch_bounds__(64) void k_amax_fold(uint32_t* __restrict__ out) {
  uint32_t m = out[threadIdx.x * kAmaxSlotWords];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (threadIdx.x == 0) out[0] = m;
}

// NVFP4 codes and scales of K_c = fp32(K - k_mean) (k_mean NULL: K_c = K).
// One thread per (token row, 16-element block).
__global__ void k_quantize_k(const void* __restrict__ k, int is_bf16, int64_t n_groups, int N,
                             const float* __restrict__ k_mean,
                             const uint32_t* __restrict__ amax, float* __restrict__ gscale_out,
                             uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
                             const uint32_t* __restrict__ q_ext, float* __restrict__ q_amax_out) {
  const float g = nvfp4_global_scale(__uint_as_float(*amax));
  const int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gi == 0) {
    *gscale_out = g;
    if (q_amax_out) *q_amax_out = __uint_as_float(*q_ext);  // the Q_c amax, passed on
  }
  if (gi >= n_groups) return;
  float v[16];
  load16(k, gi * 16, is_bf16, v);
  if (k_mean) {
    const float* mu = k_mean + (gi / 8 / N) * kD + (int)(gi & 7) * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] - mu[j];
  }
  uint32_t w[2];
  const uint32_t sc = nvfp4_block_packed(v, g, w);
  reinterpret_cast<uint2*>(codes)[gi] = make_uint2(w[0], w[1]);
  sf[gi] = (uint8_t)sc;
}

// Delta_S[b, hk*G + g, t] = bf16(fp32(sum_d q_mean[b, hk*G+g, d] * K_c[b, hk, t, d])),
// the sum in FP64 over ascending d (each product is exact in FP64, so a
// fused multiply-add rounds exactly like an add of the product).
// Block: 64 tokens of one (b, hk) and up to 8 query heads (64 threads per
// head).  The block stages K_c = fp32(K - k_mean) of its tokens in LDS with
// coalesced loads (rows padded to 129 words, so the per-token reads below
// hit 64 different banks), then thread (token, head) runs its FP64 sum.
// With codes non-NULL the first block of every (b, hk) column of the grid
// (blockIdx.z == 0) also writes the NVFP4 codes and scales of its 64 centred
// rows from the same LDS copy (the K quantizer's bytes: the same fp32 K_c
// values and block steps), so K is read once for both.
constexpr int kDsRows = 64;

__global__ __launch_bounds__(512) void k_delta_s(const void* __restrict__ k, int is_bf16, int Hkv,
                                                 int G, int N, const float* __restrict__ k_mean,
                                                 const float* __restrict__ q_mean,
                                                 uint16_t* __restrict__ delta,
                                                 const uint32_t* __restrict__ amax,
                                                 float* __restrict__ gscale_out,
                                                 uint2* __restrict__ codes,
                                                 uint8_t* __restrict__ sf,
                                                 const uint32_t* __restrict__ q_ext,
                                                 float* __restrict__ q_amax_out) {
  __shared__ float kc[kDsRows * (kD + 1)];
  __shared__ float qm[8 * kD];
  const int bhk = blockIdx.y;  // b * Hkv + hk
  const int g0 = blockIdx.z * 8;
  const int ng = min(8, G - g0);
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int64_t hq0 = (int64_t)b * Hkv * G + (int64_t)hk * G + g0;
  const int t0 = blockIdx.x * kDsRows;
  const float* km = k_mean + (int64_t)bhk * kD;
  for (int e = threadIdx.x * 8; e < kDsRows * kD; e += blockDim.x * 8) {
    const int r = e >> 7, d = e & 127;
    float v[8];
    load8(k, ((int64_t)bhk * N + min(t0 + r, N - 1)) * kD + d, is_bf16, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) kc[r * (kD + 1) + d + j] = v[j] - km[d + j];
  }
  for (int e = threadIdx.x; e < ng * kD; e += blockDim.x) qm[e] = q_mean[hq0 * kD + e];
  __syncthreads();
  if (codes && blockIdx.z == 0) {  // uniform across the block
    const float gk = nvfp4_global_scale(__uint_as_float(*amax));
    if (blockIdx.x == 0 && bhk == 0 && threadIdx.x == 0) {
      *gscale_out = gk;
      if (q_amax_out) *q_amax_out = __uint_as_float(*q_ext);  // the Q_c amax, passed on
    }
    for (int gi = threadIdx.x; gi < kDsRows * 8; gi += blockDim.x) {
      const int rr = gi >> 3, c = gi & 7;
      if (t0 + rr >= N) continue;
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = kc[rr * (kD + 1) + 16 * c + j];
      uint32_t w[2];
      const uint32_t sc = nvfp4_block_packed(x, gk, w);
      const int64_t o = ((int64_t)bhk * N + t0 + rr) * 8 + c;
      codes[o] = make_uint2(w[0], w[1]);
      sf[o] = (uint8_t)sc;
    }
  }
  const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = t0 + r;
  if (t >= N || g >= ng) return;
  const float* row = kc + r * (kD + 1);
  const float* q = qm + g * kD;
  double acc = 0.0;
#pragma unroll 16
  for (int d = 0; d < kD; ++d) acc = __builtin_fma((double)q[d], (double)row[d], acc);
  delta[(hq0 + g) * N + t] = (uint16_t)bf16_rne((float)acc);
}

// FP8 E4M3 V in 32-token tiles; inside a tile, two halves of 16 tokens,
// each head-dim major: token t, channel d at [t / 32][(t % 32) / 16][d][t % 16],
// so that 16 consecutive tokens of one channel are one 16-byte piece and the
// pieces of consecutive channels are adjacent.  Block: 128 threads x one
// tile; positions past N are written as 0.  Thread (tr, cg) reads channels
// 8 cg .. 8 cg + 7 of tokens 4 tr .. 4 tr + 3 of the tile (16-byte loads of
// bf16), encodes them and keeps one word per channel (its four tokens'
// codes); LDS turns the tile around so that thread d then writes channel
// d's two 16-token pieces (each store instruction of the block covers 2 KB
// contiguously).  Channel c's 32-byte LDS row sits in slot
// 8 (c / 8) + (c + c / 8) % 8, which spreads the word writes of one
// instruction over the banks.
__device__ __forceinline__ int v_tile_slot(int c) { return 8 * (c >> 3) + ((c + (c >> 3)) & 7); }
__global__ __launch_bounds__(128) void k_quantize_v(const void* __restrict__ v, int is_bf16, int N,
                                                    int n_tiles, const uint32_t* __restrict__ amax,
                                                    float* __restrict__ vscale_out,
                                                    uint8_t* __restrict__ out) {
  __shared__ __align__(16) uint32_t rows[kD * 8];  // [slot of channel][token / 4]
  const float A = __uint_as_float(*amax);
  const float s = A > 0.0f ? A / kE4M3Max : 1.0f;
  // every element is divided by s: one rounded reciprocal and two residual
  // corrections (block_quotient) give the correctly rounded quotient
  // wherever the E4M3 code depends on it.  That is for quotients of
  // magnitude >= 2^-10, half the smallest subnormal; with the divisor scaled
  // into [2^-64, 2^64], their residuals are multiples of at least 2^-120 and
  // stay exact.  Smaller quotients give a zero code, with the sign of x,
  // either way.
  const BlockDivisor dv = block_divisor(s, false);
  const int tile = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (tile == 0 && bh == 0 && threadIdx.x == 0) *vscale_out = s;
  const int cg = threadIdx.x & 15, tr = threadIdx.x >> 4;
  float x[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tile * 32 + 4 * tr + i;
    if (t < N) {
      load8(v, (bh * N + t) * kD + 8 * cg, is_bf16, x[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tile * 32 + 4 * tr + i;
      const uint32_t c = t < N ? e4m3_encode(block_quotient(dv, x[i][j])) : 0u;
      word |= c << (8 * i);
    }
    rows[v_tile_slot(8 * cg + j) * 8 + tr] = word;
  }
  __syncthreads();
  const int d = threadIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(rows + v_tile_slot(d) * 8);
  uint8_t* tbase = out + (bh * n_tiles + tile) * kD * 32;
  *reinterpret_cast<uint4*>(tbase + d * 16) = src[0];           // tokens 0 .. 15
  *reinterpret_cast<uint4*>(tbase + kD * 16 + d * 16) = src[1];  // tokens 16 .. 31
}

// NVFP4 V for the NVFP4 P.V variant (paper section 3.1, Fig. 3(a)): the P.V
// contraction runs over the keys, so the 16-element blocks run along the keys
// of one channel.  One 128-thread block per (16-key block, batch x KV head):
// thread d gathers channel d's 16 keys (each key row is read coalesced
// across the block; keys past N are zero), quantizes them with the global
// scale of the tensor amax and stores 8 code bytes and the scale byte.
__global__ __launch_bounds__(128) void k_quantize_v_nvfp4(const void* __restrict__ v, int is_bf16,
                                                          int N, int nb16,
                                                          const uint32_t* __restrict__ amax,
                                                          float* __restrict__ gscale_out,
                                                          uint2* __restrict__ codes,
                                                          uint8_t* __restrict__ sf) {
  const float g = nvfp4_global_scale(__uint_as_float(*amax));
  const int kb = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int d = threadIdx.x;
  if (kb == 0 && bh == 0 && d == 0) *gscale_out = g;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = 16 * kb + i;
    x[i] = t < N ? load_elem(v, (bh * N + t) * kD + d, is_bf16) : 0.0f;
  }
  uint32_t w[2];
  const uint32_t sc = nvfp4_block_packed(x, g, w);
  const int64_t o = (bh * nb16 + kb) * kD + d;
  codes[o] = make_uint2(w[0], w[1]);
  sf[o] = (uint8_t)sc;
}

// Decode-time cache write (paper section 6 "Online quantization": the new
// token is centred against the frozen per-request means and quantized with
// the cache's frozen scales; its compensation entries are written in the
// same pass).  Block = 128 threads for one (b, hk, token): thread d centres
// channel d into LDS and writes its FP8 V byte; threads 0-7 then quantize
// the row's eight NVFP4 blocks and threads 8 .. 8+G-1 its G Delta_S entries
// (FP64 over ascending channels).
//
// Where one appended token goes: its K code row (64 bytes), scale row (8
// bytes), the V byte of channel 0 (channel d at + 16 d), and the Delta_S
// entry of the group's first query head (head g at + g * dstride).
struct AppendDst {
  uint8_t* k;
  uint8_t* s;
  uint8_t* v;
  uint16_t* d;
  int64_t dstride;
};

__device__ __forceinline__ void append_token(const void* k_new, const void* v_new, int is_bf16,
                                             int64_t src_row, const float* k_mean_row,
                                             const float* q_mean_g0, int G, float gK, float vS,
                                             const AppendDst& o, float* kc) {
  const int d = threadIdx.x;
  const int64_t src = src_row * kD + d;
  float x = load_elem(k_new, src, is_bf16);
  if (k_mean_row) x = x - k_mean_row[d];
  kc[d] = x;
  o.v[d * 16] = (uint8_t)e4m3_encode(load_elem(v_new, src, is_bf16) / vS);
  __syncthreads();
  if (d < 8) {
    float xb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) xb[j] = kc[16 * d + j];
    uint32_t c[16];
    const uint32_t sc = nvfp4_block(xb, gK, c);
    uint2 packed;
    packed.x = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) |
               (c[6] << 24) | (c[7] << 28);
    packed.y = c[8] | (c[9] << 4) | (c[10] << 8) | (c[11] << 12) | (c[12] << 16) | (c[13] << 20) |
               (c[14] << 24) | (c[15] << 28);
    reinterpret_cast<uint2*>(o.k)[d] = packed;
    o.s[d] = (uint8_t)sc;
  } else if (k_mean_row && d < 8 + G) {
    const float* qm = q_mean_g0 + (int64_t)(d - 8) * kD;
    double acc = 0.0;
    for (int c = 0; c < kD; ++c) acc = __builtin_fma((double)qm[c], (double)kc[c], acc);
    o.d[(int64_t)(d - 8) * o.dstride] = (uint16_t)bf16_rne((float)acc);
  }
}

// Contiguous caches [B, Hkv, N_cap, ...]: T new tokens per (batch, KV head)
// at positions pos[b] .. pos[b] + T - 1; a batch entry whose position is
// outside [0, N_cap - T] is skipped whole.
__global__ __launch_bounds__(128) void k_append_kv(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int is_bf16, int Hkv, int G,
    int T, int N_cap, const int32_t* __restrict__ pos, const float* __restrict__ q_mean,
    const float* __restrict__ k_mean, const float* __restrict__ k_gscale,
    const float* __restrict__ v_scale, uint8_t* __restrict__ k_fp4, uint8_t* __restrict__ k_sf,
    uint8_t* __restrict__ v_fp8, uint16_t* __restrict__ delta) {
  __shared__ float kc[kD];
  const int t = blockIdx.x;
  const int bhk = blockIdx.y;  // b * Hkv + hk
  const int b = bhk / Hkv;
  const int p0 = pos[b];
  if (p0 < 0 || p0 > N_cap - T) return;  // uniform over the block
  const int p = p0 + t;
  const int ntiles = (N_cap + 31) / 32;
  const int64_t row = (int64_t)bhk * N_cap + p;
  AppendDst o;
  o.k = k_fp4 + row * 64;
  o.s = k_sf + row * 8;
  o.v = v_fp8 + ((int64_t)bhk * ntiles + p / 32) * kD * 32 + ((p & 31) >> 4) * kD * 16 + (p & 15);
  o.d = k_mean ? delta + (int64_t)bhk * G * N_cap + p : nullptr;  // head b*Hq + hk*G = bhk*G
  o.dstride = N_cap;
  append_token(k_new, v_new, is_bf16, (int64_t)bhk * T + t, k_mean ? k_mean + (int64_t)bhk * kD : nullptr,
               k_mean ? q_mean + (int64_t)bhk * G * kD : nullptr, G, *k_gscale, *v_scale, o, kc);
}

// Paged caches (128-token pages; pool [num_pages, Hkv, 128, ...], Delta_S
// [num_pages, Hq, 128]): one new token per request at position pos[b], i.e.
// slot pos[b] % 128 of page block_table[b * max_pages + pos[b] / 128], with
// the request's own frozen scales.  A request whose position is outside its
// table row or whose page index is outside the pool writes nothing.
__global__ __launch_bounds__(128) void k_append_kv_paged(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int is_bf16, int Hkv, int G,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ table, int max_pages,
    int num_pages, const float* __restrict__ q_mean, const float* __restrict__ k_mean,
    const float* __restrict__ k_gscale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ k_fp4, uint8_t* __restrict__ k_sf, uint8_t* __restrict__ v_fp8,
    uint16_t* __restrict__ delta) {
  __shared__ float kc[kD];
  const int bhk = blockIdx.x;  // b * Hkv + hk
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int p = pos[b];
  if (p < 0 || p >= max_pages * kBlk) return;  // uniform over the block
  const int pg = table[(int64_t)b * max_pages + p / kBlk];
  if (pg < 0 || pg >= num_pages) return;
  const int slot = p % kBlk;
  const int64_t slab = (int64_t)pg * Hkv + hk;
  AppendDst o;
  o.k = k_fp4 + (slab * kBlk + slot) * 64;
  o.s = k_sf + (slab * kBlk + slot) * 8;
  o.v = v_fp8 + (slab * 4 + slot / 32) * kD * 32 + ((slot & 31) >> 4) * kD * 16 + (slot & 15);
  o.d = k_mean ? delta + ((int64_t)pg * Hkv * G + (int64_t)hk * G) * kBlk + slot : nullptr;
  o.dstride = kBlk;
  append_token(k_new, v_new, is_bf16, bhk, k_mean ? k_mean + (int64_t)bhk * kD : nullptr,
               k_mean ? q_mean + (int64_t)bhk * G * kD : nullptr, G, k_gscale[b], v_scale[b], o,
               kc);
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

// Rows per block so that the whole pass has about kStatBlocks blocks.
static inline int stat_rows_per_block(int BH, int N, int align) {
  const int64_t xb = (kStatBlocks + BH - 1) / BH;
  int64_t rows = (N + xb - 1) / xb;
  rows = (rows + align - 1) / align * align;
  return (int)(rows < align ? align : rows);
}

void launch_channel_means(const ChannelMeanJob* jobs, int n_jobs, int N, hipStream_t st) {
  StatJobs J{};
  J.N = N;
  int64_t nblk = 0, bytes = 0;
  for (int t = 0; t < n_jobs; ++t)
    bytes += (int64_t)jobs[t].BH * N * kD * (jobs[t].is_bf16 ? 2 : 4);
  const bool stream = bytes > kLastLevelCacheBytes;
  for (int t = 0; t < 2; ++t) {
    const ChannelMeanJob& c = jobs[t < n_jobs ? t : 0];
    J.x[t] = c.x;
    J.is_bf16[t] = c.is_bf16;
    J.BH[t] = c.BH;
    J.rows[t] = stat_rows_per_block(c.BH, N, stream ? 64 : 128);
    J.gx[t] = (N + J.rows[t] - 1) / J.rows[t];
    J.range[t] = c.range;
    J.sums[t] = c.sums;
    J.mean[t] = c.mean;
    J.extent[t] = c.extent;
    if (t < n_jobs) nblk += (int64_t)J.gx[t] * c.BH;
  }
  J.nblk0 = J.gx[0] * J.BH[0];
  if (stream) {
    hipLaunchKernelGGL((k_channel_absmax<true, 4>), dim3((unsigned)nblk), dim3(256), 0, st, J);
    hipLaunchKernelGGL((k_channel_fixsum<true, 4>), dim3((unsigned)nblk), dim3(256), 0, st, J);
  } else {
    hipLaunchKernelGGL((k_channel_absmax<false, 8>), dim3((unsigned)nblk), dim3(256), 0, st, J);
    hipLaunchKernelGGL((k_channel_fixsum<false, 8>), dim3((unsigned)nblk), dim3(256), 0, st, J);
  }
  const int n0 = J.BH[0] * kD;
  const int n = n0 + (n_jobs > 1 ? J.BH[1] * kD : 0);
  hipLaunchKernelGGL(k_mean_finalize, dim3((n + 255) / 256), dim3(256), 0, st, J, n0, n);
}

void launch_centered_amax(const void* x, int is_bf16, int BH, int N, const float* mean,
                          uint32_t* out, hipStream_t st) {
  const int rows = stat_rows_per_block(BH, N, 128);
  dim3 grid((unsigned)((N + rows - 1) / rows), BH);
  hipLaunchKernelGGL(k_centered_amax, grid, dim3(256), 0, st, x, is_bf16, N, rows, mean, out,
                     (float*)nullptr);
  hipLaunchKernelGGL(k_amax_fold, dim3(1), dim3(kAmaxSlots), 0, st, out);
}

int launch_centered_amax_partials(const void* x, int is_bf16, int BH, int N, const float* mean,
                                  float* partials, hipStream_t st) {
  if (BH > kAmaxPartials) return -1;
  // at most kAmaxPartials / BH blocks per head, whole multiples of 128 rows
  const int per_bh = kAmaxPartials / BH;
  int rows = (N + per_bh - 1) / per_bh;
  rows = (rows + 127) / 128 * 128;
  dim3 grid((unsigned)((N + rows - 1) / rows), BH);
  hipLaunchKernelGGL(k_centered_amax, grid, dim3(256), 0, st, x, is_bf16, N, rows, mean,
                     (uint32_t*)nullptr, partials);
  return (int)(grid.x * grid.y);
}

void launch_partials_fold(const float* partials, int n, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_partials_fold, dim3(1), dim3(256), 0, st, partials, n, out);
}

void launch_rows_amax(const void* x, int is_bf16, int rows, const float* mean, float* slots,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_rows_amax, dim3(kRowsAmaxSlots), dim3(256), 0, st, x, is_bf16, rows, mean,
                     slots);
}

void launch_tile_mean(const void* x, int is_bf16, int BH, int N, float* mean, uint32_t* amax,
                      hipStream_t st) {
  dim3 grid((unsigned)((N + kBlk - 1) / kBlk), BH);
  hipLaunchKernelGGL(k_tile_mean, grid, dim3(256), 0, st, x, is_bf16, N, mean, amax);
  if (amax) hipLaunchKernelGGL(k_amax_fold, dim3(1), dim3(kAmaxSlots), 0, st, amax);
}

void launch_quantize_k_codes(const void* k, int is_bf16, int BH, int N, const float* k_mean,
                             const uint32_t* amax, float* gscale, uint8_t* codes, uint8_t* sf,
                             const uint32_t* q_ext, float* q_amax, hipStream_t st) {
  const int64_t n_groups = (int64_t)BH * N * (kD / 16);
  hipLaunchKernelGGL(k_quantize_k, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, st, k,
                     is_bf16, n_groups, N, k_mean, amax, gscale, codes, sf, q_ext, q_amax);
}

void launch_delta_s(const void* k, int is_bf16, int B, int Hkv, int G, int N, const float* k_mean,
                    const float* q_mean, uint16_t* delta, hipStream_t st, const uint32_t* amax,
                    float* gscale, uint8_t* codes, uint8_t* sf, const uint32_t* q_ext,
                    float* q_amax) {
  dim3 grid((N + kDsRows - 1) / kDsRows, B * Hkv, (G + 7) / 8);
  hipLaunchKernelGGL(k_delta_s, grid, dim3(kDsRows * min(G, 8)), 0, st, k, is_bf16, Hkv, G, N,
                     k_mean, q_mean, delta, amax, gscale, reinterpret_cast<uint2*>(codes), sf,
                     q_ext, q_amax);
}

void launch_quantize_v_codes(const void* v, int is_bf16, int BH, int N, const uint32_t* amax,
                             float* vscale, uint8_t* out, hipStream_t st) {
  const int n_tiles = (N + 31) / 32;
  hipLaunchKernelGGL(k_quantize_v, dim3(n_tiles, BH), dim3(128), 0, st, v, is_bf16, N, n_tiles,
                     amax, vscale, out);
}

void launch_quantize_v_nvfp4(const void* v, int is_bf16, int BH, int N, const uint32_t* amax,
                             float* gscale, uint8_t* codes, uint8_t* sf, hipStream_t st) {
  const int nb16 = (N + 15) / 16;
  hipLaunchKernelGGL(k_quantize_v_nvfp4, dim3(nb16, BH), dim3(128), 0, st, v, is_bf16, N, nb16, amax,
                     gscale, reinterpret_cast<uint2*>(codes), sf);
}

void launch_append_kv(const void* k_new, const void* v_new, int is_bf16, int B, int Hkv, int G,
                      int T, int N_cap, const int32_t* pos, const float* q_mean,
                      const float* k_mean, const float* k_gscale, const float* v_scale,
                      uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_append_kv, dim3(T, B * Hkv), dim3(kD), 0, st, k_new, v_new, is_bf16, Hkv, G,
                     T, N_cap, pos, q_mean, k_mean, k_gscale, v_scale, k_fp4, k_sf, v_fp8, delta);
}

void launch_append_kv_paged(const void* k_new, const void* v_new, int is_bf16, int B, int Hkv,
                            int G, const int32_t* pos, const int32_t* block_table, int max_pages,
                            int num_pages, const float* q_mean, const float* k_mean,
                            const float* k_gscale, const float* v_scale, uint8_t* k_fp4,
                            uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta, hipStream_t st) {
  hipLaunchKernelGGL(k_append_kv_paged, dim3(B * Hkv), dim3(kD), 0, st, k_new, v_new, is_bf16, Hkv,
                     G, pos, block_table, max_pages, num_pages, q_mean, k_mean, k_gscale, v_scale,
                     k_fp4, k_sf, v_fp8, delta);
}

}  // namespace mpfa
