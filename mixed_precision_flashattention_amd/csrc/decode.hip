// Split-KV QK4PV8 decode for gfx950 (paper "MpFA: ...", section 5.3
// "Decode-Specific Optimizations").
//
// One wave per (batch, KV head, partition).  The G <= 8 query heads of the
// GQA group are packed into the M dimension of the score MFMA (S = Q~ K~^T,
// 32 x 32 x 16 f16; only rows 0..G-1 are real), so each lane holds one key
// and the real rows sit in 4 accumulator registers of each lane half:
// softmax work is spent on those registers only, never on the padded rows.
// K codes go from HBM straight into registers and are expanded to exact
// FP16 operands there; the rank-one compensation is one bf16 MFMA step with
// the group's Delta_S rows as the B operand.  P is rounded to E4M3, turned
// by LDS into the head-major B operand of a 16 x 16 x 128 FP8 MFMA whose A
// operand (V^T) is read directly from the head-dim-major V tiles.  Each
// partition leaves (m, l, acc) in the workspace; a second kernel merges the
// partitions by log-sum-exp.
//
// The same kernels serve a paged cache (paper section 6 "Serving system"):
// 128-token pages (one softmax block each), a block table per request, the
// Delta_S side cache indexed by the same physical pages, per-request lengths
// and frozen scales; the number of partitions stays fixed and each request
// is cut into them by its own length.
#include "mpfa_internal.hpp"

namespace mpfa {

constexpr int kQStride = 272;  // LDS row of Q~ (f16)
constexpr int kPStride = 144;  // LDS row of P^ (128 keys + 16 bytes)
constexpr int kVTileBytes = kD * 32;

// amax of the decode queries from launch_rows_amax's partial maxima: one
// slot per lane, folded across the wave (every lane of the wave must call).
__device__ __forceinline__ float query_amax(const float* slots) {
  static_assert(kRowsAmaxSlots == 64, "one slot per lane");
  float a = slots[threadIdx.x & 63];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  return a;
}

// Everything one 128-key block needs from HBM, per lane: the K codes of its
// key in each of the 4 score tiles (32 bytes = its head-dim half), their 4
// E4M3 scales, 8 x 32 bytes of V^T operands, and a share of the group's
// Delta_S rows: keys 8 (lane % 16) .. + 7 of rows lane / 16 and 4 + lane / 16
// (whole 16-byte pieces of the rows; LDS hands each lane the entries of its
// own keys).  Two of these are live: block j+1 is loaded while block j is
// computed.
struct DecodeBlockRegs {
  uint4 k[4][2];
  uint32_t sc[4];
  uint4 dl[2];
  i32x8 v[8];
};

// Where the 128-key block starting at key k0 lives: its first K code row,
// scale row, V tile and Delta_S entry (row g of the group at d + g * dstride),
// and the last key / tile index inside the block that holds data.
struct DecodeBlockPtrs {
  const uint8_t* k;
  const uint8_t* s;
  const uint8_t* v;
  const uint16_t* d;
  int64_t dstride;
  int klast, vlast;
};

struct DecodeCtx {
  const uint8_t* kbase;
  const uint8_t* sbase;
  const uint8_t* vbase;
  const uint16_t* dbase;  // Delta_S row of the group's first query head
  int N, G, ntiles32;
  bool dvec;  // Delta_S rows start 16-byte aligned (contiguous cache: N % 8 == 0)
  // paged cache: this request's block-table row, the pool size and strides
  const int32_t* table;
  int num_pages, Hkv, hk, Hq;
  int64_t hq0;
};

template <bool PAGED>
__device__ __forceinline__ DecodeBlockPtrs block_ptrs(const DecodeCtx& c, int k0) {
  DecodeBlockPtrs b;
  if (PAGED) {
    // a page index outside the pool is clamped into it (the result for such
    // a request is unspecified, but every access stays inside the pool)
    const int pg = min(max(c.table[k0 / kBlk], 0), c.num_pages - 1);
    const int64_t slab = (int64_t)pg * c.Hkv + c.hk;
    b.k = c.kbase + slab * kBlk * 64;
    b.s = c.sbase + slab * kBlk * 8;
    b.v = c.vbase + slab * 4 * kVTileBytes;
    b.d = c.dbase ? c.dbase + ((int64_t)pg * c.Hq + c.hq0) * kBlk : nullptr;
    b.dstride = kBlk;
    b.klast = kBlk - 1;
    b.vlast = 3;
  } else {
    b.k = c.kbase + (int64_t)k0 * 64;
    b.s = c.sbase + (int64_t)k0 * 8;
    b.v = c.vbase + (int64_t)(k0 / 32) * kVTileBytes;
    b.d = c.dbase ? c.dbase + k0 : nullptr;
    b.dstride = c.N;
    b.klast = c.N - 1 - k0;  // keys past the end are clamped to the last one (masked later)
    b.vlast = c.ntiles32 - 1 - k0 / 32;
  }
  return b;
}

// Streaming loads: every KV byte is read once per call, so the loads carry
// the non-temporal hint and do not displace reusable lines from the caches
// (a plain streaming-read probe on MI355X moves ~6.5 TB/s with the hint
// against ~5.9 TB/s without it).
template <typename T>
__device__ __forceinline__ T ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

template <bool SMOOTH, bool PAGED>
__device__ __forceinline__ void decode_load(DecodeBlockRegs& r, const DecodeCtx& c, int k0,
                                            int lane) {
  const int h = lane >> 5, col = lane & 31;
  const DecodeBlockPtrs bp = block_ptrs<PAGED>(c, k0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int key = min(32 * t + col, bp.klast);
    const uint8_t* src = bp.k + (int64_t)key * 64 + 32 * h;
    const i32x4 k0v = ld_stream<i32x4>(src), k1v = ld_stream<i32x4>(src + 16);
    r.k[t][0] = make_uint4(k0v[0], k0v[1], k0v[2], k0v[3]);
    r.k[t][1] = make_uint4(k1v[0], k1v[1], k1v[2], k1v[3]);
    r.sc[t] = ld_stream<uint32_t>(bp.s + (int64_t)key * 8 + 4 * h);
  }
  if (SMOOTH) {
    // A whole 16-byte piece when the block is full and the rows are aligned
    // (always in a page); otherwise entry by entry, keys clamped to the end.
    const bool vec = PAGED || (c.dvec && bp.klast >= kBlk - 1);
    const int j8 = 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 4 * i + (lane >> 4);
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if ((i == 0 || c.G > 4) && g < c.G) {
        const uint16_t* row = bp.d + (int64_t)g * bp.dstride;
        if (vec) {
          const i32x4 x = ld_stream<i32x4>(row + j8);
          w = make_uint4(x[0], x[1], x[2], x[3]);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) e[u] = ld_stream<uint16_t>(row + min(j8 + u, bp.klast));
          w = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                         e[6] | (e[7] << 16));
        }
      }
      r.dl[i] = w;
    }
  }
  // V^T operand of lane (n, kg): channel 16 dt + n, the 32 tokens of tile
  // kg, as its two 16-token pieces (each load instruction reads 256
  // contiguous bytes per tile)
  const int n = lane & 15, kg = lane >> 4;
  const uint8_t* vt = bp.v + (int64_t)min(kg, bp.vlast) * kVTileBytes;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const i32x4 lo = ld_stream<i32x4>(vt + (16 * dt + n) * 16);
    const i32x4 hi = ld_stream<i32x4>(vt + kD * 16 + (16 * dt + n) * 16);
    r.v[dt] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

struct DecodeState {
  float m[4], l[4];
  f32x4 o[8];
};

template <bool SMOOTH>
__device__ __forceinline__ void decode_compute(const DecodeBlockRegs& r, DecodeState& st, int k0,
                                               int p1, int lane, float lam, const i32x4* qa,
                                               const i32x4& dA, uint8_t* sp, float* salpha,
                                               uint16_t* sdl, int G) {
  const int h = lane >> 5, col = lane & 31;
  if (SMOOTH) {
    // the group's Delta_S rows of this block into LDS, [row][key] (rows past
    // the group hold zeros from the kernel's start)
    *reinterpret_cast<uint4*>(sdl + (lane >> 4) * kBlk + 8 * (lane & 15)) = r.dl[0];
    if (G > 4) *reinterpret_cast<uint4*>(sdl + (4 + (lane >> 4)) * kBlk + 8 * (lane & 15)) = r.dl[1];
    __syncthreads();
  }
  // ---- scores S = Q~ K~^T: 4 tiles of 32 keys, lane col = key ------------
  f32x16 s[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t w[8] = {r.k[t][0].x, r.k[t][0].y, r.k[t][0].z, r.k[t][0].w,
                           r.k[t][1].x, r.k[t][1].y, r.k[t][1].z, r.k[t][1].w};
    uint32_t e[4];
    expand_fp4x8(w[0], e4m3_scale_f16x2(r.sc[t] & 0xFFu), e);
    const i32x4 kb0 = {(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
    if (SMOOTH) {
      // Delta_S[g][key] in slot g: the B operand of the rank-one step
      uint32_t dg[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) dg[g] = sdl[g * kBlk + 32 * t + col];
      const i32x4 dB = {(int)(dg[0] | (dg[1] << 16)), (int)(dg[2] | (dg[3] << 16)),
                        (int)(dg[4] | (dg[5] << 16)), (int)(dg[6] | (dg[7] << 16))};
      s[t] = mfma32_bf16(dA, dB, f32x16{});
      s[t] = mfma32_f16(qa[0], kb0, s[t]);
    } else {
      s[t] = mfma32_f16(qa[0], kb0, f32x16{});
    }
#pragma unroll
    for (int kc = 1; kc < 8; ++kc) {
      expand_fp4x8(w[kc], e4m3_scale_f16x2((r.sc[t] >> (8 * (kc >> 1))) & 0xFFu), e);
      s[t] = mfma32_f16(qa[kc], i32x4{(int)e[0], (int)e[1], (int)e[2], (int)e[3]}, s[t]);
    }
  }

  // ---- softmax on rows 4h + v (v < 4), keys across the 32 lanes ----------
  float alpha[4], nb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t][v] = (k0 + 32 * t + col < p1) ? s[t][v] : -INFINITY;
      mx = fmaxf(mx, s[t][v]);
    }
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
    const float m_new = fmaxf(st.m[v], mx);
    alpha[v] = fast_exp2(lam * (st.m[v] - m_new));
    nb[v] = kLog2_448 - lam * m_new;
    st.m[v] = m_new;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float lsum = 0.0f;
    uint8_t* prow = sp + (4 * h + v) * kPStride + col;
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      const float e0 = fast_exp2(fmaf(s[t][v], lam, nb[v]));
      const float e1 = fast_exp2(fmaf(s[t + 1][v], lam, nb[v]));
      lsum += e0 + e1;
      const uint32_t wd = cvt_fp8x2<false>(e0, e1, 0u);
      prow[32 * t] = (uint8_t)(wd & 0xFFu);
      prow[32 * (t + 1)] = (uint8_t)((wd >> 8) & 0xFFu);
    }
    st.l[v] = fmaf(alpha[v], st.l[v], lsum);
  }
  if (col == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) salpha[4 * h + v] = alpha[v];
  }
  __syncthreads();

  // ---- O^T += V^T P^T on FP8 16x16x128 -----------------------------------
  const int n = lane & 15, kg = lane >> 4;  // query column, 32-key group
  const i32x8 pbv = n < 8 ? *reinterpret_cast<const i32x8*>(sp + n * kPStride + 32 * kg)
                          : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  const float a_o = n < 8 ? salpha[n] : 1.0f;
  if (k0 + kBlk > p1) {
    // The last block of the range: V bytes of keys past its end may be bytes
    // nobody wrote (a NaN code times P = 0 would still be NaN), so they are
    // cleared.  Lane group kg holds keys k0 + 32 kg .. + 31, 4 per dword.
    const int nv = min(max(p1 - (k0 + 32 * kg), 0), 32);
    i32x8 vm;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int keep = min(max(nv - 4 * w, 0), 4);
      vm[w] = keep == 4 ? -1 : (int)((1u << (8 * keep)) - 1u);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma16_fp8(r.v[dt] & vm, pbv, st.o[dt] * a_o);
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma16_fp8(r.v[dt], pbv, st.o[dt] * a_o);
  }
  __syncthreads();
}

template <bool SMOOTH, bool PAGED>
__global__ __launch_bounds__(64) void k_decode_split(DecodeParams p) {
  __shared__ __align__(16) uint8_t sq[8 * kQStride];
  __shared__ __align__(16) uint8_t sp[8 * kPStride];
  __shared__ float salpha[8];
  __shared__ __align__(16) uint16_t sdl[8 * kBlk];  // Delta_S rows of the block (smoothing)

  const int N = p.N, G = p.G, P = p.P;
  const int part = blockIdx.x % P;
  const int bhk = blockIdx.x / P;
  // paged: workgroups are dealt longest request first (ragged lengths would
  // otherwise leave the longest partitions for the end of the grid)
  const int b = PAGED ? p.order[bhk / p.Hkv] : bhk / p.Hkv, hk = bhk % p.Hkv;
  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int64_t hq0 = (int64_t)b * p.Hq + (int64_t)hk * G;  // first query head of the group
  // paged: this request's length, clamped to its block-table row, cut into
  // P partitions of whole 128-key blocks
  const int Nb = PAGED ? min(max(p.seq_lens[b], 0), p.max_pages * kBlk) : N;
  const int chunk = PAGED ? (Nb + kBlk * P - 1) / (kBlk * P) * kBlk : p.chunk;
  const int p0 = part * chunk;
  const int p1 = min(p0 + chunk, Nb);

  if (p0 >= p1) {  // empty partition: neutral state
    if (lane < G) {
      p.ws_m[(hq0 + lane) * P + part] = -INFINITY;
      p.ws_l[(hq0 + lane) * P + part] = 0.0f;
    }
    for (int i = lane; i < G * kD; i += 64)
      p.ws_acc[((hq0 + i / kD) * P + part) * kD + (i % kD)] = 0.0f;
    return;
  }

  const float gQ = nvfp4_global_scale(query_amax(p.q_amax_slots));
  const float gK = PAGED ? p.k_gscale[b] : *p.k_gscale;
  const float gg = gQ * gK;
  const float lam = p.scale * kLog2e * gg;

  {  // NVFP4 of the group's query rows: lane -> (row g = lane / 8, block lane % 8)
    const int g = lane >> 3, blk = lane & 7;
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (g < G) {
      float x[16];
      load16(p.q, (hq0 + g) * kD + blk * 16, p.q_bf16, x);
      if (SMOOTH) {
        const float* mu = p.q_mean + (hq0 + g) * kD + blk * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = x[j] - mu[j];
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
    uint4* dst = reinterpret_cast<uint4*>(sq + g * kQStride + blk * 32);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
  __syncthreads();

  // A operand (Q~): row col (real for col < G), head-dim slots 64h + 8kc .. +7.
  i32x4 qa[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qa[kc] = col < 8 ? *reinterpret_cast<const i32x4*>(sq + col * kQStride + (64 * h + 8 * kc) * 2)
                     : i32x4{0, 0, 0, 0};
  // A operand of the rank-one step: row g < G has 1/(gQ gK) (hi part in lane
  // half 0, lo part in half 1) in slot g; the B operand holds Delta_S[g, key]
  // in slot g of both halves, so the step adds Delta_S / (gQ gK) to row g.
  i32x4 dA = {0, 0, 0, 0};
  if (SMOOTH && col < G) {
    const float cinv = 1.0f / gg;
    const uint32_t c_hi = bf16_rne(cinv);
    const uint32_t c_lo = bf16_rne(cinv - __uint_as_float(c_hi << 16));
    const int cv = (int)((h == 0 ? c_hi : c_lo) << (16 * (col & 1)));
#pragma unroll
    for (int i = 0; i < 4; ++i) dA[i] = ((col >> 1) == i) ? cv : 0;
  }

  DecodeCtx c;
  c.N = N;
  c.G = G;
  c.ntiles32 = (N + 31) / 32;
  c.dvec = (N & 7) == 0;
  if (SMOOTH) {  // rows past the group stay zero for the whole loop
    for (int i = lane; i < 8 * kBlk; i += 64) sdl[i] = 0;
    __syncthreads();
  }
  if (PAGED) {
    c.kbase = p.k_fp4;
    c.sbase = p.k_sf;
    c.vbase = p.v_fp8;
    c.dbase = SMOOTH ? p.delta_s : nullptr;
    c.table = p.block_table + (int64_t)b * p.max_pages;
    c.num_pages = p.num_pages;
    c.Hkv = p.Hkv;
    c.hk = hk;
    c.Hq = p.Hq;
    c.hq0 = (int64_t)hk * G;  // the group's first query head within the page's Hq rows
  } else {
    const int64_t kvh = (int64_t)b * p.Hkv + hk;
    c.kbase = p.k_fp4 + kvh * N * 64;
    c.sbase = p.k_sf + kvh * N * 8;
    c.vbase = p.v_fp8 + kvh * c.ntiles32 * kVTileBytes;
    c.dbase = SMOOTH ? p.delta_s + hq0 * N : nullptr;
  }

  DecodeState st;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    st.m[v] = -INFINITY;
    st.l[v] = 0.0f;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{};

  // Two register stages: the loads of the next block are in flight while
  // the current one is computed.
  DecodeBlockRegs ra, rb;
  decode_load<SMOOTH, PAGED>(ra, c, p0, lane);
  for (int k0 = p0; k0 < p1; k0 += 2 * kBlk) {
    if (k0 + kBlk < p1) decode_load<SMOOTH, PAGED>(rb, c, k0 + kBlk, lane);
    decode_compute<SMOOTH>(ra, st, k0, p1, lane, lam, qa, dA, sp, salpha, sdl, G);
    if (k0 + kBlk >= p1) break;
    if (k0 + 2 * kBlk < p1) decode_load<SMOOTH, PAGED>(ra, c, k0 + 2 * kBlk, lane);
    decode_compute<SMOOTH>(rb, st, k0 + kBlk, p1, lane, lam, qa, dA, sp, salpha, sdl, G);
  }

  // ---- partition state -------------------------------------------------
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float l = st.l[v];
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) l += __shfl_xor(l, o2);
    const int g = 4 * h + v;
    if (col == 0 && g < G) {
      p.ws_m[(hq0 + g) * P + part] = st.m[v];
      p.ws_l[(hq0 + g) * P + part] = l;
    }
  }
  const int n = lane & 15, kg = lane >> 4;
  if (n < G) {
    float* dst = p.ws_acc + ((hq0 + n) * P + part) * kD + 4 * kg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt) =
          make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
  }
}

// Log-sum-exp merge of the partitions (paper section 5.3): one block of 256
// threads per (batch, query head).  Thread t takes channels 2 (t % 64) and
// 2 (t % 64) + 1 of partitions t / 64, t / 64 + 4, ...; its loads are issued
// together (a loop of dependent loads over the partitions would wait on
// each), and the four partial sums meet in LDS in a fixed order.
constexpr int kCombineThreads = 256, kCombineGroups = kCombineThreads / 64;
__global__ __launch_bounds__(kCombineThreads) void k_decode_combine(DecodeParams p) {
  __shared__ float2 sacc[kCombineGroups][64];
  __shared__ float sl[kCombineGroups];
  __shared__ float red[kD];
  const int bhq = blockIdx.x;
  const int t = threadIdx.x, c2 = t & 63, pg = t >> 6;
  const int P = p.P;
  const int b = bhq / p.Hq;
  const float gQ = nvfp4_global_scale(query_amax(p.q_amax_slots));
  const float gK = p.paged ? p.k_gscale[b] : *p.k_gscale;
  const float lam = p.scale * kLog2e * gQ * gK;
  const float* wm = p.ws_m + (int64_t)bhq * P;
  const float* wl = p.ws_l + (int64_t)bhq * P;
  const float* wa = p.ws_acc + (int64_t)bhq * P * kD + 2 * c2;
  float m = -INFINITY;
  for (int i = 0; i < P; ++i) m = fmaxf(m, wm[i]);
  float l = 0.0f, a0 = 0.0f, a1 = 0.0f;
  constexpr int kU = 8;  // partitions per batch of loads
  for (int i0 = pg; i0 < P; i0 += kU * kCombineGroups) {
    float mi[kU], li[kU];
    float2 ai[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u * kCombineGroups, P - 1);
      mi[u] = wm[i];
      li[u] = wl[i];
      ai[u] = *reinterpret_cast<const float2*>(wa + (int64_t)i * kD);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // an empty partition (m = -inf, l = 0, acc = 0) and a clamped repeat
      // past P weigh nothing
      const bool use = i0 + u * kCombineGroups < P && mi[u] != -INFINITY;
      const float w = use ? fast_exp2(lam * (mi[u] - m)) : 0.0f;
      l = fmaf(w, li[u], l);
      a0 = fmaf(w, ai[u].x, a0);
      a1 = fmaf(w, ai[u].y, a1);
    }
  }
  sacc[pg][c2] = make_float2(a0, a1);
  if (c2 == 0) sl[pg] = l;
  __syncthreads();
  const int d = t & (kD - 1);  // threads 0..127 write channel d
  float sum = 0.0f, lsum = 0.0f;
#pragma unroll
  for (int g = 0; g < kCombineGroups; ++g) {
    const float2 a = sacc[g][d >> 1];
    sum += (d & 1) ? a.y : a.x;
    lsum += sl[g];
  }
  // a request with no keys (paged, length 0) has l = 0: O = 0, LSE = -inf
  const float vs = p.paged ? p.v_scale[b] : *p.v_scale;
  const float o = lsum > 0.0f ? sum * (vs / lsum) : 0.0f;
  if (t < kD) {
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[(int64_t)bhq * kD + d] = (uint16_t)bf16_rne(o);
    else
      reinterpret_cast<float*>(p.out)[(int64_t)bhq * kD + d] = o;
  }
  if (p.lse) {
    float off = 0.0f;
    if (p.delta_s) {
      const int hk = (bhq % p.Hq) / p.G;
      if (t < kD)
        red[t] = load_elem(p.q, (int64_t)bhq * kD + t, p.q_bf16) *
                 p.k_mean[((int64_t)b * p.Hkv + hk) * kD + t];
      __syncthreads();
      for (int s2 = kD / 2; s2 > 0; s2 >>= 1) {
        if (t < s2) red[t] += red[t + s2];
        __syncthreads();
      }
      off = p.scale * red[0];
    }
    if (t == 0)
      p.lse[bhq] = lsum > 0.0f ? kLn2 * (lam * m + log2f(lsum)) - kLn2 * kLog2_448 + off : -INFINITY;
  }
}

// Requests ranked by descending clamped length (ties by index): order[rank]
// = request, one thread per request counting the longer ones (B^2 work, so
// batches above kOrderMaxB keep their own order).
constexpr int kOrderMaxB = 4096;
__global__ __launch_bounds__(256) void k_decode_order(const int32_t* __restrict__ seq_lens, int B,
                                                      int cap, int* __restrict__ order) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  if (B > kOrderMaxB) {
    order[b] = b;
    return;
  }
  const int lb = min(max(seq_lens[b], 0), cap);
  int rank = 0;
  for (int i = 0; i < B; ++i) {
    const int li = min(max(seq_lens[i], 0), cap);
    rank += (li > lb) || (li == lb && i < b);
  }
  order[rank] = b;
}

void launch_decode(const DecodeParams& p, hipStream_t st) {
  if (p.paged)
    hipLaunchKernelGGL(k_decode_order, dim3((p.B + 255) / 256), dim3(256), 0, st, p.seq_lens, p.B,
                       p.max_pages * kBlk, p.order);
  const unsigned grid = (unsigned)((int64_t)p.B * p.Hkv * p.P);
  if (p.paged) {
    if (p.delta_s)
      hipLaunchKernelGGL((k_decode_split<true, true>), dim3(grid), dim3(64), 0, st, p);
    else
      hipLaunchKernelGGL((k_decode_split<false, true>), dim3(grid), dim3(64), 0, st, p);
  } else if (p.delta_s) {
    hipLaunchKernelGGL((k_decode_split<true, false>), dim3(grid), dim3(64), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_decode_split<false, false>), dim3(grid), dim3(64), 0, st, p);
  }
  hipLaunchKernelGGL(k_decode_combine, dim3((unsigned)(p.B * p.Hq)), dim3(kCombineThreads), 0, st,
                     p);
}

}  // namespace mpfa
