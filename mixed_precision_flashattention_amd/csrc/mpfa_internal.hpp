// Internal declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include "mpfa_device.hpp"

namespace mpfa {

// Precision / placement variants of the prefill attention kernel
// (PrefillParams::variant): the library's kernel, element-wise compensation,
// polynomial exp2 for one exponential in four, bf16 P.V, NVFP4 P.V, the
// compensation as a separate rank-one bf16 MMA step.
constexpr int kVarNone = 0, kVarElementwise = 1, kVarPolyExp2 = 2, kVarPvBf16 = 3,
              kVarPvNvfp4 = 4, kVarRankOne = 5;
// The fixed NVFP4 global scale of P in the NVFP4 P.V variant: fp32(1/2688)
// maps the bound p <= 1 to the largest E2M1 x E4M3 product, 6 x 448.
constexpr float kNvfp4PScale = 1.0f / 2688.0f;

struct PrefillParams {
  const void* q;
  int q_bf16;
  int B, Hq, Hkv, N, G;
  const float* q_mean;  // smoothing only
  const float* k_mean;  // smoothing and per-tile mean mode (LSE offset)
  const float* q_tile_mean;  // per-tile mean mode: [B, Hq, ceil(N/128), 128]; else NULL
  const uint8_t* k_f16;  // K~ block images from the pre-pass (BF16 in the per-tile mode)
  const float* k_gscale;
  const uint8_t* v_fp8;
  const float* v_scale;
  const uint16_t* delta_s;  // NULL: direct mode
  float scale;
  int causal;
  void* out;
  int out_bf16;
  float* lse;
  const uint32_t* q_amax;  // amax of Q_c, computed by the pre-pass
  int n_units;             // 256-row query units per (batch, head)
  // precision / placement variant of the attention kernel (0: the library's
  // kernel; 1: element-wise compensation; 2: polynomial exp2 for one
  // exponential in four; 3: bf16 P.V over v_bf16; 4: NVFP4 P.V over v_bf16
  // holding the FP16 image of the NVFP4 V cache, v_scale its global scale)
  int variant;
  const uint16_t* v_bf16;  // variants 3 and 4: tiled 16-bit V, else NULL
};

struct DecodeParams {
  const void* q;
  int q_bf16;
  int B, Hq, Hkv, N, G, P, chunk;
  const float* q_mean;
  const float* k_mean;
  const uint8_t* k_fp4;
  const uint8_t* k_sf;
  const float* k_gscale;
  const uint8_t* v_fp8;
  const float* v_scale;
  const uint16_t* delta_s;
  float scale;
  const float* q_amax_slots;  // partial maxima of |Q_c| (launch_rows_amax)
  float* ws_m;    // [B*Hq, P]
  float* ws_l;    // [B*Hq, P]
  float* ws_acc;  // [B*Hq, P, 128]
  void* out;
  int out_bf16;
  float* lse;
  // paged cache (k_gscale and v_scale are then per request, [B]): logical
  // 128-token page i of request b is physical page block_table[b * max_pages + i]
  int paged;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_pages, num_pages;
  int* order;  // paged: requests by descending length (written by the launch)
};

// quant.hip
// A tensor amax is reduced into kAmaxSlots words, one per 128-byte line
// (atomics on one address serialize across the GPU), then folded into the
// first word, which is what every consumer reads.
constexpr int kAmaxSlots = 64;
constexpr int kAmaxSlotWords = 32;
constexpr size_t kAmaxBytes = (size_t)kAmaxSlots * kAmaxSlotWords * 4;
void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);
// Sequence channel means of one or two [BH, N, 128] tensors (K and Q) in
// three launches: channel ranges, fixed-point sums (both into cleared
// buffers), finalize into mean, and, with extent non-NULL (a cleared word),
// the centred amax max |fp32(x - mean)| derived from the ranges.
struct ChannelMeanJob {
  const void* x;
  int is_bf16, BH;
  uint32_t* range;  // 2 * BH * 128 words
  unsigned long long* sums;
  float* mean;
  uint32_t* extent;
};
void launch_channel_means(const ChannelMeanJob* jobs, int n_jobs, int N, hipStream_t st);
void launch_centered_amax(const void* x, int is_bf16, int BH, int N, const float* mean,
                          uint32_t* out, hipStream_t st);
// The same amax as per-workgroup maxima in partials[0 .. n) (no clearing, no
// fold launch; the consumer folds them): returns n <= kAmaxPartials, or -1
// (nothing launched) when the tensor has more than kAmaxPartials heads.
constexpr int kAmaxPartials = (int)(kAmaxBytes / 4);
int launch_centered_amax_partials(const void* x, int is_bf16, int BH, int N, const float* mean,
                                  float* partials, hipStream_t st);
// Fold n such maxima into out[0] (one workgroup; out may alias partials).
void launch_partials_fold(const float* partials, int n, uint32_t* out, hipStream_t st);
// Partial maxima of |x - mean| over the rows of a [rows, 128] tensor, one
// per slot (kRowsAmaxSlots floats, all written): the decode query amax.
constexpr int kRowsAmaxSlots = 64;
void launch_rows_amax(const void* x, int is_bf16, int rows, const float* mean, float* slots,
                      hipStream_t st);
// Per-tile channel means; with amax non-NULL (cleared beforehand) also the
// amax of the tile-centred tensor into amax[0], as launch_centered_amax does.
void launch_tile_mean(const void* x, int is_bf16, int BH, int N, float* mean, uint32_t* amax,
                      hipStream_t st);
// q_amax non-NULL: also copies the word q_ext (a Q_c amax) into *q_amax
void launch_quantize_k_codes(const void* k, int is_bf16, int BH, int N, const float* k_mean,
                             const uint32_t* amax, float* gscale, uint8_t* codes, uint8_t* sf,
                             const uint32_t* q_ext, float* q_amax, hipStream_t st);
// codes non-NULL: the same launch also writes the NVFP4 K codes and scales
// (and gscale, and q_amax from q_ext when q_amax is non-NULL), as
// launch_quantize_k_codes would with k_mean
void launch_delta_s(const void* k, int is_bf16, int B, int Hkv, int G, int N, const float* k_mean,
                    const float* q_mean, uint16_t* delta, hipStream_t st,
                    const uint32_t* amax = nullptr, float* gscale = nullptr,
                    uint8_t* codes = nullptr, uint8_t* sf = nullptr,
                    const uint32_t* q_ext = nullptr, float* q_amax = nullptr);
// NVFP4 V along the keys: codes [BH, ceil(N/16), 128, 8 bytes] (key 2t of a
// block in the low nibble of byte t), scales [BH, ceil(N/16), 128], global
// scale from *amax written to gscale.
void launch_quantize_v_nvfp4(const void* v, int is_bf16, int BH, int N, const uint32_t* amax,
                             float* gscale, uint8_t* codes, uint8_t* sf, hipStream_t st);
void launch_quantize_v_codes(const void* v, int is_bf16, int BH, int N, const uint32_t* amax,
                             float* vscale, uint8_t* out, hipStream_t st);

void launch_append_kv(const void* k_new, const void* v_new, int is_bf16, int B, int Hkv, int G,
                      int T, int N_cap, const int32_t* pos, const float* q_mean,
                      const float* k_mean, const float* k_gscale, const float* v_scale,
                      uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta,
                      hipStream_t st);
void launch_append_kv_paged(const void* k_new, const void* v_new, int is_bf16, int B, int Hkv,
                            int G, const int32_t* pos, const int32_t* block_table, int max_pages,
                            int num_pages, const float* q_mean, const float* k_mean,
                            const float* k_gscale, const float* v_scale, uint8_t* k_fp4,
                            uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta, hipStream_t st);

// prefill.hip
// partials non-NULL: also fold n_partials maxima of launch_centered_amax_partials
// into amax_out[0] (amax_out may alias partials).
void launch_expand_k(const uint8_t* k_fp4, const uint8_t* k_sf, int64_t bhk, int N,
                     uint8_t* k_img, hipStream_t st, bool bf16 = false,
                     const float* partials = nullptr, int n_partials = 0,
                     uint32_t* amax_out = nullptr);
void launch_prefill(const PrefillParams& p, hipStream_t st);
// bf16 V cache of the bf16 P.V variant: [BH, ceil(N/32), 4, 128, 8] bf16
// (token t, channel d at [t/32][(t%32)/8][d][t%8]), zero past N.
void launch_pack_v_bf16(const void* v, int is_bf16, int BH, int N, uint16_t* out, hipStream_t st);
// FP16 image of an NVFP4 V cache (launch_quantize_v_nvfp4) in the layout of
// the bf16 V cache: code value x block scale, exact in FP16 (the global scale
// stays out); zero past N.
void launch_expand_v_nvfp4(const uint8_t* codes, const uint8_t* sf, int BH, int N, uint16_t* out,
                           hipStream_t st);

// decode.hip
void launch_decode(const DecodeParams& p, hipStream_t st);

}  // namespace mpfa
