// C ABI of the library: argument validation, workspace layout and the
// launch order of each entry point.  Everything runs on the caller's stream;
// nothing is allocated, freed or synchronised here.
#include <atomic>
#include <mutex>

#include "../../include/mpfa.h"
#include "mpfa_internal.hpp"

using namespace mpfa;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool dtype_ok(int t) { return t == MPFA_F32 || t == MPFA_BF16; }

// Workspace layouts (byte offsets from ws).
struct QuantKWs {
  size_t kmax, qmax, ksum, qsum, amax, total;
};
inline QuantKWs quant_k_layout(int B, int Hq, int Hkv) {
  QuantKWs w;
  const size_t nk = (size_t)B * Hkv * kD, nq = (size_t)B * Hq * kD;
  w.kmax = 0;  // channel ranges: two words per channel
  w.qmax = align_up(w.kmax + nk * 8);
  w.ksum = align_up(w.qmax + nq * 8);
  w.qsum = align_up(w.ksum + nk * 8);
  w.amax = align_up(w.qsum + nq * 8);
  w.total = align_up(w.amax + kAmaxBytes);
  return w;
}

struct DecodeWs {
  size_t amax, m, l, acc, order, total;
};
inline DecodeWs decode_layout(int B, int Hq, int P) {
  DecodeWs w;
  const size_t ns = (size_t)B * Hq * P;
  w.amax = 0;
  w.m = align_up(kAmaxBytes);
  w.l = align_up(w.m + ns * 4);
  w.acc = align_up(w.l + ns * 4);
  w.order = align_up(w.acc + ns * kD * 4);  // paged decode: request order
  w.total = align_up(w.order + (size_t)B * 4);
  return w;
}

// Prefill: the Q amax slots, then K~ (the K cache expanded to FP16 block
// images).
struct PrefillWs {
  size_t amax, k_f16, v_img, total;
};
// v_image: also the FP16 image of an NVFP4 V cache (NVFP4 P.V variant)
inline PrefillWs prefill_layout(int B, int Hkv, int N, bool v_image = false) {
  PrefillWs w;
  w.amax = 0;
  w.k_f16 = kAmaxBytes;
  // K~ block images: 32 KB per (batch, KV head, 128-key block)
  w.total = align_up(w.k_f16 + (size_t)B * Hkv * ((N + kBlk - 1) / kBlk) * kBlk * kD * 2);
  w.v_img = w.total;
  // V image: 8 KB per (batch, KV head, 32-key tile)
  if (v_image) w.total = align_up(w.v_img + (size_t)B * Hkv * ((N + 31) / 32) * 32 * kD * 2);
  return w;
}

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MPFA_OK : MPFA_ERR_LAUNCH;
}

// Sizes shared by every entry point.
inline int check_sizes(int B, int Hkv, int N, int D) {
  if (D != kD) return MPFA_ERR_UNSUPPORTED;
  if (B < 1 || Hkv < 1 || N < 1) return MPFA_ERR_INVALID;
  if ((int64_t)B * Hkv > 65535) return MPFA_ERR_INVALID;
  if ((int64_t)N * kD > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;
  return MPFA_OK;
}

inline int check_heads(int Hq, int Hkv, int B) {
  if (Hq < 1 || Hq % Hkv != 0) return MPFA_ERR_INVALID;
  if ((int64_t)B * Hq > 65535) return MPFA_ERR_INVALID;
  return MPFA_OK;
}

}  // namespace

extern "C" {

size_t mpfa_workspace_bytes(int op, int B, int Hq, int Hkv, int N, int D, int num_splits) {
  if (B < 1 || Hkv < 1 || N < 1 || D < 1) return 0;
  switch (op) {
    case MPFA_OP_QUANTIZE_K:
      return quant_k_layout(B, Hq > 0 ? Hq : 0, Hkv).total;
    case MPFA_OP_QUANTIZE_V:
      return kAmaxBytes;
    case MPFA_OP_PREFILL:
      return prefill_layout(B, Hkv, N).total;
    case MPFA_OP_PREFILL_PV_NVFP4:
      return prefill_layout(B, Hkv, N, true).total;
    case MPFA_OP_DECODE:
      if (num_splits < 1 || Hq < 1) return 0;
      return decode_layout(B, Hq, num_splits).total;
    default:
      return 0;
  }
}

const char* mpfa_status_string(int status) {
  switch (status) {
    case MPFA_OK: return "ok";
    case MPFA_ERR_INVALID: return "invalid argument";
    case MPFA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MPFA_ERR_WORKSPACE: return "workspace too small";
    case MPFA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Stage one for K; q_amax (smoothing mode with q only) receives the Q_c amax.
int quantize_k_impl(const void* k, int k_dtype, int B, int Hkv, int N, int D, const void* q,
                    int q_dtype, int Hq, float* q_mean, float* k_mean, uint8_t* k_fp4,
                    uint8_t* k_sf, float* k_gscale, uint16_t* delta_s, float* q_amax, void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if (!dtype_ok(k_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (!k || !k_fp4 || !k_sf || !k_gscale || !ws) return MPFA_ERR_INVALID;
  if (!aligned16(k) || !aligned16(k_fp4) || !aligned16(k_sf) || !aligned16(ws))
    return MPFA_ERR_INVALID;
  // smooth: K centred and delta_s written; centred only (k_mean without
  // delta_s, no q): the cache of the per-tile mean prefill; direct: neither.
  const bool center = k_mean != nullptr;
  const bool smooth = delta_s != nullptr;
  if (smooth) {
    if (!k_mean || !q_mean) return MPFA_ERR_INVALID;
    if ((st = check_heads(Hq, Hkv, B))) return st;
    if (q) {
      if (!dtype_ok(q_dtype)) return MPFA_ERR_UNSUPPORTED;
      if (!aligned16(q)) return MPFA_ERR_INVALID;
    }
    if (!aligned16(q_mean) || !aligned16(delta_s)) return MPFA_ERR_INVALID;
  } else if (center && q) {
    return MPFA_ERR_INVALID;  // a Q mean is only needed for delta_s
  }
  if (center && !aligned16(k_mean)) return MPFA_ERR_INVALID;
  const int Hq_ws = (smooth && q) ? Hq : 0;
  const QuantKWs L = quant_k_layout(B, Hq_ws, Hkv);
  if (ws_bytes < L.total) return MPFA_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  uint32_t* amax = (uint32_t*)(w + L.amax);
  // the Q_c amax (second slot of the cleared amax block) when it is asked for
  uint32_t* q_ext = (smooth && q && q_amax) ? amax + kAmaxSlotWords : nullptr;
  const int kb = k_dtype == MPFA_BF16;
  launch_fill_u32((uint32_t*)w, (int64_t)(L.total / 4), 0u, s);
  const float* kc_mean = nullptr;
  if (center) {
    // K and Q in the same launches; the K_c amax comes from K's channel
    // ranges and means, with no pass of its own
    const ChannelMeanJob kjob = {k, kb, B * Hkv, (uint32_t*)(w + L.kmax),
                                 (unsigned long long*)(w + L.ksum), k_mean, amax};
    const ChannelMeanJob qjob = {q, q_dtype == MPFA_BF16, B * Hq, (uint32_t*)(w + L.qmax),
                                 (unsigned long long*)(w + L.qsum), q_mean, q_ext};
    // the query tensor (G times the keys) first: its long row blocks go out
    // before the short key blocks, which then fill the pass's tail
    const bool two = smooth && q;
    const ChannelMeanJob jobs[2] = {two ? qjob : kjob, kjob};
    launch_channel_means(jobs, two ? 2 : 1, N, s);
    kc_mean = k_mean;
  } else {
    launch_centered_amax(k, kb, B * Hkv, N, nullptr, amax, s);
  }
  // the K quantizer also copies the Q_c amax word out (it runs after the
  // finalize); in smoothing mode it rides in the Delta_S launch, which holds
  // the centred rows anyway
  if (smooth)
    launch_delta_s(k, kb, B, Hkv, Hq / Hkv, N, k_mean, q_mean, delta_s, s, amax, k_gscale, k_fp4,
                   k_sf, q_ext, q_ext ? q_amax : nullptr);
  else
    launch_quantize_k_codes(k, kb, B * Hkv, N, kc_mean, amax, k_gscale, k_fp4, k_sf, q_ext,
                            q_ext ? q_amax : nullptr, s);
  return launch_status();
}

}  // namespace

extern "C" {

int mpfa_quantize_k_nvfp4(const void* k, int k_dtype, int B, int Hkv, int N, int D,
                          const void* q_or_null, int q_dtype, int Hq, float* q_mean, float* k_mean,
                          uint8_t* k_fp4, uint8_t* k_sf, float* k_gscale, uint16_t* delta_s,
                          void* ws, size_t ws_bytes, void* stream) {
  return quantize_k_impl(k, k_dtype, B, Hkv, N, D, q_or_null, q_dtype, Hq, q_mean, k_mean, k_fp4,
                         k_sf, k_gscale, delta_s, nullptr, ws, ws_bytes, stream);
}

int mpfa_quantize_k_nvfp4_with_q_amax(const void* k, int k_dtype, int B, int Hkv, int N, int D,
                                      const void* q_or_null, int q_dtype, int Hq, float* q_mean,
                                      float* k_mean, uint8_t* k_fp4, uint8_t* k_sf,
                                      float* k_gscale, uint16_t* delta_s, float* q_amax, void* ws,
                                      size_t ws_bytes, void* stream) {
  // the Q_c amax exists only where Q is centred by its own means
  if (!q_or_null || !delta_s || !k_mean || !q_amax || !aligned16(q_amax)) return MPFA_ERR_INVALID;
  return quantize_k_impl(k, k_dtype, B, Hkv, N, D, q_or_null, q_dtype, Hq, q_mean, k_mean, k_fp4,
                         k_sf, k_gscale, delta_s, q_amax, ws, ws_bytes, stream);
}

int mpfa_quantize_v_fp8(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint8_t* v_fp8,
                        float* v_scale, void* ws, size_t ws_bytes, void* stream) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if (!dtype_ok(v_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (!v || !v_fp8 || !v_scale || !ws) return MPFA_ERR_INVALID;
  if (!aligned16(v) || !aligned16(v_fp8) || !aligned16(ws)) return MPFA_ERR_INVALID;
  if (ws_bytes < kAmaxBytes) return MPFA_ERR_WORKSPACE;
  if ((N + 31) / 32 > 65535 * 64) return MPFA_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = (uint32_t*)ws;
  const int vb = v_dtype == MPFA_BF16;
  // per-workgroup maxima stored plainly into the workspace and folded into
  // its first word: no clearing launch (the slotted atomics past the limit)
  const int n_part = launch_centered_amax_partials(v, vb, B * Hkv, N, nullptr, (float*)ws, s);
  if (n_part > 0) {
    launch_partials_fold((const float*)ws, n_part, amax, s);
  } else {
    launch_fill_u32(amax, kAmaxBytes / 4, 0u, s);
    launch_centered_amax(v, vb, B * Hkv, N, nullptr, amax, s);
  }
  launch_quantize_v_codes(v, vb, B * Hkv, N, amax, v_scale, v_fp8, s);
  return launch_status();
}

int mpfa_append_kv(const void* k_new, const void* v_new, int kv_dtype, int B, int Hkv, int T,
                   int D, int N_cap, const int32_t* pos, int Hq, const float* q_mean,
                   const float* k_mean, const float* k_gscale, const float* v_scale,
                   uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta_s,
                   void* stream) {
  int st = check_sizes(B, Hkv, N_cap, D);
  if (st) return st;
  if (!dtype_ok(kv_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (T < 1 || T > N_cap || T > 65535) return MPFA_ERR_INVALID;
  if (!k_new || !v_new || !pos || !k_gscale || !v_scale || !k_fp4 || !k_sf || !v_fp8)
    return MPFA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_fp4) || !aligned16(k_sf) ||
      !aligned16(v_fp8))
    return MPFA_ERR_INVALID;
  const bool smooth = k_mean != nullptr;
  int G = 0;
  if (smooth) {
    if (!q_mean || !delta_s) return MPFA_ERR_INVALID;
    if ((st = check_heads(Hq, Hkv, B))) return st;
    G = Hq / Hkv;
    if (G > kD - 8) return MPFA_ERR_UNSUPPORTED;
  } else if (delta_s) {
    return MPFA_ERR_INVALID;  // a compensation cache needs the means
  }
  launch_append_kv(k_new, v_new, kv_dtype == MPFA_BF16, B, Hkv, G, T, N_cap, pos,
                   smooth ? q_mean : nullptr, k_mean, k_gscale, v_scale, k_fp4, k_sf, v_fp8,
                   smooth ? delta_s : nullptr, (hipStream_t)stream);
  return launch_status();
}

int mpfa_append_kv_paged(const void* k_new, const void* v_new, int kv_dtype, int B, int Hkv, int D,
                         const int32_t* pos, const int32_t* block_table, int max_pages,
                         int num_pages, int page_size, int Hq, const float* q_mean,
                         const float* k_mean, const float* k_gscale, const float* v_scale,
                         uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta_s,
                         void* stream) {
  int st = check_sizes(B, Hkv, 1, D);
  if (st) return st;
  if (!dtype_ok(kv_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (page_size != kBlk) return MPFA_ERR_UNSUPPORTED;
  if (max_pages < 1 || num_pages < 1 || (int64_t)max_pages * kBlk > (int64_t)INT32_MAX)
    return MPFA_ERR_INVALID;
  if ((int64_t)B * Hkv > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;
  if (!k_new || !v_new || !pos || !block_table || !k_gscale || !v_scale || !k_fp4 || !k_sf ||
      !v_fp8)
    return MPFA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_fp4) || !aligned16(k_sf) ||
      !aligned16(v_fp8))
    return MPFA_ERR_INVALID;
  const bool smooth = k_mean != nullptr;
  int G = 0;
  if (smooth) {
    if (!q_mean || !delta_s) return MPFA_ERR_INVALID;
    if ((st = check_heads(Hq, Hkv, B))) return st;
    G = Hq / Hkv;
    if (G > kD - 8) return MPFA_ERR_UNSUPPORTED;
  } else if (delta_s) {
    return MPFA_ERR_INVALID;  // a compensation cache needs the means
  }
  launch_append_kv_paged(k_new, v_new, kv_dtype == MPFA_BF16, B, Hkv, G, pos, block_table,
                         max_pages, num_pages, smooth ? q_mean : nullptr, k_mean, k_gscale,
                         v_scale, k_fp4, k_sf, v_fp8, smooth ? delta_s : nullptr,
                         (hipStream_t)stream);
  return launch_status();
}

}  // extern "C"

namespace {

// The prefill call; q_amax NULL: the Q_c amax comes from a pass over Q here.
// variant: the attention kernel's precision / placement variant (0 = the
// method); variant 3 reads V from v_bf16 instead of v_fp8 and v_scale;
// variant 4 reads the NVFP4 V cache v_fp4 / v_sf with its global scale in
// v_scale and expands it into the workspace first.
int prefill_impl(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                 const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                 const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                 const float* v_scale, const uint16_t* delta_s, const float* q_amax,
                 float softmax_scale, int causal, void* out, int out_dtype, float* lse, void* ws,
                 size_t ws_bytes, void* stream, int variant = 0,
                 const uint16_t* v_bf16 = nullptr, const uint8_t* v_fp4 = nullptr,
                 const uint8_t* v_sf = nullptr) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if ((st = check_heads(Hq, Hkv, B))) return st;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return MPFA_ERR_UNSUPPORTED;
  const bool v16 = variant == kVarPvBf16, v4 = variant == kVarPvNvfp4;
  if (!q || !k_fp4 || !k_sf || !k_gscale || !out || !ws) return MPFA_ERR_INVALID;
  if (v16 ? !v_bf16 : (v4 ? (!v_fp4 || !v_sf || !v_scale) : (!v_fp8 || !v_scale)))
    return MPFA_ERR_INVALID;
  const void* v_main = v16 ? (const void*)v_bf16 : (v4 ? (const void*)v_fp4 : (const void*)v_fp8);
  if (!aligned16(q) || !aligned16(k_fp4) || !aligned16(k_sf) || !aligned16(v_main) ||
      (v4 && !aligned16(v_sf)) || !aligned16(out) || !aligned16(ws) || (lse && !aligned16(lse)))
    return MPFA_ERR_INVALID;
  if (delta_s && (!q_mean || !k_mean || !aligned16(q_mean) || !aligned16(k_mean) ||
                  !aligned16(delta_s)))
    return MPFA_ERR_INVALID;
  if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return MPFA_ERR_INVALID;
  const PrefillWs L = prefill_layout(B, Hkv, N, v4);
  if (ws_bytes < L.total) return MPFA_ERR_WORKSPACE;
  const int n_units = (N + 255) / 256;
  if ((int64_t)n_units * B * Hq > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;

  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = (uint32_t*)((uint8_t*)ws + L.amax);
  uint8_t* k_f16 = (uint8_t*)ws + L.k_f16;
  uint16_t* v_img = (uint16_t*)((uint8_t*)ws + L.v_img);
  if (v4) launch_expand_v_nvfp4(v_fp4, v_sf, B * Hkv, N, v_img, s);
  // Q_c amax as per-workgroup maxima, folded by the K expansion that follows
  // (more heads than partial slots: cleared slots, atomics and a fold)
  // (given by the caller: no pass at all)
  const float* qm = delta_s ? q_mean : nullptr;
  int n_part = 0;
  if (!q_amax) {
    n_part = launch_centered_amax_partials(q, q_dtype == MPFA_BF16, B * Hq, N, qm, (float*)amax,
                                           s);
    if (n_part < 0) {
      launch_fill_u32(amax, kAmaxBytes / 4, 0u, s);
      launch_centered_amax(q, q_dtype == MPFA_BF16, B * Hq, N, qm, amax, s);
    }
  }
  launch_expand_k(k_fp4, k_sf, (int64_t)B * Hkv, N, k_f16, s, /*bf16=*/false,
                  n_part > 0 ? (const float*)amax : nullptr, n_part, amax);
  PrefillParams p;
  p.q = q;
  p.q_bf16 = q_dtype == MPFA_BF16;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.G = Hq / Hkv;
  p.q_mean = delta_s ? q_mean : nullptr;
  p.k_mean = delta_s ? k_mean : nullptr;
  p.q_tile_mean = nullptr;
  p.k_f16 = k_f16;
  p.k_gscale = k_gscale;
  p.v_fp8 = v_fp8;
  p.v_scale = v_scale;
  p.delta_s = delta_s;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.out = out;
  p.out_bf16 = out_dtype == MPFA_BF16;
  p.lse = lse;
  p.q_amax = q_amax ? reinterpret_cast<const uint32_t*>(q_amax) : amax;
  p.n_units = n_units;
  p.variant = variant;
  p.v_bf16 = v16 ? v_bf16 : (v4 ? v_img : nullptr);
  launch_prefill(p, s);
  return launch_status();
}

}  // namespace

extern "C" {

int mpfa_prefill(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                 const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                 const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                 const float* v_scale, const uint16_t* delta_s, float softmax_scale, int causal,
                 void* out, int out_dtype, float* lse_or_null, void* ws, size_t ws_bytes,
                 void* stream) {
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                      v_scale, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream);
}

int mpfa_prefill_with_q_amax(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                             const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                             const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                             const float* v_scale, const uint16_t* delta_s, const float* q_amax,
                             float softmax_scale, int causal, void* out, int out_dtype,
                             float* lse_or_null, void* ws, size_t ws_bytes, void* stream) {
  // the first stage derives the amax of the centred Q only
  if (!delta_s || !q_amax || !aligned16(q_amax)) return MPFA_ERR_INVALID;
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                      v_scale, delta_s, q_amax, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream);
}

int mpfa_prefill_elementwise(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                             const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                             const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                             const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                             int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!delta_s) return MPFA_ERR_INVALID;  // a placement of the compensation needs one
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                      v_scale, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream, kVarElementwise);
}

int mpfa_prefill_rank_one(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                          const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                          const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                          const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                          int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!delta_s) return MPFA_ERR_INVALID;  // a placement of the compensation needs one
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                      v_scale, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream, kVarRankOne);
}

int mpfa_prefill_poly_exp2(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                           const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                           const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                           const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                           int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                           size_t ws_bytes, void* stream) {
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                      v_scale, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream, kVarPolyExp2);
}

int mpfa_prefill_pv_bf16(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                         const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                         const uint8_t* k_sf, const float* k_gscale, const uint16_t* v_bf16,
                         const uint16_t* delta_s, float softmax_scale, int causal, void* out,
                         int out_dtype, float* lse_or_null, void* ws, size_t ws_bytes,
                         void* stream) {
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, nullptr,
                      nullptr, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream, kVarPvBf16, v_bf16);
}

int mpfa_prefill_pv_nvfp4(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                          const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                          const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp4,
                          const uint8_t* v_sf, const float* v_gscale, const uint16_t* delta_s,
                          float softmax_scale, int causal, void* out, int out_dtype,
                          float* lse_or_null, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(q, q_dtype, B, Hq, Hkv, N, D, q_mean, k_mean, k_fp4, k_sf, k_gscale, nullptr,
                      v_gscale, delta_s, nullptr, softmax_scale, causal, out, out_dtype,
                      lse_or_null, ws, ws_bytes, stream, kVarPvNvfp4, nullptr, v_fp4, v_sf);
}

int mpfa_quantize_v_nvfp4(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint8_t* v_fp4,
                          uint8_t* v_sf, float* v_gscale, void* ws, size_t ws_bytes,
                          void* stream) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if (!dtype_ok(v_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (!v || !v_fp4 || !v_sf || !v_gscale || !ws) return MPFA_ERR_INVALID;
  if (!aligned16(v) || !aligned16(v_fp4) || !aligned16(v_sf) || !aligned16(ws))
    return MPFA_ERR_INVALID;
  if (ws_bytes < kAmaxBytes) return MPFA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = (uint32_t*)ws;
  const int vb = v_dtype == MPFA_BF16;
  const int n_part = launch_centered_amax_partials(v, vb, B * Hkv, N, nullptr, (float*)ws, s);
  if (n_part > 0) {
    launch_partials_fold((const float*)ws, n_part, amax, s);
  } else {
    launch_fill_u32(amax, kAmaxBytes / 4, 0u, s);
    launch_centered_amax(v, vb, B * Hkv, N, nullptr, amax, s);
  }
  launch_quantize_v_nvfp4(v, vb, B * Hkv, N, amax, v_gscale, v_fp4, v_sf, s);
  return launch_status();
}

int mpfa_pack_v_bf16(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint16_t* v_bf16,
                     void* stream) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if (!dtype_ok(v_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (!v || !v_bf16 || !aligned16(v) || !aligned16(v_bf16)) return MPFA_ERR_INVALID;
  launch_pack_v_bf16(v, v_dtype == MPFA_BF16, B * Hkv, N, v_bf16, (hipStream_t)stream);
  return launch_status();
}

int mpfa_prefill_tile_mean(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                           const float* k_mean, const uint8_t* k_fp4, const uint8_t* k_sf,
                           const float* k_gscale, const uint8_t* v_fp8, const float* v_scale,
                           float softmax_scale, int causal, void* out, int out_dtype, float* lse,
                           float* q_tile_mean, void* ws, size_t ws_bytes, void* stream) {
  int st = check_sizes(B, Hkv, N, D);
  if (st) return st;
  if ((st = check_heads(Hq, Hkv, B))) return st;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (!q || !k_mean || !k_fp4 || !k_sf || !k_gscale || !v_fp8 || !v_scale || !out ||
      !q_tile_mean || !ws)
    return MPFA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_mean) || !aligned16(k_fp4) || !aligned16(k_sf) ||
      !aligned16(v_fp8) || !aligned16(out) || !aligned16(q_tile_mean) || !aligned16(ws) ||
      (lse && !aligned16(lse)))
    return MPFA_ERR_INVALID;
  if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return MPFA_ERR_INVALID;
  const PrefillWs L = prefill_layout(B, Hkv, N);
  if (ws_bytes < L.total) return MPFA_ERR_WORKSPACE;
  const int n_units = (N + 255) / 256;
  if ((int64_t)n_units * B * Hq > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;

  hipStream_t s = (hipStream_t)stream;
  const int qb = q_dtype == MPFA_BF16;
  uint32_t* amax = (uint32_t*)((uint8_t*)ws + L.amax);
  uint8_t* k_img = (uint8_t*)ws + L.k_f16;
  launch_fill_u32(amax, kAmaxBytes / 4, 0u, s);
  launch_tile_mean(q, qb, B * Hq, N, q_tile_mean, amax, s);
  launch_expand_k(k_fp4, k_sf, (int64_t)B * Hkv, N, k_img, s, /*bf16=*/true);
  PrefillParams p;
  p.q = q;
  p.q_bf16 = qb;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.G = Hq / Hkv;
  p.q_mean = nullptr;
  p.k_mean = k_mean;
  p.q_tile_mean = q_tile_mean;
  p.k_f16 = k_img;
  p.k_gscale = k_gscale;
  p.v_fp8 = v_fp8;
  p.v_scale = v_scale;
  p.delta_s = nullptr;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.out = out;
  p.out_bf16 = out_dtype == MPFA_BF16;
  p.lse = lse;
  p.q_amax = amax;
  p.n_units = n_units;
  p.variant = 0;
  p.v_bf16 = nullptr;
  launch_prefill(p, s);
  return launch_status();
}

}  // extern "C"

namespace {

// Argument checks of mpfa_decode except the workspace.
int decode_validate(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D,
                    const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                    const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                    const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                    int num_splits, const void* out, int out_dtype, const float* lse) {
  int st = check_sizes(B, Hkv, N_kv, D);
  if (st) return st;
  if ((st = check_heads(Hq, Hkv, B))) return st;
  if (Hq / Hkv > MPFA_DECODE_MAX_GROUP) return MPFA_ERR_UNSUPPORTED;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (num_splits < 1) return MPFA_ERR_INVALID;
  if (!q || !k_fp4 || !k_sf || !k_gscale || !v_fp8 || !v_scale || !out) return MPFA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_fp4) || !aligned16(k_sf) || !aligned16(v_fp8) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return MPFA_ERR_INVALID;
  if (delta_s && (!q_mean || !k_mean || !aligned16(q_mean) || !aligned16(k_mean) ||
                  !aligned16(delta_s)))
    return MPFA_ERR_INVALID;
  if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return MPFA_ERR_INVALID;
  if ((int64_t)B * Hkv * num_splits > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;
  return MPFA_OK;
}

// The decode launches over a validated call and a workspace of at least
// decode_layout(B, Hq, num_splits).total bytes.  Every workspace word the
// kernels read is written by an earlier kernel of the same call (the query
// amax slots, each partition's state, empty partitions included), so the
// workspace needs no clearing.
int decode_run(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, const float* q_mean,
               const float* k_mean, const uint8_t* k_fp4, const uint8_t* k_sf,
               const float* k_gscale, const uint8_t* v_fp8, const float* v_scale,
               const uint16_t* delta_s, float softmax_scale, int num_splits, void* out,
               int out_dtype, float* lse, void* ws, void* stream) {
  const DecodeWs L = decode_layout(B, Hq, num_splits);
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  uint32_t* amax = (uint32_t*)(w + L.amax);
  launch_rows_amax(q, q_dtype == MPFA_BF16, B * Hq, delta_s ? q_mean : nullptr, (float*)amax, s);
  DecodeParams p;
  p.q = q;
  p.q_bf16 = q_dtype == MPFA_BF16;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N_kv;
  p.G = Hq / Hkv;
  p.P = num_splits;
  const int64_t per = ((int64_t)N_kv + (int64_t)kBlk * num_splits - 1) / ((int64_t)kBlk * num_splits);
  p.chunk = (int)(per * kBlk);
  p.q_mean = delta_s ? q_mean : nullptr;
  p.k_mean = delta_s ? k_mean : nullptr;
  p.k_fp4 = k_fp4;
  p.k_sf = k_sf;
  p.k_gscale = k_gscale;
  p.v_fp8 = v_fp8;
  p.v_scale = v_scale;
  p.delta_s = delta_s;
  p.scale = softmax_scale;
  p.q_amax_slots = (const float*)amax;
  p.ws_m = (float*)(w + L.m);
  p.ws_l = (float*)(w + L.l);
  p.ws_acc = (float*)(w + L.acc);
  p.out = out;
  p.out_bf16 = out_dtype == MPFA_BF16;
  p.lse = lse;
  p.paged = 0;
  p.block_table = nullptr;
  p.seq_lens = nullptr;
  p.max_pages = p.num_pages = 0;
  p.order = nullptr;
  launch_decode(p, s);
  return launch_status();
}

// Scratch of mpfa_decode_static: a fixed array in every GPU's memory (each
// device holds its own copy, at its own address, until the process ends).
// Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, looked up once per device with that device
// current and kept in scratch_ptr.
constexpr size_t kStaticScratchBytes = (size_t)MPFA_DECODE_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 256;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// This device's scratch address, or nullptr if it cannot be found.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  ptr = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

int mpfa_decode(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D,
                const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                int num_splits, void* out, int out_dtype, float* lse, void* ws, size_t ws_bytes,
                void* stream) {
  int st = decode_validate(q, q_dtype, B, Hq, Hkv, N_kv, D, q_mean, k_mean, k_fp4, k_sf, k_gscale,
                           v_fp8, v_scale, delta_s, softmax_scale, num_splits, out, out_dtype, lse);
  if (st) return st;
  if (!ws || !aligned16(ws)) return MPFA_ERR_INVALID;
  if (ws_bytes < decode_layout(B, Hq, num_splits).total) return MPFA_ERR_WORKSPACE;
  return decode_run(q, q_dtype, B, Hq, Hkv, N_kv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                    v_scale, delta_s, softmax_scale, num_splits, out, out_dtype, lse, ws, stream);
}

int mpfa_decode_static(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D,
                       const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                       const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                       const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                       int num_splits, void* out, int out_dtype, float* lse, void* stream) {
  int st = decode_validate(q, q_dtype, B, Hq, Hkv, N_kv, D, q_mean, k_mean, k_fp4, k_sf, k_gscale,
                           v_fp8, v_scale, delta_s, softmax_scale, num_splits, out, out_dtype, lse);
  if (st) return st;
  if (decode_layout(B, Hq, num_splits).total > kStaticScratchBytes) return MPFA_ERR_WORKSPACE;
  void* ws = static_scratch();
  if (!ws) return MPFA_ERR_LAUNCH;
  return decode_run(q, q_dtype, B, Hq, Hkv, N_kv, q_mean, k_mean, k_fp4, k_sf, k_gscale, v_fp8,
                    v_scale, delta_s, softmax_scale, num_splits, out, out_dtype, lse, ws, stream);
}

int mpfa_decode_paged(const void* q, int q_dtype, int B, int Hq, int Hkv, int D,
                      const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                      const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                      const float* v_scale, const uint16_t* delta_s, const int32_t* block_table,
                      const int32_t* seq_lens, int max_pages, int num_pages, int page_size,
                      float softmax_scale, int num_splits, void* out, int out_dtype, float* lse,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_sizes(B, Hkv, 1, D);
  if (st) return st;
  if ((st = check_heads(Hq, Hkv, B))) return st;
  if (Hq / Hkv > MPFA_DECODE_MAX_GROUP) return MPFA_ERR_UNSUPPORTED;
  if (page_size != kBlk) return MPFA_ERR_UNSUPPORTED;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return MPFA_ERR_UNSUPPORTED;
  if (num_splits < 1 || max_pages < 1 || num_pages < 1) return MPFA_ERR_INVALID;
  if ((int64_t)max_pages * kBlk + (int64_t)kBlk * num_splits > (int64_t)INT32_MAX)
    return MPFA_ERR_INVALID;
  if (!q || !k_fp4 || !k_sf || !k_gscale || !v_fp8 || !v_scale || !block_table || !seq_lens ||
      !out || !ws)
    return MPFA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_fp4) || !aligned16(k_sf) || !aligned16(v_fp8) ||
      !aligned16(out) || !aligned16(ws) || (lse && !aligned16(lse)))
    return MPFA_ERR_INVALID;
  if (delta_s && (!q_mean || !k_mean || !aligned16(q_mean) || !aligned16(k_mean) ||
                  !aligned16(delta_s)))
    return MPFA_ERR_INVALID;
  if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return MPFA_ERR_INVALID;
  if ((int64_t)B * Hkv * num_splits > (int64_t)INT32_MAX) return MPFA_ERR_INVALID;
  const DecodeWs L = decode_layout(B, Hq, num_splits);
  if (ws_bytes < L.total) return MPFA_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  uint32_t* amax = (uint32_t*)(w + L.amax);
  launch_rows_amax(q, q_dtype == MPFA_BF16, B * Hq, delta_s ? q_mean : nullptr, (float*)amax, s);
  DecodeParams p;
  p.q = q;
  p.q_bf16 = q_dtype == MPFA_BF16;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = 0;  // per request
  p.G = Hq / Hkv;
  p.P = num_splits;
  p.chunk = 0;
  p.q_mean = delta_s ? q_mean : nullptr;
  p.k_mean = delta_s ? k_mean : nullptr;
  p.k_fp4 = k_fp4;
  p.k_sf = k_sf;
  p.k_gscale = k_gscale;
  p.v_fp8 = v_fp8;
  p.v_scale = v_scale;
  p.delta_s = delta_s;
  p.scale = softmax_scale;
  p.q_amax_slots = (const float*)amax;
  p.ws_m = (float*)(w + L.m);
  p.ws_l = (float*)(w + L.l);
  p.ws_acc = (float*)(w + L.acc);
  p.out = out;
  p.out_bf16 = out_dtype == MPFA_BF16;
  p.lse = lse;
  p.paged = 1;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.order = (int*)(w + L.order);
  launch_decode(p, s);
  return launch_status();
}

}  // extern "C"
