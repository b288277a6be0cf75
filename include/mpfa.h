/*
 * mpfa.h -- C ABI of the QK4PV8 attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * Method: "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels
 * on Blackwell GPUs" (paperpeel.com page).  Q.K^T is computed from NVFP4
 * operands (E2M1 elements, one E4M3 scale per 16 head-dim elements, one FP32
 * scale per tensor), P.V from FP8 E4M3 operands, with an FP32 online softmax
 * (paper section 4.1).  With smoothing, Q and K are centred on their
 * per-head sequence means and the score correction Delta_S = Qbar . K_c
 * enters the score accumulator of the matrix product (its input, before the
 * Q.K^T terms), before the mask and the running-max update (sections 3.2,
 * 5.1, 5.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers.  The caller owns every buffer,
 *   the workspace included.  The library never allocates, frees or
 *   synchronises, keeps no state between calls and retains no pointer.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   The call returns once the kernels are enqueued; device-side faults
 *   surface at the caller's next synchronisation.
 * - Head dimension D must be 128 (the head size of the models the paper
 *   measures, section 7.1).
 * - Input dtypes: MPFA_F32 or MPFA_BF16, contiguous row-major [B, H, N, D].
 * - GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 * - Every pointer must be 16-byte aligned.
 * - Non-finite inputs violate the precondition; results are then
 *   unspecified.
 * - Return value: MPFA_OK (0) or a negative MPFA_ERR_* code.  Arguments are
 *   validated on the host before anything is enqueued; an invalid call
 *   enqueues nothing.
 *
 * Quantized cache layouts (produced by the two quantizers, consumed by
 * prefill and decode):
 *   k_fp4    uint8 [B, Hkv, N, 64]   E2M1 codes, element 2t in the low
 *                                     nibble of byte t (bit 3 = sign)
 *   k_sf     uint8 [B, Hkv, N, 8]    E4M3 scale code of each 16-element block
 *   k_gscale float [1]               per-tensor FP32 scale of the K codes
 *   v_fp8    uint8 [B, Hkv, ceil(N/32), 2, 128, 16]  E4M3 codes of V, stored
 *                                     in tiles of 32 tokens, each two halves
 *                                     of 16 tokens, head-dim major inside a
 *                                     half: element (t, d) sits at
 *                                     [t/32][(t%32)/16][d][t%16]; positions
 *                                     t >= N of the last tile hold code 0
 *   v_scale  float [1]               per-tensor FP32 scale of the V codes
 *   delta_s  uint16 [B, Hq, N]       bf16 bits of Delta_S (smoothing only)
 *   q_mean   float [B, Hq, 128], k_mean float [B, Hkv, 128]
 *
 * The value represented by a K code is e2m1(code) * e4m3(sf) * k_gscale and
 * by a V code e4m3(code) * v_scale.
 *
 * The V cache holds the same bytes as a row-major [B, Hkv, N, 128] FP8 cache
 * (one byte per element, paper section 6), permuted inside each 32-token
 * tile: the FP8 matrix instruction of P.V takes, per lane, 32 consecutive
 * tokens of one channel, which this layout serves as two 16-byte pieces, the
 * pieces of consecutive channels adjacent, so the operand loads of a wave
 * read whole contiguous runs and need no transpose.  Its size is
 * 128 * 32 * ceil(N / 32) bytes per (batch, KV head): N * 128 rounded up to
 * whole tiles.  Converting to or from the row layout is a pure byte
 * permutation (byte (t, d) of the row layout is byte
 * [t / 32][(t % 32) / 16][d][t % 16] here).
 */
#ifndef MPFA_H_
#define MPFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input / output element types. */
#define MPFA_F32 0
#define MPFA_BF16 1

/* Status codes. */
#define MPFA_OK 0
#define MPFA_ERR_INVALID (-1)     /* null / misaligned pointer, bad size, Hq % Hkv != 0 ... */
#define MPFA_ERR_UNSUPPORTED (-2) /* D != 128, unknown dtype, GQA group above the limit */
#define MPFA_ERR_WORKSPACE (-3)   /* ws_bytes smaller than mpfa_workspace_bytes() */
#define MPFA_ERR_LAUNCH (-4)      /* the HIP runtime rejected a kernel launch */

/* Operation selectors for mpfa_workspace_bytes(). */
#define MPFA_OP_QUANTIZE_K 0
#define MPFA_OP_QUANTIZE_V 1
#define MPFA_OP_PREFILL 2
#define MPFA_OP_DECODE 3
#define MPFA_OP_PREFILL_PV_NVFP4 4 /* mpfa_prefill_pv_nvfp4 */

/* Largest GQA group (Hq / Hkv) the decode kernel packs into one tile. */
#define MPFA_DECODE_MAX_GROUP 8

/* Size of the fixed per-GPU scratch array of mpfa_decode_static (16 MiB):
 * the largest mpfa_workspace_bytes(MPFA_OP_DECODE, ...) it serves. */
#define MPFA_DECODE_STATIC_SCRATCH_BYTES 16777216

/*
 * Bytes of device workspace the given operation needs for these sizes
 * (multiple of 256).  Arguments not used by an operation are ignored
 * (Hq for MPFA_OP_QUANTIZE_V, num_splits except for MPFA_OP_DECODE).  For
 * MPFA_OP_QUANTIZE_K pass Hq = 0 when no query tensor will be given.
 * Returns 0 for an unknown operation or a non-positive size.
 */
size_t mpfa_workspace_bytes(int op, int B, int Hq, int Hkv, int N, int D, int num_splits);

/* Static, human-readable name of a status code. */
const char* mpfa_status_string(int status);

/*
 * mpfa_quantize_k_nvfp4 -- first stage for K (paper section 5.1, "first
 * stage"; section 6, "Online quantization").
 *
 * Smoothing mode (k_mean and delta_s both non-NULL):
 *   - k_mean[b, hk, :] <- channel mean of K over the N tokens;
 *   - if q is non-NULL: q_mean[b, h, :] <- channel mean of Q [B, Hq, N, D]
 *     (prefill); if q is NULL, q_mean is an INPUT holding means frozen
 *     earlier in the request (decode);
 *   - K_c = fp32(K - k_mean);
 *   - delta_s[b, h, t] <- bf16(fp32(sum_d q_mean[b, h, d] * K_c[b, h/G, t, d]))
 *     with the sum in FP64 over ascending d (the per-token compensation
 *     vector computed "with one GEMV", section 5.1).
 * Centring only (k_mean non-NULL, delta_s and q NULL; q_mean ignored):
 * k_mean and K_c as above, no Q mean and no delta_s -- the K cache of
 * mpfa_prefill_tile_mean, which computes its compensation itself.  q
 * non-NULL without delta_s returns MPFA_ERR_INVALID.
 * Direct mode (q_mean, k_mean, delta_s all NULL; q ignored): K_c = K.
 * Then NVFP4 of K_c: k_gscale <- amax(|K_c|) / 2688 (1 if the amax is 0),
 * per 16-element block an E4M3 scale code of amax_block / (6 * k_gscale) and
 * E2M1 codes of x / (scale * k_gscale), rounding to nearest, ties to the
 * even code, saturating, sign kept.
 *
 * Means are exact up to one final rounding and independent of summation
 * order: each channel is summed in 64-bit fixed point at 2^-30 of its
 * largest magnitude.
 *
 * k, q: [B, Hkv, N, 128] and [B, Hq, N, 128] in k_dtype / q_dtype.
 * Hq: number of query heads (needed in smoothing mode; Hq % Hkv == 0).
 * ws: mpfa_workspace_bytes(MPFA_OP_QUANTIZE_K, B, q ? Hq : 0, Hkv, N, 128, 1).
 */
int mpfa_quantize_k_nvfp4(const void* k, int k_dtype, int B, int Hkv, int N, int D,
                          const void* q_or_null, int q_dtype, int Hq, float* q_mean, float* k_mean,
                          uint8_t* k_fp4, uint8_t* k_sf, float* k_gscale, uint16_t* delta_s,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * mpfa_quantize_k_nvfp4_with_q_amax -- mpfa_quantize_k_nvfp4 in smoothing
 * mode with the query tensor given (q_or_null and delta_s non-NULL; any
 * other mode returns MPFA_ERR_INVALID), which also writes
 *   q_amax[0] <- max |fp32(Q - q_mean)| over the whole Q tensor,
 * the amax that sets the NVFP4 global scale of the in-kernel query
 * quantization of mpfa_prefill for this Q (paper section 5.1: the first stage
 * feeds the second).  It is derived from the channel statistics the call
 * computes anyway (each channel's largest and smallest value and its mean:
 * fp32 subtraction is monotone, so the value is the one a pass over Q finds),
 * so it costs no pass over Q.  Hand it to mpfa_prefill_with_q_amax with the
 * same Q.  q_amax: device float [1], 16-byte aligned.  Other arguments,
 * workspace and errors as mpfa_quantize_k_nvfp4.
 */
int mpfa_quantize_k_nvfp4_with_q_amax(const void* k, int k_dtype, int B, int Hkv, int N, int D,
                                      const void* q_or_null, int q_dtype, int Hq, float* q_mean,
                                      float* k_mean, uint8_t* k_fp4, uint8_t* k_sf,
                                      float* k_gscale, uint16_t* delta_s, float* q_amax, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * mpfa_quantize_v_fp8 -- FP8 E4M3 V cache (paper section 4.2: V is neither
 * centred nor smoothed; section 6: one byte per V element).
 *   v_scale <- amax(|V|) / 448 (1 if the amax is 0);
 *   v_fp8   <- E4M3 codes of V / v_scale (round to nearest even, saturating),
 *              in the tiled layout described above.
 * v: [B, Hkv, N, 128] in v_dtype.
 * ws: mpfa_workspace_bytes(MPFA_OP_QUANTIZE_V, ...).
 */
int mpfa_quantize_v_fp8(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint8_t* v_fp8,
                        float* v_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * mpfa_append_kv -- decode-time cache write of new tokens (paper section 6,
 * "Online quantization": a newly appended token is centred against the
 * per-request means frozen at prefill and written to the low-bit caches in
 * the same pass that produces its compensation entries).
 *
 * k_new, v_new: [B, Hkv, T, D] in kv_dtype; token t of batch entry b is
 * written to cache position pos[b] + t, where pos is a device int32 array
 * [B] (the caller's per-request lengths).  Caches of capacity N_cap tokens,
 * in the layouts mpfa_quantize_k_nvfp4 / mpfa_quantize_v_fp8 write:
 * k_fp4 [B, Hkv, N_cap, 64], k_sf [B, Hkv, N_cap, 8], v_fp8
 * [B, Hkv, ceil(N_cap/32), 2, 128, 16], delta_s [B, Hq, N_cap] (bf16 bits).
 * The new rows are quantized exactly as the first stage would quantize
 * them with the same statistics: K_c = fp32(K - k_mean) (k_mean may be NULL:
 * direct mode), NVFP4 with the frozen global scale *k_gscale, FP8 with the
 * frozen *v_scale (values out of range saturate), and in smoothing mode
 * delta_s[b, h, p] = bf16(q_mean[b, h] . K_c) for the Hq / Hkv query heads
 * of each KV head.  Smoothing iff k_mean != NULL; then q_mean [B, Hq, 128]
 * and delta_s are required and Hq / Hkv <= 120.
 *
 * Only the T rows of each batch entry are written.  Positions are read on
 * the device: an entry with pos[b] < 0 or pos[b] + T > N_cap is skipped
 * (nothing written for it), which the host cannot report.
 * No workspace.  Returns MPFA_ERR_INVALID for T < 1 or T > N_cap, null or
 * misaligned pointers, delta_s without k_mean.
 */
int mpfa_append_kv(const void* k_new, const void* v_new, int kv_dtype, int B, int Hkv, int T,
                   int D, int N_cap, const int32_t* pos, int Hq, const float* q_mean,
                   const float* k_mean, const float* k_gscale, const float* v_scale,
                   uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta_s,
                   void* stream);

/*
 * Paged caches (paper section 6 "Serving system": fixed-size cache pages, a
 * constant number of KV partitions, the Delta_S side cache following the
 * same physical page indices).  A pool of num_pages pages of page_size = 128
 * tokens (one softmax block; other sizes give MPFA_ERR_UNSUPPORTED):
 *   k_fp4   [num_pages, Hkv, 128, 64]      NVFP4 codes (element 2t low nibble)
 *   k_sf    [num_pages, Hkv, 128, 8]       E4M3 block scales
 *   v_fp8   [num_pages, Hkv, 4, 2, 128, 16] FP8 V, four 32-token tiles (layout above)
 *   delta_s [num_pages, Hq, 128]           bf16 compensation entries (smoothing)
 * block_table: device int32 [B, max_pages]; logical page i of request b
 * (its positions 128 i .. 128 i + 127) is physical page block_table[b, i].
 * A page belongs to one request: its Delta_S rows are that request's query
 * heads.  k_gscale and v_scale are per request: device float [B], the
 * scales each request's cache was quantized with (frozen at its prefill).
 */

/*
 * mpfa_append_kv_paged -- decode-time write of one new token per request
 * into a paged cache (paper section 6 "Online quantization" and "Serving
 * system"); the quantization is that of mpfa_append_kv with request b's
 * frozen scales k_gscale[b], v_scale[b] and means.
 *
 * k_new, v_new: [B, Hkv, 1, 128] in kv_dtype; the token of request b goes to
 * position pos[b] (device int32 [B]), i.e. slot pos[b] % 128 of page
 * block_table[b, pos[b] / 128].  Read on the device: a request with pos[b]
 * outside [0, 128 max_pages) or a page index outside [0, num_pages) is
 * skipped (nothing written for it).  Smoothing iff k_mean != NULL; then
 * q_mean [B, Hq, 128] and delta_s are required and Hq / Hkv <= 120.
 * No workspace.  Returns MPFA_ERR_INVALID for max_pages < 1, num_pages < 1,
 * null or misaligned pointers, delta_s without k_mean.
 */
int mpfa_append_kv_paged(const void* k_new, const void* v_new, int kv_dtype, int B, int Hkv, int D,
                         const int32_t* pos, const int32_t* block_table, int max_pages,
                         int num_pages, int page_size, int Hq, const float* q_mean,
                         const float* k_mean, const float* k_gscale, const float* v_scale,
                         uint8_t* k_fp4, uint8_t* k_sf, uint8_t* v_fp8, uint16_t* delta_s,
                         void* stream);

/*
 * mpfa_prefill -- QK4PV8 attention over a whole sequence (paper section 5.1,
 * "second stage"; sections 5.2, 4.1).
 *
 * Q is centred (smoothing: Q_c = fp32(Q - q_mean)) and quantized to NVFP4 on
 * the fly with a per-call global scale amax(|Q_c|) / 2688.  Per row i and KV
 * block of 128 keys (ascending, skipping blocks with no visible key):
 *   S_ij = Q~_i . K~_j + Delta_S[j]      (compensation before mask and max)
 *   m    = running max of S; p = 2^(lambda (S - m)), lambda = scale * log2(e)
 *   l    = alpha l + sum p               (FP32, unquantized p)
 *   acc  = alpha acc + e4m3(448 p) . V~  (FP8 P.V, the only in-loop rounding)
 * out_i = acc * v_scale / (448 l); lse_i = scale * m + ln l, plus
 * scale * (Q_i . k_mean) in smoothing mode (so it estimates the LSE of the
 * uncentred scores).
 *
 * Smoothing iff delta_s != NULL (then q_mean and k_mean are required).
 * The NVFP4 global scale of Q comes from a pass over Q_c in this call.
 * causal != 0: key j is visible to row i iff j <= i; else every key.
 * out: [B, Hq, N, 128] in out_dtype (MPFA_BF16, the paper's output, or
 * MPFA_F32).  lse_or_null: [B, Hq, N] float, or NULL.
 * ws: mpfa_workspace_bytes(MPFA_OP_PREFILL, B, Hq, Hkv, N, 128, 1) bytes
 * (8192 + B * Hkv * ceil(N / 128) * 32768, rounded up to 256): the per-call
 * Q amax and the K cache expanded once per call to exact FP16 operands
 * (code value x block scale, 32 KB per 128-key block, 256 bytes per key
 * against the cache's 72, zero past N), which the attention kernel copies
 * into LDS block by block.  It is caller-owned scratch: nothing in it
 * outlives the call.
 */
int mpfa_prefill(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                 const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                 const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                 const float* v_scale, const uint16_t* delta_s, float softmax_scale, int causal,
                 void* out, int out_dtype, float* lse_or_null, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * mpfa_prefill_with_q_amax -- mpfa_prefill in smoothing mode that takes the
 * Q_c amax from the first stage (mpfa_quantize_k_nvfp4_with_q_amax on the
 * same Q) instead of a pass over Q: identical results, one launch less.
 * q_amax: device float [1] holding max |fp32(Q - q_mean)| for this Q and
 * q_mean; a value that belongs to another Q gives another global scale, and
 * the library cannot detect that (it never reads device memory on the host).
 * delta_s == NULL or q_amax == NULL returns MPFA_ERR_INVALID.  Other
 * arguments, workspace and errors as mpfa_prefill.
 */
int mpfa_prefill_with_q_amax(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                             const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                             const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                             const float* v_scale, const uint16_t* delta_s, const float* q_amax,
                             float softmax_scale, int causal, void* out, int out_dtype,
                             float* lse_or_null, void* ws, size_t ws_bytes, void* stream);

/*
 * Precision and placement variants of the smoothing-mode prefill (paper
 * section 3.1, Fig. 3(a): NVFP4 + FP8 against NVFP4 + BF16 and NVFP4 +
 * NVFP4; section 7.4
 * "Compensation placement": the compensation inside the matrix product
 * against an element-wise add, here in two forms of the former -- the score
 * accumulator's input (mpfa_prefill) and a rank-one MMA step;
 * section 5.1: part of the exponentials by a polynomial on the FMA units).
 * They exist to measure those choices on gfx950; each computes what its
 * description says and is checked against the oracle like mpfa_prefill.
 * Arguments, workspace and errors are those of mpfa_prefill unless stated.
 *
 * mpfa_prefill_elementwise -- Delta_S * 1/(gQ gK) added to every score on the
 * vector ALUs at the start of the softmax of each block (before the mask and
 * the running max), instead of entering the score accumulator before the
 * products; the scores are the same up to FP32 rounding.  delta_s == NULL
 * returns MPFA_ERR_INVALID.
 */
int mpfa_prefill_elementwise(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                             const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                             const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                             const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                             int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * mpfa_prefill_rank_one -- the compensation as its own rank-one matrix step
 * (paper section 5.2's MMA placement): per 32-key score tile one bf16
 * 32x32x16 matrix instruction with A = the bf16 Delta_S of each key and B =
 * 1/(gQ gK) as three bf16 parts writes the term into the score accumulator
 * before the Q.K^T products, where mpfa_prefill instead loads Delta_S *
 * 1/(gQ gK) (fp32) as that accumulator's input; the scores are the same up to
 * FP32 rounding.  delta_s == NULL returns MPFA_ERR_INVALID.
 */
int mpfa_prefill_rank_one(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                          const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                          const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                          const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                          int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * mpfa_prefill_poly_exp2 -- mpfa_prefill with one exponential in four
 * computed as 2^rint(x) * c(x - rint(x)), c a cubic fitted to 2^f on
 * [-1/2, 1/2] (largest relative error 7.5e-5), instead of the hardware exp2;
 * P is then that much less accurate before its E4M3 rounding.  Smoothing or
 * direct as mpfa_prefill.
 */
int mpfa_prefill_poly_exp2(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                           const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                           const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                           const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                           int causal, void* out, int out_dtype, float* lse_or_null, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * mpfa_pack_v_bf16 -- the bf16 V cache of mpfa_prefill_pv_bf16: V rounded to
 * bf16 (nearest even) in tiles of 32 tokens, [B, Hkv, ceil(N/32), 4, 128, 8]
 * uint16: token t, channel d at [t / 32][(t % 32) / 8][d][t % 8] (8 tokens of
 * one channel per 16 bytes, the operand of a bf16 matrix instruction); zero
 * past N.  v: [B, Hkv, N, 128] in v_dtype.  No workspace.
 */
int mpfa_pack_v_bf16(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint16_t* v_bf16,
                     void* stream);

/*
 * mpfa_prefill_pv_bf16 -- the NVFP4 + BF16 precision assignment: Q.K^T as in
 * mpfa_prefill, P rounded to bf16 (of 448 p, round to nearest even) instead
 * of E4M3, and P.V on bf16 matrix instructions over the bf16 V cache of
 * mpfa_pack_v_bf16 (v_bf16 replaces v_fp8 and v_scale); l sums the
 * unrounded p as in mpfa_prefill; out_i = acc / (448 l).  Smoothing or direct
 * as mpfa_prefill.
 */
int mpfa_prefill_pv_bf16(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                         const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                         const uint8_t* k_sf, const float* k_gscale, const uint16_t* v_bf16,
                         const uint16_t* delta_s, float softmax_scale, int causal, void* out,
                         int out_dtype, float* lse_or_null, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * mpfa_quantize_v_nvfp4 -- the NVFP4 V cache of mpfa_prefill_pv_nvfp4.  The
 * P.V contraction runs over the keys, so V's 16-element blocks run along the
 * keys of each channel (paper section 3.1: block-scaled NVFP4 P.V).  With A
 * the amax of the whole V tensor, g = A > 0 ? fp32(A / 2688) : 1 -> *v_gscale;
 * per (16-key block kb, channel d): s = E4M3(fp32(amax / fp32(6 g))),
 * code_t = E2M1(fp32(v_t / fp32(s g))) (the steps of mpfa_quantize_k_nvfp4),
 * keys past N counting as zero.
 *   v      [B, Hkv, N, 128] in v_dtype.
 *   v_fp4  [B, Hkv, ceil(N/16), 128, 8] uint8: byte t of (kb, d) holds key
 *          16 kb + 2t in the low nibble and key 16 kb + 2t + 1 in the high.
 *   v_sf   [B, Hkv, ceil(N/16), 128] uint8 E4M3 block scales.
 *   ws: mpfa_workspace_bytes(MPFA_OP_QUANTIZE_V, ...).
 */
int mpfa_quantize_v_nvfp4(const void* v, int v_dtype, int B, int Hkv, int N, int D, uint8_t* v_fp4,
                          uint8_t* v_sf, float* v_gscale, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * mpfa_prefill_pv_nvfp4 -- the NVFP4 + NVFP4 precision assignment (paper
 * section 3.1, Fig. 3(a)): Q.K^T as in mpfa_prefill; in each 128-key block
 * the p of every 16 consecutive keys (groups aligned at the block start,
 * masked keys zero) are quantized on the softmax path to NVFP4 with the
 * fixed global scale G_P = fp32(1/2688) (so p <= 1 maps to at most 6 x 448):
 * amax, E4M3 scale s = E4M3(fp32(amax / fp32(6 G_P))), codes
 * E2M1(fp32(p / fp32(s G_P))); V from mpfa_quantize_v_nvfp4 (v_fp4, v_sf,
 * v_gscale replace v_fp8 and v_scale).  P.V multiplies the exact values
 * (code x block scale, in FP16) on f16 matrix instructions with FP32
 * accumulation; l sums the unquantized p; out_i = acc G_P g_V / l; lse as
 * mpfa_prefill.  Smoothing or direct as mpfa_prefill.
 *   ws: mpfa_workspace_bytes(MPFA_OP_PREFILL_PV_NVFP4, B, Hq, Hkv, N, 128, 1)
 *       (mpfa_prefill's, plus the FP16 image of V: 256 bytes per key and KV
 *       head, written by this call).
 */
int mpfa_prefill_pv_nvfp4(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                          const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                          const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp4,
                          const uint8_t* v_sf, const float* v_gscale, const uint16_t* delta_s,
                          float softmax_scale, int causal, void* out, int out_dtype,
                          float* lse_or_null, void* ws, size_t ws_bytes, void* stream);

/*
 * mpfa_prefill_tile_mean -- mpfa_prefill with the queries smoothed per
 * 128-row query tile instead of per sequence (the query smoothing of paper
 * sections 3.2 and 5.1 at the granularity of the attention stage's query
 * tile; the compensation is computed in the attention stage, so no Delta_S
 * side cache exists in this mode).
 *
 *   q_tile_mean[b, h, t, :] <- channel mean of rows 128 t .. min(128 t + 127,
 *     N - 1) of Q [b, h], by the order-free fixed-point rule of the sequence
 *     means (the last tile averages only its rows);
 *   Q_c = fp32(Q_i - q_tile_mean[tile of i]); NVFP4 with global scale
 *     gQ = amax(|Q_c|) / 2688 over the whole call;
 *   Delta_tile[t, j] = bf16(fp32(q_tile_mean[t] . K~_c[j])), K~_c the
 *     dequantized centred key, the column term of the tile's mean, carried
 *     in BF16 like Delta_S (section 5.2) and computed in the attention kernel
 *     one 128-key block ahead by a matrix product of the mean's three exact
 *     bf16 parts with the K operands (FP32 accumulation);
 *   S_ij = Q~_c,i . K~_c,j + Delta_tile[tile of i, j], the offset entering
 *     the score accumulator as Delta_S does in mpfa_prefill;
 * then the online softmax, P.V and epilogue of mpfa_prefill; lse adds back
 * scale * (Q_i . k_mean).
 *
 * K must be cached centred (mpfa_quantize_k_nvfp4 in centring-only or
 * smoothing mode; k_mean is that call's k_mean).  q_tile_mean: OUTPUT,
 * device float [B, Hq, ceil(N / 128), 128].  The other arguments, the output
 * layouts and the workspace (mpfa_workspace_bytes(MPFA_OP_PREFILL, ...); the
 * K cache is expanded to BF16 operands here, same size) are those of
 * mpfa_prefill.  Returns MPFA_ERR_INVALID for a null k_mean or q_tile_mean
 * and as mpfa_prefill does.
 */
int mpfa_prefill_tile_mean(const void* q, int q_dtype, int B, int Hq, int Hkv, int N, int D,
                           const float* k_mean, const uint8_t* k_fp4, const uint8_t* k_sf,
                           const float* k_gscale, const uint8_t* v_fp8, const float* v_scale,
                           float softmax_scale, int causal, void* out, int out_dtype, float* lse,
                           float* q_tile_mean, void* ws, size_t ws_bytes, void* stream);

/*
 * mpfa_decode -- one query token per (batch, query head) against N_kv cached
 * keys (paper section 5.3): the KV history is cut into num_splits contiguous
 * partitions of whole 128-key blocks (partition length
 * 128 * ceil(N_kv / (128 * num_splits))); each partition runs the prefill
 * block loop from its own start with every key visible, the GQA group's
 * query heads packed into one tile, and the partial (m, l, acc) states are
 * merged by log-sum-exp.
 *
 * q: [B, Hq, 1, 128].  q_mean: the frozen per-request means (smoothing).
 * out: [B, Hq, 128]; lse: [B, Hq] or NULL.  Hq / Hkv <= MPFA_DECODE_MAX_GROUP.
 * ws: mpfa_workspace_bytes(MPFA_OP_DECODE, B, Hq, Hkv, N_kv, 128, num_splits).
 */
int mpfa_decode(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D,
                const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                int num_splits, void* out, int out_dtype, float* lse, void* ws, size_t ws_bytes,
                void* stream);

/*
 * mpfa_decode_static -- mpfa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace argument and allocates nothing:
 * the decode's scratch (query amax slots, per-partition m, l and acc) lives in
 * a fixed array of MPFA_DECODE_STATIC_SCRATCH_BYTES in each GPU's memory,
 * part of the library's device code, held until the process ends.  The first
 * call on a device looks up that device's copy (hipGetSymbolAddress; no
 * allocation); make one call before a graph capture.  Results are those of
 * mpfa_decode with the same arguments, bit for bit.
 *
 * Limit: mpfa_workspace_bytes(MPFA_OP_DECODE, B, Hq, Hkv, N_kv, 128,
 * num_splits) <= MPFA_DECODE_STATIC_SCRATCH_BYTES (about B * Hq * num_splits
 * <= 32000), else MPFA_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and give unspecified
 * results; calls on one stream are ordered and safe.  The array keeps the
 * last call's contents; every word a call reads is written earlier in the
 * same call, so nothing needs clearing.  Returns MPFA_ERR_LAUNCH if the
 * array cannot be located on the current device.  Other arguments and errors
 * as mpfa_decode.
 */
int mpfa_decode_static(const void* q, int q_dtype, int B, int Hq, int Hkv, int N_kv, int D,
                       const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                       const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                       const float* v_scale, const uint16_t* delta_s, float softmax_scale,
                       int num_splits, void* out, int out_dtype, float* lse, void* stream);

/*
 * mpfa_decode_paged -- mpfa_decode over a paged cache (layout above) with
 * per-request lengths: request b attends to its positions
 * 0 .. seq_lens[b] - 1 (seq_lens: device int32 [B], read on the device and
 * clamped to [0, 128 max_pages]), cut into num_splits partitions of whole
 * 128-key blocks by its own length (partition length
 * 128 * ceil(seq_lens[b] / (128 * num_splits))), with its own frozen scales
 * k_gscale[b], v_scale[b].  Q is quantized once over the whole [B, Hq]
 * query tensor of the call, as in mpfa_decode.  A request with no positions
 * returns O = 0 and LSE = -inf.  Page slots past a request's length are
 * never used (their V bytes are masked, whatever they hold).  Page indices
 * are read on the device; one outside [0, num_pages) is clamped into the
 * pool (every access stays inside it; that request's result is unspecified).
 *
 * q: [B, Hq, 1, 128]; q_mean [B, Hq, 128] and k_mean [B, Hkv, 128] the frozen
 * per-request means (smoothing iff delta_s != NULL).  out: [B, Hq, 128];
 * lse: [B, Hq] or NULL.  Hq / Hkv <= MPFA_DECODE_MAX_GROUP.
 * ws: mpfa_workspace_bytes(MPFA_OP_DECODE, B, Hq, Hkv, 1, 128, num_splits)
 * (the decode workspace does not depend on the lengths).
 * Returns MPFA_ERR_INVALID for num_splits, max_pages or num_pages < 1, null or
 * misaligned pointers, 128 max_pages + 128 num_splits >= 2^31.
 */
int mpfa_decode_paged(const void* q, int q_dtype, int B, int Hq, int Hkv, int D,
                      const float* q_mean, const float* k_mean, const uint8_t* k_fp4,
                      const uint8_t* k_sf, const float* k_gscale, const uint8_t* v_fp8,
                      const float* v_scale, const uint16_t* delta_s, const int32_t* block_table,
                      const int32_t* seq_lens, int max_pages, int num_pages, int page_size,
                      float softmax_scale, int num_splits, void* out, int out_dtype, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MPFA_H_ */
