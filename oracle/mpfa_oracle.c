/*
 * mpfa_oracle.c -- plain, slow, host-only reference of the QK4PV8 attention
 * path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the benchmark may call it; the library under
 * mixed_precision_flashattention_amd/ never does, and the two share no code.
 *
 * Source of the method: the MpFA paper page, "MpFA: Hardware-Efficient
 * Train-Free QK4V8 FlashAttention Kernels on Blackwell GPUs" (cited below as
 * "MpFA §x").  The page names the number formats but prints no equations, so
 * every rounding step below is a reading, written out explicitly next to the
 * function that takes it.
 *
 * Arithmetic: FP64 wherever the method names no rounding; fp32 exactly where
 * a reading fixes an fp32 step (centering, scale computation, quantizer
 * divisions), so that the device quantizers can be compared byte for byte.
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fused multiply-add, so every
 * C expression rounds exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define E2M1_MAX 6.0
#define E4M3_MAX 448.0

/* ---------------------------------------------------------------- codecs --
 * E2M1 (MpFA §4.1 "NVFP4", 4-bit element): bits s|e1 e0|m, exponent bias 1,
 * e == 0 is subnormal (m * 0.5).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.      */
double oracle_e2m1_decode(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? m * 0.5 : (1.0 + m * 0.5) * ldexp(1.0, e - 1);
  return s ? -v : v;
}

/* E4M3 in the OCP "FN" variant (MpFA §4.1 "e4m3" scale factors and FP8
 * P and V): bits s|eeee|mmm, bias 7, e == 0 subnormal m/8 * 2^-6, no
 * infinities, 0x7F / 0xFF are NaN, largest finite 448 (code 0x7E).          */
double oracle_e4m3_decode(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  v = (e == 0) ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

/* Round to the nearest representable magnitude of a code table whose codes
 * 0..n-1 decode to increasing magnitudes; ties go to the even code; anything
 * beyond the largest magnitude saturates to it.  The sign bit is attached by
 * the caller, so -0 and negative values that round to zero keep their sign. */
static int nearest_code(double a, const double* mag, int n) {
  int lo = 0, hi = n - 1;
  if (a >= mag[n - 1]) return n - 1;
  /* binary search for mag[lo] <= a < mag[lo+1] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (mag[mid] <= a) lo = mid; else hi = mid;
  }
  {
    double dlo = a - mag[lo], dhi = mag[hi] - a;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo; /* tie: even code */
  }
}

static double g_e2m1_mag[8];
static double g_e4m3_mag[127];
static int g_tables_ready = 0;
static void init_tables(void) {
  int c;
  if (g_tables_ready) return;
  for (c = 0; c < 8; ++c) g_e2m1_mag[c] = oracle_e2m1_decode(c);
  for (c = 0; c < 127; ++c) g_e4m3_mag[c] = oracle_e4m3_decode(c);
  g_tables_ready = 1;
}

/* Encoders take a double so that a value computed in FP64 is rounded once;
 * a float argument converts to double exactly.  NaN inputs are outside the
 * method's domain (unspecified); they encode as the saturated magnitude.     */
int oracle_e2m1_encode(double x) {
  int sign = signbit(x) ? 8 : 0;
  double a = fabs(x);
  init_tables();
  if (isnan(a)) a = E2M1_MAX;
  return sign | nearest_code(a, g_e2m1_mag, 8);
}

int oracle_e4m3_encode(double x) {
  int sign = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  init_tables();
  if (isnan(a)) a = E4M3_MAX;
  return sign | nearest_code(a, g_e4m3_mag, 127);
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t oracle_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

double oracle_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------ statistics --
 * Per-channel mean over tokens (MpFA §6 "Online quantization": per-head means
 * of Q and K over the valid tokens; §3.2 "subtracting the means").  Reading:
 * the mean must not depend on summation order, so it is defined through an
 * exact fixed-point sum:
 *   M = max_t |x_t|;  M == 0 -> mean 0
 *   E with M in [2^(E-1), 2^E);  u = 2^(E-30)
 *   q_t = round-half-even(x_t / u)            (exact power-of-two scaling)
 *   S = sum q_t in int64                       (exact, order free)
 *   mean = fp32( (double)S / (double)T * u )   (FP64 ops, round to nearest)
 * x is [T][D] row-major, one (batch, head) slice; out is [D].               */
void oracle_channel_mean(const float* x, int64_t T, int D, float* out) {
  /* Rows are walked in memory order; per channel this is the same max and
   * the same exact integer sum as a walk down the column. */
  double* M = (double*)calloc((size_t)D, sizeof(double));
  double* u_inv = (double*)calloc((size_t)D, sizeof(double));
  int* E = (int*)calloc((size_t)D, sizeof(int));
  int64_t* S = (int64_t*)calloc((size_t)D, sizeof(int64_t));
  int64_t t;
  int d;
  for (t = 0; t < T; ++t)
    for (d = 0; d < D; ++d) {
      double a = fabs((double)x[t * D + d]);
      if (a > M[d]) M[d] = a;
    }
  for (d = 0; d < D; ++d) {
    if (M[d] > 0.0) frexp(M[d], &E[d]); /* M = f * 2^E with f in [0.5, 1) */
    u_inv[d] = ldexp(1.0, 30 - E[d]);    /* 1/u, a power of two: x * u_inv is exact */
  }
  for (t = 0; t < T; ++t)
    for (d = 0; d < D; ++d)
      S[d] += (int64_t)nearbyint((double)x[t * D + d] * u_inv[d]); /* half to even */
  for (d = 0; d < D; ++d) {
    if (M[d] == 0.0 || T == 0) {
      out[d] = 0.0f;
    } else {
      double mean = (double)S[d] / (double)T;
      mean = mean * ldexp(1.0, E[d] - 30);
      out[d] = (float)mean;
    }
  }
  free(M);
  free(u_inv);
  free(E);
  free(S);
}

/* max |x| over n elements (exact). */
float oracle_amax(const float* x, int64_t n) {
  float m = 0.0f;
  int64_t i;
  for (i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  return m;
}

/* ------------------------------------------------------------ quantizers --
 * NVFP4 block quantization (MpFA §4.1: one e4m3 scale per 16 head-dim
 * elements; the per-tensor FP32 global scale is the format's second level,
 * named on the crashtech article's NVFP4 paragraph).  Reading:
 *   g   = A > 0 ? fp32(A / 2688) : 1        (A = tensor amax, 2688 = 6*448)
 *   s_b = dec(enc_e4m3( fp32(a_b / fp32(6*g)) ))   a_b = block amax
 *   c   = (s_b == 0 or fp32(s_b*g) == 0) ? signed zero
 *                                         : enc_e2m1( fp32(x / fp32(s_b*g)) )
 *   value represented: dec(c) * s_b * g
 * Packing: byte t of a row holds element 2t in the low nibble.
 * x is [rows][D], D a multiple of 16; codes is [rows][D/2]; sf is [rows][D/16]. */
float oracle_nvfp4_global_scale(float amax) {
  return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/* One block of 16 values, the steps above: returns the scale code and
 * writes the 16 element codes. */
static int nvfp4_block_codes(const float* xb, float g, int* c) {
  const float six_g = 6.0f * g;
  float ab = 0.0f, s, sg;
  int sc, j;
  for (j = 0; j < 16; ++j) if (fabsf(xb[j]) > ab) ab = fabsf(xb[j]);
  sc = oracle_e4m3_encode((double)(ab / six_g));
  s = (float)oracle_e4m3_decode(sc);
  sg = s * g;
  for (j = 0; j < 16; ++j) {
    if (s == 0.0f || sg == 0.0f) c[j] = signbit(xb[j]) ? 8 : 0;
    else c[j] = oracle_e2m1_encode((double)(xb[j] / sg));
  }
  return sc;
}

void oracle_nvfp4_quantize(const float* x, int64_t rows, int D, float g,
                           uint8_t* codes, uint8_t* sf) {
  int64_t r;
  init_tables();
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    int b, j, c[16];
    for (b = 0; b < D / 16; ++b) {
      sf[r * (D / 16) + b] = (uint8_t)nvfp4_block_codes(x + r * D + b * 16, g, c);
      for (j = 0; j < 16; j += 2)
        codes[r * (D / 2) + b * 8 + j / 2] = (uint8_t)(c[j] | (c[j + 1] << 4));
    }
  }
}

/* Dequantize NVFP4 rows to FP64: dec(code) * s * g, exact in FP64. */
void oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* sf, int64_t rows, int D,
                             float g, double* out) {
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    int e;
    for (e = 0; e < D; ++e) {
      int byte = codes[r * (D / 2) + e / 2];
      int c = (e & 1) ? (byte >> 4) : (byte & 15);
      double s = oracle_e4m3_decode(sf[r * (D / 16) + e / 16]);
      out[r * D + e] = oracle_e2m1_decode(c) * s * (double)g;
    }
  }
}

/* FP8 E4M3 per-tensor quantization of V (MpFA §4.2: V is not centered and
 * uses FP8 e4m3).  Reading: s_V = A > 0 ? fp32(A / 448) : 1, A = tensor amax;
 * code = enc_e4m3(fp32(v / s_V)); value represented dec(code) * s_V.        */
float oracle_fp8_scale(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

void oracle_fp8_quantize(const float* x, int64_t n, float s, uint8_t* codes) {
  int64_t i;
  init_tables();
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) codes[i] = (uint8_t)oracle_e4m3_encode((double)(x[i] / s));
}

/* Rank-one compensation vector (MpFA §5.1: "one GEMV", §5.2, §7.4: carried in
 * BF16).  Reading: Delta_S[j] = bf16_rne( fp32( sum_d qmean_d * kc[j][d] ) ),
 * the sum taken in FP64 in ascending d (each product is exact in FP64).     */
void oracle_delta_s(const float* qmean, const float* kc, int64_t T, int D, uint16_t* out) {
  int64_t j;
#pragma omp parallel for schedule(static)
  for (j = 0; j < T; ++j) {
    double acc = 0.0;
    int d;
    for (d = 0; d < D; ++d) acc += (double)qmean[d] * (double)kc[j * D + d];
    out[j] = oracle_bf16_rne((float)acc);
  }
}

/* --------------------------------------------------------------- attention --
 * Online-softmax attention over one key range for R query rows of one head
 * (MpFA §4.1: m, l and the PV accumulator in FP32 -- here FP64 -- and P the
 * only in-loop quantization with a fixed scale; §3.2: the compensation is in
 * the score before masking and before the running-max update; §5.1: the
 * softmax constant is folded into a base-2 exponent).
 *
 *   keys [kv_begin, kv_end) are cut into blocks of `block` keys aligned at
 *   kv_begin and taken in ascending order; key j is visible to row r iff
 *   row_pos[r] < 0 or j <= row_pos[r]; a block with no visible key is skipped.
 *   S_rj = sum_d q[r][d] * k[j][d] + delta[j]           (FP64)
 *   per block:  m' = max(m, max_j S_rj);  alpha = 2^(lam (m - m'))  (0 first)
 *               p_rj = 2^(lam (S_rj - m'))
 *               l   = alpha l + sum_j p_rj                (unquantized p)
 *               ph  = quant_p ? dec(enc_e4m3(448 p)) : 448 p
 *               acc = alpha acc + sum_j ph * v[j][:]
 *   lam = scale * log2(e).
 * Outputs the partial state (m, l, acc); m = -inf and l = 0 when the row saw
 * no key.  q is [R][D], k and v are [*][D] indexed by absolute key, delta is
 * indexed by absolute key or NULL.                                          */
/* The other E4M3 magnitude a value a >= 0 may round to when it lies within
 * `rel` (relative) of the midpoint between two neighbouring magnitudes --
 * closer than the kernel's own computation of p can place it -- else the
 * rounded value ph itself.                                                  */
static double table_alternative(double a, double ph, double rel, const double* mag, int n) {
  int lo = 0, hi = n - 1;
  double mid;
  if (a >= mag[n - 1] || a <= 0.0) return ph;
  while (hi - lo > 1) {
    int m = (lo + hi) / 2;
    if (mag[m] <= a) lo = m; else hi = m;
  }
  mid = 0.5 * (mag[lo] + mag[hi]);
  if (fabs(a - mid) > rel * a) return ph;
  return ph == mag[lo] ? mag[hi] : mag[lo];
}
static double e4m3_alternative(double a, double ph, double rel) {
  return table_alternative(a, ph, rel, g_e4m3_mag, 127);
}

/* NVFP4 P (the NVFP4 + NVFP4 precision assignment of MpFA §3.1, Fig. 3(a):
 * P quantized with a scale per 16 elements along the keys, computed on the
 * softmax path).  Reading: the O3 block steps above applied to x = fp32(p)
 * over 16 consecutive keys (groups aligned at the KV block start; masked or
 * absent keys count as p = 0), with the global scale fixed at
 * G_P = fp32(1/2688), the NVFP4 scale that maps the bound p <= 1 to the
 * largest representable product 6 * 448 (as the fixed 448 does for FP8 P).
 * ph[i] = 448 * dec(code) * s * G_P, in the 448 units of the other formats.
 * alt[i]: the value farthest from ph[i] among the other roundings that are
 * equally valid when the scale decision (amax / fp32(6 G_P)) or the element
 * decision (x / fp32(s G_P)) lies within `rel` of a midpoint; ph[i] when
 * there is none.                                                            */
static const float G_P = 1.0f / 2688.0f;
static void nvfp4_p_values(int sc, const int* c, double* ph) {
  const double s = oracle_e4m3_decode(sc);
  int i;
  for (i = 0; i < 16; ++i) ph[i] = 448.0 * oracle_e2m1_decode(c[i]) * s * (double)G_P;
}
static void nvfp4_p_block(const float* x, double rel, double* ph, double* alt) {
  const float six_g = 6.0f * G_P;
  double cand[16];
  float ab = 0.0f;
  int c[16], i, k, sc, scs[2], nsc = 1;
  for (i = 0; i < 16; ++i) if (x[i] > ab) ab = x[i];
  sc = nvfp4_block_codes(x, G_P, c);
  nvfp4_p_values(sc, c, ph);
  for (i = 0; i < 16; ++i) alt[i] = ph[i];
  scs[0] = sc;
  {
    const double qs = (double)(ab / six_g), s = oracle_e4m3_decode(sc);
    const double s_alt = e4m3_alternative(qs, s, rel);
    if (s_alt != s) scs[nsc++] = oracle_e4m3_encode(s_alt);
  }
  for (k = 0; k < nsc; ++k) {
    const float s = (float)oracle_e4m3_decode(scs[k]), sg = s * G_P;
    int ck[16];
    for (i = 0; i < 16; ++i)
      ck[i] = (s == 0.0f || sg == 0.0f) ? 0 : oracle_e2m1_encode((double)(x[i] / sg));
    nvfp4_p_values(scs[k], ck, cand);
    for (i = 0; i < 16; ++i) {
      const double qe = (s == 0.0f || sg == 0.0f) ? 0.0 : (double)(x[i] / sg);
      const double e = oracle_e2m1_decode(ck[i]);
      const double e_alt = table_alternative(qe, e, rel, g_e2m1_mag, 8);
      const double v_alt = 448.0 * e_alt * (double)s * (double)G_P;
      if (fabs(cand[i] - ph[i]) > fabs(alt[i] - ph[i])) alt[i] = cand[i];
      if (fabs(v_alt - ph[i]) > fabs(alt[i] - ph[i])) alt[i] = v_alt;
    }
  }
}

/* Nearest bf16 value (8 significant bits) to a >= 0, ties to the even
 * significand, from the FP64 value directly (one rounding).  Normal bf16
 * range only: the P values it rounds (448 p) are 0 or above 2^-120 wherever
 * they can matter.                                                          */
static double bf16_round_pos(double a) {
  int e;
  if (a <= 0.0) return 0.0;
  frexp(a, &e);
  return ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);
}

/* The other bf16 neighbour of a >= 0 when a lies within `rel` of the midpoint
 * between its two bf16 neighbours, else ph.                                 */
static double bf16_alternative(double a, double ph, double rel) {
  int e;
  double lo, hi, mid;
  if (a <= 0.0) return ph;
  frexp(a, &e);
  lo = ldexp(floor(ldexp(a, 8 - e)), e - 8);
  hi = lo + ldexp(1.0, e - 8);
  mid = 0.5 * (lo + hi);
  if (fabs(a - mid) > rel * a) return ph;
  return ph == lo ? hi : lo;
}

/* out_amb (NULL or [R][D]): alongside acc, the sum over keys whose 448 p is
 * that close to a rounding midpoint of its P format of
 * |other rounding - p^| * |v|, rescaled with acc -- the most a different
 * (equally valid) rounding of those keys can move acc.  It does not change
 * m, l or acc.
 * p_format: 0 = P not rounded (p^ = 448 p), 1 = E4M3 of 448 p (the method's
 * FP8 P), 2 = bf16 of 448 p (the BF16 P.V precision assignment), 3 = 448 x
 * the NVFP4 value of p (nvfp4_p_block; the NVFP4 P.V assignment).
 * amb_rel: the relative distance to a midpoint below which both roundings
 * count as valid (2^-16 for an FP32 exp2; wider for an approximate one).    */
void oracle_attn_state(int D, int R, const double* q, const int64_t* row_pos,
                       const double* k, const double* v, const double* delta,
                       int64_t kv_begin, int64_t kv_end, int block, double scale, int p_format,
                       double amb_rel, double* out_m, double* out_l, double* out_acc,
                       double* out_amb) {
  const double lam = scale / log(2.0);
  int r;
  init_tables();
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < R; ++r) {
    double m = -INFINITY, l = 0.0;
    double* acc = out_acc + (int64_t)r * D;
    double* amb = out_amb ? out_amb + (int64_t)r * D : NULL;
    double* s = (double*)malloc(sizeof(double) * (size_t)block);
    int64_t b0;
    int d;
    for (d = 0; d < D; ++d) acc[d] = 0.0;
    if (amb)
      for (d = 0; d < D; ++d) amb[d] = 0.0;
    for (b0 = kv_begin; b0 < kv_end; b0 += block) {
      int64_t b1 = b0 + block < kv_end ? b0 + block : kv_end;
      int64_t last = b1; /* exclusive end of visible keys in this block */
      int64_t j;
      double mb = -INFINITY, mn, alpha;
      if (row_pos[r] >= 0 && row_pos[r] + 1 < last) last = row_pos[r] + 1;
      if (last <= b0) break; /* blocks are ascending: nothing further is visible */
      for (j = b0; j < last; ++j) {
        double acc_s = 0.0;
        for (d = 0; d < D; ++d) acc_s += q[(int64_t)r * D + d] * k[j * D + d];
        if (delta) acc_s += delta[j];
        s[j - b0] = acc_s;
        if (acc_s > mb) mb = acc_s;
      }
      mn = m > mb ? m : mb;
      alpha = (m == -INFINITY) ? 0.0 : exp2(lam * (m - mn));
      l *= alpha;
      for (d = 0; d < D; ++d) acc[d] *= alpha;
      if (amb)
        for (d = 0; d < D; ++d) amb[d] *= alpha;
      if (p_format == 3) {
        int64_t g0;
        for (g0 = b0; g0 < last; g0 += 16) {
          const int n = (int)(last - g0 < 16 ? last - g0 : 16);
          float x[16];
          double ph[16], alt[16];
          int i;
          for (i = 0; i < 16; ++i) {
            const double p = i < n ? exp2(lam * (s[g0 + i - b0] - mn)) : 0.0;
            x[i] = (float)p;
            l += p;
          }
          nvfp4_p_block(x, amb_rel, ph, alt);
          for (i = 0; i < n; ++i) {
            for (d = 0; d < D; ++d) acc[d] += ph[i] * v[(g0 + i) * D + d];
            if (amb && alt[i] != ph[i])
              for (d = 0; d < D; ++d) amb[d] += fabs(alt[i] - ph[i]) * fabs(v[(g0 + i) * D + d]);
          }
        }
        m = mn;
        continue;
      }
      for (j = b0; j < last; ++j) {
        double p = exp2(lam * (s[j - b0] - mn));
        double ph = 448.0 * p, alt = ph;
        if (p_format == 1) {
          ph = oracle_e4m3_decode(oracle_e4m3_encode(448.0 * p));
          alt = e4m3_alternative(448.0 * p, ph, amb_rel);
        } else if (p_format == 2) {
          ph = bf16_round_pos(448.0 * p);
          alt = bf16_alternative(448.0 * p, ph, amb_rel);
        }
        l += p;
        for (d = 0; d < D; ++d) acc[d] += ph * v[j * D + d];
        if (amb && alt != ph)
          for (d = 0; d < D; ++d) amb[d] += fabs(alt - ph) * fabs(v[j * D + d]);
      }
      m = mn;
    }
    out_m[r] = m;
    out_l[r] = l;
    free(s);
  }
}

/* Log-sum-exp merge of P partial states per row (MpFA §5.3: local (m, l, O)
 * states of the KV partitions merged by log-sum-exp):
 *   m = max_p m_p;  w_p = 2^(lam (m_p - m));  l = sum w_p l_p;  acc = sum w_p acc_p
 * Partitions with m_p = -inf (no keys) contribute nothing.
 * m_in/l_in are [R][P], acc_in is [R][P][D].                                */
void oracle_merge_states(int D, int R, int P, const double* m_in, const double* l_in,
                         const double* acc_in, double scale, double* out_m, double* out_l,
                         double* out_acc) {
  const double lam = scale / log(2.0);
  int r;
  for (r = 0; r < R; ++r) {
    double m = -INFINITY, l = 0.0;
    int p, d;
    for (p = 0; p < P; ++p) if (m_in[r * P + p] > m) m = m_in[r * P + p];
    for (d = 0; d < D; ++d) out_acc[(int64_t)r * D + d] = 0.0;
    for (p = 0; p < P; ++p) {
      double w;
      if (m_in[r * P + p] == -INFINITY) continue;
      w = exp2(lam * (m_in[r * P + p] - m));
      l += w * l_in[r * P + p];
      for (d = 0; d < D; ++d)
        out_acc[(int64_t)r * D + d] += w * acc_in[((int64_t)r * P + p) * D + d];
    }
    out_m[r] = m;
    out_l[r] = l;
  }
}

/* ---------------------------------------------------- array conveniences -- */
void oracle_e4m3_encode_array(const double* x, int64_t n, uint8_t* out) {
  int64_t i;
  init_tables();
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_encode(x[i]);
}

void oracle_e2m1_encode_array(const double* x, int64_t n, uint8_t* out) {
  int64_t i;
  init_tables();
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_encode(x[i]);
}

void oracle_bf16_rne_array(const float* x, int64_t n, uint16_t* out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}
