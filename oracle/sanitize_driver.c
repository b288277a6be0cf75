/*
 * sanitize_driver.c -- TEST INFRASTRUCTURE ONLY.  A standalone program that
 * links mpfa_oracle.c and calls every function it exports on small inputs,
 * edge cases included (one token, one row, ragged key blocks, empty key
 * ranges, zero tensors, signed zeros, saturating values), so that the oracle
 * can be built and run under AddressSanitizer and UndefinedBehaviorSanitizer
 * on the host.  Besides the sanitizers' own checks it verifies a few closed-
 * form facts (codec round trips, the mean of a constant, a one-key attention
 * state) and exits non-zero if one fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1_decode(int code);
double oracle_e4m3_decode(int code);
int oracle_e2m1_encode(double x);
int oracle_e4m3_encode(double x);
uint16_t oracle_bf16_rne(float x);
double oracle_bf16_decode(uint16_t h);
void oracle_channel_mean(const float* x, int64_t T, int D, float* out);
float oracle_amax(const float* x, int64_t n);
float oracle_nvfp4_global_scale(float amax);
void oracle_nvfp4_quantize(const float* x, int64_t rows, int D, float g, uint8_t* codes,
                           uint8_t* sf);
void oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* sf, int64_t rows, int D,
                             float g, double* out);
float oracle_fp8_scale(float amax);
void oracle_fp8_quantize(const float* x, int64_t n, float s, uint8_t* codes);
void oracle_delta_s(const float* qmean, const float* kc, int64_t T, int D, uint16_t* out);
void oracle_attn_state(int D, int R, const double* q, const int64_t* row_pos, const double* k,
                       const double* v, const double* delta, int64_t kv_begin, int64_t kv_end,
                       int block, double scale, int p_format, double amb_rel, double* out_m,
                       double* out_l, double* out_acc, double* out_amb);
void oracle_merge_states(int D, int R, int P, const double* m_in, const double* l_in,
                         const double* acc_in, double scale, double* out_m, double* out_l,
                         double* out_acc);
void oracle_e4m3_encode_array(const double* x, int64_t n, uint8_t* out);
void oracle_e2m1_encode_array(const double* x, int64_t n, uint8_t* out);
void oracle_bf16_rne_array(const float* x, int64_t n, uint16_t* out);

static int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

/* xorshift64* test data: deterministic, not part of the method */
static uint64_t rs = 0x9E3779B97F4A7C15ull;
static double urand(void) {
  rs ^= rs >> 12;
  rs ^= rs << 25;
  rs ^= rs >> 27;
  return (double)((rs * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void) { /* sum of uniforms: bounded, roughly normal */
  double s = 0.0;
  int i;
  for (i = 0; i < 12; ++i) s += urand();
  return s - 6.0;
}

static void codecs(void) {
  int c;
  for (c = 0; c < 16; ++c) {
    const double v = oracle_e2m1_decode(c);
    CHECK(oracle_e2m1_encode(v) == c, "e2m1 round trip of code %d", c);
  }
  for (c = 0; c < 256; ++c) {
    const double v = oracle_e4m3_decode(c);
    if ((c & 0x7F) == 0x7F) {
      CHECK(isnan(v), "e4m3 code %d is NaN", c);
      continue;
    }
    CHECK(oracle_e4m3_encode(v) == c, "e4m3 round trip of code %d", c);
  }
  {
    const double odd[] = {0.0, -0.0, 1e-300, -1e-300, 1e300, -1e300, INFINITY, -INFINITY, NAN,
                          0.25, 0.75, 5.0, 7.0, 464.0, 480.0, -1e-9};
    double arr[sizeof(odd) / sizeof(odd[0])];
    uint8_t o1[sizeof(odd) / sizeof(odd[0])], o2[sizeof(odd) / sizeof(odd[0])];
    const int n = (int)(sizeof(odd) / sizeof(odd[0]));
    int i;
    for (i = 0; i < n; ++i) {
      arr[i] = odd[i];
      (void)oracle_e2m1_encode(odd[i]);
      (void)oracle_e4m3_encode(odd[i]);
    }
    oracle_e4m3_encode_array(arr, n, o1);
    oracle_e2m1_encode_array(arr, n, o2);
    CHECK(o1[6] == 0x7E && o1[7] == 0xFE, "e4m3 saturates +-inf");
    CHECK(o2[1] == 8, "e2m1 keeps the sign of -0");
  }
  {
    const float f[] = {0.0f, -0.0f, 1.0f, 1.00390625f, 1.01171875f, 3.4e38f, -3.4e38f, 1e-40f,
                       -2.5f, 65504.0f};
    uint16_t h[10];
    int i;
    oracle_bf16_rne_array(f, 10, h);
    for (i = 0; i < 10; ++i) CHECK(h[i] == oracle_bf16_rne(f[i]), "bf16 array entry %d", i);
    CHECK(oracle_bf16_decode(h[3]) == 1.0, "bf16 tie 1 + 2^-8 rounds to even (1)");
    CHECK(oracle_bf16_decode(h[4]) == 1.015625, "bf16 tie 1 + 3*2^-8 rounds to even");
  }
}

static void statistics(void) {
  const int D = 128;
  int64_t T;
  for (T = 1; T <= 300; T += 299) {
    float* x = (float*)malloc(sizeof(float) * (size_t)(T * D));
    float mean[128];
    int64_t i;
    int d;
    for (i = 0; i < T * D; ++i) x[i] = (float)(0.75 * (double)((i % D) - 64) / 8.0);
    oracle_channel_mean(x, T, D, mean);
    for (d = 0; d < D; ++d) CHECK(mean[d] == x[d], "mean of a constant channel %d (T=%lld)", d,
                                  (long long)T);
    for (i = 0; i < T * D; ++i) x[i] = (float)nrand();
    oracle_channel_mean(x, T, D, mean);
    CHECK(oracle_amax(x, T * D) >= 0.0f, "amax");
    memset(x, 0, sizeof(float) * (size_t)(T * D));
    oracle_channel_mean(x, T, D, mean);
    for (d = 0; d < D; ++d) CHECK(mean[d] == 0.0f, "mean of zeros");
    CHECK(oracle_amax(x, T * D) == 0.0f, "amax of zeros");
    free(x);
  }
  CHECK(oracle_nvfp4_global_scale(0.0f) == 1.0f, "global scale of a zero tensor");
  CHECK(oracle_fp8_scale(0.0f) == 1.0f, "fp8 scale of a zero tensor");
}

static void quantizers(void) {
  const int D = 128;
  int64_t rows;
  for (rows = 1; rows <= 37; rows += 36) {
    float* x = (float*)malloc(sizeof(float) * (size_t)(rows * D));
    uint8_t* codes = (uint8_t*)malloc((size_t)(rows * D / 2));
    uint8_t* sf = (uint8_t*)malloc((size_t)(rows * D / 16));
    uint8_t* v8 = (uint8_t*)malloc((size_t)(rows * D));
    double* back = (double*)malloc(sizeof(double) * (size_t)(rows * D));
    uint16_t* delta = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)rows);
    float qmean[128];
    int64_t i;
    float g;
    for (i = 0; i < rows * D; ++i) x[i] = (float)(nrand() * (i % 17 == 0 ? 40.0 : 1.0));
    x[0] = -0.0f;
    for (i = 0; i < D; ++i) qmean[i] = (float)(0.1 * nrand());
    g = oracle_nvfp4_global_scale(oracle_amax(x, rows * D));
    oracle_nvfp4_quantize(x, rows, D, g, codes, sf);
    oracle_nvfp4_dequantize(codes, sf, rows, D, g, back);
    for (i = 0; i < rows * D; ++i) CHECK(isfinite(back[i]), "NVFP4 value finite");
    oracle_fp8_quantize(x, rows * D, oracle_fp8_scale(oracle_amax(x, rows * D)), v8);
    oracle_delta_s(qmean, x, rows, D, delta);
    /* a block of zeros: zero scale, signed-zero codes */
    memset(x, 0, sizeof(float) * (size_t)(rows * D));
    x[1] = -0.0f;
    oracle_nvfp4_quantize(x, rows, D, 1.0f, codes, sf);
    CHECK(sf[0] == 0 && (codes[0] >> 4) == 8, "zero block: zero scale, -0 keeps its sign");
    free(x);
    free(codes);
    free(sf);
    free(v8);
    free(back);
    free(delta);
  }
}

static void attention(void) {
  const int D = 128;
  const int64_t N = 300; /* two full 128-key blocks and a ragged one */
  double* k = (double*)malloc(sizeof(double) * (size_t)(N * D));
  double* v = (double*)malloc(sizeof(double) * (size_t)(N * D));
  double* delta = (double*)malloc(sizeof(double) * (size_t)N);
  const int R = 5;
  double q[5 * 128];
  int64_t pos[5] = {0, 127, 128, 299, -1};
  double m[5], l[5], acc[5 * 128], amb[5 * 128];
  int64_t i;
  int fmt, r, d;
  for (i = 0; i < N * D; ++i) {
    k[i] = nrand();
    v[i] = nrand();
  }
  for (i = 0; i < N; ++i) delta[i] = 0.1 * nrand();
  for (i = 0; i < R * D; ++i) q[i] = nrand();
  for (fmt = 0; fmt <= 3; ++fmt) {
    oracle_attn_state(D, R, q, pos, k, v, delta, 0, N, 128, 0.0883883476, fmt, 0x1p-16, m, l,
                      acc, amb);
    for (r = 0; r < R; ++r) CHECK(isfinite(m[r]) && l[r] >= 1.0, "state of row %d", r);
    oracle_attn_state(D, R, q, pos, k, v, NULL, 7, N, 128, 0.0883883476, fmt, 0x1p-13, m, l,
                      acc, NULL);
  }
  /* empty key range and a row that sees no key */
  oracle_attn_state(D, R, q, pos, k, v, delta, 5, 5, 128, 0.1, 1, 0x1p-16, m, l, acc, amb);
  for (r = 0; r < R; ++r) CHECK(m[r] == -INFINITY && l[r] == 0.0, "empty range row %d", r);
  /* one visible key: l = 1 and acc = 448 v0 exactly without P rounding */
  oracle_attn_state(D, 1, q, pos, k, v, NULL, 0, N, 128, 0.1, 0, 0x1p-16, m, l, acc, NULL);
  CHECK(l[0] == 1.0, "one key: l = 1");
  for (d = 0; d < D; ++d) CHECK(acc[d] == 448.0 * v[d], "one key: acc = 448 v");
  {
    /* merge: three partitions, one of them empty */
    const int P = 3;
    double mi[2 * 3], li[2 * 3], ai[2 * 3 * 128], mo[2], lo[2], ao[2 * 128];
    for (i = 0; i < 2 * P; ++i) {
      mi[i] = (i % P == 1) ? -INFINITY : nrand();
      li[i] = (i % P == 1) ? 0.0 : 1.0 + urand();
    }
    for (i = 0; i < 2 * P * D; ++i) ai[i] = nrand();
    oracle_merge_states(D, 2, P, mi, li, ai, 0.1, mo, lo, ao);
    for (r = 0; r < 2; ++r) CHECK(isfinite(mo[r]) && lo[r] > 0.0, "merged row %d", r);
  }
  free(k);
  free(v);
  free(delta);
}

int main(void) {
  codecs();
  statistics();
  quantizers();
  attention();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: all calls completed, all checks passed\n");
  return 0;
}
