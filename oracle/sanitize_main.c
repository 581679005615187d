/*
 * sanitize_main.c -- a standalone driver that runs every oracle entry point on
 * small seeded inputs, built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer by tests/test_oracle_sanitize.py (host code only; test
 * infrastructure like the oracle itself).  Buffers are allocated at their
 * exact sizes so any read or write past them is reported; every result is
 * also checked against a property that holds for it (round trip, sign of the
 * bound, zero rows).  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qblk_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static float weight(int r, int i) {
  switch (r % 4) {
    case 0: return (float)((uniform() - 0.5) * 0.08);
    case 1: return (float)((uniform() - 0.5) * 1e-6); /* fp16-subnormal scales */
    case 2: return 0.0f;                              /* all-zero rows */
    default: return (i % 32 == 0) ? 3.0f : (float)((uniform() - 0.5) * 0.02);
  }
}

static int fail(const char* what) {
  fprintf(stderr, "sanitize driver: %s\n", what);
  return 1;
}

int main(void) {
  const int64_t rows = 6, k = 512, n = 3;
  const int fmts[4] = {ORC_Q4_0, ORC_SB4, ORC_SB4_AFFINE, ORC_Q4_K};
  float* w = malloc(sizeof(float) * rows * k);
  uint16_t* w16 = malloc(sizeof(uint16_t) * rows * k);
  float* back = malloc(sizeof(float) * rows * k);
  double* x = malloc(sizeof(double) * k);
  double* X = malloc(sizeof(double) * n * k);
  double* y = malloc(sizeof(double) * rows);
  double* yb = malloc(sizeof(double) * rows);
  double* Y = malloc(sizeof(double) * n * rows);
  double* Yb = malloc(sizeof(double) * n * rows);
  if (!w || !w16 || !back || !x || !X || !y || !yb || !Y || !Yb) return fail("out of memory");
  for (int64_t r = 0; r < rows; r++)
    for (int64_t i = 0; i < k; i++) w[r * k + i] = weight((int)r, (int)i);
  for (int64_t i = 0; i < rows * k; i++) w16[i] = orc_f32_to_f16(w[i]);
  for (int64_t i = 0; i < k; i++) x[i] = uniform() - 0.5;
  for (int64_t i = 0; i < n * k; i++) X[i] = uniform() - 0.5;

  for (int f = 0; f < 4; f++) {
    const int fmt = fmts[f];
    const size_t nbytes = (size_t)(rows * (k / orc_block_elems(fmt)) * orc_block_bytes(fmt));
    uint8_t* b = malloc(nbytes);
    uint8_t* b2 = malloc(nbytes);
    if (!b || !b2) return fail("out of memory");
    for (int dt = 0; dt < 3; dt++) {
      const void* src = dt == ORC_F32 ? (const void*)w : (const void*)w16;
      if (dt == ORC_BF16) {
        for (int64_t i = 0; i < rows * k; i++) w16[i] = orc_f32_to_bf16(w[i]);
      } else if (dt == ORC_F16) {
        for (int64_t i = 0; i < rows * k; i++) w16[i] = orc_f32_to_f16(w[i]);
      }
      const int st = fmt == ORC_Q4_0   ? orc_quantize_q4_0(src, dt, rows, k, b)
                     : fmt == ORC_Q4_K ? orc_quantize_q4_k(src, dt, rows, k, b)
                                       : orc_quantize_sb4(src, dt, rows, k, fmt == ORC_SB4_AFFINE, b);
      if (st != 0) return fail("quantize failed");
    }
    if (orc_dequant(fmt, b, rows, k, back) != 0) return fail("dequant failed");
    for (int64_t i = 2 * k; i < 3 * k; i++)
      if (back[i] != 0.0f) return fail("an all-zero row did not rebuild to zeros");
    if (fmt == ORC_Q4_0) {
      /* quantizing the rebuilt values of normal-scale blocks gives the same bytes */
      if (orc_quantize_q4_0(back, ORC_F32, 1, k, b2) != 0) return fail("requantize failed");
      if (memcmp(b, b2, (size_t)(k / 32 * 18)) != 0) return fail("Q4_0 round trip changed row 0");
      if (orc_quantize_q4_0_ref(w, rows, k, b2) != 0) return fail("reference quantizer failed");
    }
    if (orc_gemv(fmt, b, rows, k, x, NULL, rows, y, yb) != 0) return fail("gemv failed");
    if (orc_gemm(fmt, b, rows, k, X, n, NULL, rows, Y, Yb) != 0) return fail("gemm failed");
    for (int64_t r = 0; r < rows; r++)
      if (!(yb[r] >= fabs(y[r]))) return fail("gemv bound below |y|");
    if (y[2] != 0.0 || yb[2] != 0.0) return fail("zero row gave a nonzero product");
    const int64_t sel[2] = {rows - 1, 0};
    if (orc_gemv(fmt, b, rows, k, x, sel, 2, y, yb) != 0) return fail("sampled gemv failed");
    free(b);
    free(b2);
  }
  {
    /* group-128 W4 weights (two planes at exact sizes) and int8 activations */
    const size_t wb = (size_t)(rows * k / 2 + rows * (k / 128) * 2);
    uint8_t* b = malloc(wb);
    int8_t* xq = malloc((size_t)(n * k));
    float* xs = malloc(sizeof(float) * (size_t)n);
    if (!b || !xq || !xs) return fail("out of memory");
    if (orc_quantize_w4g128(w, ORC_F32, rows, k, b) != 0) return fail("quantize_w4g128 failed");
    if (orc_quantize_w4g128(w16, ORC_F16, rows, k, b) != 0) return fail("quantize_w4g128 f16 failed");
    if (orc_dequant(ORC_W4G128, b, rows, k, back) != 0) return fail("w4g128 dequant failed");
    float* Xf = malloc(sizeof(float) * (size_t)(n * k));
    if (!Xf) return fail("out of memory");
    for (int64_t i = 0; i < n * k; i++) Xf[i] = (float)X[i];
    if (orc_quantize_act_i8(Xf, ORC_F32, n, k, xq, xs) != 0) return fail("quantize_act_i8 failed");
    if (orc_gemm_w4a8(b, rows, k, xq, xs, n, NULL, rows, Y, Yb) != 0) return fail("gemm_w4a8 failed");
    const int64_t sel[2] = {rows - 1, 1};
    if (orc_gemm_w4a8(b, rows, k, xq, xs, n, sel, 2, Y, Yb) != 0) return fail("sampled gemm_w4a8 failed");
    if (orc_gemv(ORC_W4G128, b, rows, k, x, NULL, rows, y, yb) != 0) return fail("w4g128 gemv failed");
    free(Xf);
    free(b);
    free(xq);
    free(xs);
  }
  {
    const float s[8] = {0.10f, 0.14f, 0.11f, 0.18f, 0.08f, 0.16f, 0.13f, 0.09f};
    int8_t codes[8];
    uint16_t S16 = 0;
    float S_used = 0.0f;
    if (orc_meta_int8(s, 8, 0.0f, codes, &S16, &S_used) != 0) return fail("meta_int8 failed");
    if (orc_meta_int8(s, 8, 0.00142f, codes, &S16, &S_used) != 0) return fail("meta_int8 (forced) failed");
  }
  for (uint32_t u = 0; u < 65536; u++) {
    const float v = orc_f16_to_f32((uint16_t)u);
    if (v == v && orc_f32_to_f16(v) != (uint16_t)u) return fail("fp16 round trip");
    (void)orc_bf16_to_f32((uint16_t)u);
    (void)orc_rha(v);
  }
  free(w);
  free(w16);
  free(back);
  free(x);
  free(X);
  free(y);
  free(yb);
  free(Y);
  free(Yb);
  puts("sanitize driver: clean");
  return 0;
}
