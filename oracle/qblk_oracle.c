/*
 * qblk_oracle.c -- the CPU oracle: the block formats and their products
 * written out as the pages define them, one weight at a time.
 *
 * TEST INFRASTRUCTURE ONLY (see qblk_oracle.h).  Build:
 *   gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fexcess-precision=standard
 *       -fPIC -shared qblk_oracle.c -o libqblk_oracle.so -lm
 * x86-64 evaluates float in SSE registers, so every float operation below is
 * one IEEE-754 binary32 operation rounded to nearest even.
 *
 * Readings taken where the pages leave a step open (each is listed, with its
 * reason, in the design notes of the repository):
 *   R1  Q4_0 scale d = absmax/7, code = clamp(rha(w/d), -8, 7) + 8 (the
 *       global-scale rule of [Q40] 4.1.1 applied per 32-block).
 *   R2  codes are computed against the STORED (fp16-rounded) scale.
 *   R4  ties round away from zero; R5 true IEEE division, not reciprocal.
 *   R6  a zero scale gives quotient 0.
 *   R7  fp16 rounding is round-to-nearest-even with subnormals kept.
 *   R8  super-block field order [S16][sc x8][qs x128] (Type 0) and
 *       [Ss16][Sa16][sc x8][ac x8][qs x128] (Type 1), little-endian.
 *   R9  inside a super-block, sub-block j owns qs[16j .. 16j+15], split
 *       lo/hi as in a Q4_0 block.
 *   R10 Type 0 stores n = q+8; Type 1 stores n = q in [0, 15].
 *   R11 the scales that enter the meta step are the fp16-rounded ones.
 *   R12 4-bit codes use the first-level fp16 scales, not the INT8-rebuilt ones.
 *   R13 Type 1 offsets alpha are meta-quantized symmetrically under their own
 *       fp16 super-offset max|alpha|/127.
 *   R14 dequant operation order: (S*sc)*(n-8) for Type 0 and
 *       (Ss*sc)*n + (Sa*ac) for Type 1, no fused multiply-add.
 *   R23 Q4_K field order [d16][dmin16][12 bytes of 6-bit fields][qs x128]
 *       (144 bytes); field i (s_0..s_7, then m_0..m_7) occupies bits
 *       6i..6i+5 of the 96-bit little-endian integer in bytes 4..15.
 *   R24 Q4_K sub-block range: lo = min(0, min w), hi = max w; first-level
 *       scale (hi - lo)/15 and min -lo (>= 0, so m_j is unsigned), in fp32.
 *   R25 Q4_K second level: d = fp16(max scale / 63), dmin = fp16(max min / 63);
 *       6-bit codes clamp(rha(v / stored), 0, 63).
 *   R26 Q4_K 4-bit codes against the rebuilt S_j = d*s_j and M_j = dmin*m_j:
 *       clamp(rha((w + M_j) / S_j), 0, 15).
 *   R27 Q4_K dequant fl(S_j*q - M_j) (S_j*q and M_j are exact in fp32).
 *   R28 group-128 W4 layout (the TurboQuant article gives none): planar, the
 *       code plane (rows x k/2 bytes; byte j of group g holds weight 128g+j
 *       in its low nibble and weight 128g+64+j in its high nibble) followed
 *       by the fp16 scale plane (rows x k/128, row-major).
 *   R29 group-128 W4 rule: symmetric, d = fp16(absmax/7) per group, code
 *       clamp(rha(w/d), -8, 7) stored +8 (R1 with groups of 128).
 *   R30 8-bit activations: one symmetric scale per token (row of X),
 *       s = absmax/127 kept in fp32, codes clamp(rha(x/s), -127, 127).
 *   R31 the W4A8 product is that of the rebuilt weights and the rebuilt
 *       activations s*xq (fp64 sums here).
 */
#include "qblk_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* fp16 bits -> value.  IEEE binary16: 1 sign, 5 exponent (bias 15), 10
 * fraction bits; exponent 0 holds subnormals f * 2^-24.  The Q4_0 chapter
 * (4.1.2) stores the scale as this bit pattern, little-endian. */
float orc_f16_to_f32(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 10) & 0x1F;
  int frac = bits & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)frac, -24);
  else if (e == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + frac), e - 25);
  return (float)(sign ? -v : v);
}

/* value -> fp16 bits, round to nearest, ties to even, subnormals kept,
 * overflow to infinity.  Written on magnitudes: a normal result is
 * (1 + f/1024) * 2^E, a subnormal one is f * 2^-24. */
uint16_t orc_f32_to_f16(float v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return (uint16_t)(sign | 0x7E00);
  if (isinf(v)) return (uint16_t)(sign | 0x7C00);
  double a = fabs((double)v);
  if (a < 0x1p-14) {
    /* multiples of 2^-24; the product is exact in double and nearbyint
     * rounds ties to even.  q == 1024 is exactly the smallest normal,
     * whose encoding is the same integer. */
    double q = nearbyint(a * 0x1p24);
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  double q = nearbyint(m * 2048.0); /* 11 significant bits, in [1024, 2048] */
  int E = e - 1;
  if (q == 2048.0) {
    q = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* bfloat16 is the upper half of a binary32 pattern. */
float orc_bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float v;
  memcpy(&v, &u, 4);
  return v;
}

/* value -> bf16 bits, nearest-even, 8 significant bits, fp32's exponent
 * range (subnormals are multiples of 2^-133). */
uint16_t orc_f32_to_bf16(float v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0);
  if (isinf(v)) return (uint16_t)(sign | 0x7F80);
  double a = fabs((double)v);
  if (a < 0x1p-126) {
    double q = nearbyint(a * 0x1p133);
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  double m = frexp(a, &e);
  double q = nearbyint(m * 256.0); /* in [128, 256] */
  int E = e - 1;
  if (q == 256.0) {
    q = 128.0;
    E += 1;
  }
  if (E > 127) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(q - 128.0));
}

/* round half away from zero: C99 roundf is exactly this operation. */
float orc_rha(float v) { return roundf(v); }

static float qdiv(float v, float s) { return s == 0.0f ? 0.0f : v / s; }

/* clamp a rounded quotient into [lo, hi] (NaN, never produced for finite
 * inputs with finite scales, lands on lo). */
static int clamp_code(float v, int lo, int hi) {
  if (!(v >= (float)lo)) return lo;
  if (v > (float)hi) return hi;
  return (int)v;
}

static float load_elem(const void* w, int dtype, int64_t i) {
  if (dtype == ORC_F32) return ((const float*)w)[i];
  if (dtype == ORC_F16) return orc_f16_to_f32(((const uint16_t*)w)[i]);
  return orc_bf16_to_f32(((const uint16_t*)w)[i]);
}

static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t* p) {
  return (uint16_t)(p[0] | (p[1] << 8));
}

int orc_block_elems(int fmt) {
  if (fmt == ORC_Q4_0) return 32;
  if (fmt == ORC_W4G128) return 128;
  if (fmt == ORC_SB4 || fmt == ORC_SB4_AFFINE || fmt == ORC_Q4_K) return 256;
  return 0;
}

/* Q4_0: 2-byte scale + 16 bytes of codes ([Q40] 4.1.2).  Super-block:
 * 8 x 8-bit sub-scales + one 16-bit super-scale in place of eight 16-bit
 * scales ([KQ] storage table), i.e. 10 + 128 bytes; Type 1 adds another
 * 8 + 2 bytes for the offsets. */
int orc_block_bytes(int fmt) {
  if (fmt == ORC_Q4_0) return 2 + 32 / 2;
  if (fmt == ORC_SB4) return 2 + 8 + 256 / 2;
  if (fmt == ORC_SB4_AFFINE) return 2 + 2 + 8 + 8 + 256 / 2;
  /* Q4_K: fp16 d and dmin, 16 six-bit fields (96 bits), 128 bytes of codes */
  if (fmt == ORC_Q4_K) return 2 + 2 + 16 * 6 / 8 + 256 / 2;
  /* group-128 W4: 64 code bytes and one fp16 scale, in two planes (R28) */
  if (fmt == ORC_W4G128) return 128 / 2 + 2;
  return 0;
}

/* ------------------------------------------------------------------ */
/* [KQ] "套娃": quantize a handful of scale values to INT8.           */
/* ------------------------------------------------------------------ */
int orc_meta_int8(const float* s, int n, float S_forced, int8_t* codes,
                  uint16_t* S16, float* S_used) {
  if (!s || !codes || n < 1) return -1;
  /* step 1: the largest magnitude fixes the symmetric interval [-d, d] */
  float d = 0.0f;
  for (int i = 0; i < n; i++)
    if (fabsf(s[i]) > d) d = fabsf(s[i]);
  /* step 2: INT8 levels -127 .. +127 (254 intervals), zero in the middle */
  const int lo = -127, hi = 127;
  /* step 3: the super-scale is the interval width over the level span */
  float S = (d - (-d)) / (float)(hi - lo);
  float Su;
  uint16_t Sb = 0;
  if (S_forced > 0.0f) {
    Su = S_forced;
  } else {
    Sb = orc_f32_to_f16(S); /* stored as FP16 */
    Su = orc_f16_to_f32(Sb);
  }
  /* step 4: each scale divided by the super-scale, rounded, kept in range */
  for (int i = 0; i < n; i++)
    codes[i] = (int8_t)clamp_code(orc_rha(qdiv(s[i], Su)), lo, hi);
  if (S16) *S16 = Sb;
  if (S_used) *S_used = Su;
  return 0;
}

/* ------------------------------------------------------------------ */
/* Q4_0 block (reading R1-R2)                                          */
/* ------------------------------------------------------------------ */

/* One block of 32 weights -> the fp16 scale and 32 codes n in [0, 15]. */
static uint16_t q4_0_codes(const float* w, uint8_t* n) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++)
    if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
  /* signed range [-8, 7]: the largest magnitude maps to 7 */
  uint16_t d16 = orc_f32_to_f16(amax / 7.0f);
  float d = orc_f16_to_f32(d16);
  for (int i = 0; i < 32; i++) {
    int q = clamp_code(orc_rha(qdiv(w[i], d)), -8, 7);
    n[i] = (uint8_t)(q + 8); /* stored unsigned, zero point 8 ([Q40] 4.2.2) */
  }
  return d16;
}

/* [Q40] 4.2.1: byte j carries weight j in its low nibble and weight j+16 in
 * its high nibble. */
static void pack_nibbles(const uint8_t* n, uint8_t* qs) {
  for (int j = 0; j < 16; j++) qs[j] = (uint8_t)(n[j] | (n[j + 16] << 4));
}

int orc_quantize_q4_0(const void* w, int dtype, int64_t rows, int64_t k,
                      uint8_t* out) {
  if (!w || !out || rows < 0 || k < 0 || k % 32 != 0) return -1;
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -1;
  const int64_t nb = k / 32;
  float buf[32];
  uint8_t n[32];
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      for (int i = 0; i < 32; i++) buf[i] = load_elem(w, dtype, r * k + b * 32 + i);
      uint8_t* blk = out + (r * nb + b) * 18;
      put_u16(blk, q4_0_codes(buf, n));
      pack_nibbles(n, blk + 2);
    }
  return 0;
}

/* [Q40] 4.4: the scale is the signed value of largest magnitude (first one
 * met when several tie) divided by -8, so that value lands on code 0; codes
 * are the product with the fp32 reciprocal, shifted by 8.5, truncated and
 * capped at 15. */
int orc_quantize_q4_0_ref(const float* w, int64_t rows, int64_t k,
                          uint8_t* out) {
  if (!w || !out || rows < 0 || k < 0 || k % 32 != 0) return -1;
  const int64_t nb = k / 32;
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      const float* x = w + r * k + b * 32;
      float amax = 0.0f, extreme = 0.0f;
      for (int i = 0; i < 32; i++)
        if (fabsf(x[i]) > amax) {
          amax = fabsf(x[i]);
          extreme = x[i];
        }
      float d = extreme / -8.0f;
      float inv = (d != 0.0f) ? 1.0f / d : 0.0f;
      uint8_t n[32];
      for (int i = 0; i < 32; i++) {
        float t = x[i] * inv + 8.5f;
        int c = (int)t; /* truncation toward zero; t >= 0 here */
        n[i] = (uint8_t)(c < 15 ? c : 15);
      }
      uint8_t* blk = out + (r * nb + b) * 18;
      put_u16(blk, orc_f32_to_f16(d));
      pack_nibbles(n, blk + 2);
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* super-blocks                                                        */
/* ------------------------------------------------------------------ */

/* Type 0 ([KQ] "套娃"): eight Q4_0 sub-blocks whose fp16 scales are then
 * quantized to INT8 under one fp16 super-scale. */
static void sb4_type0(const float* w, uint8_t* blk) {
  float s[8];
  uint8_t n[32];
  for (int j = 0; j < 8; j++) {
    uint16_t d16 = q4_0_codes(w + 32 * j, n);
    s[j] = orc_f16_to_f32(d16);
    pack_nibbles(n, blk + 10 + 16 * j);
  }
  int8_t sc[8];
  uint16_t S16;
  orc_meta_int8(s, 8, 0.0f, sc, &S16, NULL);
  put_u16(blk, S16);
  memcpy(blk + 2, sc, 8);
}

/* Type 1 (affine): per sub-block scale (max-min)/15 and offset min, codes
 * 0..15; the eight scales and the eight offsets are each meta-quantized. */
static void sb4_type1(const float* w, uint8_t* blk) {
  float s[8], a[8];
  uint8_t n[32];
  for (int j = 0; j < 8; j++) {
    const float* x = w + 32 * j;
    float mn = x[0], mx = x[0];
    for (int i = 1; i < 32; i++) {
      if (x[i] < mn) mn = x[i];
      if (x[i] > mx) mx = x[i];
    }
    s[j] = orc_f16_to_f32(orc_f32_to_f16((mx - mn) / 15.0f));
    a[j] = orc_f16_to_f32(orc_f32_to_f16(mn));
    for (int i = 0; i < 32; i++)
      n[i] = (uint8_t)clamp_code(orc_rha(qdiv(x[i] - a[j], s[j])), 0, 15);
    pack_nibbles(n, blk + 20 + 16 * j);
  }
  int8_t sc[8], ac[8];
  uint16_t Ss16, Sa16;
  orc_meta_int8(s, 8, 0.0f, sc, &Ss16, NULL);
  orc_meta_int8(a, 8, 0.0f, ac, &Sa16, NULL);
  put_u16(blk, Ss16);
  put_u16(blk + 2, Sa16);
  memcpy(blk + 4, sc, 8);
  memcpy(blk + 12, ac, 8);
}

int orc_quantize_sb4(const void* w, int dtype, int64_t rows, int64_t k,
                     int affine, uint8_t* out) {
  if (!w || !out || rows < 0 || k < 0 || k % 256 != 0) return -1;
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -1;
  const int64_t nb = k / 256;
  const int bytes = affine ? 148 : 138;
  float buf[256];
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      for (int i = 0; i < 256; i++) buf[i] = load_elem(w, dtype, r * k + b * 256 + i);
      uint8_t* blk = out + (r * nb + b) * bytes;
      if (affine)
        sb4_type1(buf, blk);
      else
        sb4_type0(buf, blk);
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Q4_K form ([Q40] 4.6): one fp16 scale d and one fp16 min-scale dmin */
/* per super-block, a 6-bit scale s_j and a 6-bit min m_j per 32-weight */
/* sub-block; a weight is d*s_j*q - dmin*m_j with q in [0, 15].         */
/* The page names the 6-bit packing without describing it (R23).        */
/* ------------------------------------------------------------------ */
static void put_field6(uint8_t* f, int i, int v) {
  for (int b = 0; b < 6; b++)
    if ((v >> b) & 1) f[(6 * i + b) / 8] |= (uint8_t)(1u << ((6 * i + b) % 8));
}
static int get_field6(const uint8_t* f, int i) {
  int v = 0;
  for (int b = 0; b < 6; b++) v |= ((f[(6 * i + b) / 8] >> ((6 * i + b) % 8)) & 1) << b;
  return v;
}

static void q4_k_superblock(const float* w, uint8_t* blk) {
  float sc[8], mn[8];
  float smax = 0.0f, mmax = 0.0f;
  for (int j = 0; j < 8; j++) {
    const float* x = w + 32 * j;
    float lo = 0.0f, hi = x[0]; /* R24: the range always reaches down to 0 */
    for (int i = 0; i < 32; i++) {
      if (x[i] < lo) lo = x[i];
      if (x[i] > hi) hi = x[i];
    }
    sc[j] = (hi - lo) / 15.0f; /* 16 levels, 15 steps */
    mn[j] = -lo;
    if (sc[j] > smax) smax = sc[j];
    if (mn[j] > mmax) mmax = mn[j];
  }
  /* R25: the largest scale and the largest min map to the 6-bit top, 63 */
  const uint16_t d16 = orc_f32_to_f16(smax / 63.0f);
  const uint16_t m16 = orc_f32_to_f16(mmax / 63.0f);
  const float D = orc_f16_to_f32(d16), Dm = orc_f16_to_f32(m16);
  put_u16(blk, d16);
  put_u16(blk + 2, m16);
  memset(blk + 4, 0, 12);
  for (int j = 0; j < 8; j++) {
    const int s6 = clamp_code(orc_rha(qdiv(sc[j], D)), 0, 63);
    const int m6 = clamp_code(orc_rha(qdiv(mn[j], Dm)), 0, 63);
    put_field6(blk + 4, j, s6);
    put_field6(blk + 4, 8 + j, m6);
    /* R26: codes against the values the block rebuilds */
    const float S = D * (float)s6, M = Dm * (float)m6;
    uint8_t n[32];
    for (int i = 0; i < 32; i++)
      n[i] = (uint8_t)clamp_code(orc_rha(qdiv(w[32 * j + i] + M, S)), 0, 15);
    pack_nibbles(n, blk + 16 + 16 * j);
  }
}

int orc_quantize_q4_k(const void* w, int dtype, int64_t rows, int64_t k,
                      uint8_t* out) {
  if (!w || !out || rows < 0 || k < 0 || k % 256 != 0) return -1;
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -1;
  const int64_t nb = k / 256;
  float buf[256];
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      for (int i = 0; i < 256; i++) buf[i] = load_elem(w, dtype, r * k + b * 256 + i);
      q4_k_superblock(buf, out + (r * nb + b) * 144);
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Group-128 W4 weights with 8-bit activations (TurboQuant article,    */
/* sections 2.1-2.2): per row, groups of 128 weights share one scale   */
/* from their own maximum and map to 4-bit integers; activations are  */
/* 8-bit.  Readings R28-R31.                                           */
/* ------------------------------------------------------------------ */
int orc_quantize_w4g128(const void* w, int dtype, int64_t rows, int64_t k,
                        uint8_t* out) {
  if (!w || !out || rows < 0 || k < 0 || k % 128 != 0) return -1;
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -1;
  const int64_t ng = k / 128;
  uint8_t* scales = out + rows * (k / 2);
  for (int64_t r = 0; r < rows; r++)
    for (int64_t g = 0; g < ng; g++) {
      float x[128];
      float amax = 0.0f;
      for (int i = 0; i < 128; i++) {
        x[i] = load_elem(w, dtype, r * k + g * 128 + i);
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
      }
      /* symmetric: the largest magnitude maps to 7, the codes span [-8, 7] */
      const uint16_t d16 = orc_f32_to_f16(amax / 7.0f);
      const float d = orc_f16_to_f32(d16);
      uint8_t* qs = out + r * (k / 2) + g * 64;
      for (int j = 0; j < 64; j++) {
        const int lo = clamp_code(orc_rha(qdiv(x[j], d)), -8, 7) + 8;
        const int hi = clamp_code(orc_rha(qdiv(x[64 + j], d)), -8, 7) + 8;
        qs[j] = (uint8_t)(lo | (hi << 4));
      }
      put_u16(scales + (r * ng + g) * 2, d16);
    }
  return 0;
}

int orc_quantize_act_i8(const void* x, int dtype, int64_t n, int64_t k,
                        int8_t* xq, float* scale) {
  if (!x || !xq || !scale || n < 0 || k < 0) return -1;
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -1;
  for (int64_t t = 0; t < n; t++) {
    float amax = 0.0f;
    for (int64_t i = 0; i < k; i++) {
      const float v = fabsf(load_elem(x, dtype, t * k + i));
      if (v > amax) amax = v;
    }
    const float s = amax / 127.0f; /* INT8 levels -127 .. 127 */
    for (int64_t i = 0; i < k; i++)
      xq[t * k + i] = (int8_t)clamp_code(orc_rha(qdiv(load_elem(x, dtype, t * k + i), s)), -127, 127);
    scale[t] = s;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* dequantization                                                      */
/* ------------------------------------------------------------------ */

/* code of weight i (0..31) inside a 16-byte nibble group */
static int nib(const uint8_t* qs, int i) {
  return i < 16 ? (qs[i] & 0x0F) : ((qs[i - 16] >> 4) & 0x0F);
}

static int64_t row_bytes(int fmt, int64_t k);

/* row r of an m x k packed matrix -> k fp32 values */
static void dequant_row(int fmt, const uint8_t* blocks, int64_t m, int64_t k,
                        int64_t r, float* y) {
  const uint8_t* row = blocks + r * row_bytes(fmt, k);
  if (fmt == ORC_W4G128) {
    const uint8_t* codes = blocks + r * (k / 2);
    const uint8_t* scales = blocks + m * (k / 2) + r * (k / 128) * 2;
    for (int64_t g = 0; g < k / 128; g++) {
      const float d = orc_f16_to_f32(get_u16(scales + 2 * g));
      for (int j = 0; j < 64; j++) {
        const uint8_t b = codes[g * 64 + j];
        y[g * 128 + j] = d * (float)((b & 0x0F) - 8);
        y[g * 128 + 64 + j] = d * (float)((b >> 4) - 8);
      }
    }
  } else if (fmt == ORC_Q4_0) {
    for (int64_t b = 0; b < k / 32; b++) {
      const uint8_t* blk = row + b * 18;
      float d = orc_f16_to_f32(get_u16(blk));
      for (int i = 0; i < 32; i++) y[b * 32 + i] = d * (float)(nib(blk + 2, i) - 8);
    }
  } else if (fmt == ORC_SB4) {
    for (int64_t b = 0; b < k / 256; b++) {
      const uint8_t* blk = row + b * 138;
      float S = orc_f16_to_f32(get_u16(blk));
      for (int j = 0; j < 8; j++) {
        float sj = S * (float)(int8_t)blk[2 + j]; /* rebuilt sub-scale */
        for (int i = 0; i < 32; i++)
          y[b * 256 + 32 * j + i] = sj * (float)(nib(blk + 10 + 16 * j, i) - 8);
      }
    }
  } else if (fmt == ORC_Q4_K) {
    for (int64_t b = 0; b < k / 256; b++) {
      const uint8_t* blk = row + b * 144;
      float D = orc_f16_to_f32(get_u16(blk));
      float Dm = orc_f16_to_f32(get_u16(blk + 2));
      for (int j = 0; j < 8; j++) {
        float S = D * (float)get_field6(blk + 4, j);
        float M = Dm * (float)get_field6(blk + 4, 8 + j);
        for (int i = 0; i < 32; i++) {
          float t = S * (float)nib(blk + 16 + 16 * j, i);
          y[b * 256 + 32 * j + i] = t - M;
        }
      }
    }
  } else {
    for (int64_t b = 0; b < k / 256; b++) {
      const uint8_t* blk = row + b * 148;
      float Ss = orc_f16_to_f32(get_u16(blk));
      float Sa = orc_f16_to_f32(get_u16(blk + 2));
      for (int j = 0; j < 8; j++) {
        float sj = Ss * (float)(int8_t)blk[4 + j];
        float aj = Sa * (float)(int8_t)blk[12 + j];
        for (int i = 0; i < 32; i++) {
          float t = sj * (float)nib(blk + 20 + 16 * j, i);
          y[b * 256 + 32 * j + i] = t + aj;
        }
      }
    }
  }
}

static int fmt_ok(int fmt, int64_t k) {
  int e = orc_block_elems(fmt);
  return e > 0 && k >= 0 && k % e == 0;
}

/* bytes of one row in the packed stream (for the planar group-128 format,
 * only rows of the same plane are this far apart) */
static int64_t row_bytes(int fmt, int64_t k) {
  return k / orc_block_elems(fmt) * orc_block_bytes(fmt);
}

int orc_dequant(int fmt, const uint8_t* blocks, int64_t rows, int64_t k,
                float* out) {
  if (!blocks || !out || rows < 0 || !fmt_ok(fmt, k)) return -1;
  for (int64_t r = 0; r < rows; r++)
    dequant_row(fmt, blocks, rows, k, r, out + r * k);
  return 0;
}

/* ------------------------------------------------------------------ */
/* products: fp64 sums over the dequantized fp32 weights               */
/* ------------------------------------------------------------------ */
int orc_gemv(int fmt, const uint8_t* blocks, int64_t m, int64_t k,
             const double* x, const int64_t* row_idx, int64_t nrows,
             double* y, double* bound) {
  if (!blocks || !x || !y || m < 0 || !fmt_ok(fmt, k)) return -1;
  if (!row_idx) nrows = m;
  float* w = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  if (!w) return -2;
  for (int64_t i = 0; i < nrows; i++) {
    int64_t r = row_idx ? row_idx[i] : i;
    if (r < 0 || r >= m) {
      free(w);
      return -1;
    }
    dequant_row(fmt, blocks, m, k, r, w);
    double acc = 0.0, b = 0.0;
    for (int64_t c = 0; c < k; c++) {
      double p = (double)w[c] * x[c];
      acc += p;
      b += fabs(p);
    }
    y[i] = acc;
    if (bound) bound[i] = b;
  }
  free(w);
  return 0;
}

int orc_gemm(int fmt, const uint8_t* blocks, int64_t m, int64_t k,
             const double* X, int64_t n, const int64_t* row_idx,
             int64_t nrows, double* Y, double* bound) {
  if (!blocks || !X || !Y || m < 0 || n < 0 || !fmt_ok(fmt, k)) return -1;
  if (!row_idx) nrows = m;
  float* w = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  if (!w) return -2;
  for (int64_t i = 0; i < nrows; i++) {
    int64_t r = row_idx ? row_idx[i] : i;
    if (r < 0 || r >= m) {
      free(w);
      return -1;
    }
    dequant_row(fmt, blocks, m, k, r, w);
    for (int64_t t = 0; t < n; t++) {
      const double* xr = X + t * k;
      double acc = 0.0, b = 0.0;
      for (int64_t c = 0; c < k; c++) {
        double p = (double)w[c] * xr[c];
        acc += p;
        b += fabs(p);
      }
      Y[t * nrows + i] = acc;
      if (bound) bound[t * nrows + i] = b;
    }
  }
  free(w);
  return 0;
}

/* W4A8 product (R31): Y[t, i] = sum_k W[row_i, k] * (scale[t] * xq[t, k]),
 * fp64 sums over the fp32 rebuilt weights and the fp32 rebuilt activations
 * (scale * code is exact in fp64). */
int orc_gemm_w4a8(const uint8_t* blocks, int64_t m, int64_t k,
                  const int8_t* xq, const float* scale, int64_t n,
                  const int64_t* row_idx, int64_t nrows, double* Y,
                  double* bound) {
  if (!blocks || !xq || !scale || !Y || m < 0 || n < 0 || !fmt_ok(ORC_W4G128, k)) return -1;
  if (!row_idx) nrows = m;
  float* w = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  if (!w) return -2;
  for (int64_t i = 0; i < nrows; i++) {
    int64_t r = row_idx ? row_idx[i] : i;
    if (r < 0 || r >= m) {
      free(w);
      return -1;
    }
    dequant_row(ORC_W4G128, blocks, m, k, r, w);
    for (int64_t t = 0; t < n; t++) {
      double acc = 0.0, b = 0.0;
      for (int64_t c = 0; c < k; c++) {
        double p = (double)w[c] * ((double)scale[t] * (double)xq[t * k + c]);
        acc += p;
        b += fabs(p);
      }
      Y[t * nrows + i] = acc;
      if (bound) bound[t * nrows + i] = b;
    }
  }
  free(w);
  return 0;
}
