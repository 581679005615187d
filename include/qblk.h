/*
 * qblk.h -- C ABI of libqblk: 4-bit block quantization of weight matrices and
 * the fused dequantize-and-multiply that streams the blocks, for AMD Instinct
 * MI355X (gfx950).
 *
 * Formats (all little-endian, no padding: the packed bytes are the storage
 * format itself):
 *
 *   QBLK_Q4_0        32 weights in 18 bytes (4.5 bit/weight):
 *                      [d: fp16][qs: 16 bytes]
 *                    byte qs[j] holds the 4-bit code of weight j in its low
 *                    nibble and of weight j+16 in its high nibble; a weight is
 *                    d * (code - 8).
 *                    ("GGUF 量化内幕 第4章 Q4_0" (sxkj888.cn), sections 4.1.2,
 *                    4.2.1, 4.2.2, 4.3.)
 *
 *   QBLK_SB4         super-block of 256 weights in 138 bytes (4.3125 bit/weight):
 *                      [S: fp16][sc: 8 x int8][qs: 8 x 16 bytes]
 *                    eight Q4_0-style sub-blocks of 32 whose fp16 scales are
 *                    themselves quantized to INT8 in [-127, 127] under the fp16
 *                    super-scale S = max(scale)/127; a weight of sub-block j is
 *                    (S * sc[j]) * (code - 8).
 *                    ("GGUF K-quants" blog (hugo-blog-2v1.pages.dev), section
 *                    "套娃": the super-block, steps 1-5 and the storage table.)
 *
 *   QBLK_SB4_AFFINE  affine super-block of 256 weights in 148 bytes (4.625 b/w):
 *                      [Ss: fp16][Sa: fp16][sc: 8 x int8][ac: 8 x int8][qs: 128]
 *                    per sub-block scale (max-min)/15 and offset min with codes
 *                    0..15; scales and offsets are each INT8-quantized under
 *                    their own fp16 super-scale; a weight is
 *                    (Ss * sc[j]) * code + (Sa * ac[j]).
 *                    (Same blog, section "套娃": Type 1 blocks also carry an
 *                    offset whose fp16 value is compressed to INT8.)
 *
 *   QBLK_Q4_K        super-block of 256 weights in 144 bytes (4.5 bit/weight):
 *                      [d: fp16][dmin: fp16][f: 12 bytes][qs: 8 x 16 bytes]
 *                    per 32-weight sub-block j a 6-bit scale s_j and a 6-bit
 *                    min m_j; field i of the sixteen 6-bit fields (s_0..s_7,
 *                    then m_0..m_7) sits at bits 6i..6i+5 of f read as one
 *                    little-endian integer; codes 0..15 stored as in Q4_0;
 *                    a weight is (d * s_j) * code - dmin * m_j.
 *                    (Q4_0 chapter, section 4.6, which names the 6-bit
 *                    packing without describing it: the field order is this
 *                    library's.)
 *
 *   QBLK_W4G128      groups of 128 weights along a row, one fp16 scale each
 *                    (66 bytes per group, 4.125 bit/weight), stored as two
 *                    planes: first the codes, k/2 bytes per row (byte j of
 *                    group g holds weight 128g+j in its low nibble and weight
 *                    128g+64+j in its high nibble, codes stored +8), then the
 *                    scales, k/128 fp16 values per row.  Symmetric: scale
 *                    d = absmax/7, a weight is d * (code - 8).  Products take
 *                    8-bit activations (qblk_quantize_act_i8, qblk_gemm_w4a8).
 *                    (TurboQuant W4A8 article (codechina.net), sections 2.1
 *                    and 2.2; the layout is this library's, the page gives
 *                    none.)
 *
 * Matrices are dense row-major.  A packed matrix of rows x k weights stores row
 * r, block b at byte (r * k/E + b) * B, with E weights and B bytes per block
 * (QBLK_W4G128: the two planes above, rows * k/E * B bytes in all).
 *
 * Quantization rule (the same for all formats; both the codes and the INT8
 * or 6-bit scales are computed against the scale the block STORES, decoded
 * back from fp16): code = clamp(round_half_away(v / s), lo, hi), with IEEE
 * fp32 division, a zero scale giving code 0 (Q4_0/Type 0: stored code 8),
 * fp16 rounding to nearest even with subnormals kept.  Q4_0 uses s = absmax/7
 * per 32 weights.  The GPU library reproduces the CPU definition bit for bit.
 *
 * Conventions for every entry point:
 *   - Pointers to data are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no mutable state, so calls are reentrant.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Device faults surface at the caller's
 *     next synchronization.
 *   - Arguments are checked on the host before any launch; on error nothing is
 *     launched and nothing is written.  A failed launch returns
 *     QBLK_ERR_LAUNCH.
 *   - Data pointers must be 16-byte aligned (QBLK_ERR_ALIGN); the fp32
 *     per-token scale arrays of the 8-bit activations only 4-byte aligned.
 *   - k must be a multiple of the format's block size (QBLK_ERR_SHAPE);
 *     rows/m/n/k may be 0 (an empty product writes zeros to y when m, n > 0).
 *   - rows, m, n and k must each stay below 2^31, and a packed matrix below
 *     2^40 bytes (QBLK_ERR_SHAPE); qblk_gemm and qblk_gemm_w4a8 take at most
 *     m = 2^28 rows (QBLK_ERR_SHAPE).  A call whose grid would exceed the
 *     2^32 - 1 threads one launch can hold (the quantizers, dequant, the
 *     activation quantizer and the batch-1 products at very large sizes)
 *     is run as several launches in stream order.
 *   - Inputs must be finite; non-finite inputs give unspecified results.
 *     A block whose scale overflows fp16 (|w| > 7 * 65504 for Q4_0 and
 *     Type 0, a 32-weight range above 15 * 65504 for Type 1) is stored with an
 *     infinite scale; that is well defined for Q4_0 but not for super-blocks.
 */
#ifndef QBLK_H
#define QBLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QBLK_Q4_0 = 0,       /* 32 weights, 18 bytes  */
  QBLK_SB4 = 1,        /* 256 weights, 138 bytes */
  QBLK_SB4_AFFINE = 2, /* 256 weights, 148 bytes */
  QBLK_Q4_K = 3,       /* 256 weights, 144 bytes */
  QBLK_W4G128 = 4      /* 128 weights, 66 bytes (two planes) */
} qblk_format_t;

typedef enum {
  QBLK_F32 = 0,  /* IEEE binary32 */
  QBLK_F16 = 1,  /* IEEE binary16 */
  QBLK_BF16 = 2  /* bfloat16      */
} qblk_dtype_t;

typedef enum {
  QBLK_OK = 0,
  QBLK_ERR_NULL = 1,        /* a required pointer is NULL               */
  QBLK_ERR_SHAPE = 2,       /* negative/too large size, k not a multiple */
  QBLK_ERR_DTYPE = 3,       /* element type not accepted by this call   */
  QBLK_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned    */
  QBLK_ERR_UNSUPPORTED = 5, /* format/type combination not implemented  */
  QBLK_ERR_LAUNCH = 6,      /* the kernel launch failed                 */
  QBLK_ERR_FORMAT = 7       /* unknown format                           */
} qblk_status_t;

typedef void* qblk_stream_t; /* hipStream_t */

/* One product of qblk_gemv_batch: y (m fp32) = W x with W (m x k) in blocks
 * and x (k elements); device pointers owned by the caller. */
typedef struct {
  const void* blocks;
  int64_t m;
  const void* x;
  float* y;
} qblk_gemv_item_t;

/* Most products one qblk_gemv_batch call takes. */
#define QBLK_GEMV_BATCH_MAX 32

/* Geometry.  qblk_block_bytes/elems return 0 for an unknown format;
 * qblk_packed_bytes returns 0 if k is not a multiple of the block size or a
 * size is negative. */
size_t qblk_block_bytes(qblk_format_t fmt);
int qblk_block_elems(qblk_format_t fmt);
size_t qblk_packed_bytes(qblk_format_t fmt, int64_t rows, int64_t k);

/* Quantize w (rows x k, element type wt in {F32, F16, BF16}, read exactly as
 * fp32 values) into Q4_0 blocks (qblk_packed_bytes(QBLK_Q4_0, rows, k) bytes).
 * Q4_0 chapter section 4.1.1 gives the absmax/7 scale; sections 4.1.2-4.2.2
 * the layout and the +8 code offset. */
qblk_status_t qblk_quantize_q4_0(const void* w, qblk_dtype_t wt, int64_t rows,
                                 int64_t k, void* blocks, qblk_stream_t stream);

/* Quantize w into super-blocks: affine = 0 gives QBLK_SB4 (Type 0), affine = 1
 * gives QBLK_SB4_AFFINE (Type 1).  K-quants blog, section "套娃", steps 1-4
 * for the INT8 sub-scales (and offsets). */
qblk_status_t qblk_quantize_sb4(const void* w, qblk_dtype_t wt, int64_t rows,
                                int64_t k, int affine, void* blocks,
                                qblk_stream_t stream);

/* Quantize w (element type F32, F16 or BF16) into QBLK_Q4_K super-blocks.
 * Q4_0 chapter, section 4.6 gives the form y = d*s_j*q - dmin*m_j; the steps
 * it leaves open are taken as: sub-block range lo = min(0, min w), hi = max w;
 * first-level scale (hi - lo)/15 and min -lo in fp32; d = fp16(max scale/63),
 * dmin = fp16(max min/63); s_j, m_j = clamp(round_half_away(v / stored), 0, 63);
 * codes clamp(round_half_away((w + dmin*m_j) / (d*s_j)), 0, 15) with the
 * rebuilt (exact fp32) d*s_j and dmin*m_j. */
qblk_status_t qblk_quantize_q4_k(const void* w, qblk_dtype_t wt, int64_t rows,
                                 int64_t k, void* blocks, qblk_stream_t stream);

/* Quantize w (element type F32, F16 or BF16, k a multiple of 128) into
 * QBLK_W4G128 groups: per row, each group of 128 weights takes the scale
 * d = fp16(max|w| / 7) and codes clamp(round_half_away(w / d), -8, 7) + 8
 * against the stored d (TurboQuant article, section 2.1: per-row symmetric
 * groups of 128, scale from the group's own maximum, 4-bit integers). */
qblk_status_t qblk_quantize_w4g128(const void* w, qblk_dtype_t wt, int64_t rows,
                                   int64_t k, void* blocks, qblk_stream_t stream);

/* 8-bit activations (TurboQuant article, section 2.2, which leaves the
 * activation scaling open): for each of the n rows (tokens) of x (n x k,
 * type xt, k a multiple of 8), one symmetric scale s = max|x| / 127 kept in
 * fp32 (scale[t], n floats) and codes xq = clamp(round_half_away(x / s),
 * -127, 127) (n x k int8, row-major); a zero row gives s = 0 and codes 0. */
qblk_status_t qblk_quantize_act_i8(const void* x, qblk_dtype_t xt, int64_t n,
                                   int64_t k, int8_t* xq, float* scale,
                                   qblk_stream_t stream);

/* W4A8 product Y = X W^T with W (m x k) in QBLK_W4G128 and X given as the
 * int8 codes xq (n x k) and token scales (n floats) of
 * qblk_quantize_act_i8: Y[t,i] = scale[t] * sum_g d[i,g] *
 * sum_{k in g} (code - 8) * xq[t,k], Y n x m fp32 row-major.  The integer
 * sums are exact; Y is within 2e-5 * sum_k |W[i,k] * scale[t] * xq[t,k]| of
 * the exact product of the rebuilt weights and activations.  n = 1 runs a
 * batch-1 kernel (k <= 16384); otherwise int8 matrix cores, with the k range
 * split over the grid (partial sums added into Y, zeroed first by this call)
 * when m*n is small.  qblk_gemv and qblk_gemm return QBLK_ERR_UNSUPPORTED
 * for QBLK_W4G128. */
qblk_status_t qblk_gemm_w4a8(const void* blocks, int64_t m, int64_t k,
                             const int8_t* xq, const float* scale, int64_t n,
                             float* y, qblk_stream_t stream);

/* Q4_0 quantization as the Q4_0 chapter's section 4.4 prints it: the signed
 * value of largest magnitude divided by -8 is the scale, codes are
 * min(15, trunc(w * (1/d) + 8.5)) with the fp32 reciprocal.  Input F32 only
 * (QBLK_ERR_DTYPE otherwise).  Output layout as QBLK_Q4_0. */
qblk_status_t qblk_quantize_q4_0_ref(const void* w, qblk_dtype_t wt,
                                     int64_t rows, int64_t k, void* blocks,
                                     qblk_stream_t stream);

/* Rebuild the weights from blocks into out (rows x k, type ot in {F32, F16,
 * BF16}).  F32 output is the fp32 value of the format's formula (Q4_0
 * chapter section 4.3 for Q4_0; K-quants blog step 5 for the super-blocks;
 * chapter section 4.6 for Q4_K, one rounding of the exact product minus the
 * exact min); F16/BF16 outputs are that value rounded to nearest even. */
qblk_status_t qblk_dequant(qblk_format_t fmt, const void* blocks, int64_t rows,
                           int64_t k, void* out, qblk_dtype_t ot,
                           qblk_stream_t stream);

/* Batch-1 product y = W x for W (m x k) in blocks: x has k elements of type xt
 * in {F32, F16, BF16}; y has m fp32 elements.  Products are formed from the
 * exact codes and x, accumulated in fp32; the result is within
 * 2e-5 * sum_k |W[i,k] x[k]| of the exact sum of the rebuilt weights times x. */
qblk_status_t qblk_gemv(qblk_format_t fmt, const void* blocks, int64_t m,
                        int64_t k, const void* x, qblk_dtype_t xt, float* y,
                        qblk_stream_t stream);

/* Several batch-1 products that share the format, k and the type of x, in
 * one launch: items[i].y = W_i x_i for i < count (count <= 32, the items
 * read during the call only).  Each product is the one qblk_gemv computes,
 * with the same bound; a layer's matrices of equal k (a transformer's q, k, v
 * and o projections, or gate and up) then share one grid instead of paying a
 * kernel boundary each.  Items with m = 0 are skipped; argument errors in any
 * item are returned before any launch.  fp16 x with k <= 12288 runs as one
 * launch; other x types or longer rows run one launch per item. */
qblk_status_t qblk_gemv_batch(qblk_format_t fmt, int64_t k, qblk_dtype_t xt,
                              const qblk_gemv_item_t* items, int count,
                              qblk_stream_t stream);

/* Small-batch product Y = X W^T: X is n x k row-major (token-major) of type xt,
 * Y is n x m row-major fp32.  All four formats run on the bf16 matrix cores
 * with xt = BF16; F32/F16 activations, and Q4_0 with k % 256 != 0, return
 * QBLK_ERR_UNSUPPORTED.  Same error bound as qblk_gemv, per output element.
 * When k spans many groups and m*n is small the k range is split over the
 * grid and partial sums are added into Y (zeroed first by this call), so the
 * summation order, not the bound, varies between tilings and between runs
 * (qblk_set_deterministic turns the split off). */
qblk_status_t qblk_gemm(qblk_format_t fmt, const void* blocks, int64_t m,
                        int64_t k, const void* x, qblk_dtype_t xt, int64_t n,
                        float* y, qblk_stream_t stream);

/* Reproducible products.  With on != 0, qblk_gemm and qblk_gemm_w4a8 never
 * split the k range over workgroups: every output is summed by one
 * workgroup in a fixed order, so identical inputs and sizes give bitwise
 * identical Y on the same device, run after run (split sums are added into
 * Y with fp32 atomics, whose order varies).  Slower where the split paid: few
 * tokens, or few rows with a long k.  The setting is process-wide, applies to
 * calls made after it, and is off at load.  Always returns QBLK_OK.  (Not an
 * operation of the pages: a property of this implementation's sums.) */
qblk_status_t qblk_set_deterministic(int on);

/* 1 when reproducible products are on (qblk_set_deterministic), else 0. */
int qblk_deterministic(void);

/* Static English text for a status code (never NULL). */
const char* qblk_status_string(qblk_status_t st);

/* Library version as "major.minor.patch" (static string). */
const char* qblk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QBLK_H */
