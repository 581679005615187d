/*
 * qblk_oracle.h -- plain, slow, single-threaded CPU definitions of the block
 * formats, their codecs and the products that stream them.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker, not the product:
 * only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or constant with
 * the GPU library, and neither side includes or links the other.
 *
 * Sources (the pages the method is defined on):
 *   [KQ]  "GGUF K-quants" blog post (hugo-blog-2v1.pages.dev/2025/gguf-k-quants/),
 *         section "套娃" (the super-block and the five-step quantization of
 *         its eight block scales, with the worked example and the storage table).
 *   [Q40] "GGUF 量化内幕 第4章 Q4_0：块量化的起点" (sxkj888.cn), sections
 *         4.1.2 (block layout), 4.2.1 (nibble order), 4.2.2 (code range and
 *         the minus-8 offset), 4.3 (dequantization), 4.4 (quantizer), 4.5
 *         (outlier example), 4.6 (the Q4_K form: d, dmin, 6-bit s_j and m_j).
 *   [TQ]  the TurboQuant W4A8 article (codechina.net), sections 2.1 (per-row
 *         symmetric groups of 128 weights, 4-bit) and 2.2 (8-bit activations).
 *
 * Conventions (fp32 IEEE arithmetic, no FMA contraction, true division):
 *   h(v)  fp32 -> fp16 bits, round-to-nearest-even, subnormals kept.
 *   f(b)  fp16 bits -> fp32, exact.
 *   rha   round half away from zero (C99 roundf).
 *   qdiv(v, s) = (s == 0) ? 0 : v / s.
 *   Every integer code is computed against the scale its level STORES,
 *   decoded back to fp32 (so encode and decode see the same number).
 *
 * All buffers are host memory owned by the caller.  Functions return 0 on
 * success and a negative value on a bad argument; nothing is written then.
 */
#ifndef QBLK_ORACLE_H
#define QBLK_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* formats */
#define ORC_Q4_0 0       /* 32 weights, 18 bytes            */
#define ORC_SB4 1        /* 256 weights, 138 bytes (Type 0) */
#define ORC_SB4_AFFINE 2 /* 256 weights, 148 bytes (Type 1) */
#define ORC_Q4_K 3       /* 256 weights, 144 bytes ([Q40] 4.6 form) */
#define ORC_W4G128 4     /* 128 weights: 64 code bytes + fp16 scale, two planes ([TQ]) */

/* element types of dense inputs */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* scalar helpers (exposed so the tests can pin them one by one) */
float orc_f16_to_f32(uint16_t bits);
uint16_t orc_f32_to_f16(float v);
float orc_bf16_to_f32(uint16_t bits);
uint16_t orc_f32_to_bf16(float v);
float orc_rha(float v);

/* geometry */
int orc_block_elems(int fmt);
int orc_block_bytes(int fmt);

/* Meta-quantization of n (>= 1) scale values to INT8, [KQ] "套娃" steps 1-4.
 * s:        the scales as fp32 values.
 * S_forced: if > 0, use this value as the super-scale as it is (the page's
 *           rounded 0.00142); otherwise compute it and store it as fp16.
 * codes:    n int8 outputs; S16: the stored fp16 super-scale (0 if forced);
 * S_used:   the fp32 super-scale the codes were computed against.        */
int orc_meta_int8(const float* s, int n, float S_forced, int8_t* codes,
                  uint16_t* S16, float* S_used);

/* Quantize a dense rows x k matrix (dtype ORC_F32/F16/BF16, row-major) into
 * the packed block stream (row r, block b at (r*k/elems + b)*block_bytes;
 * the group-128 W4 format is planar instead, see R28). */
int orc_quantize_q4_0(const void* w, int dtype, int64_t rows, int64_t k,
                      uint8_t* out);
int orc_quantize_sb4(const void* w, int dtype, int64_t rows, int64_t k,
                     int affine, uint8_t* out);

/* Q4_K form of [Q40] 4.6: y = d*s_j*q - dmin*m_j (layout and the steps the
 * page leaves open are the readings R23-R27 listed in qblk_oracle.c). */
int orc_quantize_q4_k(const void* w, int dtype, int64_t rows, int64_t k,
                      uint8_t* out);

/* [TQ] group-128 symmetric 4-bit weights (readings R28-R29 in qblk_oracle.c)
 * and per-token symmetric 8-bit activations (R30): xq is n x k int8, scale
 * has n fp32 entries.  gemm_w4a8 is the product of the rebuilt operands
 * (R31), fp64 sums, rows as in orc_gemm. */
int orc_quantize_w4g128(const void* w, int dtype, int64_t rows, int64_t k,
                        uint8_t* out);
int orc_quantize_act_i8(const void* x, int dtype, int64_t n, int64_t k,
                        int8_t* xq, float* scale);
int orc_gemm_w4a8(const uint8_t* blocks, int64_t m, int64_t k,
                  const int8_t* xq, const float* scale, int64_t n,
                  const int64_t* row_idx, int64_t nrows, double* Y,
                  double* bound);

/* Q4_0 quantizer as [Q40] 4.4 prints it (signed extreme / -8, reciprocal
 * multiply, +8.5 and truncation, upper clamp at 15). */
int orc_quantize_q4_0_ref(const float* w, int64_t rows, int64_t k,
                          uint8_t* out);

/* Dequantize the packed stream to fp32 values. */
int orc_dequant(int fmt, const uint8_t* blocks, int64_t rows, int64_t k,
                float* out);

/* Products in fp64 over the fp32 dequantized weights.
 * gemv: y[i] = sum_k W[row_i, k] * x[k] and bound[i] = sum_k |W x| for the
 *       rows listed in row_idx (nrows of them; row_idx NULL = all m rows).
 * gemm: Y[n, i] = sum_k W[row_i, k] * X[n, k], X is n x k row-major, Y is
 *       n x nrows row-major, bound likewise.                                */
int orc_gemv(int fmt, const uint8_t* blocks, int64_t m, int64_t k,
             const double* x, const int64_t* row_idx, int64_t nrows,
             double* y, double* bound);
int orc_gemm(int fmt, const uint8_t* blocks, int64_t m, int64_t k,
             const double* X, int64_t n, const int64_t* row_idx,
             int64_t nrows, double* Y, double* bound);

#ifdef __cplusplus
}
#endif
#endif
