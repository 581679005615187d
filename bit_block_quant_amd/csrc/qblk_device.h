// qblk_device.h -- device-side helpers shared by the gfx950 kernels of libqblk:
// number conversions, the rounding rule, wave reductions and loads of the
// 2-byte-aligned fields of the packed block streams.
//
// Every kernel is compiled with -ffp-contract=off (no implicit fused
// multiply-add; dequantization must reproduce separate IEEE products), with
// correctly rounded fp32 division and with fp32/fp16 denormals kept; fused
// multiply-adds that are wanted (accumulation) are written explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qblk {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
// 16 bytes with only dword alignment: global_load_dwordx4 needs 4-byte
// alignment, and the fields of the block streams sit at 2-byte granularity.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- numbers
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default
// round mode; fp16 denormals are kept by the default FP16/64 denorm mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<half_t>(v));
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(b)));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}
// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Round half away from zero (roundf is exactly that operation).
__device__ __forceinline__ float rha(float v) { return __builtin_roundf(v); }

// Quotient used by every quantizer: zero scale -> 0.  True IEEE division.
__device__ __forceinline__ float qdiv(float v, float s) { return s == 0.0f ? 0.0f : v / s; }

// round-half-away quotient clamped into [lo, hi]; NaN lands on lo.
__device__ __forceinline__ int code_of(float v, float s, float lo, float hi) {
  float t = rha(qdiv(v, s));
  t = __builtin_fmaxf(t, lo);  // fmax(NaN, lo) = lo
  t = __builtin_fminf(t, hi);
  return static_cast<int>(t);
}

// The same codes for 8 values against one scale s, with the division done
// once: r = 1/s (IEEE; 0 when s = 0).  The rounded product y = v*r is within
// 2.5 ulp of the IEEE quotient v/s (r and the product each add at most half an
// ulp of relative error), so when y is more than 2^-14 from every
// half-integer -- 3 ulp or more while |y| < 256; larger quotients clamp
// either way -- the quotient rounds (half away from zero) to the integer
// nearest y, which v_rndne gives.  Values that close to a half-integer take
// the exact quotient (a rare, wave-uniform branch).
__device__ __forceinline__ void codes8(const float v[8], float s, float lo, float hi, int n[8]) {
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  float q[8];
  uint64_t m[8], any = 0;  // per value: the lanes whose product is near a half-integer
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float y = v[i] * r;
    q[i] = __builtin_rintf(y);
    m[i] = __builtin_amdgcn_ballot_w64(__builtin_fabsf(y - q[i]) >= 0.5f - 0x1p-14f);  // y - q exact
    any |= m[i];
  }
  if (any) {
    const uint64_t bit = uint64_t(1) << (threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (m[i] & bit) q[i] = rha(qdiv(v[i], s));
  }
#pragma unroll
  for (int i = 0; i < 8; i++) n[i] = static_cast<int>(__builtin_amdgcn_fmed3f(q[i], lo, hi));
}

// The clamped codes as floats (same rule as codes8) for N values whose
// products y = v*r are already formed (v: the exact dividends, used only on
// the slow path).
template <int N>
__device__ __forceinline__ void codes_f(const float v[N], float y[N], float s, float lo, float hi) {
  uint64_t m[N], any = 0;
#pragma unroll
  for (int i = 0; i < N; i++) {
    const float q = __builtin_rintf(y[i]);
    m[i] = __builtin_amdgcn_ballot_w64(__builtin_fabsf(y[i] - q) >= 0.5f - 0x1p-14f);
    any |= m[i];
    y[i] = q;
  }
  if (any) {
    const uint64_t bit = uint64_t(1) << (threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < N; i++)
      if (m[i] & bit) y[i] = rha(qdiv(v[i], s));
  }
#pragma unroll
  for (int i = 0; i < N; i++) y[i] = __builtin_amdgcn_fmed3f(y[i], lo, hi);
}

// fp16 half (lo or hi) of a packed word times m plus c, one rounding
// (v_fma_mix: the fp16 operand is widened exactly).
__device__ __forceinline__ float mix_lo(uint32_t h, float m, float c) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(m), "v"(c));
  return r;
}
__device__ __forceinline__ float mix_hi(uint32_t h, float m, float c) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(m), "v"(c));
  return r;
}

// 16 qs bytes from 32 clamped codes (as floats): byte b = c[b] + 16*c[b+16] + add
__device__ __forceinline__ void pack32f(const float c[32], float add, uint32_t qw[4]) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t x = 0;
#pragma unroll
    for (int b = 0; b < 4; b++)
      x = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c[4 * q + b + 16], 16.0f, c[4 * q + b]) + add, b, x);
    qw[q] = x;
  }
}

// Optimisation barrier: the value is materialised in a VGPR, so a following
// narrowing conversion cannot be fused with the arithmetic that produced it
// (a fused v_fma_mix with a +0 addend would turn -0 into +0).
__device__ __forceinline__ float opaque(float v) {
  asm("" : "+v"(v));
  return v;
}

// (a & mask) | bits in one v_and_or_b32 (mask from an SGPR, bits from a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(bits));
  return r;
}

// a.lo*b.lo + a.hi*b.hi in fp32 (v_dot2_f32_f16 with a zero addend in the
// instruction itself, so no register has to be zeroed first)
__device__ __forceinline__ float dot2_first(half2_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---------------------------------------------------------------- waves
// Sum over the 64 lanes of a wave with DPP moves; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)); // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)); // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)); // row_bcast:15
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)); // row_bcast:31
  return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
template <int W>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = __builtin_fminf(v, __shfl_xor(v, m, kWave));
  return v;
}

// ---------------------------------------------------------------- loads
// 16 bytes starting at a 2-byte-aligned address p: a dword-aligned 16-byte
// load from p rounded down to 4, plus the 2 bytes that spill past it, realigned
// with v_alignbyte.  Every byte read lies inside [p - 2, p + 16).
__device__ __forceinline__ void load16_a2(const uint8_t* p, uint32_t out[4]) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(a & ~uintptr_t(3));
  const uint32_t tail = *reinterpret_cast<const uint16_t*>(p + 14);
  const uint32_t sh = static_cast<uint32_t>(a & 3u);  // 0 or 2
  out[0] = __builtin_amdgcn_alignbyte(v.y, v.x, sh);
  out[1] = __builtin_amdgcn_alignbyte(v.z, v.y, sh);
  out[2] = __builtin_amdgcn_alignbyte(v.w, v.z, sh);
  out[3] = __builtin_amdgcn_alignbyte(tail, v.w, sh);
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// ---------------------------------------------------------------- Q4_K
// The 16-byte header of a Q4_K super-block as dwords h0..h3: fp16 d (low half
// of h0) and dmin (high half), then sixteen 6-bit fields, field i at bit
// 32 + 6i: the scale s_j is field j (inside h1:h2), the min m_j field 8 + j
// (inside h2:h3).
__device__ __forceinline__ uint32_t q4k_scale6(uint32_t h1, uint32_t h2, int j) {
  return static_cast<uint32_t>(((static_cast<uint64_t>(h2) << 32) | h1) >> (6 * j)) & 63u;
}
__device__ __forceinline__ uint32_t q4k_min6(uint32_t h2, uint32_t h3, int j) {
  return static_cast<uint32_t>(((static_cast<uint64_t>(h3) << 32) | h2) >> (16 + 6 * j)) & 63u;
}

}  // namespace qblk
