// qblk_quant.hip -- quantization kernels (dense fp32/fp16/bf16 -> packed blocks)
// and dequantization kernels (packed blocks -> dense fp32/fp16/bf16) for gfx950.
//
// A dense row-major matrix and its packed stream are both contiguous, so these
// kernels work on the flat sequence of blocks: block g covers weights
// [g*E, (g+1)*E) and bytes [g*B, (g+1)*B).  A workgroup of 256 threads owns
// 2048 consecutive weights (64 Q4_0 blocks or 8 super-blocks), 8 weights per
// thread; since 64*18 = 1152, 8*138 = 1104 and 8*148 = 1184 are multiples of
// 16, each workgroup's slice of the packed stream is 16-byte aligned and is
// moved between HBM and LDS with 16-byte loads/stores.
//
// Definitions followed (field order and the rounding readings are stated in
// qblk.h):
//   Q4_0 block ("GGUF 量化内幕 第4章 Q4_0", 4.1.1 absmax/7 scale, 4.1.2 layout,
//     4.2.1 low nibble = weight j / high nibble = weight j+16, 4.2.2 code+8,
//     4.3 value = d*(code-8)).
//   Super-block ("GGUF K-quants" blog, "套娃"): eight sub-block scales stored
//     as fp16, then quantized to INT8 in [-127, 127] against the fp16
//     super-scale max/127 (steps 1-4), rebuilt as code*super-scale (step 5).
//   Q4_K form (Q4_0 chapter 4.6): fp16 d and dmin per super-block, 6-bit
//     scale s_j and min m_j per sub-block, weight (d*s_j)*code - dmin*m_j.
#include "qblk_device.h"
#include "qblk_launch.h"

namespace qblk {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kWgWeights = kThreads * kPerThread;  // 2048

// ------------------------------------------------------------- dense I/O
template <int DT>
__device__ __forceinline__ void load8(const void* w, int64_t idx, bool valid, float v[8]) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0.0f;
    return;
  }
  if constexpr (DT == QBLK_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + idx);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + idx);
    const uint32_t r[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (DT == QBLK_F16) {
        v[2 * i] = f16_bits_to_f32(r[i] & 0xffffu);
        v[2 * i + 1] = f16_bits_to_f32(r[i] >> 16);
      } else {
        v[2 * i] = bf16_bits_to_f32(r[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* out, int64_t idx, const float v[8]) {
  if constexpr (DT == QBLK_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t a, b;
      if constexpr (DT == QBLK_F16) {
        a = f32_to_f16_bits(opaque(v[2 * i]));
        b = f32_to_f16_bits(opaque(v[2 * i + 1]));
      } else {
        a = f32_to_bf16_bits(v[2 * i]);
        b = f32_to_bf16_bits(v[2 * i + 1]);
      }
      r[i] = a | (b << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + idx) = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// ------------------------------------------------------ LDS <-> packed stream
// Copy `nbytes` (even) of the workgroup's packed slice between LDS and global
// memory.  Whole 16-byte pieces move as uint4, a 2-byte-granular tail as u16.
__device__ __forceinline__ void lds_to_global(const uint8_t* lds, uint8_t* g, int nbytes) {
  const int n16 = nbytes >> 4;
  for (int i = threadIdx.x; i < n16; i += kThreads)
    reinterpret_cast<uint4*>(g)[i] = reinterpret_cast<const uint4*>(lds)[i];
  for (int i = (n16 << 3) + threadIdx.x; i < (nbytes >> 1); i += kThreads)
    reinterpret_cast<uint16_t*>(g)[i] = reinterpret_cast<const uint16_t*>(lds)[i];
}
__device__ __forceinline__ void global_to_lds(const uint8_t* g, uint8_t* lds, int nbytes) {
  const int n16 = nbytes >> 4;
  for (int i = threadIdx.x; i < n16; i += kThreads)
    reinterpret_cast<uint4*>(lds)[i] = reinterpret_cast<const uint4*>(g)[i];
  for (int i = (n16 << 3) + threadIdx.x; i < (nbytes >> 1); i += kThreads)
    reinterpret_cast<uint16_t*>(lds)[i] = reinterpret_cast<const uint16_t*>(g)[i];
}

// Nibble packing.  Inside a 32-weight group, thread u (0..3) holds weights
// 8u..8u+7.  Byte b of the group stores weight b (low nibble) and weight b+16
// (high nibble), so thread u < 2 combines its codes with those of thread u+2.
// Returns the 8 bytes 8u..8u+7 (meaningful for u < 2) as two words.
__device__ __forceinline__ void pack_group(const int n[8], uint32_t& w0, uint32_t& w1) {
  uint32_t a0 = n[0] | (n[1] << 8) | (n[2] << 16) | (n[3] << 24);
  uint32_t a1 = n[4] | (n[5] << 8) | (n[6] << 16) | (n[7] << 24);
  uint32_t b0 = __shfl_xor(a0, 2, kWave);
  uint32_t b1 = __shfl_xor(a1, 2, kWave);
  w0 = a0 | (b0 << 4);
  w1 = a1 | (b1 << 4);
}

__device__ __forceinline__ void lds_put8(uint8_t* lds, int off, uint32_t w0, uint32_t w1) {
  uint16_t* p = reinterpret_cast<uint16_t*>(lds + off);  // off is even
  p[0] = static_cast<uint16_t>(w0);
  p[1] = static_cast<uint16_t>(w0 >> 16);
  p[2] = static_cast<uint16_t>(w1);
  p[3] = static_cast<uint16_t>(w1 >> 16);
}

// ------------------------------------------------------------- Q4_0 quantize
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_q4_0(const void* __restrict__ w,
                                                         uint8_t* __restrict__ out,
                                                         int64_t nblocks) {
  __shared__ uint4 stage4[64 * 18 / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int bl = t >> 2, u = t & 3;
  const bool valid = blk0 + bl < nblocks;
  float v[8];
  load8<DT>(w, (blk0 + bl) * 32 + u * 8, valid, v);

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  amax = group_max<4>(amax);
  const uint16_t d16 = f32_to_f16_bits(amax / 7.0f);
  const float d = f16_bits_to_f32(d16);
  int n[8];
  codes8(v, d, -8.0f, 7.0f, n);
#pragma unroll
  for (int i = 0; i < 8; i++) n[i] += 8;
  uint32_t w0, w1;
  pack_group(n, w0, w1);
  if (valid) {
    if (u == 0) *reinterpret_cast<uint16_t*>(stage + bl * 18) = d16;
    if (u < 2) lds_put8(stage, bl * 18 + 2 + 8 * u, w0, w1);
  }
  __syncthreads();
  const int64_t nb = nblocks - blk0 < 64 ? nblocks - blk0 : 64;
  lds_to_global(stage, out + blk0 * 18, static_cast<int>(nb * 18));
}

// Q4_0 as the chapter's reference listing computes it (section 4.4): the
// signed value of largest magnitude (first one on ties) over -8 is the scale,
// codes min(15, trunc(w * (1/d) + 8.5)) with the fp32 reciprocal.
__global__ __launch_bounds__(kThreads) void k_quant_q4_0_ref(const float* __restrict__ w,
                                                             uint8_t* __restrict__ out,
                                                             int64_t nblocks) {
  __shared__ uint4 stage4[64 * 18 / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int bl = t >> 2, u = t & 3;
  const bool valid = blk0 + bl < nblocks;
  float v[8];
  load8<QBLK_F32>(w, (blk0 + bl) * 32 + u * 8, valid, v);
  // first element of largest magnitude in weight order: reduce (|v|, -index)
  float amax = 0.0f, ext = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++)
    if (__builtin_fabsf(v[i]) > amax) {
      amax = __builtin_fabsf(v[i]);
      ext = v[i];
    }
#pragma unroll
  for (int m = 1; m < 4; m <<= 1) {
    const float oa = __shfl_xor(amax, m, kWave);
    const float oe = __shfl_xor(ext, m, kWave);
    const bool other_first = (u ^ m) < u;  // the partner holds earlier weights
    if (oa > amax || (oa == amax && other_first && oa != 0.0f)) {
      amax = oa;
      ext = oe;
    }
  }
  const float d = ext / -8.0f;
  const float inv = d != 0.0f ? 1.0f / d : 0.0f;
  int n[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float s = v[i] * inv + 8.5f;  // separate multiply and add (no contraction)
    const int c = static_cast<int>(s);
    n[i] = c < 15 ? c : 15;
  }
  uint32_t w0, w1;
  pack_group(n, w0, w1);
  if (valid) {
    if (u == 0) *reinterpret_cast<uint16_t*>(stage + bl * 18) = f32_to_f16_bits(d);
    if (u < 2) lds_put8(stage, bl * 18 + 2 + 8 * u, w0, w1);
  }
  __syncthreads();
  const int64_t nb = nblocks - blk0 < 64 ? nblocks - blk0 : 64;
  lds_to_global(stage, out + blk0 * 18, static_cast<int>(nb * 18));
}

// ---------------------------------------------------------- super-blocks
// Threads 32*s .. 32*s+31 of the workgroup own super-block s (0..7); thread
// v = t % 32 holds weights 8v..8v+7, i.e. sub-block j = v/4, part u = v%4.
template <int DT, bool AFFINE>
__global__ __launch_bounds__(kThreads) void k_quant_sb4(const void* __restrict__ w,
                                                        uint8_t* __restrict__ out,
                                                        int64_t nsb) {
  constexpr int B = AFFINE ? 148 : 138;
  __shared__ uint4 stage4[8 * B / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t sb0 = static_cast<int64_t>(blockIdx.x) * 8;
  const int sl = t >> 5, v = t & 31, j = v >> 2, u = v & 3;
  const bool valid = sb0 + sl < nsb;
  float x[8];
  load8<DT>(w, (sb0 + sl) * 256 + v * 8, valid, x);
  uint8_t* blk = stage + sl * B;
  int n[8];
  if constexpr (!AFFINE) {
    // first level: a Q4_0 block per sub-block
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = group_max<4>(amax);
    const float d = f16_bits_to_f32(f32_to_f16_bits(amax / 7.0f));
    codes8(x, d, -8.0f, 7.0f, n);
#pragma unroll
    for (int i = 0; i < 8; i++) n[i] += 8;
    // second level: the eight fp16 scales -> INT8 under one fp16 super-scale
    float smax = d;
#pragma unroll
    for (int m = 4; m < 32; m <<= 1) smax = __builtin_fmaxf(smax, __shfl_xor(smax, m, kWave));
    const uint16_t S16 = f32_to_f16_bits(smax / 127.0f);
    const int sc = code_of(d, f16_bits_to_f32(S16), -127.0f, 127.0f);
    if (valid) {
      if (v == 0) *reinterpret_cast<uint16_t*>(blk) = S16;
      if (u == 0) blk[2 + j] = static_cast<uint8_t>(sc);
    }
  } else {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; i++) {
      mn = __builtin_fminf(mn, x[i]);
      mx = __builtin_fmaxf(mx, x[i]);
    }
    mn = group_min<4>(mn);
    mx = group_max<4>(mx);
    const float s = f16_bits_to_f32(f32_to_f16_bits((mx - mn) / 15.0f));
    const float a = f16_bits_to_f32(f32_to_f16_bits(mn));
    float xa[8];
#pragma unroll
    for (int i = 0; i < 8; i++) xa[i] = x[i] - a;
    codes8(xa, s, 0.0f, 15.0f, n);
    float smax = s, amax = __builtin_fabsf(a);
#pragma unroll
    for (int m = 4; m < 32; m <<= 1) {
      smax = __builtin_fmaxf(smax, __shfl_xor(smax, m, kWave));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, kWave));
    }
    const uint16_t Ss16 = f32_to_f16_bits(smax / 127.0f);
    const uint16_t Sa16 = f32_to_f16_bits(amax / 127.0f);
    const int sc = code_of(s, f16_bits_to_f32(Ss16), -127.0f, 127.0f);
    const int ac = code_of(a, f16_bits_to_f32(Sa16), -127.0f, 127.0f);
    if (valid) {
      if (v == 0) reinterpret_cast<uint32_t*>(blk)[0] = Ss16 | (static_cast<uint32_t>(Sa16) << 16);
      if (u == 0) {
        blk[4 + j] = static_cast<uint8_t>(sc);
        blk[12 + j] = static_cast<uint8_t>(ac);
      }
    }
  }
  uint32_t w0, w1;
  pack_group(n, w0, w1);
  if (valid && u < 2) lds_put8(stage, sl * B + (AFFINE ? 20 : 10) + 16 * j + 8 * u, w0, w1);
  __syncthreads();
  const int64_t ns = nsb - sb0 < 8 ? nsb - sb0 : 8;
  lds_to_global(stage, out + sb0 * B, static_cast<int>(ns * B));
}

// ------------------------------------------ one 32-weight group per thread
// The same quantizers with each thread owning a whole 32-weight group (a
// Q4_0 block or a sub-block): the group's extremes, its scale and its nibble
// pairs (byte b = code b | code b+16 << 4) need no cross-lane traffic, and
// the per-group divisions are done once per 32 weights instead of once per 8.
// A workgroup covers 256 groups (8192 weights): 256 Q4_0 blocks (4608 bytes)
// or 32 super-blocks (4416 / 4736 bytes), all multiples of 16.
// 16-bit inputs stay packed (two per word) until the products: extremes
// with packed 16-bit max/min, dividends and products with v_fma_mix (fp16)
// or an exact widening to fp32 (bf16).
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_h16(const void* w, int64_t idx, bool valid, uint32_t h[16]) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (valid) u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + idx + 8 * q);
    h[4 * q] = u.x;
    h[4 * q + 1] = u.y;
    h[4 * q + 2] = u.z;
    h[4 * q + 3] = u.w;
  }
}

template <int DT>
__device__ __forceinline__ float widen16(uint32_t bits) {
  return DT == QBLK_F16 ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
}

// max |x| of the 32 values: with the sign cleared, finite fp16 and bf16
// patterns order like unsigned integers
template <int DT>
__device__ __forceinline__ float absmax16(const uint32_t h[16]) {
  u16x2_t m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; i++) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, h[i] & 0x7fff7fffu));
  return widen16<DT>(m.x > m.y ? m.x : m.y);
}

template <int DT>
__device__ __forceinline__ void minmax16(const uint32_t h[16], float& mn, float& mx) {
  if constexpr (DT == QBLK_F16) {
    half2_t lo = __builtin_bit_cast(half2_t, h[0]), hi = lo;
#pragma unroll
    for (int i = 1; i < 16; i++) {
      lo = __builtin_elementwise_min(lo, __builtin_bit_cast(half2_t, h[i]));
      hi = __builtin_elementwise_max(hi, __builtin_bit_cast(half2_t, h[i]));
    }
    mn = __builtin_fminf(static_cast<float>(lo.x), static_cast<float>(lo.y));
    mx = __builtin_fmaxf(static_cast<float>(hi.x), static_cast<float>(hi.y));
  } else {
    mn = mx = widen16<DT>(h[0] & 0xffffu);
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float a = widen16<DT>(h[i] & 0xffffu), b = widen16<DT>(h[i] >> 16);
      mn = __builtin_fminf(mn, __builtin_fminf(a, b));
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(a, b));
    }
  }
}

// Codes of the 32 values (x - a)/s (a = 0: x/s) clamped to [lo, hi], packed
// as byte b = code b + 16 * code b+16 + add (add = 136 stores code+8 for the
// signed formats).  Dividend fl(x - a) and product as in codes8.
template <int DT, bool OFFSET>
__device__ __forceinline__ void codes16(const uint32_t h[16], float a, float s, float lo, float hi,
                                        float add, uint32_t qw[4]) {
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  float v[32], y[32];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    if constexpr (DT == QBLK_F16) {
      if constexpr (OFFSET) {
        v[2 * i] = mix_lo(h[i], 1.0f, -a);
        v[2 * i + 1] = mix_hi(h[i], 1.0f, -a);
        y[2 * i] = v[2 * i] * r;
        y[2 * i + 1] = v[2 * i + 1] * r;
      } else {
        v[2 * i] = f16_bits_to_f32(h[i] & 0xffffu);  // only read on the slow path
        v[2 * i + 1] = f16_bits_to_f32(h[i] >> 16);
        y[2 * i] = mix_lo(h[i], r, 0.0f);
        y[2 * i + 1] = mix_hi(h[i], r, 0.0f);
      }
    } else {
      v[2 * i] = widen16<DT>(h[i] & 0xffffu);
      v[2 * i + 1] = widen16<DT>(h[i] >> 16);
      if constexpr (OFFSET) {
        v[2 * i] = v[2 * i] - a;
        v[2 * i + 1] = v[2 * i + 1] - a;
      }
      y[2 * i] = v[2 * i] * r;
      y[2 * i + 1] = v[2 * i + 1] * r;
    }
  }
  codes_f<32>(v, y, s, lo, hi);
  pack32f(y, add, qw);
}

__device__ __forceinline__ void lds_put16_a2(uint8_t* lds, int off, const uint32_t qw[4]) {
  uint16_t* p = reinterpret_cast<uint16_t*>(lds + off);  // off is even
#pragma unroll
  for (int q = 0; q < 4; q++) {
    p[2 * q] = static_cast<uint16_t>(qw[q]);
    p[2 * q + 1] = static_cast<uint16_t>(qw[q] >> 16);
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_q4_0_g(const void* __restrict__ w,
                                                           uint8_t* __restrict__ out,
                                                           int64_t nblocks) {
  __shared__ uint4 stage4[kThreads * 18 / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * kThreads;
  const bool valid = blk0 + t < nblocks;
  uint32_t h[16];
  load_h16(w, (blk0 + t) * 32, valid, h);
  const float amax = absmax16<DT>(h);
  const uint16_t d16 = f32_to_f16_bits(amax / 7.0f);
  const float d = f16_bits_to_f32(d16);
  uint32_t qw[4];
  codes16<DT, false>(h, 0.0f, d, -8.0f, 7.0f, 136.0f, qw);
  if (valid) {
    *reinterpret_cast<uint16_t*>(stage + t * 18) = d16;
    lds_put16_a2(stage, t * 18 + 2, qw);
  }
  __syncthreads();
  const int64_t nb = nblocks - blk0 < kThreads ? nblocks - blk0 : kThreads;
  lds_to_global(stage, out + blk0 * 18, static_cast<int>(nb * 18));
}

// Threads 8s..8s+7 own super-block s (0..31) of the workgroup, thread j of
// the eight owning sub-block j.
template <int DT, bool AFFINE>
__global__ __launch_bounds__(kThreads) void k_quant_sb4_g(const void* __restrict__ w,
                                                          uint8_t* __restrict__ out,
                                                          int64_t nsb) {
  constexpr int B = AFFINE ? 148 : 138;
  constexpr int SBW = kThreads / 8;  // super-blocks per workgroup
  __shared__ uint4 stage4[SBW * B / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t sb0 = static_cast<int64_t>(blockIdx.x) * SBW;
  const int sl = t >> 3, j = t & 7;
  const bool valid = sb0 + sl < nsb;
  uint32_t h[16];
  load_h16(w, (sb0 + sl) * 256 + 32 * j, valid, h);
  uint8_t* blk = stage + sl * B;
  uint32_t qw[4];
  if constexpr (!AFFINE) {
    const float amax = absmax16<DT>(h);
    const float d = f16_bits_to_f32(f32_to_f16_bits(amax / 7.0f));
    codes16<DT, false>(h, 0.0f, d, -8.0f, 7.0f, 136.0f, qw);
    float smax = d;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) smax = __builtin_fmaxf(smax, __shfl_xor(smax, m, kWave));
    const uint16_t S16 = f32_to_f16_bits(smax / 127.0f);
    const int sc = code_of(d, f16_bits_to_f32(S16), -127.0f, 127.0f);
    if (valid) {
      if (j == 0) *reinterpret_cast<uint16_t*>(blk) = S16;
      blk[2 + j] = static_cast<uint8_t>(sc);
      lds_put16_a2(blk, 10 + 16 * j, qw);
    }
  } else {
    float mn, mx;
    minmax16<DT>(h, mn, mx);
    const float s = f16_bits_to_f32(f32_to_f16_bits((mx - mn) / 15.0f));
    const float a = f16_bits_to_f32(f32_to_f16_bits(mn));
    codes16<DT, true>(h, a, s, 0.0f, 15.0f, 0.0f, qw);
    float smax = s, amax = __builtin_fabsf(a);
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      smax = __builtin_fmaxf(smax, __shfl_xor(smax, m, kWave));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, kWave));
    }
    const uint16_t Ss16 = f32_to_f16_bits(smax / 127.0f);
    const uint16_t Sa16 = f32_to_f16_bits(amax / 127.0f);
    const int sc = code_of(s, f16_bits_to_f32(Ss16), -127.0f, 127.0f);
    const int ac = code_of(a, f16_bits_to_f32(Sa16), -127.0f, 127.0f);
    if (valid) {
      if (j == 0) reinterpret_cast<uint32_t*>(blk)[0] = Ss16 | (static_cast<uint32_t>(Sa16) << 16);
      blk[4 + j] = static_cast<uint8_t>(sc);
      blk[12 + j] = static_cast<uint8_t>(ac);
      uint32_t* qd = reinterpret_cast<uint32_t*>(blk + 20 + 16 * j);  // 4-byte aligned
#pragma unroll
      for (int q = 0; q < 4; q++) qd[q] = qw[q];
    }
  }
  __syncthreads();
  const int64_t ns = nsb - sb0 < SBW ? nsb - sb0 : SBW;
  lds_to_global(stage, out + sb0 * B, static_cast<int>(ns * B));
}

// ------------------------------------------------------------------ Q4_K
// Sub-block range lo = min(0, min w), hi = max w; first-level scale
// (hi - lo)/15 and min -lo; d and dmin are fp16 of the largest of each over
// 63; the 6-bit codes are taken against the stored d and dmin, the 4-bit codes
// of (w + M_j)/S_j against the rebuilt S_j = d*s_j and M_j = dmin*m_j (both
// exact in fp32).  Header dwords: d | dmin << 16, then the sixteen 6-bit
// fields (s_0..s_7, m_0..m_7) at bits 6i of the next three dwords.  Each lane
// forms the bits of its own sub-block's two fields; an OR over the lanes of a
// super-block assembles the words.
__device__ __forceinline__ void q4k_field_bits(uint32_t s6, uint32_t m6, int j, uint32_t& h1,
                                               uint32_t& h2, uint32_t& h3) {
  const uint64_t fs = static_cast<uint64_t>(s6) << (6 * j);  // field bits 0..47
  const uint64_t fm = static_cast<uint64_t>(m6) << (6 * j);  // field bits 48..95, shifted down 48
  h1 = static_cast<uint32_t>(fs);
  h2 = static_cast<uint32_t>(fs >> 32) | (static_cast<uint32_t>(fm) << 16);
  h3 = static_cast<uint32_t>(fm >> 16);
}

// The second level of one super-block, given this lane's sub-block scale and
// min and the OR/max partners at lane distances m0, 2*m0, ... < mend.
struct Q4kMeta {
  uint32_t d16, m16, s6, m6;
  float S, M;
};
template <int M0, int MEND>
__device__ __forceinline__ Q4kMeta q4k_meta(float sc, float mn) {
  float smax = sc, mmax = mn;
#pragma unroll
  for (int m = M0; m < MEND; m <<= 1) {
    smax = __builtin_fmaxf(smax, __shfl_xor(smax, m, kWave));
    mmax = __builtin_fmaxf(mmax, __shfl_xor(mmax, m, kWave));
  }
  Q4kMeta r;
  // maxima are >= 0; a zero may carry a sign here, the stored value has none
  r.d16 = f32_to_f16_bits(smax / 63.0f) & 0x7fffu;
  r.m16 = f32_to_f16_bits(mmax / 63.0f) & 0x7fffu;
  const float D = f16_bits_to_f32(r.d16), Dm = f16_bits_to_f32(r.m16);
  r.s6 = static_cast<uint32_t>(code_of(sc, D, 0.0f, 63.0f));
  r.m6 = static_cast<uint32_t>(code_of(mn, Dm, 0.0f, 63.0f));
  r.S = D * static_cast<float>(r.s6);
  r.M = Dm * static_cast<float>(r.m6);
  return r;
}

template <int M0, int MEND>
__device__ __forceinline__ uint4 q4k_header(const Q4kMeta& q, int j) {
  uint32_t h1, h2, h3;
  q4k_field_bits(q.s6, q.m6, j, h1, h2, h3);
#pragma unroll
  for (int m = M0; m < MEND; m <<= 1) {
    h1 |= __shfl_xor(h1, m, kWave);
    h2 |= __shfl_xor(h2, m, kWave);
    h3 |= __shfl_xor(h3, m, kWave);
  }
  return make_uint4(q.d16 | (q.m16 << 16), h1, h2, h3);
}

// fp32 input, 8 weights per thread: threads 32s..32s+31 own super-block s,
// thread v holding weights 8v..8v+7 (sub-block v/4).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_q4k(const void* __restrict__ w,
                                                        uint8_t* __restrict__ out, int64_t nsb) {
  constexpr int B = 144;
  __shared__ uint4 stage4[8 * B / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t sb0 = static_cast<int64_t>(blockIdx.x) * 8;
  const int sl = t >> 5, v = t & 31, j = v >> 2, u = v & 3;
  const bool valid = sb0 + sl < nsb;
  float x[8];
  load8<DT>(w, (sb0 + sl) * 256 + v * 8, valid, x);
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < 8; i++) {
    lo = __builtin_fminf(lo, x[i]);
    hi = __builtin_fmaxf(hi, x[i]);
  }
  lo = group_min<4>(lo);
  hi = group_max<4>(hi);
  lo = lo < 0.0f ? lo : 0.0f;  // the range always reaches down to 0
  const Q4kMeta q = q4k_meta<4, 32>((hi - lo) / 15.0f, -lo);
  float xm[8];
#pragma unroll
  for (int i = 0; i < 8; i++) xm[i] = x[i] + q.M;
  int n[8];
  codes8(xm, q.S, 0.0f, 15.0f, n);
  const uint4 hd = q4k_header<4, 32>(q, j);
  uint32_t w0, w1;
  pack_group(n, w0, w1);
  if (valid) {
    if (v == 0) *reinterpret_cast<uint4*>(stage + sl * B) = hd;
    if (u < 2) *reinterpret_cast<uint2*>(stage + sl * B + 16 + 16 * j + 8 * u) = make_uint2(w0, w1);
  }
  __syncthreads();
  const int64_t ns = nsb - sb0 < 8 ? nsb - sb0 : 8;
  lds_to_global(stage, out + sb0 * B, static_cast<int>(ns * B));
}

// 16-bit input, one sub-block per thread: threads 8s..8s+7 own super-block s.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_q4k_g(const void* __restrict__ w,
                                                          uint8_t* __restrict__ out, int64_t nsb) {
  constexpr int B = 144;
  constexpr int SBW = kThreads / 8;
  __shared__ uint4 stage4[SBW * B / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t sb0 = static_cast<int64_t>(blockIdx.x) * SBW;
  const int sl = t >> 3, j = t & 7;
  const bool valid = sb0 + sl < nsb;
  uint32_t h[16];
  load_h16(w, (sb0 + sl) * 256 + 32 * j, valid, h);
  float lo, hi;
  minmax16<DT>(h, lo, hi);
  lo = lo < 0.0f ? lo : 0.0f;
  const Q4kMeta q = q4k_meta<1, 8>((hi - lo) / 15.0f, -lo);
  uint32_t qw[4];
  codes16<DT, true>(h, -q.M, q.S, 0.0f, 15.0f, 0.0f, qw);  // dividends fl(x + M)
  const uint4 hd = q4k_header<1, 8>(q, j);
  if (valid) {
    uint8_t* blk = stage + sl * B;
    if (j == 0) *reinterpret_cast<uint4*>(blk) = hd;
    *reinterpret_cast<uint4*>(blk + 16 + 16 * j) = make_uint4(qw[0], qw[1], qw[2], qw[3]);
  }
  __syncthreads();
  const int64_t ns = nsb - sb0 < SBW ? nsb - sb0 : SBW;
  lds_to_global(stage, out + sb0 * B, static_cast<int>(ns * B));
}

// ------------------------------------------- group-128 W4 and int8 activations
// TurboQuant article, sections 2.1-2.2: per row, groups of 128 weights with
// one symmetric scale from their own maximum, 4-bit codes; 8-bit activations.
// Weight layout (planar): the code plane (byte j of group G holds weight
// 128G+j in its low nibble and 128G+64+j in its high nibble, codes stored +8)
// followed by the fp16 scale plane, one entry per group.  The flat group
// index G = row * k/128 + g addresses both planes.  A workgroup takes 16
// groups, 16 threads per group with 8 weights each: thread u < 8 holds
// weights 8u..8u+7 (low nibbles of bytes 8u..8u+7), thread u + 8 the weights
// 64 further (their high nibbles).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_w4g128(const void* __restrict__ w,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           int64_t ngroups) {
  const int t = threadIdx.x;
  const int64_t G = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (t >> 4);
  const int u = t & 15;
  const bool valid = G < ngroups;
  float v[8];
  load8<DT>(w, G * 128 + u * 8, valid, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  amax = group_max<16>(amax);
  const uint16_t d16 = f32_to_f16_bits(amax / 7.0f);
  int n[8];
  codes8(v, f16_bits_to_f32(d16), -8.0f, 7.0f, n);
  const uint32_t a0 = (n[0] + 8) | ((n[1] + 8) << 8) | ((n[2] + 8) << 16) | ((n[3] + 8) << 24);
  const uint32_t a1 = (n[4] + 8) | ((n[5] + 8) << 8) | ((n[6] + 8) << 16) | ((n[7] + 8) << 24);
  const uint32_t b0 = __shfl_xor(a0, 8, kWave), b1 = __shfl_xor(a1, 8, kWave);
  if (valid && u < 8) *reinterpret_cast<uint2*>(codes + G * 64 + 8 * u) = make_uint2(a0 | (b0 << 4), a1 | (b1 << 4));
  if (valid && u == 0) *reinterpret_cast<uint16_t*>(scales + 2 * G) = d16;
}

template <int OT>
__global__ __launch_bounds__(kThreads) void k_dequant_w4g128(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             void* __restrict__ out, int64_t ngroups) {
  const int t = threadIdx.x;
  const int64_t G = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (t >> 4);
  const int u = t & 15;
  if (G >= ngroups) return;
  const float d = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(scales + 2 * G));
  const uint2 c = *reinterpret_cast<const uint2*>(codes + G * 64 + 8 * (u & 7));
  const int sh = (u >> 3) * 4;  // high nibbles for the upper 64 weights
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    y[i] = d * static_cast<float>(static_cast<int>((c.x >> (8 * i + sh)) & 15u) - 8);
    y[4 + i] = d * static_cast<float>(static_cast<int>((c.y >> (8 * i + sh)) & 15u) - 8);
  }
  store8<OT>(out, G * 128 + 8 * u, y);
}

// One workgroup per token (row of X): the row's largest magnitude, then
// codes clamp(round_half_away(x / s), -127, 127) with s = max/127 (fp32).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_act_i8(const void* __restrict__ x,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ scale, int64_t k) {
  __shared__ float red[kThreads / kWave];
  const int64_t row = blockIdx.x;
  float amax = 0.0f;
  for (int64_t i = threadIdx.x * 8; i < k; i += kThreads * 8) {
    float v[8];
    load8<DT>(x, row * k + i, true, v);
#pragma unroll
    for (int j = 0; j < 8; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) scale[row] = s;
  for (int64_t i = threadIdx.x * 8; i < k; i += kThreads * 8) {
    float v[8];
    load8<DT>(x, row * k + i, true, v);
    int n[8];
    codes8(v, s, -127.0f, 127.0f, n);
    const uint32_t a0 = (n[0] & 0xff) | ((n[1] & 0xff) << 8) | ((n[2] & 0xff) << 16) | (static_cast<uint32_t>(n[3]) << 24);
    const uint32_t a1 = (n[4] & 0xff) | ((n[5] & 0xff) << 8) | ((n[6] & 0xff) << 16) | (static_cast<uint32_t>(n[7]) << 24);
    *reinterpret_cast<uint2*>(xq + row * k + i) = make_uint2(a0, a1);
  }
}

// ------------------------------------------------------------- dequantize
// 4-bit code of weight i (0..7 of this thread's 8) from the staged qs bytes of
// a 32-weight group: threads u = 0,1 take low nibbles of bytes 8u..8u+7,
// threads u = 2,3 the high nibbles of bytes 8(u-2)..8(u-2)+7.
__device__ __forceinline__ void group_codes(const uint8_t* qs, int u, int c[8]) {
  const uint8_t* p = qs + 8 * (u & 1);
  const int sh = (u >> 1) * 4;
#pragma unroll
  for (int i = 0; i < 8; i++) c[i] = (p[i] >> sh) & 0xF;
}

template <int FMT, int OT>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ blocks,
                                                      void* __restrict__ out, int64_t nblocks) {
  constexpr int E = FMT == QBLK_Q4_0 ? 32 : 256;
  constexpr int B = FMT == QBLK_Q4_0 ? 18 : FMT == QBLK_SB4 ? 138 : FMT == QBLK_Q4_K ? 144 : 148;
  constexpr int PER_WG = kWgWeights / E;  // 64 or 8
  __shared__ uint4 stage4[PER_WG * B / 16];
  uint8_t* stage = reinterpret_cast<uint8_t*>(stage4);
  const int t = threadIdx.x;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * PER_WG;
  const int64_t ng = nblocks - g0 < PER_WG ? nblocks - g0 : PER_WG;
  global_to_lds(blocks + g0 * B, stage, static_cast<int>(ng * B));
  __syncthreads();
  const int gl = t / (E / 8);  // block of this thread inside the workgroup
  if (gl >= ng) return;
  const uint8_t* blk = stage + gl * B;
  const int u = t & 3;
  int c[8];
  float y[8];
  if constexpr (FMT == QBLK_Q4_0) {
    const float d = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(blk));
    group_codes(blk + 2, u, c);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = d * static_cast<float>(c[i] - 8);
  } else if constexpr (FMT == QBLK_SB4) {
    const int j = (t & 31) >> 2;
    const float S = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(blk));
    const float sj = S * static_cast<float>(static_cast<int8_t>(blk[2 + j]));
    group_codes(blk + 10 + 16 * j, u, c);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = sj * static_cast<float>(c[i] - 8);
  } else if constexpr (FMT == QBLK_Q4_K) {
    const int j = (t & 31) >> 2;
    const uint4 hd = *reinterpret_cast<const uint4*>(blk);
    const float S = f16_bits_to_f32(hd.x & 0xffffu) * static_cast<float>(q4k_scale6(hd.y, hd.z, j));
    const float M = f16_bits_to_f32(hd.x >> 16) * static_cast<float>(q4k_min6(hd.z, hd.w, j));
    group_codes(blk + 16 + 16 * j, u, c);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float p = S * static_cast<float>(c[i]);  // exact
      y[i] = p - M;
    }
  } else {
    const int j = (t & 31) >> 2;
    const uint32_t hdr = *reinterpret_cast<const uint32_t*>(blk);
    const float sj = f16_bits_to_f32(hdr & 0xffffu) * static_cast<float>(static_cast<int8_t>(blk[4 + j]));
    const float aj = f16_bits_to_f32(hdr >> 16) * static_cast<float>(static_cast<int8_t>(blk[12 + j]));
    group_codes(blk + 20 + 16 * j, u, c);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float p = sj * static_cast<float>(c[i]);
      y[i] = p + aj;
    }
  }
  store8<OT>(out, (g0 + gl) * E + (t % (E / 8)) * 8, y);
}

// Bytes per input or output element of a float type id.
inline int64_t elem_bytes(int t) { return t == QBLK_F32 ? 4 : 2; }

// Workgroups for `units` units of `per_wg` each (one launch's piece).
inline unsigned wgs(int64_t units, int64_t per_wg) { return static_cast<unsigned>((units + per_wg - 1) / per_wg); }

}  // namespace

// ------------------------------------------------------------- launchers
// Every launcher walks a flat sequence of independent blocks (or rows); a
// sequence longer than one dispatch can hold runs in pieces of whole
// workgroups, each with its pointers moved to its first block.
hipError_t launch_quantize_q4_0(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                hipStream_t s) {
  const int64_t nb = rows * k / 32;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* out = static_cast<uint8_t*>(blocks);
  const int64_t es = elem_bytes(wt);
  // fp32: 8 weights per thread (32-byte coalesced loads), 64 blocks per
  // workgroup; 16-bit inputs: one 32-weight block per thread (64-byte loads)
  const int64_t per = wt == QBLK_F32 ? kWgWeights / 32 : kThreads;
  if (log_enabled())
    log_launch("quantize %s in=%d rows=%lld k=%lld grid=%u", wt == QBLK_F32 ? "k_quant_q4_0" : "k_quant_q4_0_g", wt,
               (long long)rows, (long long)k, wgs(nb, per));
  return in_pieces(nb, per, kThreads, [&](int64_t b0, int64_t n) {
    const void* wp = wb + b0 * 32 * es;
    uint8_t* op = out + b0 * 18;
    if (wt == QBLK_F32) hipLaunchKernelGGL(k_quant_q4_0<QBLK_F32>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else if (wt == QBLK_F16) hipLaunchKernelGGL(k_quant_q4_0_g<QBLK_F16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else hipLaunchKernelGGL(k_quant_q4_0_g<QBLK_BF16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    return hipGetLastError();
  });
}

hipError_t launch_quantize_q4_0_ref(const float* w, int64_t rows, int64_t k, void* blocks,
                                    hipStream_t s) {
  const int64_t nb = rows * k / 32, per = kWgWeights / 32;
  if (log_enabled())
    log_launch("quantize k_quant_q4_0_ref rows=%lld k=%lld grid=%u", (long long)rows, (long long)k, wgs(nb, per));
  return in_pieces(nb, per, kThreads, [&](int64_t b0, int64_t n) {
    hipLaunchKernelGGL(k_quant_q4_0_ref, dim3(wgs(n, per)), dim3(kThreads), 0, s, w + b0 * 32,
                       static_cast<uint8_t*>(blocks) + b0 * 18, n);
    return hipGetLastError();
  });
}

template <bool A>
static hipError_t launch_sb4_t(const void* w, int wt, int64_t nsb, uint8_t* out, hipStream_t s) {
  constexpr int64_t B = A ? 148 : 138;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const int64_t es = elem_bytes(wt);
  // fp32: 8 weights per thread, 8 super-blocks per workgroup; 16-bit inputs:
  // one sub-block per thread (64-byte loads), 32 super-blocks per workgroup
  const int64_t per = wt == QBLK_F32 ? 8 : kThreads / 8;
  return in_pieces(nsb, per, kThreads, [&](int64_t b0, int64_t n) {
    const void* wp = wb + b0 * 256 * es;
    uint8_t* op = out + b0 * B;
    if (wt == QBLK_F32) hipLaunchKernelGGL((k_quant_sb4<QBLK_F32, A>), dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else if (wt == QBLK_F16) hipLaunchKernelGGL((k_quant_sb4_g<QBLK_F16, A>), dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else hipLaunchKernelGGL((k_quant_sb4_g<QBLK_BF16, A>), dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    return hipGetLastError();
  });
}

hipError_t launch_quantize_sb4(const void* w, int wt, int64_t rows, int64_t k, int affine,
                               void* blocks, hipStream_t s) {
  const int64_t nsb = rows * k / 256;
  uint8_t* out = static_cast<uint8_t*>(blocks);
  if (log_enabled())
    log_launch("quantize %s affine=%d in=%d rows=%lld k=%lld super-blocks=%lld",
               wt == QBLK_F32 ? "k_quant_sb4" : "k_quant_sb4_g", affine, wt, (long long)rows, (long long)k,
               (long long)nsb);
  if (affine) return launch_sb4_t<true>(w, wt, nsb, out, s);
  return launch_sb4_t<false>(w, wt, nsb, out, s);
}

hipError_t launch_quantize_w4g128(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                  hipStream_t s) {
  const int64_t ng = rows * k / 128, per = kThreads / 16;  // 16 threads per 128-weight group
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* codes = static_cast<uint8_t*>(blocks);
  uint8_t* scales = codes + rows * k / 2;
  const int64_t es = elem_bytes(wt);
  if (log_enabled())
    log_launch("quantize k_quant_w4g128 in=%d rows=%lld k=%lld grid=%u", wt, (long long)rows, (long long)k, wgs(ng, per));
  return in_pieces(ng, per, kThreads, [&](int64_t g0, int64_t n) {
    const void* wp = wb + g0 * 128 * es;
    uint8_t* cp = codes + g0 * 64;
    uint8_t* sp = scales + g0 * 2;
    if (wt == QBLK_F32) hipLaunchKernelGGL(k_quant_w4g128<QBLK_F32>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, cp, sp, n);
    else if (wt == QBLK_F16) hipLaunchKernelGGL(k_quant_w4g128<QBLK_F16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, cp, sp, n);
    else hipLaunchKernelGGL(k_quant_w4g128<QBLK_BF16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, cp, sp, n);
    return hipGetLastError();
  });
}

hipError_t launch_quantize_act_i8(const void* x, int xt, int64_t n, int64_t k, int8_t* xq, float* scale,
                                  hipStream_t s) {
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const int64_t es = elem_bytes(xt);
  if (log_enabled()) log_launch("quantize k_quant_act_i8 in=%d n=%lld k=%lld grid=%lld", xt, (long long)n, (long long)k, (long long)n);
  // one workgroup per row
  return in_pieces(n, 1, kThreads, [&](int64_t r0, int64_t nr) {
    const void* xp = xb + r0 * k * es;
    int8_t* qp = xq + r0 * k;
    float* sp = scale + r0;
    const dim3 g(static_cast<unsigned>(nr));
    if (xt == QBLK_F32) hipLaunchKernelGGL(k_quant_act_i8<QBLK_F32>, g, dim3(kThreads), 0, s, xp, qp, sp, k);
    else if (xt == QBLK_F16) hipLaunchKernelGGL(k_quant_act_i8<QBLK_F16>, g, dim3(kThreads), 0, s, xp, qp, sp, k);
    else hipLaunchKernelGGL(k_quant_act_i8<QBLK_BF16>, g, dim3(kThreads), 0, s, xp, qp, sp, k);
    return hipGetLastError();
  });
}

hipError_t launch_quantize_q4_k(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                hipStream_t s) {
  const int64_t nsb = rows * k / 256;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* out = static_cast<uint8_t*>(blocks);
  const int64_t es = elem_bytes(wt);
  const int64_t per = wt == QBLK_F32 ? 8 : kThreads / 8;
  if (log_enabled())
    log_launch("quantize %s in=%d rows=%lld k=%lld super-blocks=%lld", wt == QBLK_F32 ? "k_quant_q4k" : "k_quant_q4k_g",
               wt, (long long)rows, (long long)k, (long long)nsb);
  return in_pieces(nsb, per, kThreads, [&](int64_t b0, int64_t n) {
    const void* wp = wb + b0 * 256 * es;
    uint8_t* op = out + b0 * 144;
    if (wt == QBLK_F32) hipLaunchKernelGGL(k_quant_q4k<QBLK_F32>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else if (wt == QBLK_F16) hipLaunchKernelGGL(k_quant_q4k_g<QBLK_F16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    else hipLaunchKernelGGL(k_quant_q4k_g<QBLK_BF16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, wp, op, n);
    return hipGetLastError();
  });
}

template <int FMT>
static hipError_t launch_deq_t(const uint8_t* b, int64_t nblk, void* out, int ot, hipStream_t s) {
  constexpr int64_t E = FMT == QBLK_Q4_0 ? 32 : 256;
  constexpr int64_t B = FMT == QBLK_Q4_0 ? 18 : FMT == QBLK_SB4 ? 138 : FMT == QBLK_Q4_K ? 144 : 148;
  constexpr int64_t per = kWgWeights / E;  // blocks per workgroup
  uint8_t* ob = static_cast<uint8_t*>(out);
  const int64_t es = elem_bytes(ot);
  return in_pieces(nblk, per, kThreads, [&](int64_t b0, int64_t n) {
    const uint8_t* bp = b + b0 * B;
    void* op = ob + b0 * E * es;
    if (ot == QBLK_F32) hipLaunchKernelGGL((k_dequant<FMT, QBLK_F32>), dim3(wgs(n, per)), dim3(kThreads), 0, s, bp, op, n);
    else if (ot == QBLK_F16) hipLaunchKernelGGL((k_dequant<FMT, QBLK_F16>), dim3(wgs(n, per)), dim3(kThreads), 0, s, bp, op, n);
    else hipLaunchKernelGGL((k_dequant<FMT, QBLK_BF16>), dim3(wgs(n, per)), dim3(kThreads), 0, s, bp, op, n);
    return hipGetLastError();
  });
}

hipError_t launch_dequant(int fmt, const void* blocks, int64_t rows, int64_t k, void* out, int ot,
                          hipStream_t s) {
  const uint8_t* b = static_cast<const uint8_t*>(blocks);
  if (log_enabled())
    log_launch("dequant %s fmt=%d out=%d rows=%lld k=%lld", fmt == QBLK_W4G128 ? "k_dequant_w4g128" : "k_dequant", fmt,
               ot, (long long)rows, (long long)k);
  if (fmt == QBLK_W4G128) {
    const int64_t ng = rows * k / 128, per = kThreads / 16;
    const uint8_t* sc = b + rows * k / 2;
    uint8_t* ob = static_cast<uint8_t*>(out);
    const int64_t es = elem_bytes(ot);
    return in_pieces(ng, per, kThreads, [&](int64_t g0, int64_t n) {
      const uint8_t* cp = b + g0 * 64;
      const uint8_t* sp = sc + g0 * 2;
      void* op = ob + g0 * 128 * es;
      if (ot == QBLK_F32) hipLaunchKernelGGL(k_dequant_w4g128<QBLK_F32>, dim3(wgs(n, per)), dim3(kThreads), 0, s, cp, sp, op, n);
      else if (ot == QBLK_F16) hipLaunchKernelGGL(k_dequant_w4g128<QBLK_F16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, cp, sp, op, n);
      else hipLaunchKernelGGL(k_dequant_w4g128<QBLK_BF16>, dim3(wgs(n, per)), dim3(kThreads), 0, s, cp, sp, op, n);
      return hipGetLastError();
    });
  }
  if (fmt == QBLK_Q4_0) return launch_deq_t<QBLK_Q4_0>(b, rows * k / 32, out, ot, s);
  if (fmt == QBLK_SB4) return launch_deq_t<QBLK_SB4>(b, rows * k / 256, out, ot, s);
  if (fmt == QBLK_Q4_K) return launch_deq_t<QBLK_Q4_K>(b, rows * k / 256, out, ot, s);
  return launch_deq_t<QBLK_SB4_AFFINE>(b, rows * k / 256, out, ot, s);
}

}  // namespace qblk
