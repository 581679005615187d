// qblk_gemm.hip -- small-batch (prefill) product Y = X W^T on gfx950 matrix
// cores, W in super-blocks (Type 0), X bf16 (n x k, token-major), Y fp32 (n x m).
//
// What is computed: Y[t,i] = sum_k X[t,k] W[i,k] with W[i,k] = (S*sc_j)*(code-8)
// ("GGUF K-quants" blog, "套娃" step 5; code offset from "GGUF 量化内幕 第4章
// Q4_0" 4.2.2).
//
// One v_mfma_f32_16x16x32_bf16 spans K = 32, exactly one sub-block, so the
// weight operand holds the exact integers (code - 8) in bf16 and the
// sub-block's fp32 scale S*sc_j multiplies each 16x16 partial product before
// it is added to the fp32 accumulator.  (Rounding the scaled weights to bf16
// instead would break the 2e-5 relative error bound.)
//
// Operand layout of the 16x16x32 MFMA: lane l holds row (l % 16) of A and
// column (l % 16) of B, each with 8 consecutive-in-register k values of the
// k-group (l / 16); lane l receives D[4*(l/16) + r][l % 16], r = 0..3.  Only
// A and B having the same k assignment matters, so lane group g takes the
// codes of qs bytes 4g..4g+3 of the sub-block -- weights 4g..4g+3 (low
// nibbles) and 4g+16..4g+19 (high nibbles) -- and the same eight X entries.
//
// Tiling: A = X (16 tokens per tile), B = W^T (16 weight rows per tile), so a
// lane's outputs share one weight row and one scale.  A workgroup of 4 waves
// owns 64*TM weight rows (16*TM per wave) and 16*TN tokens; the X tile of the
// current super-block (16*TN x 256 bf16) is staged in LDS once and read by all
// four waves; weight codes go from HBM straight to registers.
#include "qblk_device.h"
#include "qblk_launch.h"

namespace qblk {
namespace {

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kLdsRow = 256 + 8;  // bf16 per staged X row (+16 B pad against bank conflicts)

__device__ __forceinline__ uint32_t pack_bf16_ints(float a, float b) {
  // a, b are small integers: their bf16 patterns are the upper halves exactly
  return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xffff0000u);
}

// (code - 8) of weights 4g..4g+3 and 4g+16..4g+19 as 8 bf16 values.
__device__ __forceinline__ bf16x8v_t decode_codes(uint32_t q) {
  float lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    lo[i] = static_cast<float>((q >> (8 * i)) & 0xFu) - 8.0f;
    hi[i] = static_cast<float>((q >> (8 * i + 4)) & 0xFu) - 8.0f;
  }
  const uint4 w = make_uint4(pack_bf16_ints(lo[0], lo[1]), pack_bf16_ints(lo[2], lo[3]),
                             pack_bf16_ints(hi[0], hi[1]), pack_bf16_ints(hi[2], hi[3]));
  return __builtin_bit_cast(bf16x8v_t, w);
}

template <int TM, int TN>
__global__ __launch_bounds__(kThreads) void k_gemm_sb4(const uint8_t* __restrict__ W,
                                                       const uint16_t* __restrict__ X,
                                                       float* __restrict__ Y, int M, int K,
                                                       int N) {
  constexpr int NT = 16 * TN;
  __shared__ uint4 xs4[NT * kLdsRow / 8];
  uint16_t* xs = reinterpret_cast<uint16_t*>(xs4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t mw = static_cast<int64_t>(blockIdx.x) * 64 * TM + wave * 16 * TM;
  const int n0 = blockIdx.y * NT;
  const int64_t rowbytes = static_cast<int64_t>(K / 256) * 138;
  const uint8_t* rowp[TM];
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
    int64_t m = mw + 16 * tm + l16;
    m = m < M ? m : M - 1;
    rowp[tm] = W + m * rowbytes;
  }
  float4_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; tm++)
#pragma unroll
    for (int tn = 0; tn < TN; tn++) acc[tm][tn] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};

  const int nsb = K / 256;
  for (int b = 0; b < nsb; b++) {
    __syncthreads();
    for (int i = threadIdx.x; i < NT * 32; i += kThreads) {
      const int r = i >> 5, c = i & 31;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n0 + r < N) v = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(n0 + r) * K + 256 * b + 8 * c);
      *reinterpret_cast<uint4*>(xs + r * kLdsRow + 8 * c) = v;
    }
    __syncthreads();
    // super-block header of each of this lane's weight rows
    float S[TM];
    uint32_t scw[TM][2];  // sc_0..sc_7 as bytes
#pragma unroll
    for (int tm = 0; tm < TM; tm++) {
      const uint8_t* p = rowp[tm] + static_cast<int64_t>(b) * 138;
      const uintptr_t a = reinterpret_cast<uintptr_t>(p);
      const u32x3_a4 h = *reinterpret_cast<const u32x3_a4*>(a & ~uintptr_t(3));
      const uint32_t sh = static_cast<uint32_t>(a & 3u);
      const uint32_t w0 = __builtin_amdgcn_alignbyte(h.y, h.x, sh);  // S16, sc0, sc1
      const uint32_t w1 = __builtin_amdgcn_alignbyte(h.z, h.y, sh);  // sc2..sc5
      const uint32_t w2 = h.z >> (8 * sh);                           // sc6, sc7
      S[tm] = f16_bits_to_f32(w0 & 0xffffu);
      scw[tm][0] = (w0 >> 16) | (w1 << 16);  // sc0..sc3
      scw[tm][1] = (w1 >> 16) | (w2 << 16);  // sc4..sc7
    }
#pragma unroll 2
    for (int j = 0; j < 8; j++) {
      bf16x8v_t Bop[TM];
      float scale[TM];
#pragma unroll
      for (int tm = 0; tm < TM; tm++) {
        const uint8_t* o = rowp[tm] + static_cast<int64_t>(b) * 138 + 10 + 16 * j + 4 * g;
        const uint32_t q = load_u16(o) | (load_u16(o + 2) << 16);
        Bop[tm] = decode_codes(q);
        const int8_t scj = static_cast<int8_t>((scw[tm][j >> 2] >> (8 * (j & 3))) & 0xffu);
        scale[tm] = S[tm] * static_cast<float>(scj);
      }
#pragma unroll
      for (int tn = 0; tn < TN; tn++) {
        const uint16_t* xr = xs + (16 * tn + l16) * kLdsRow + 32 * j + 4 * g;
        const uint2 a0 = *reinterpret_cast<const uint2*>(xr);
        const uint2 a1 = *reinterpret_cast<const uint2*>(xr + 16);
        const bf16x8v_t Aop = __builtin_bit_cast(bf16x8v_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
        for (int tm = 0; tm < TM; tm++) {
          const float4_t P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop, Bop[tm], zero, 0, 0, 0);
          float4_t& A = acc[tm][tn];
          A.x = __builtin_fmaf(scale[tm], P.x, A.x);
          A.y = __builtin_fmaf(scale[tm], P.y, A.y);
          A.z = __builtin_fmaf(scale[tm], P.z, A.z);
          A.w = __builtin_fmaf(scale[tm], P.w, A.w);
        }
      }
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
    const int64_t m = mw + 16 * tm + l16;
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; tn++) {
      const float v[4] = {acc[tm][tn].x, acc[tm][tn].y, acc[tm][tn].z, acc[tm][tn].w};
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int n = n0 + 16 * tn + 4 * g + r;
        if (n < N) Y[static_cast<int64_t>(n) * M + m] = v[r];
      }
    }
  }
}

template <int TM, int TN>
hipError_t launch_t(const void* blocks, int64_t m, int64_t k, const void* x, int64_t n, float* y,
                    hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((m + 64 * TM - 1) / (64 * TM)),
                  static_cast<unsigned>((n + 16 * TN - 1) / (16 * TN)));
  hipLaunchKernelGGL((k_gemm_sb4<TM, TN>), grid, dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                     static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       int64_t n, float* y, hipStream_t s) {
  (void)fmt;
  (void)xt;  // only QBLK_SB4 x QBLK_BF16 reaches this point
  if (n <= 16) return launch_t<1, 1>(blocks, m, k, x, n, y, s);
  if (n <= 32) return launch_t<1, 2>(blocks, m, k, x, n, y, s);
  if (n <= 64) return launch_t<1, 4>(blocks, m, k, x, n, y, s);
  return launch_t<2, 4>(blocks, m, k, x, n, y, s);
}

}  // namespace qblk
