// qblk_gemm.hip -- small-batch (prefill) product Y = X W^T on gfx950 matrix
// cores, W in any of the block formats, X bf16 (n x k, token-major), Y fp32
// (n x m).
//
// What is computed: Y[t,i] = sum_k X[t,k] W[i,k] with W[i,k] the rebuilt
// weight: Type 0 (S*sc_j)*(code-8) ("GGUF K-quants" blog, "套娃" step 5; code
// offset from "GGUF 量化内幕 第4章 Q4_0" 4.2.2), Q4_0 d*(code-8) (chapter 4.3),
// Type 1 (Ss*sc_j)*code + Sa*ac_j (blog, "套娃"), Q4_K (d*s_j)*code - dmin*m_j
// (chapter 4.6).  The affine formats are run as s*(code-8) + (8s + offset).
//
// One v_mfma_f32_16x16x32_bf16 spans K = 32, exactly one sub-block, so the
// weight operand holds the exact integers (code - 8)/16 in bf16 and the
// sub-block's fp32 scale 16*S*sc_j multiplies each 16x16 partial product
// before it is added to the fp32 accumulator.  (Rounding the scaled weights
// to bf16 instead would break the 2e-5 relative error bound.)  The codes are
// widened with v_cvt_off_f32_i4 (a 4-bit two's-complement field / 16; code
// XOR 8 is exactly code - 8 in that form), selecting bytes with SDWA, and
// packed with v_cvt_pk_bf16_f32 (exact: at most 4 significant bits).
//
// Operand layout of the 16x16x32 MFMA: lane l holds row (l % 16) of A and
// column (l % 16) of B, each with 8 k values of the k-group (l / 16); lane l
// receives D[4*(l/16) + r][l % 16], r = 0..3.  Only A and B having the same k
// assignment matters, so lane group g takes the codes of qs bytes 4g..4g+3 of
// the sub-block -- weights 4g..4g+3 (low nibbles) and 4g+16..4g+19 (high
// nibbles) -- and the same eight X entries.
//
// Tiling: A = X (16 tokens per tile), B = W^T (16 weight rows per tile), so a
// lane's outputs share one weight row and one scale.  Three kernels: up to 16
// tokens k_gemm_u (one stage of 64 rows x 2 super-blocks per workgroup, every
// load issued up front, K split over the grid), up to 64 tokens k_gemm_s (the
// same stages walked over the whole K range, the next stage's loads in flight
// while the current one is multiplied), beyond that k_gemm_w (32x32x16
// matrix ops, 128 rows x 128 tokens per workgroup; Type 1 and Q4_K 128 x 64
// when that fills the GPU better).  When a K range is split over a third
// grid dimension the partial products are added into Y (zeroed first); with
// reproducible products on (qblk_set_deterministic) nothing is split.
#include "qblk_device.h"
#include "qblk_launch.h"

namespace qblk {
namespace {

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
// A staged X row holds one super-block (256 bf16) in MFMA order: for sub-block
// j and k-group g, the 8 entries 32j+4g..+3 and 32j+16+4g..+3 sit together at
// 32j+8g, so a lane's A operand is one 16-byte LDS read.  Rows are padded by
// 16 bf16 (8 dwords) so that 16 rows read at the same column fall in
// different banks.
constexpr int kLdsRow = 256 + 16;

template <int BYTE>
__device__ __forceinline__ float off_i4(uint32_t v) {
  float r;
  if constexpr (BYTE == 0)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(v));
  else if constexpr (BYTE == 1)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(v));
  else if constexpr (BYTE == 2)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(v));
  else
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(v));
  return r;
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2v_t));
}

// (code - 8)/16 of weights 4g..4g+3 and 4g+16..4g+19 as 8 bf16 values.
__device__ __forceinline__ bf16x8v_t decode_codes(uint32_t q) {
  const uint32_t lo = q ^ 0x88888888u;  // each nibble n -> n XOR 8, a 4-bit field worth n-8
  const uint32_t hi = lo >> 4;           // high nibbles moved into the low half of each byte
  const uint4 w = make_uint4(pk_bf16(off_i4<0>(lo), off_i4<1>(lo)), pk_bf16(off_i4<2>(lo), off_i4<3>(lo)),
                             pk_bf16(off_i4<0>(hi), off_i4<1>(hi)), pk_bf16(off_i4<2>(hi), off_i4<3>(hi)));
  return __builtin_bit_cast(bf16x8v_t, w);
}

// sum over the 4 lanes of a quad (lanes 4i..4i+3)
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  return v;
}

// ---------------------------------------------------------------------------
// Wide tiles on the 32x32x16 matrix op.
//
// Operand layout of v_mfma_f32_32x32x16_bf16: lane l holds row (l % 32) of A
// and column (l % 32) of B, each with the 8 k values 8*(l / 32) .. +7 of the
// 16-wide step; lane l receives D[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.
// A sub-block (32 k) is two steps.  In natural k order, step 0 holds weights
// 0..15 of the sub-block (the low nibbles of its 16 code bytes) and step 1
// weights 16..31 (the high nibbles), so lane half h needs code bytes
// 8h..8h+7 -- low nibbles for step 0, high for step 1 -- and X entries
// 16*step + 8h .. +7, one contiguous 16-byte piece of the token row.
//
// A workgroup of 4 waves owns 128 weight rows (32 per wave, decoded in the
// wave's registers) and 32*T32 tokens shared by the 4 waves through LDS.
// X is staged per half super-block (128 k = 16 pieces of 16 bytes per token),
// double-buffered; piece c of token t is stored at slot c ^ (t % 16) so that
// the 16 lanes of one LDS read phase hit 16 different bank groups.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 16 codes (8 bytes, two dwords) -> (code - 8)/16 in bf16: low nibbles (step 0)
// and high nibbles (step 1), each in byte order.
__device__ __forceinline__ void decode16(uint32_t d0, uint32_t d1, bf16x8v_t& lo, bf16x8v_t& hi) {
  const uint32_t a = d0 ^ 0x88888888u, b = d1 ^ 0x88888888u;
  const uint32_t ah = a >> 4, bh = b >> 4;
  lo = __builtin_bit_cast(bf16x8v_t, make_uint4(pk_bf16(off_i4<0>(a), off_i4<1>(a)), pk_bf16(off_i4<2>(a), off_i4<3>(a)),
                                                pk_bf16(off_i4<0>(b), off_i4<1>(b)), pk_bf16(off_i4<2>(b), off_i4<3>(b))));
  hi = __builtin_bit_cast(bf16x8v_t, make_uint4(pk_bf16(off_i4<0>(ah), off_i4<1>(ah)), pk_bf16(off_i4<2>(ah), off_i4<3>(ah)),
                                                pk_bf16(off_i4<0>(bh), off_i4<1>(bh)), pk_bf16(off_i4<2>(bh), off_i4<3>(bh))));
}

// Per lane half h, the wide kernel needs code bytes 8h..8h+7 of every
// sub-block of a 256-weight group (16 codes), the 8 sub-block scales and, for
// Type 1, the offsets of sub-blocks 2q+h (q = 0..3).
struct SbRegsW {
  uint32_t code[8][2];
  float scale[8];  // 16 * (scale of sub-block j)
  float corr[4];   // Type 1: 8*s_j + a_j for j = 2q + h
};

template <int FMT>
struct GroupW;

template <>
struct GroupW<QBLK_SB4> {
  static constexpr int GB = 138, RAW = 3 + 8 * 3;
  // the header (dword aligned 12 bytes holding its 10 bytes, never before the
  // row's first byte since row starts are even) and, per sub-block, code
  // bytes 8h..8h+7 at A from the dwords at A & ~3: three of them for
  // sub-blocks 0..6 (the extra bytes belong to the next sub-block), for
  // sub-block 7 two dwords plus the 2 bytes at A+6, so nothing past the
  // super-block is read
  static __device__ __forceinline__ void load(const uint8_t* p, int h, uint32_t raw[RAW]) {
    // p - (p & 3) keeps the pointer's provenance, so these stay global loads
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
    const u32x3_a4 hd = *reinterpret_cast<const u32x3_a4*>(p - mis);
    raw[0] = hd.x;
    raw[1] = hd.y;
    raw[2] = hd.z;
    const uint8_t* a = p + 10 + 8 * h;                      // code bytes of sub-block 0
    const uint8_t* c = p - mis + ((mis + 10 + 8 * h) & ~3u);  // a & ~3
#pragma unroll
    for (int s = 0; s < 7; s++) {
      const u32x3_a4 v = *reinterpret_cast<const u32x3_a4*>(c + 16 * s);
      raw[3 + 3 * s] = v.x;
      raw[4 + 3 * s] = v.y;
      raw[5 + 3 * s] = v.z;
    }
    const u32x2_a4 v = *reinterpret_cast<const u32x2_a4*>(c + 16 * 7);
    raw[3 + 3 * 7] = v.x;
    raw[4 + 3 * 7] = v.y;
    raw[5 + 3 * 7] = load_u16(a + 16 * 7 + 6);
  }
  static __device__ __forceinline__ void finish(const uint8_t* p, int, const uint32_t raw[RAW], SbRegsW& r) {
    const uint32_t sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
    const uint32_t w0 = __builtin_amdgcn_alignbyte(raw[1], raw[0], sh);  // S16, sc0, sc1
    const uint32_t w1 = __builtin_amdgcn_alignbyte(raw[2], raw[1], sh);  // sc2..sc5
    const uint32_t w2 = raw[2] >> (8 * sh);                              // sc6, sc7
    const float S16 = f16_bits_to_f32(w0 & 0xffffu) * 16.0f;
    const uint32_t sc03 = (w0 >> 16) | (w1 << 16), sc47 = (w1 >> 16) | (w2 << 16);
    // code bytes start at p + 10 (+ 8h): offset (sh + 2) & 3 inside the aligned dwords
    const uint32_t cs = (sh + 2) & 3u;
#pragma unroll
    for (int s = 0; s < 8; s++) {
      r.code[s][0] = __builtin_amdgcn_alignbyte(raw[4 + 3 * s], raw[3 + 3 * s], cs);
      r.code[s][1] = __builtin_amdgcn_alignbyte(raw[5 + 3 * s], raw[4 + 3 * s], cs);
      const uint32_t word = s < 4 ? sc03 : sc47;
      const int8_t c = static_cast<int8_t>((word >> (8 * (s & 3))) & 0xffu);
      r.scale[s] = S16 * static_cast<float>(c);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) r.corr[q] = 0.0f;
  }
};

template <>
struct GroupW<QBLK_Q4_0> {
  // p is 4-byte aligned (rows are whole multiples of 144 bytes).  Block j
  // starts at 18j: for even j its code bytes 8h.. sit 2 bytes past a dword
  // boundary (three dwords from 18j+8h, ending at most at byte 128 of the
  // group), for odd j on one (two dwords, ending at most at byte 144).
  static constexpr int GB = 144, RAW = 8 + 4 * 3 + 4 * 2;
  static __device__ __forceinline__ void load(const uint8_t* p, int h, uint32_t raw[RAW]) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      raw[j] = *reinterpret_cast<const uint32_t*>(p + ((18 * j) & ~3));  // d16 in the low or high half
      uint32_t* r = raw + 8 + (j >> 1) * 5 + (j & 1) * 3;
      if (j & 1) {
        const u32x2_a4 v = *reinterpret_cast<const u32x2_a4*>(p + 18 * j + 2 + 8 * h);
        r[0] = v.x;
        r[1] = v.y;
      } else {
        const u32x3_a4 v = *reinterpret_cast<const u32x3_a4*>(p + 18 * j + 8 * h);
        r[0] = v.x;
        r[1] = v.y;
        r[2] = v.z;
      }
    }
  }
  static __device__ __forceinline__ void finish(const uint8_t*, int, const uint32_t raw[RAW], SbRegsW& r) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t d = (j & 1) ? raw[j] >> 16 : raw[j] & 0xffffu;
      r.scale[j] = f16_bits_to_f32(d) * 16.0f;
      const uint32_t* c = raw + 8 + (j >> 1) * 5 + (j & 1) * 3;
      if (j & 1) {
        r.code[j][0] = c[0];
        r.code[j][1] = c[1];
      } else {
        r.code[j][0] = __builtin_amdgcn_alignbyte(c[1], c[0], 2);
        r.code[j][1] = __builtin_amdgcn_alignbyte(c[2], c[1], 2);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; q++) r.corr[q] = 0.0f;
  }
};

template <>
struct GroupW<QBLK_SB4_AFFINE> {
  // 148-byte groups are dword aligned: header dwords 0..4, codes at 20 + 16j
  static constexpr int GB = 148, RAW = 5 + 8 * 2;
  static __device__ __forceinline__ void load(const uint8_t* p, int h, uint32_t raw[RAW]) {
    const u32x4_a4 hd = *reinterpret_cast<const u32x4_a4*>(p);
    raw[0] = hd.x;
    raw[1] = hd.y;
    raw[2] = hd.z;
    raw[3] = hd.w;
    raw[4] = *reinterpret_cast<const uint32_t*>(p + 16);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const u32x2_a4 v = *reinterpret_cast<const u32x2_a4*>(p + 20 + 16 * s + 8 * h);
      raw[5 + 2 * s] = v.x;
      raw[6 + 2 * s] = v.y;
    }
  }
  static __device__ __forceinline__ void finish(const uint8_t*, int h, const uint32_t raw[RAW], SbRegsW& r) {
    const float Ss = f16_bits_to_f32(raw[0] & 0xffffu), Sa = f16_bits_to_f32(raw[0] >> 16);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      r.code[s][0] = raw[5 + 2 * s];
      r.code[s][1] = raw[6 + 2 * s];
      const int8_t c = static_cast<int8_t>((raw[1 + (s >> 2)] >> (8 * (s & 3))) & 0xffu);
      r.scale[s] = (Ss * static_cast<float>(c)) * 16.0f;
    }
    // w = s*n + a = s*(n-8) + (8s + a): the codes decode to n-8 as for Type 0
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int sb = 2 * q + h;
      const int8_t c = static_cast<int8_t>((raw[1 + (sb >> 2)] >> (8 * (sb & 3))) & 0xffu);
      const int8_t o = static_cast<int8_t>((raw[3 + (sb >> 2)] >> (8 * (sb & 3))) & 0xffu);
      r.corr[q] = __builtin_fmaf(8.0f, Ss * static_cast<float>(c), Sa * static_cast<float>(o));
    }
  }
};

template <>
struct GroupW<QBLK_Q4_K> {
  // 144-byte groups are 16-byte aligned: header dwordx4, codes at 16 + 16j
  static constexpr int GB = 144, RAW = 4 + 8 * 2;
  static __device__ __forceinline__ void load(const uint8_t* p, int h, uint32_t raw[RAW]) {
    const uint4 hd = *reinterpret_cast<const uint4*>(p);
    raw[0] = hd.x;
    raw[1] = hd.y;
    raw[2] = hd.z;
    raw[3] = hd.w;
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + 16 + 16 * s + 8 * h);
      raw[4 + 2 * s] = v.x;
      raw[5 + 2 * s] = v.y;
    }
  }
  static __device__ __forceinline__ void finish(const uint8_t*, int h, const uint32_t raw[RAW], SbRegsW& r) {
    const float D = f16_bits_to_f32(raw[0] & 0xffffu), Dm = f16_bits_to_f32(raw[0] >> 16);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      r.code[s][0] = raw[4 + 2 * s];
      r.code[s][1] = raw[5 + 2 * s];
      r.scale[s] = (D * static_cast<float>(q4k_scale6(raw[1], raw[2], s))) * 16.0f;
    }
    // w = S*n - M = S*(n-8) + (8S - M)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int sb = 2 * q + h;
      const float S = D * static_cast<float>(q4k_scale6(raw[1], raw[2], sb));
      r.corr[q] = __builtin_fmaf(8.0f, S, -(Dm * static_cast<float>(q4k_min6(raw[2], raw[3], sb))));
    }
  }
};

template <int FMT, int T32, int OCC, bool SPLIT>
__global__ __launch_bounds__(kThreads, OCC) void k_gemm_w(const uint8_t* __restrict__ W,
                                                          const uint16_t* __restrict__ X,
                                                          float* __restrict__ Y, int M, int K, int N,
                                                          int sb_per_split) {
  constexpr int NT = 32 * T32;             // tokens per workgroup
  constexpr int kPieces = NT * 16;         // 16-byte pieces per stage (128 k per token)
  constexpr int kPer = kPieces / kThreads; // pieces moved per thread per stage
  static_assert(kPieces % kThreads == 0, "stage must split evenly over the workgroup");
  using G = GroupW<FMT>;
  constexpr bool AFFINE = FMT == QBLK_SB4_AFFINE || FMT == QBLK_Q4_K;
  __shared__ uint4 xs[2][kPieces];
  __shared__ float xsum[2][AFFINE ? NT * 4 : 1];  // Type 1: sum(x) [token][sub-block of the stage]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j32 = lane & 31, h = lane >> 5;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + j32;
  const int n0 = blockIdx.y * NT;
  const int nsb = K / 256;
  const int b_begin = SPLIT ? blockIdx.z * sb_per_split : 0;
  const int b_end = SPLIT ? min(nsb, b_begin + sb_per_split) : nsb;
  const int64_t rowbytes = static_cast<int64_t>(nsb) * G::GB;
  const uint8_t* rowp = W + (m < M ? m : M - 1) * rowbytes;

  // stage q = 2*b + half: thread t moves pieces t, t+256, ...; piece i of the
  // stage is token i/16, 16-byte piece i%16 of that token's 128 k, so the
  // thread's piece i is token (t >> 4) + 16 i, piece t & 15 (token offsets in
  // 64 bits: a row of K bf16 is up to 4 GiB).  Tokens past N read the last
  // token's row instead: their products are never stored.
  const int tlast = N - 1 - n0;
  const uint8_t* xtile =
      reinterpret_cast<const uint8_t*>(X + static_cast<int64_t>(n0) * K) + 16 * (threadIdx.x & 15);
  auto load_x = [&](int q, uint4 xv[kPer]) {
    const uint8_t* xq = xtile + 256 * q;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int t = min(static_cast<int>(threadIdx.x >> 4) + 16 * i, tlast);
      xv[i] = *reinterpret_cast<const uint4*>(xq + static_cast<uint64_t>(t) * (2u * static_cast<uint32_t>(K)));
    }
  };
  auto store_x = [&](int buf, const uint4 xv[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = threadIdx.x + i * kThreads;
      const int t = c >> 4, pc = c & 15;
      xs[buf][t * 16 + (pc ^ (t & 15))] = xv[i];
      if constexpr (AFFINE) {
        // the 4 pieces of a sub-block sit on 4 adjacent lanes; products with
        // 1.0 are exact, the sums fp32
        const bf16x2v_t one = __builtin_bit_cast(bf16x2v_t, 0x3f803f80u);
        float part = 0.0f;
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, xv[i].x), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, xv[i].y), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, xv[i].z), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, xv[i].w), one, part, false);
        part = quad_sum(part);
        if ((c & 3) == 0) xsum[buf][t * 4 + (pc >> 2)] = part;
      }
    }
  };

  f32x16_t acc[T32];
#pragma unroll
  for (int tt = 0; tt < T32; tt++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[tt][r] = 0.0f;
  f32x16_t zero;
#pragma unroll
  for (int r = 0; r < 16; r++) zero[r] = 0.0f;

  uint4 xv[kPer];
  uint32_t raw[G::RAW];
  SbRegsW cur;
  if (b_begin < b_end) {
    load_x(2 * b_begin, xv);
    G::load(rowp + static_cast<int64_t>(b_begin) * G::GB, h, raw);
    store_x(0, xv);
    G::finish(rowp + static_cast<int64_t>(b_begin) * G::GB, h, raw, cur);
  }

  // Stage hs of super-block b reads buffer hs; the next stage's X is fetched
  // into registers meanwhile, and the next super-block's codes during stage 0.
  // The last stage fetches (and parks in the idle buffer) a copy of itself,
  // so the loop body has no data-dependent branches.
  for (int b = b_begin; b < b_end; b++) {
    const int bn = b + 1 < b_end ? b + 1 : b;
#pragma unroll
    for (int hs = 0; hs < 2; hs++) {
      __syncthreads();
      load_x(hs == 0 ? 2 * b + 1 : 2 * bn, xv);
      if (hs == 0) G::load(rowp + static_cast<int64_t>(bn) * G::GB, h, raw);
      const uint4* xb = xs[hs];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int s = 4 * hs + jj;
        bf16x8v_t B0, B1;
        decode16(cur.code[s][0], cur.code[s][1], B0, B1);
        const float sc = cur.scale[s];
#pragma unroll
        for (int tt = 0; tt < T32; tt++) {
          const int t = 32 * tt + j32;
          const bf16x8v_t A0 = __builtin_bit_cast(bf16x8v_t, xb[t * 16 + ((4 * jj + h) ^ (t & 15))]);
          const bf16x8v_t A1 = __builtin_bit_cast(bf16x8v_t, xb[t * 16 + ((4 * jj + 2 + h) ^ (t & 15))]);
          f32x16_t P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B0, zero, 0, 0, 0);
          P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1, P, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; r++) acc[tt][r] = __builtin_fmaf(sc, P[r], acc[tt][r]);
        }
#pragma unroll
        for (int tt = 0; tt < T32; tt++) asm volatile("" : "+v"(acc[tt]));
      }
      if constexpr (AFFINE) {
        // sum_j (8 s_j + a_j) sum(x_j) over the stage's 4 sub-blocks: two fp32
        // 32x32x2 matrix ops per tile, A = sum(x) [token][sub-block 2q+h of
        // the pair], B = (8 s + a) [that sub-block][row]
#pragma unroll
        for (int tt = 0; tt < T32; tt++) {
          const float* xq = xsum[hs] + (32 * tt + j32) * 4 + h;
#pragma unroll
          for (int q = 0; q < 2; q++)
            acc[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(xq[2 * q], cur.corr[2 * hs + q], acc[tt], 0, 0, 0);
        }
      }
      store_x(hs ^ 1, xv);
      if (hs == 1) G::finish(rowp + static_cast<int64_t>(bn) * G::GB, h, raw, cur);
    }
  }

  if (m < M) {
#pragma unroll
    for (int tt = 0; tt < T32; tt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int n = n0 + 32 * tt + 8 * (r / 4) + 4 * h + (r % 4);
        if (n < N) {
          float* dst = Y + static_cast<int64_t>(n) * M + m;
          if constexpr (SPLIT) atomicAdd(dst, acc[tt][r]);
          else *dst = acc[tt][r];
        }
      }
  }
}


// Grid of the wide kernel: 128-row by nt-token tiles, K split into pieces
// when the tiles alone leave workgroup slots (slots = workgroups resident at
// once) idle -- floor(slots / tiles) pieces, so that the grid still fits one
// round, of at least two super-blocks each.
struct WideGrid {
  unsigned gx, gy;
  int split, per;  // K pieces and super-blocks per piece
};

WideGrid wide_grid(int64_t m, int64_t n, int nsb, int nt, int64_t slots) {
  WideGrid g;
  g.gx = static_cast<unsigned>((m + 127) / 128);
  g.gy = static_cast<unsigned>((n + nt - 1) / nt);
  const int64_t tiles = static_cast<int64_t>(g.gx) * g.gy;
  int64_t split = 1;
  if (tiles < slots) {
    split = slots / tiles;
    const int64_t max_split = nsb / 2 > 1 ? nsb / 2 : 1;
    split = split > max_split ? max_split : split;
  }
  g.per = static_cast<int>((nsb + split - 1) / split);
  g.split = (nsb + g.per - 1) / g.per;
  return g;
}

template <int FMT, int T32, int OCC>
hipError_t launch_w_t(const void* blocks, int64_t m, int64_t k, const void* x, int64_t n, float* y,
                      const WideGrid& g, hipStream_t s) {
  const int nsb = static_cast<int>(k / 256);
  if (log_enabled())
    log_launch("gemm k_gemm_w fmt=%d tile=128x%d (%d per CU) m=%lld k=%lld n=%lld grid=%ux%ux%d "
               "super-blocks/piece=%d", FMT, 32 * T32, OCC, (long long)m, (long long)k, (long long)n, g.gx, g.gy,
               g.split, g.per);
  if (g.split > 1) {
    const hipError_t e = launch_fill_zero(y, m * n, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_w<FMT, T32, OCC, true>), dim3(g.gx, g.gy, g.split), dim3(kThreads), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), g.per);
  } else {
    hipLaunchKernelGGL((k_gemm_w<FMT, T32, OCC, false>), dim3(g.gx, g.gy, 1), dim3(kThreads), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), nsb);
  }
  return hipGetLastError();
}

// 128-token tiles, two workgroups per CU.  The affine formats switch to
// 64-token tiles, three workgroups per CU (their registers allow it), when
// 128-token tiles would fill under 3/4 of the slots without splitting K.
template <int FMT>
hipError_t launch_w(const void* blocks, int64_t m, int64_t k, const void* x, int64_t n, float* y,
                    hipStream_t s) {
  constexpr bool AFFINE = FMT == QBLK_SB4_AFFINE || FMT == QBLK_Q4_K;
  const int nsb = static_cast<int>(k / 256);
  const int64_t cus = cu_count();
  const int64_t split_ok = deterministic() ? 0 : 1;  // slots 0: K never split
  const WideGrid g4 = wide_grid(m, n, nsb, 128, split_ok * 2 * cus);
  if constexpr (AFFINE) {
    if (static_cast<int64_t>(g4.gx) * g4.gy * 4 < 3 * 2 * cus)
      return launch_w_t<FMT, 2, 3>(blocks, m, k, x, n, y, wide_grid(m, n, nsb, 64, split_ok * 3 * cus), s);
  }
  return launch_w_t<FMT, 4, 2>(blocks, m, k, x, n, y, g4, s);
}

// ---------------------------------------------------------------------------
// Few tokens, weights loaded by whole 16-byte code units (all formats).
//
// Loading the codes directly in matrix-operand order (a dword per lane and
// sub-block, lanes spread over 16 rows) asks for every cache line of a
// super-block about eight times.  Here the workgroup's tile -- 64*R16 rows
// by NSB 256-weight groups -- is fetched as the batch-1 GEMV fetches it: each
// lane takes whole 32-weight units (16 code bytes and the unit's header
// fields), consecutive lanes consecutive units of a row.  The codes are
// written to LDS realigned, one 16-byte slot per (row, unit) and 16 bytes
// of padding per row, with the unit's fp32 scale (times 16: the codes
// decode to (code-8)/16) and, for the affine formats, its offset term
// 8*s + a beside them; the matrix ops then read a dword per lane from LDS
// (16 rows x 4 k-groups: 64 different banks).  Every load of the workgroup
// is issued before the first barrier, and the K range is split over the
// grid.  With KW > 1 the workgroup has 4*KW waves: KW waves share each
// 16*R16 rows, each taking NSB/KW of the groups, and add their sums in LDS
// at the end.  The affine formats add sum_j (8 s_j + a_j) * sum(x over
// sub-block j) per group with two fp32 16x16x4 matrix ops (sub-blocks 0..3
// and 4..7; the sums of x are formed while X is staged, the 4 pieces of a
// sub-block sitting on 4 adjacent lanes).
// ---------------------------------------------------------------------------

// One 32-weight unit: raw loads, then code dwords, scale*16 and offset term.
template <int FMT>
struct UnitU;

template <>
struct UnitU<QBLK_SB4> {
  static constexpr int GB = 138;  // bytes per 256-weight group
  static constexpr int RAW = 7;
  // g: the group's first byte, j: the unit in the group
  static __device__ __forceinline__ void load(const uint8_t* g, int j, uint32_t raw[RAW]) {
    const uint8_t* cp = g + 10 + 16 * j;
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(cp) & 3u);  // 0 or 2
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(cp - mis);  // inside the group
    raw[0] = v.x;
    raw[1] = v.y;
    raw[2] = v.z;
    raw[3] = v.w;
    raw[4] = load_u16(cp + 14);
    raw[5] = load_u16(g);
    raw[6] = static_cast<uint32_t>(*reinterpret_cast<const int8_t*>(g + 2 + j));
  }
  static __device__ __forceinline__ void finish(const uint8_t* g, int j, const uint32_t raw[RAW], uint4& c,
                                                float& scale, float& corr) {
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(g + 10 + 16 * j) & 3u);
    c = make_uint4(__builtin_amdgcn_alignbyte(raw[1], raw[0], a), __builtin_amdgcn_alignbyte(raw[2], raw[1], a),
                   __builtin_amdgcn_alignbyte(raw[3], raw[2], a), __builtin_amdgcn_alignbyte(raw[4], raw[3], a));
    scale = (f16_bits_to_f32(raw[5]) * 16.0f) * static_cast<float>(static_cast<int32_t>(raw[6]));
    corr = 0.0f;
  }
};

template <>
struct UnitU<QBLK_Q4_0> {
  static constexpr int GB = 144;  // eight 18-byte blocks
  static constexpr int RAW = 6;
  static __device__ __forceinline__ void load(const uint8_t* g, int j, uint32_t raw[RAW]) {
    const uint8_t* blk = g + 18 * j;
    const uint8_t* cp = blk + 2;
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(cp) & 3u);  // 0 or 2
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(cp - mis);  // starts at blk or blk + 2
    raw[0] = v.x;
    raw[1] = v.y;
    raw[2] = v.z;
    raw[3] = v.w;
    raw[4] = load_u16(cp + 14);
    raw[5] = load_u16(blk);
  }
  static __device__ __forceinline__ void finish(const uint8_t* g, int j, const uint32_t raw[RAW], uint4& c,
                                                float& scale, float& corr) {
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(g + 18 * j + 2) & 3u);
    c = make_uint4(__builtin_amdgcn_alignbyte(raw[1], raw[0], a), __builtin_amdgcn_alignbyte(raw[2], raw[1], a),
                   __builtin_amdgcn_alignbyte(raw[3], raw[2], a), __builtin_amdgcn_alignbyte(raw[4], raw[3], a));
    scale = f16_bits_to_f32(raw[5]) * 16.0f;
    corr = 0.0f;
  }
};

template <>
struct UnitU<QBLK_SB4_AFFINE> {
  static constexpr int GB = 148;  // dword aligned
  static constexpr int RAW = 7;
  static __device__ __forceinline__ void load(const uint8_t* g, int j, uint32_t raw[RAW]) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(g + 20 + 16 * j);
    raw[0] = v.x;
    raw[1] = v.y;
    raw[2] = v.z;
    raw[3] = v.w;
    raw[4] = *reinterpret_cast<const uint32_t*>(g);  // Ss | Sa << 16
    raw[5] = static_cast<uint32_t>(*reinterpret_cast<const int8_t*>(g + 4 + j));
    raw[6] = static_cast<uint32_t>(*reinterpret_cast<const int8_t*>(g + 12 + j));
  }
  static __device__ __forceinline__ void finish(const uint8_t*, int, const uint32_t raw[RAW], uint4& c,
                                                float& scale, float& corr) {
    c = make_uint4(raw[0], raw[1], raw[2], raw[3]);
    const float s = f16_bits_to_f32(raw[4] & 0xffffu) * static_cast<float>(static_cast<int32_t>(raw[5]));
    const float o = f16_bits_to_f32(raw[4] >> 16) * static_cast<float>(static_cast<int32_t>(raw[6]));
    scale = s * 16.0f;
    corr = __builtin_fmaf(8.0f, s, o);  // w = s*n + o = s*(n-8) + (8s + o)
  }
};

template <>
struct UnitU<QBLK_Q4_K> {
  static constexpr int GB = 144;  // 16-byte aligned
  static constexpr int RAW = 8;
  static __device__ __forceinline__ void load(const uint8_t* g, int j, uint32_t raw[RAW]) {
    const uint4 h = *reinterpret_cast<const uint4*>(g);
    const uint4 v = *reinterpret_cast<const uint4*>(g + 16 + 16 * j);
    raw[0] = v.x;
    raw[1] = v.y;
    raw[2] = v.z;
    raw[3] = v.w;
    raw[4] = h.x;
    raw[5] = h.y;
    raw[6] = h.z;
    raw[7] = h.w;
  }
  static __device__ __forceinline__ void finish(const uint8_t*, int j, const uint32_t raw[RAW], uint4& c,
                                                float& scale, float& corr) {
    c = make_uint4(raw[0], raw[1], raw[2], raw[3]);
    const float s = f16_bits_to_f32(raw[4] & 0xffffu) * static_cast<float>(q4k_scale6(raw[5], raw[6], j));
    const float mn = f16_bits_to_f32(raw[4] >> 16) * static_cast<float>(q4k_min6(raw[6], raw[7], j));
    scale = s * 16.0f;
    corr = __builtin_fmaf(8.0f, s, -mn);  // w = s*n - mn = s*(n-8) + (8s - mn)
  }
};

// One stage of the unit-loaded kernels: NSB 256-weight groups of a tile of
// 64*R16 rows and 16*T16 tokens, fetched into registers (load), written to
// LDS (store) and multiplied out of LDS (compute).  KW waves share each
// 16*R16 rows, each taking NSB/KW of the stage's groups.
template <int FMT, int R16, int T16, int NSB, int KW>
struct UStage {
  using UU = UnitU<FMT>;
  static constexpr bool AFFINE = FMT == QBLK_SB4_AFFINE || FMT == QBLK_Q4_K;
  static constexpr int NT = 16 * T16;
  static constexpr int RW = 64 * R16;             // weight rows per workgroup
  static constexpr int UR = NSB * 8;              // units per row in a stage
  static constexpr int kT = kThreads * KW;        // threads per workgroup
  static constexpr int kUPT = RW * UR / kT;       // units per thread
  static_assert(RW * UR % kT == 0 && NSB % KW == 0, "whole units per thread, whole groups per wave");
  static constexpr int kCodeRow = UR * 16 + 16;   // bytes per staged row of codes
  static constexpr int kScRow = UR + 1;           // floats per staged row of scales
  static constexpr int kPieces = NSB * NT * 32;   // 16-byte pieces of the X slice
  static constexpr int kPer = (kPieces + kT - 1) / kT;

  struct Lds {
    uint4 xs4[NSB * NT * kLdsRow / 8];
    uint4 cs4[RW * kCodeRow / 16];
    float scs[RW * kScRow];
    float cos_[AFFINE ? RW * kScRow : 1];   // offset terms 8s + a
    float xsum[AFFINE ? NSB * NT * 8 : 1];  // [group][token][sub-block]
  };
  struct Regs {
    uint4 xv[kPer];
    uint32_t raw[kUPT][UU::RAW];
  };

  // Issue the loads of groups [b0, b0 + nb): X first (L2-resident), then
  // every unit of the tile.  Pieces past the stage's last group or past row
  // M-1 / token N-1 re-read valid data that is never used or never stored.
  static __device__ __forceinline__ void load(const uint8_t* __restrict__ W, const uint16_t* __restrict__ X,
                                              int64_t m0, int n0, int M, int N, int K, int64_t rowbytes,
                                              int b0, int nb, Regs& r) {
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = min(static_cast<int>(threadIdx.x) + i * kT, kPieces - 1);
      const int sb = c / (NT * 32), rem = c % (NT * 32);
      const int t = min(n0 + (rem >> 5), N - 1), col = rem & 31;
      const int b = b0 + min(sb, nb - 1);
      r.xv[i] = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(t) * K + 256 * b + 8 * col);
    }
#pragma unroll
    for (int i = 0; i < kUPT; i++) {
      const int U = static_cast<int>(threadIdx.x) + i * kT;
      const int rr = U / UR, u = U % UR;
      const int64_t m = m0 + rr < M ? m0 + rr : M - 1;
      UU::load(W + m * rowbytes + static_cast<int64_t>(UU::GB) * (b0 + min(u >> 3, nb - 1)), u & 7, r.raw[i]);
    }
  }

  // Write a loaded stage to LDS: X in matrix-operand order (and, for the
  // affine formats, its sums over each sub-block), the realigned codes, the
  // unit scales and offset terms.
  static __device__ __forceinline__ void store(Lds& L, const Regs& r, const uint8_t* __restrict__ W, int64_t m0,
                                               int M, int64_t rowbytes, int b0, int nb) {
    uint16_t* xs = reinterpret_cast<uint16_t*>(L.xs4);
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = static_cast<int>(threadIdx.x) + i * kT;
      const int sb = c / (NT * 32), rem = c % (NT * 32);
      if (kPieces % kT == 0 || c < kPieces) {
        // entries 8cc..8cc+7 of sub-block j go to the k-group slots 32j + 8g (+4)
        const int j = (rem & 31) >> 2, cc = rem & 3;
        const int g0 = 2 * (cc & 1), half = cc >> 1;
        uint16_t* row = xs + (sb * NT + (rem >> 5)) * kLdsRow + 32 * j + 4 * half;
        *reinterpret_cast<uint2*>(row + 8 * g0) = make_uint2(r.xv[i].x, r.xv[i].y);
        *reinterpret_cast<uint2*>(row + 8 * (g0 + 1)) = make_uint2(r.xv[i].z, r.xv[i].w);
      }
      if constexpr (AFFINE) {
        // sum of x over the sub-block: products with 1.0 are exact, fp32 sums;
        // the 4 pieces of a sub-block sit on 4 adjacent lanes
        const bf16x2v_t one = __builtin_bit_cast(bf16x2v_t, 0x3f803f80u);
        float part = 0.0f;
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, r.xv[i].x), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, r.xv[i].y), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, r.xv[i].z), one, part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, r.xv[i].w), one, part, false);
        part = quad_sum(part);
        if ((kPieces % kT == 0 || c < kPieces) && (c & 3) == 0)
          L.xsum[(sb * NT + (rem >> 5)) * 8 + ((rem & 31) >> 2)] = part;
      }
    }
    uint8_t* cs = reinterpret_cast<uint8_t*>(L.cs4);
#pragma unroll
    for (int i = 0; i < kUPT; i++) {
      const int U = static_cast<int>(threadIdx.x) + i * kT;
      const int rr = U / UR, u = U % UR;
      const int64_t m = m0 + rr < M ? m0 + rr : M - 1;
      uint4 c;
      float scale, corr;
      UU::finish(W + m * rowbytes + static_cast<int64_t>(UU::GB) * (b0 + min(u >> 3, nb - 1)), u & 7, r.raw[i],
                 c, scale, corr);
      *reinterpret_cast<uint4*>(cs + rr * kCodeRow + 16 * u) = c;
      L.scs[rr * kScRow + u] = scale;
      if constexpr (AFFINE) L.cos_[rr * kScRow + u] = corr;
    }
  }

  // Multiply this wave's share of a staged stage (nb groups) into acc.
  static __device__ __forceinline__ void compute(const Lds& L, int nb, int wave, int kw, int lane,
                                                 float4_t (&acc)[R16][T16]) {
    const int l16 = lane & 15, g = lane >> 4;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(L.xs4);
    const uint8_t* cs = reinterpret_cast<const uint8_t*>(L.cs4);
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sq = 0; sq < NSB / KW; sq++) {
      const int sb = kw * (NSB / KW) + sq;
      if (sb >= nb) break;
      const uint16_t* xb = xs + sb * NT * kLdsRow;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int u = 8 * sb + j;
        bf16x8v_t Bop[R16];
        float sc[R16];
#pragma unroll
        for (int tm = 0; tm < R16; tm++) {
          const int rl = wave * 16 * R16 + 16 * tm + l16;
          Bop[tm] = decode_codes(*reinterpret_cast<const uint32_t*>(cs + rl * kCodeRow + 16 * u + 4 * g));
          sc[tm] = L.scs[rl * kScRow + u];
        }
#pragma unroll
        for (int tn = 0; tn < T16; tn++) {
          const bf16x8v_t Aop = *reinterpret_cast<const bf16x8v_t*>(xb + (16 * tn + l16) * kLdsRow + 32 * j + 8 * g);
#pragma unroll
          for (int tm = 0; tm < R16; tm++) {
            const float4_t P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop, Bop[tm], zero, 0, 0, 0);
            float4_t& A = acc[tm][tn];
            A.x = __builtin_fmaf(sc[tm], P.x, A.x);
            A.y = __builtin_fmaf(sc[tm], P.y, A.y);
            A.z = __builtin_fmaf(sc[tm], P.z, A.z);
            A.w = __builtin_fmaf(sc[tm], P.w, A.w);
          }
        }
#pragma unroll
        for (int tm = 0; tm < R16; tm++)
#pragma unroll
          for (int tn = 0; tn < T16; tn++)
            asm volatile("" : "+v"(acc[tm][tn].x), "+v"(acc[tm][tn].y), "+v"(acc[tm][tn].z), "+v"(acc[tm][tn].w));
      }
      if constexpr (AFFINE) {
        // A = sum(x) [token][sub-block 4q + g], B = (8 s + a) [sub-block 4q + g][row]
#pragma unroll
        for (int tn = 0; tn < T16; tn++) {
          const float* xq = L.xsum + (sb * NT + 16 * tn + l16) * 8 + g;
#pragma unroll
          for (int tm = 0; tm < R16; tm++) {
            const float* co = L.cos_ + (wave * 16 * R16 + 16 * tm + l16) * kScRow + 8 * sb + g;
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xq[0], co[0], acc[tm][tn], 0, 0, 0);
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xq[4], co[4], acc[tm][tn], 0, 0, 0);
          }
        }
      }
    }
  }

  // The K shares of a row tile meet in LDS (KW > 1; every thread calls this),
  // then the waves of share 0 write (or, with K split over the grid, add) Y.
  template <bool SPLIT>
  static __device__ __forceinline__ void finish(float4_t (&acc)[R16][T16], float4_t* red, int wave, int kw,
                                                int lane, int64_t m0, int n0, int M, int N, float* __restrict__ Y) {
    const int l16 = lane & 15, g = lane >> 4;
    if constexpr (KW > 1) {
      if (kw > 0) {
#pragma unroll
        for (int tm = 0; tm < R16; tm++)
#pragma unroll
          for (int tn = 0; tn < T16; tn++)
            red[((((kw - 1) * 4 + wave) * R16 + tm) * T16 + tn) * 64 + lane] = acc[tm][tn];
      }
      __syncthreads();
      if (kw > 0) return;
#pragma unroll
      for (int q = 1; q < KW; q++)
#pragma unroll
        for (int tm = 0; tm < R16; tm++)
#pragma unroll
          for (int tn = 0; tn < T16; tn++) {
            const float4_t o = red[((((q - 1) * 4 + wave) * R16 + tm) * T16 + tn) * 64 + lane];
            acc[tm][tn].x += o.x;
            acc[tm][tn].y += o.y;
            acc[tm][tn].z += o.z;
            acc[tm][tn].w += o.w;
          }
    }
#pragma unroll
    for (int tm = 0; tm < R16; tm++) {
      const int64_t m = m0 + wave * 16 * R16 + 16 * tm + l16;
      if (m >= M) continue;
#pragma unroll
      for (int tn = 0; tn < T16; tn++) {
        const float v[4] = {acc[tm][tn].x, acc[tm][tn].y, acc[tm][tn].z, acc[tm][tn].w};
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int n = n0 + 16 * tn + 4 * g + r;
          if (n < N) {
            float* dst = Y + static_cast<int64_t>(n) * M + m;
            if constexpr (SPLIT) atomicAdd(dst, v[r]);
            else *dst = v[r];
          }
        }
      }
    }
  }
};

// One stage per workgroup: every load issued before the single barrier
// (few tokens; the K range is split over the grid).
template <int FMT, int R16, int T16, int NSB, int KW, bool SPLIT>
__global__ __launch_bounds__(kThreads * KW) void k_gemm_u(const uint8_t* __restrict__ W,
                                                   const uint16_t* __restrict__ X,
                                                   float* __restrict__ Y, int M, int K, int N) {
  using St = UStage<FMT, R16, T16, NSB, KW>;
  __shared__ typename St::Lds L;
  __shared__ float4_t red[KW > 1 ? (KW - 1) * 4 * R16 * T16 * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);  // wave-uniform: scalar
  const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * St::RW;
  const int n0 = blockIdx.y * St::NT;
  const int ngr = K / 256;
  const int b0 = blockIdx.z * NSB;
  const int nb = min(NSB, ngr - b0);  // groups in this piece of K (>= 1)
  const int64_t rowbytes = static_cast<int64_t>(ngr) * St::UU::GB;

  typename St::Regs r;
  St::load(W, X, m0, n0, M, N, K, rowbytes, b0, nb, r);
  St::store(L, r, W, m0, M, rowbytes, b0, nb);
  __syncthreads();
  float4_t acc[R16][T16];
#pragma unroll
  for (int tm = 0; tm < R16; tm++)
#pragma unroll
    for (int tn = 0; tn < T16; tn++) acc[tm][tn] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  St::compute(L, nb, wave, kw, lane, acc);
  St::template finish<SPLIT>(acc, red, wave, kw, lane, m0, n0, M, N, Y);
}

// Many stages per workgroup (tens of tokens): the workgroup walks its K
// range NSB groups at a time; the loads of the next stage are issued into
// registers before the products of the current one, so they arrive while it
// runs, and are written to LDS between two barriers.  With the whole K range
// in one workgroup no partial products are added into Y.
template <int FMT, int R16, int T16, int NSB, int KW, bool SPLIT>
__global__ __launch_bounds__(kThreads * KW) void k_gemm_s(const uint8_t* __restrict__ W,
                                                   const uint16_t* __restrict__ X,
                                                   float* __restrict__ Y, int M, int K, int N,
                                                   int groups_per_split) {
  using St = UStage<FMT, R16, T16, NSB, KW>;
  __shared__ typename St::Lds L;
  __shared__ float4_t red[KW > 1 ? (KW - 1) * 4 * R16 * T16 * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);  // wave-uniform: scalar
  const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * St::RW;
  const int n0 = blockIdx.y * St::NT;
  const int ngr = K / 256;
  const int g_begin = blockIdx.z * groups_per_split;
  const int g_end = min(ngr, g_begin + groups_per_split);
  const int64_t rowbytes = static_cast<int64_t>(ngr) * St::UU::GB;

  float4_t acc[R16][T16];
#pragma unroll
  for (int tm = 0; tm < R16; tm++)
#pragma unroll
    for (int tn = 0; tn < T16; tn++) acc[tm][tn] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  typename St::Regs r;
  if (g_begin < g_end) St::load(W, X, m0, n0, M, N, K, rowbytes, g_begin, min(NSB, g_end - g_begin), r);
  for (int b = g_begin; b < g_end; b += NSB) {
    const int nb = min(NSB, g_end - b);
    if (b != g_begin) __syncthreads();  // every wave is done with the previous stage
    St::store(L, r, W, m0, M, rowbytes, b, nb);
    __syncthreads();
    if (b + NSB < g_end) St::load(W, X, m0, n0, M, N, K, rowbytes, b + NSB, min(NSB, g_end - b - NSB), r);
    St::compute(L, nb, wave, kw, lane, acc);
  }
  St::template finish<SPLIT>(acc, red, wave, kw, lane, m0, n0, M, N, Y);
}

template <int FMT, int R16, int T16, int NSB, int KW = 1>
hipError_t launch_u(const void* blocks, int64_t m, int64_t k, const void* x, int64_t n, float* y,
                    hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((m + 64 * R16 - 1) / (64 * R16));
  const unsigned gy = static_cast<unsigned>((n + 16 * T16 - 1) / (16 * T16));
  const int nsb = static_cast<int>(k / 256);
  const unsigned gz = static_cast<unsigned>((nsb + NSB - 1) / NSB);
  if (log_enabled())
    log_launch("gemm k_gemm_u fmt=%d tile=%dx%d waves/tile=%d m=%lld k=%lld n=%lld grid=%ux%ux%u super-blocks/piece=%d",
               FMT, 64 * R16, 16 * T16, KW, (long long)m, (long long)k, (long long)n, gx, gy, gz, NSB);
  if (gz > 1) {
    const hipError_t e = launch_fill_zero(y, m * n, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_u<FMT, R16, T16, NSB, KW, true>), dim3(gx, gy, gz), dim3(kThreads * KW), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
  } else {
    hipLaunchKernelGGL((k_gemm_u<FMT, R16, T16, NSB, KW, false>), dim3(gx, gy, 1), dim3(kThreads * KW), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
  }
  return hipGetLastError();
}

// Full K per workgroup unless the tiles alone leave CUs idle; then K is
// split over the grid, for about two workgroups per CU (partial products
// added into Y, zeroed first).
template <int FMT, int R16, int T16, int NSB, int KW>
hipError_t launch_st(const void* blocks, int64_t m, int64_t k, const void* x, int64_t n, float* y,
                     hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((m + 64 * R16 - 1) / (64 * R16));
  const unsigned gy = static_cast<unsigned>((n + 16 * T16 - 1) / (16 * T16));
  const int nsb = static_cast<int>(k / 256);
  const int64_t tiles = static_cast<int64_t>(gx) * gy;
  int split = 1;
  if (tiles < cu_count() && !deterministic()) {
    split = static_cast<int>((2 * cu_count() + tiles - 1) / tiles);
    const int max_split = nsb / (2 * NSB) > 1 ? nsb / (2 * NSB) : 1;  // >= 2 stages per piece
    split = split > max_split ? max_split : split;
  }
  const int per = (nsb + split - 1) / split;
  split = (nsb + per - 1) / per;
  if (log_enabled())
    log_launch("gemm k_gemm_s fmt=%d tile=%dx%d waves/tile=%d stage=%d m=%lld k=%lld n=%lld grid=%ux%ux%d "
               "super-blocks/piece=%d", FMT, 64 * R16, 16 * T16, KW, NSB, (long long)m, (long long)k, (long long)n,
               gx, gy, split, split > 1 ? per : nsb);
  if (split > 1) {
    const hipError_t e = launch_fill_zero(y, m * n, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_s<FMT, R16, T16, NSB, KW, true>), dim3(gx, gy, split), dim3(kThreads * KW), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), per);
  } else {
    hipLaunchKernelGGL((k_gemm_s<FMT, R16, T16, NSB, KW, false>), dim3(gx, gy, 1), dim3(kThreads * KW), 0, s,
                       static_cast<const uint8_t*>(blocks), static_cast<const uint16_t*>(x), y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), nsb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       int64_t n, float* y, hipStream_t s) {
  (void)xt;  // only BF16 activations reach this point
  // (sweeps at 14336 x 4096: up to 16 tokens one stage per workgroup with
  // K split over the grid, 15.5-16.0 us for every format -- Type 1 and Q4_K
  // with two waves per row tile, 16.9 us with one; up to 64 tokens the
  // streaming kernel over the whole K range with 32-token tiles (Q4_K: 16
  // up to 32 tokens), N = 32: 19.9-22.3 us against 24.1-26.8 us for the
  // double-buffered kernel it replaced, N = 64: 27.2-29.8 us against
  // 35.1-44.9 us; 64-token tiles were 29-36 us at N = 64)
  // (reproducible products: the streaming kernel up to 64 tokens, K whole)
  if (n <= 16 && !deterministic()) {
    if (fmt == QBLK_SB4) return launch_u<QBLK_SB4, 1, 1, 2>(blocks, m, k, x, n, y, s);
    if (fmt == QBLK_Q4_0) return launch_u<QBLK_Q4_0, 1, 1, 2>(blocks, m, k, x, n, y, s);
    if (fmt == QBLK_Q4_K) return launch_u<QBLK_Q4_K, 1, 1, 2, 2>(blocks, m, k, x, n, y, s);
    return launch_u<QBLK_SB4_AFFINE, 1, 1, 2, 2>(blocks, m, k, x, n, y, s);
  }
  if (n <= 64) {
    if (fmt == QBLK_SB4) return launch_st<QBLK_SB4, 1, 2, 2, 2>(blocks, m, k, x, n, y, s);
    if (fmt == QBLK_Q4_0) return launch_st<QBLK_Q4_0, 1, 2, 2, 2>(blocks, m, k, x, n, y, s);
    if (fmt == QBLK_Q4_K) {
      if (n <= 32) return launch_st<QBLK_Q4_K, 1, 1, 2, 2>(blocks, m, k, x, n, y, s);
      return launch_st<QBLK_Q4_K, 1, 2, 2, 2>(blocks, m, k, x, n, y, s);
    }
    return launch_st<QBLK_SB4_AFFINE, 1, 2, 2, 2>(blocks, m, k, x, n, y, s);
  }
  if (fmt == QBLK_SB4) return launch_w<QBLK_SB4>(blocks, m, k, x, n, y, s);
  if (fmt == QBLK_Q4_0) return launch_w<QBLK_Q4_0>(blocks, m, k, x, n, y, s);
  if (fmt == QBLK_Q4_K) return launch_w<QBLK_Q4_K>(blocks, m, k, x, n, y, s);
  return launch_w<QBLK_SB4_AFFINE>(blocks, m, k, x, n, y, s);
}

}  // namespace qblk
