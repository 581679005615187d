// qblk_gemv.hip -- batch-1 dequantize-and-multiply y = W x on gfx950.
//
// What is computed: y[i] = sum_k W[i,k] x[k] where W[i,k] is the block
// format's rebuilt weight (Q4_0: d*(code-8), "GGUF 量化内幕 第4章 Q4_0" 4.3;
// super-block Type 0: (S*sc_j)*(code-8) and Type 1: (Ss*sc_j)*code + Sa*ac_j,
// "GGUF K-quants" blog, "套娃" step 5; Q4_K: (d*s_j)*code - dmin*m_j, Q4_0
// chapter 4.6).  The pages only say that dequantized
// weights feed the matrix product; this kernel never materialises W.
//
// Work split.  A 32-weight unit (a Q4_0 block or one super-block sub-block)
// shares one scale.  Lane l of a wave takes units l, l+64, ... of a row and
// R rows at once (x is read once per unit and used R times); each wave then
// reduces its R partial sums across the 64 lanes.  Adjacent lanes read
// adjacent 16-byte code groups, so each load instruction of a wave covers a
// contiguous ~1 KB stretch of the packed stream.
//
// Arithmetic (x in fp16).  Codes are turned into exact fp16 values by OR-ing a
// nibble into the mantissa of 1024.0 (0x6400) and subtracting 1032 (or, for
// the high nibbles, which sit 4 bits up, 1024 + 16*8 giving 16*(code-8));
// v_dot2_f32_f16 then forms exact fp16 x fp16 products and accumulates them in
// fp32.  To pair codes with x without shuffling the codes, x is put in the
// matching order once (in LDS by the generic kernel, in registers with v_perm
// by the fp16-x kernel below): for code word t (bytes 4t..4t+3 of a unit) the pairs
// are (x[4t], x[4t+2]), (x[4t+16], x[4t+18]), (x[4t+1], x[4t+3]),
// (x[4t+17], x[4t+19]).  The unit's fp32 scale multiplies the two partial
// sums; Type 1 and Q4_K add offset * sum(x over the unit) (Q4_K's offset is
// -dmin*m_j).
// With x in fp32 (or bf16, widened exactly to fp32) the codes are converted
// with v_cvt_f32_ubyte and accumulated with fp32 fused multiply-adds.
#include "qblk_device.h"
#include "qblk_launch.h"

namespace qblk {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunkF16 = 16384;  // x elements staged per pass (32 KB of fp16)
constexpr int kChunkF32 = 8192;   // (32 KB of fp32)

template <int FMT>
struct Fmt;
template <>
struct Fmt<QBLK_Q4_0> {
  static constexpr int E = 32, B = 18;
};
template <>
struct Fmt<QBLK_SB4> {
  static constexpr int E = 256, B = 138;
};
template <>
struct Fmt<QBLK_SB4_AFFINE> {
  static constexpr int E = 256, B = 148;
};
template <>
struct Fmt<QBLK_Q4_K> {
  static constexpr int E = 256, B = 144;
};

// formats whose codes are 0..15 plus a per-unit offset
constexpr bool affine_fmt(int f) { return f == QBLK_SB4_AFFINE || f == QBLK_Q4_K; }

// Scale, offset and the 16 code bytes of unit s of a row.
template <int FMT>
__device__ __forceinline__ void load_unit(const uint8_t* row, int s, float& sc, float& off,
                                          uint32_t q[4]) {
  if constexpr (FMT == QBLK_Q4_0) {
    const uint8_t* p = row + static_cast<int64_t>(s) * 18;
    sc = f16_bits_to_f32(load_u16(p));
    off = 0.0f;
    load16_a2(p + 2, q);
  } else if constexpr (FMT == QBLK_SB4) {
    const int b = s >> 3, j = s & 7;
    const uint8_t* p = row + static_cast<int64_t>(b) * 138;
    const float S = f16_bits_to_f32(load_u16(p));
    sc = S * static_cast<float>(static_cast<int8_t>(p[2 + j]));
    off = 0.0f;
    load16_a2(p + 10 + 16 * j, q);
  } else if constexpr (FMT == QBLK_Q4_K) {
    const int b = s >> 3, j = s & 7;
    const uint8_t* p = row + static_cast<int64_t>(b) * 144;  // 16-byte aligned
    const uint4 h = *reinterpret_cast<const uint4*>(p);
    sc = f16_bits_to_f32(h.x & 0xffffu) * static_cast<float>(q4k_scale6(h.y, h.z, j));
    off = -(f16_bits_to_f32(h.x >> 16) * static_cast<float>(q4k_min6(h.z, h.w, j)));
    const uint4 v = *reinterpret_cast<const uint4*>(p + 16 + 16 * j);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  } else {
    const int b = s >> 3, j = s & 7;
    const uint8_t* p = row + static_cast<int64_t>(b) * 148;
    const uint32_t h = *reinterpret_cast<const uint32_t*>(p);
    sc = f16_bits_to_f32(h & 0xffffu) * static_cast<float>(static_cast<int8_t>(p[4 + j]));
    off = f16_bits_to_f32(h >> 16) * static_cast<float>(static_cast<int8_t>(p[12 + j]));
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(p + 20 + 16 * j);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  }
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// sum over a unit of (code - 8) * x (signed formats) or code * x (affine),
// returned as lo + hi/16 in two fp32 partials.
template <bool AFFINE>
__device__ __forceinline__ void dot_unit_f16(const uint32_t q[4], const uint4 X[4], float& lo,
                                             float& hi) {
  // 1024+n -> n-8: subtract 1032; 1024+16n -> 16(n-8): subtract 1152.
  const half2_t kLo = AFFINE ? half2_t{-1024.0f16, -1024.0f16} : half2_t{-1032.0f16, -1032.0f16};
  const half2_t kHi = AFFINE ? half2_t{-1024.0f16, -1024.0f16} : half2_t{-1152.0f16, -1152.0f16};
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint32_t a = q[t], b = q[t] >> 8;
    const half2_t v0 = as_h2((a & 0x000F000Fu) | 0x64006400u) + kLo;
    const half2_t v1 = as_h2((a & 0x00F000F0u) | 0x64006400u) + kHi;
    const half2_t v2 = as_h2((b & 0x000F000Fu) | 0x64006400u) + kLo;
    const half2_t v3 = as_h2((b & 0x00F000F0u) | 0x64006400u) + kHi;
    const uint4 x = X[t];
    lo = __builtin_amdgcn_fdot2(v0, as_h2(x.x), lo, false);
    hi = __builtin_amdgcn_fdot2(v1, as_h2(x.y), hi, false);
    lo = __builtin_amdgcn_fdot2(v2, as_h2(x.z), lo, false);
    hi = __builtin_amdgcn_fdot2(v3, as_h2(x.w), hi, false);
  }
}

template <bool AFFINE>
__device__ __forceinline__ float dot_unit_f32(const uint32_t q[4], const float* xs) {
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint32_t lo = q[t] & 0x0F0F0F0Fu, hi = (q[t] >> 4) & 0x0F0F0F0Fu;
    const float4 xl = *reinterpret_cast<const float4*>(xs + 4 * t);
    const float4 xh = *reinterpret_cast<const float4*>(xs + 16 + 4 * t);
    const float xlv[4] = {xl.x, xl.y, xl.z, xl.w};
    const float xhv[4] = {xh.x, xh.y, xh.z, xh.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float cl = static_cast<float>((lo >> (8 * i)) & 0xFFu);
      float ch = static_cast<float>((hi >> (8 * i)) & 0xFFu);
      if (!AFFINE) {
        cl -= 8.0f;
        ch -= 8.0f;
      }
      acc = __builtin_fmaf(cl, xlv[i], acc);
      acc = __builtin_fmaf(ch, xhv[i], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Stage x[k0, k0+kc) into LDS.  fp16 path: permuted pairs, 16 words per unit.
// fp32 path: natural order.  Affine formats also get the per-unit sum of x.
template <int XT, bool AFFINE>
__device__ void stage_x(const void* x, int k0, int kc, uint32_t* xs, float* xsum) {
  const int nchunk = kc / 8;  // groups of 8 elements; 4 per unit
  for (int c = threadIdx.x; c < (nchunk + 3) / 4 * 4; c += kThreads) {
    float part = 0.0f;
    if (c < nchunk) {
      const int e0 = k0 + 8 * c;
      if constexpr (XT == QBLK_F16) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e0);
        const int unit = c >> 2, cc = c & 3;
        const int tb = (cc & 1) * 2, hi = cc >> 1;  // elements 8cc..8cc+7 of the unit
        uint32_t* d = xs + unit * 16;
        d[4 * tb + hi] = (u.x & 0xffffu) | (u.y << 16);            // (e0, e2)
        d[4 * tb + 2 + hi] = (u.x >> 16) | (u.y & 0xffff0000u);    // (e1, e3)
        d[4 * tb + 4 + hi] = (u.z & 0xffffu) | (u.w << 16);        // (e4, e6)
        d[4 * tb + 6 + hi] = (u.z >> 16) | (u.w & 0xffff0000u);    // (e5, e7)
        if (AFFINE) {
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; i++) part += f16_bits_to_f32(w[i] & 0xffffu) + f16_bits_to_f32(w[i] >> 16);
        }
      } else {
        float v[8];
        if constexpr (XT == QBLK_F32) {
          const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + e0);
          const float4 a = p[0], b = p[1];
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
          v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
          const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e0);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
          }
        }
        float* d = reinterpret_cast<float*>(xs) + 8 * c;
        reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
        if (AFFINE) {
#pragma unroll
          for (int i = 0; i < 8; i++) part += v[i];
        }
      }
    }
    if (AFFINE) {
      // the 4 chunks of a unit sit on 4 consecutive lanes
      part += __shfl_xor(part, 1, kWave);
      part += __shfl_xor(part, 2, kWave);
      if ((c & 3) == 0 && c < nchunk) xsum[c >> 2] = part;
    }
  }
}

template <int FMT, int XT, int R>
__global__ __launch_bounds__(kThreads) void k_gemv(const uint8_t* __restrict__ blocks,
                                                   const void* __restrict__ x,
                                                   float* __restrict__ y, int M, int K) {
  constexpr bool AFFINE = affine_fmt(FMT);
  constexpr bool XH = XT == QBLK_F16;
  constexpr int KC = XH ? kChunkF16 : kChunkF32;
  extern __shared__ uint4 smem[];
  // LDS: the staged x chunk (kcmax elements) followed by one sum per unit
  const int kcmax = K < KC ? K : KC;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  float* xsum = reinterpret_cast<float*>(xs + (XH ? kcmax / 2 : kcmax));

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * R;
  const int64_t rowbytes = static_cast<int64_t>(K / Fmt<FMT>::E) * Fmt<FMT>::B;
  const uint8_t* rowp[R];
#pragma unroll
  for (int i = 0; i < R; i++) {
    const int64_t r = r0 + i < M ? r0 + i : M - 1;  // rows past the end re-read the last row
    rowp[i] = blocks + r * rowbytes;
  }
  float acc[R];
#pragma unroll
  for (int i = 0; i < R; i++) acc[i] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += KC) {
    const int kc = K - k0 < KC ? K - k0 : KC;
    __syncthreads();
    stage_x<XT, AFFINE>(x, k0, kc, xs, xsum);
    __syncthreads();
    if (r0 >= M) continue;
    const int s0 = k0 / 32, ns = kc / 32;
#pragma unroll 2
    for (int su = lane; su < ns; su += kWave) {
      float sc[R], off[R];
      uint32_t q[R][4];
#pragma unroll
      for (int i = 0; i < R; i++) load_unit<FMT>(rowp[i], s0 + su, sc[i], off[i], q[i]);
      if constexpr (XH) {
        uint4 X[4];
#pragma unroll
        for (int t = 0; t < 4; t++) X[t] = smem[su * 4 + t];
#pragma unroll
        for (int i = 0; i < R; i++) {
          float lo = 0.0f, hi = 0.0f;
          dot_unit_f16<AFFINE>(q[i], X, lo, hi);
          acc[i] = __builtin_fmaf(sc[i], lo, acc[i]);
          acc[i] = __builtin_fmaf(sc[i] * 0.0625f, hi, acc[i]);
        }
      } else {
        const float* xf = reinterpret_cast<const float*>(xs) + su * 32;
#pragma unroll
        for (int i = 0; i < R; i++) acc[i] = __builtin_fmaf(sc[i], dot_unit_f32<AFFINE>(q[i], xf), acc[i]);
      }
      if constexpr (AFFINE) {
        const float sx = xsum[su];
#pragma unroll
        for (int i = 0; i < R; i++) acc[i] = __builtin_fmaf(off[i], sx, acc[i]);
      }
    }
  }
  if (r0 >= M) return;
#pragma unroll
  for (int i = 0; i < R; i++) {
    const float v = wave_sum(acc[i]);
    if (lane == 0 && r0 + i < M) y[r0 + i] = v;
  }
}

// ===================================================================
// fp16-x kernel: every load of a wave issued up front, no LDS; one barrier
// at the end when two waves share a row.
//
// The rows are split evenly over the workgroups (one workgroup of W = 12 or
// 16 waves per CU).  With one wave per row (KS = 1) wave w of a workgroup
// takes rows w, w+W, w+2W, ... of its slice (RMAX of them at most) and lane
// l takes units l, l+64, ... (UPL of them at most) of each row; with KS = 2
// waves 2j and 2j+1 take rows j, j+W/2, ... and split each row's units into
// two halves.  A
// lane therefore sees the same units of x in every row: it loads their 32
// halves once and forms the fp16 pairs in registers (v_perm), to be reused
// for its RMAX rows.  The weight loads go out group by group -- unit k of
// row i, unit-major -- with the row base in SGPRs and a fixed 32-bit offset
// per (lane, unit), each unit's x just before its first group; the products
// consume the groups in the same order, so each waits only for its own
// loads (the load counter drains in issue order).  No wave waits for
// another before its last product.
//
// Code groups of Q4_0 blocks and Type 0 sub-blocks start 2 bytes past a dword
// boundary every other unit: a dword-aligned 16-byte load from just below,
// plus the 2 bytes that spill past it, realigned with v_alignbyte.
// ===================================================================
constexpr int kWavesH = 16;  // waves per workgroup unless a launch says otherwise

template <int FMT>
struct UnitAddr {
  // byte offset of the 16 code bytes of unit u inside a row
  static __device__ __forceinline__ uint32_t codes(int u) {
    if constexpr (FMT == QBLK_Q4_0) return 18u * u + 2u;
    else if constexpr (FMT == QBLK_SB4) return 138u * (u >> 3) + 10u + 16u * (u & 7);
    else if constexpr (FMT == QBLK_Q4_K) return 144u * (u >> 3) + 16u + 16u * (u & 7);
    else return 148u * (u >> 3) + 20u + 16u * (u & 7);
  }
};

// KS waves share a row (KS = 2 splits the row's units in two halves whose
// sums meet in LDS after the only barrier of the kernel); WAVES waves per
// workgroup (one workgroup per CU).  XL > 0: x is
// loaded once per workgroup -- every thread a few 4-element pieces, ahead of
// its weight loads -- written to LDS already paired, published with one
// barrier and read back per unit, instead of every wave loading the x of its
// units.  XL = 1 publishes after the weight loads are issued; XL = 2 before
// any is issued: a barrier passed with loads in flight waits for them on this
// part (an 11008 x 4096 launch with the barrier after its loads took 8.4 us,
// one with it before 6.9 us), so XL = 2 pays only the latency of x first.
// (Publishing without the barrier does not help: with every wave's weight
// loads issued behind its piece of x, each wave counting itself in LDS once
// its piece is written and waiting for the count, 11008 x 4096 took 8.40 us
// against 6.61 -- 8.44 us even with every piece of x requested, behind one
// barrier, before any weight request of the workgroup: x is then fetched
// while every CU's weight requests are in flight, and arrives late.)
// The kernel's body; wg is the workgroup's index among those of its matrix.
template <int FMT, int RMAX, int UPL, int KS, int WAVES, int XL>
__device__ __forceinline__ void gemv_h_body(const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
                                            float* __restrict__ y, int M, int K, int rows_per_wg, unsigned wg) {
  constexpr bool AFFINE = affine_fmt(FMT);
  constexpr bool QK = FMT == QBLK_Q4_K;
  constexpr int E = Fmt<FMT>::E, B = Fmt<FMT>::B;
  constexpr int SLOTS = WAVES / KS;  // rows in flight per workgroup round
  const int S = K >> 5;                // units per row
  const int SP = (S + KS - 1) / KS;    // units per part
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int slot = wave / KS, part = wave % KS;
  const int row0 = wg * rows_per_wg;
  const int row_end = min(M, row0 + rows_per_wg);
  // (KS > 1 or XL: every wave meets the barrier)
  if (KS == 1 && !XL && row0 + slot >= row_end) return;
  const int64_t rowbytes = static_cast<int64_t>(K / E) * B;

  // per (lane, unit): byte offsets inside a row of the codes, the scale
  // header and the INT8 sub-scale (Type 1: offset 8 bytes further); Q4_K
  // reads its whole 16-byte header and needs the sub-block index
  uint32_t off[UPL], hoff[UPL], coff[UPL];
  int sbj[UPL];
  bool live[UPL];
#pragma unroll
  for (int k = 0; k < UPL; k++) {
    const int uu = part * SP + lane + 64 * k;
    live[k] = lane + 64 * k < SP && uu < S;
    const int u = min(uu, S - 1);
    off[k] = UnitAddr<FMT>::codes(u);
    hoff[k] = FMT == QBLK_Q4_0 ? off[k] - 2u : static_cast<uint32_t>(B) * (u >> 3);
    coff[k] = hoff[k] + (FMT == QBLK_SB4_AFFINE ? 4u : 2u) + (u & 7);
    sbj[k] = u & 7;
  }

  // (1) x of this lane's units, 32 halves each: unit 0's issued first, unit
  // k's just before the weight groups of unit k (so the first weight requests
  // are not queued behind every x request of the CU's waves: 7.47 -> 7.33 us
  // at 11008 x 4096)
  // (Q4_K with three units per lane, whose groups are not pinned below, keeps
  // the old order -- every x load first, every unit's pairs formed before the
  // first product: the later forms cost it registers it does not have.)
  constexpr bool kLateX = !XL && !(QK && UPL > 2);
  uint4 xr[UPL][4];
  // XL: this thread's pieces of x (4 elements each) for the LDS copy; units
  // past the row's last one are written as zeros
  constexpr int kPieces = XL ? KS * UPL * 64 * 8 : 0;  // 8 pieces per unit, every part's units
  constexpr int kPPT = XL ? (kPieces + WAVES * kWave - 1) / (WAVES * kWave) : 1;
  uint2 xp[kPPT];
  if constexpr (XL) {
#pragma unroll
    for (int j = 0; j < kPPT; j++) {  // unconditional loads (clamped), so the waits stay in order
      const int pc = min(static_cast<int>(threadIdx.x) + j * WAVES * kWave, 8 * S - 1);
      xp[j] = *reinterpret_cast<const uint2*>(x + 4 * pc);
    }
  }
  // XL: pairs of unit u, word t, at xs[(4 (u / 64) + t) * 64 + (u + 8t) % 64]
  // (the rotation by 8t puts the four words of a unit, written by
  // neighbouring threads, in different banks: 4-way conflicts on the writes
  // become 2-way; the reads stay conflict-free)
  __shared__ uint4 xs[XL ? KS * UPL * 4 * 64 : 1];
  auto publish_x = [&]() {
#pragma unroll
    for (int j = 0; j < kPPT; j++) {
      const int pc = static_cast<int>(threadIdx.x) + j * WAVES * kWave;
      uint2 v = xp[j];
      asm volatile("" : "+v"(v.x), "+v"(v.y)::"memory");  // waits for this piece only
      if (pc >= 8 * S) v = make_uint2(0u, 0u);  // units past the row's last one
      if (pc < kPieces) {
        const int u = pc >> 3, q = pc & 7, t = q & 3, hh = q >> 2;
        uint32_t* w = reinterpret_cast<uint32_t*>(xs + (4 * (u >> 6) + t) * 64 + ((u + 8 * t) & 63));
        w[hh] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);      // (x0, x2)
        w[2 + hh] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
      }
    }
    // LDS writes done, then the workgroup barrier; the memory clobber keeps
    // every LDS access on its side
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  if constexpr (XL == 2) {
    publish_x();
    if (KS == 1 && row0 + slot >= row_end) return;
  }
  auto load_x = [&](int k) {
    const int u = min(part * SP + lane + 64 * k, S - 1);
    const uint4* p = reinterpret_cast<const uint4*>(x + 32 * u);
#pragma unroll
    for (int c = 0; c < 4; c++) xr[k][c] = p[c];
  };
  if constexpr (!XL) {
#pragma unroll
    for (int k = 0; k < (kLateX ? 1 : UPL); k++) load_x(k);
  }
  __builtin_amdgcn_sched_barrier(0);

  // (2) every weight load of this wave, group by group
  uint32_t q[RMAX][UPL][5];
  int hs[RMAX][UPL], hc[RMAX][UPL], ha[RMAX][UPL];
  uint4 hk[RMAX][UPL];  // Q4_K headers
  uint32_t rbm[RMAX];  // 2 when the row starts 2 bytes past a dword boundary
#pragma unroll
  for (int k = 0; k < UPL; k++) {
    if (kLateX && k > 0) {
      load_x(k);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
      const int r = min(row0 + slot + SLOTS * i, row_end - 1);
      const uint8_t* rb = blocks + static_cast<int64_t>(r) * rowbytes;  // wave-uniform
      rbm[i] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(rb) & 3u);
      if constexpr (QK) {
        hk[i][k] = *reinterpret_cast<const uint4*>(rb + hoff[k]);  // 16-byte aligned
      } else {
        hs[i][k] = AFFINE ? *reinterpret_cast<const int32_t*>(rb + hoff[k])
                          : *reinterpret_cast<const uint16_t*>(rb + hoff[k]);
        if constexpr (FMT != QBLK_Q4_0) hc[i][k] = *reinterpret_cast<const int8_t*>(rb + coff[k]);
        if constexpr (AFFINE) ha[i][k] = *reinterpret_cast<const int8_t*>(rb + coff[k] + 8);
      }
      if constexpr (AFFINE) {
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(rb + off[k]);  // 4-aligned
        q[i][k][0] = v.x; q[i][k][1] = v.y; q[i][k][2] = v.z; q[i][k][3] = v.w;
        q[i][k][4] = 0;
      } else {
        // dword-aligned start at or below the code bytes; covers [o-2, o+14)
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(rb - rbm[i] + ((off[k] + rbm[i]) & ~3u));
        q[i][k][0] = v.x; q[i][k][1] = v.y; q[i][k][2] = v.z; q[i][k][3] = v.w;
        q[i][k][4] = *reinterpret_cast<const uint16_t*>(rb + off[k] + 14);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // (3) x pairs matching the code words: for word t (bytes 4t..4t+3) the pairs
  // are (x[4t], x[4t+2]), (x[4t+16], x[4t+18]), (x[4t+1], x[4t+3]),
  // (x[4t+17], x[4t+19]); Type 1 also needs the unit's sum of x.  Formed for
  // unit k just before its products (below), after an empty asm that
  // "redefines" the x registers there: nothing may use x before every weight
  // load above is issued, and unit k's pairs wait only for their own loads.
  uint4 X[UPL][4];
  float sx[UPL];
  const half2_t kOne = {1.0f16, 1.0f16};
  if constexpr (XL == 1) {
    publish_x();
    if (KS == 1 && row0 + slot >= row_end) return;
  }
  auto make_pairs = [&](int k) {
    if constexpr (XL) {
      const int uu = part * SP + lane + 64 * k;  // < KS * UPL * 64
#pragma unroll
      for (int t = 0; t < 4; t++) X[k][t] = xs[(4 * (uu >> 6) + t) * 64 + ((uu + 8 * t) & 63)];
      sx[k] = 0.0f;
      if constexpr (AFFINE) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
          sx[k] = __builtin_amdgcn_fdot2(as_h2(X[k][t].x), kOne, sx[k], false);
          sx[k] = __builtin_amdgcn_fdot2(as_h2(X[k][t].y), kOne, sx[k], false);
          sx[k] = __builtin_amdgcn_fdot2(as_h2(X[k][t].z), kOne, sx[k], false);
          sx[k] = __builtin_amdgcn_fdot2(as_h2(X[k][t].w), kOne, sx[k], false);
        }
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < 4; c++)
      asm volatile("" : "+v"(xr[k][c].x), "+v"(xr[k][c].y), "+v"(xr[k][c].z), "+v"(xr[k][c].w)::"memory");
    const uint32_t* h = reinterpret_cast<const uint32_t*>(xr[k]);  // h[d] = x[2d], x[2d+1]
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const uint32_t a0 = h[2 * t], a1 = h[2 * t + 1], b0 = h[2 * t + 8], b1 = h[2 * t + 9];
      X[k][t] = make_uint4(__builtin_amdgcn_perm(a1, a0, 0x05040100u), __builtin_amdgcn_perm(b1, b0, 0x05040100u),
                           __builtin_amdgcn_perm(a1, a0, 0x07060302u), __builtin_amdgcn_perm(b1, b0, 0x07060302u));
    }
    sx[k] = 0.0f;
    if constexpr (AFFINE) {
#pragma unroll
      for (int d = 0; d < 16; d++) sx[k] = __builtin_amdgcn_fdot2(as_h2(h[d]), kOne, sx[k], false);
    }
  };

  constexpr bool kLazyPairs = kLateX || XL;  // each unit's pairs just before its products
  if constexpr (!kLazyPairs) {
#pragma unroll
    for (int k = 0; k < UPL; k++) make_pairs(k);
  }

  // (4) products
  const uint32_t kMagic = 0x64006400u;
  const half2_t kLo = AFFINE ? half2_t{-1024.0f16, -1024.0f16} : half2_t{-1032.0f16, -1032.0f16};
  const half2_t kHi = AFFINE ? half2_t{-1024.0f16, -1024.0f16} : half2_t{-1152.0f16, -1152.0f16};
  float acc[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; i++) acc[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < UPL; k++) {
    if constexpr (kLazyPairs) make_pairs(k);
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
      // one group at a time: the accumulators (written by the groups before)
      // and this group's loaded registers are "redefined" here, in order, so
      // neither can a later group's decode move up nor an earlier group's
      // products move down (either keeps several groups' decoded codes live).
      // Not for Q4_K with three units per lane: there the pinned 16-byte
      // headers would not fit in a wave's registers.
      // A last row slot past the workgroup's rows repeats its last row
      // (loaded, to keep every wave's loads unconditional): its math is
      // skipped (the wave still meets the barrier below when KS > 1).  For the
      // affine formats the compiler sinks that row's loads into the skip
      // branch unless the pins below come first, so there the skip follows
      // them; for Type 0 and Q4_0 it does not, and skipping before the pins
      // is a little faster.
      // (one slot per wave and one wave per row: a wave without a row has
      // returned, so there is nothing to skip and no branch to merge)
      const bool dup = (RMAX > 1 || KS > 1) && i == RMAX - 1 && row0 + slot + SLOTS * i >= row_end;
      if constexpr (!AFFINE) {
        if (dup) continue;
      }
      if constexpr (!(QK && UPL > 2)) {  // (Q4_K, three units per lane: no registers to spare)
#pragma unroll
        for (int r = 0; r < RMAX; r++) asm volatile("" : "+v"(acc[r]));
        asm volatile("" : "+v"(q[i][k][0]), "+v"(q[i][k][1]), "+v"(q[i][k][2]), "+v"(q[i][k][3]), "+v"(q[i][k][4]));
        if constexpr (QK) asm volatile("" : "+v"(hk[i][k].x), "+v"(hk[i][k].y), "+v"(hk[i][k].z), "+v"(hk[i][k].w));
        else if constexpr (AFFINE) asm volatile("" : "+v"(hs[i][k]), "+v"(hc[i][k]), "+v"(ha[i][k]));
        if constexpr (AFFINE) {
          if (dup) continue;
        }
      }
      uint32_t c[4];
      if constexpr (AFFINE) {
        c[0] = q[i][k][0]; c[1] = q[i][k][1]; c[2] = q[i][k][2]; c[3] = q[i][k][3];
      } else {
        const uint32_t a = (off[k] + rbm[i]) & 3u;  // 0 or 2
        c[0] = __builtin_amdgcn_alignbyte(q[i][k][1], q[i][k][0], a);
        c[1] = __builtin_amdgcn_alignbyte(q[i][k][2], q[i][k][1], a);
        c[2] = __builtin_amdgcn_alignbyte(q[i][k][3], q[i][k][2], a);
        c[3] = __builtin_amdgcn_alignbyte(q[i][k][4], q[i][k][3], a);
      }
      float lo, hi;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const uint32_t b = c[t] >> 8;
        const half2_t v0 = as_h2(and_or(c[t], 0x000F000Fu, kMagic)) + kLo;
        const half2_t v1 = as_h2(and_or(c[t], 0x00F000F0u, kMagic)) + kHi;
        const half2_t v2 = as_h2(and_or(b, 0x000F000Fu, kMagic)) + kLo;
        const half2_t v3 = as_h2(and_or(b, 0x00F000F0u, kMagic)) + kHi;
        if (t == 0) {  // each chain starts from its first product (no zeroed accumulator to move)
          lo = dot2_first(v0, X[k][t].x);
          hi = dot2_first(v1, X[k][t].y);
        } else {
          lo = __builtin_amdgcn_fdot2(v0, as_h2(X[k][t].x), lo, false);
          hi = __builtin_amdgcn_fdot2(v1, as_h2(X[k][t].y), hi, false);
        }
        lo = __builtin_amdgcn_fdot2(v2, as_h2(X[k][t].z), lo, false);
        hi = __builtin_amdgcn_fdot2(v3, as_h2(X[k][t].w), hi, false);
      }
      float sc;
      if constexpr (FMT == QBLK_Q4_0) sc = f16_bits_to_f32(hs[i][k]);
      else if constexpr (QK)
        sc = f16_bits_to_f32(hk[i][k].x & 0xffffu) * static_cast<float>(q4k_scale6(hk[i][k].y, hk[i][k].z, sbj[k]));
      else sc = f16_bits_to_f32(hs[i][k] & 0xffff) * static_cast<float>(hc[i][k]);
      sc = live[k] ? sc : 0.0f;  // lanes past the row's last unit add 0
      acc[i] = __builtin_fmaf(sc, __builtin_fmaf(hi, 0.0625f, lo), acc[i]);
      if constexpr (AFFINE) {
        float oa;
        if constexpr (QK)
          oa = -(f16_bits_to_f32(hk[i][k].x >> 16) * static_cast<float>(q4k_min6(hk[i][k].z, hk[i][k].w, sbj[k])));
        else oa = f16_bits_to_f32(static_cast<uint32_t>(hs[i][k]) >> 16) * static_cast<float>(ha[i][k]);
        oa = live[k] ? oa : 0.0f;
        acc[i] = __builtin_fmaf(oa, sx[k], acc[i]);
      }
      // (and for the machine scheduler: hoisting the realignment of later
      // groups above this point would make the first product wait for every
      // load of the wave)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // (5) one sum per row; lane 63 holds it
  if constexpr (KS == 1) {
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
      const float v = wave_sum_dpp(acc[i]);
      const int r = row0 + slot + SLOTS * i;
      if (lane == kWave - 1 && r < row_end) y[r] = v;
    }
  } else {
    __shared__ float part_sum[WAVES][RMAX];
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
      const float v = wave_sum_dpp(acc[i]);
      if (lane == kWave - 1) part_sum[wave][i] = v;
    }
    __syncthreads();
    if (part == 0 && lane == kWave - 1) {
#pragma unroll
      for (int i = 0; i < RMAX; i++) {
        float v = part_sum[wave][i];
#pragma unroll
        for (int p = 1; p < KS; p++) v += part_sum[wave + p][i];
        const int r = row0 + slot + SLOTS * i;
        if (r < row_end) y[r] = v;
      }
    }
  }
}

template <int FMT, int RMAX, int UPL, int KS, int WAVES = kWavesH, int XL = 0>
__global__ __launch_bounds__(WAVES * kWave, WAVES == 8 ? 4 : 1) void k_gemv_h(const uint8_t* __restrict__ blocks,
                                                      const uint16_t* __restrict__ x,
                                                      float* __restrict__ y, int M, int K,
                                                      int rows_per_wg) {
  gemv_h_body<FMT, RMAX, UPL, KS, WAVES, XL>(blocks, x, y, M, K, rows_per_wg, blockIdx.x);
}

// Several matrices of equal k in one grid: matrix i takes workgroups
// [wg_end[i-1], wg_end[i]) (kernel arguments, 1 KB at most, read with scalar
// loads).
struct GemvBatch {
  const uint8_t* blocks[QBLK_GEMV_BATCH_MAX];
  const uint16_t* x[QBLK_GEMV_BATCH_MAX];
  float* y[QBLK_GEMV_BATCH_MAX];
  int m[QBLK_GEMV_BATCH_MAX];
  unsigned wg_end[QBLK_GEMV_BATCH_MAX];
  int count;
};

template <int FMT, int RMAX, int UPL, int KS, int WAVES = kWavesH, int XL = 0>
__global__ __launch_bounds__(WAVES * kWave, WAVES == 8 ? 4 : 1) void k_gemv_hb(const GemvBatch b, int K, int rows_per_wg) {
  const unsigned w = blockIdx.x;
  int i = 0;
  while (i + 1 < b.count && w >= b.wg_end[i]) i++;
  const unsigned first = i > 0 ? b.wg_end[i - 1] : 0u;
  gemv_h_body<FMT, RMAX, UPL, KS, WAVES, XL>(b.blocks[i], b.x[i], b.y[i], b.m[i], K, rows_per_wg, w - first);
}

// y[0, n) = 0: 16-byte stores (y is 16-byte aligned), a scalar tail.
__global__ __launch_bounds__(256) void k_fill_zero(float* y, int64_t n) {
  const int64_t n4 = n >> 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<float4*>(y)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) y[(n4 << 2) + threadIdx.x] = 0.0f;
}

// Rows per wave of the generic kernel (fp32 or bf16 x, or rows past 12288
// weights): 2 measured faster than 4 at every size tried, by the number of
// workgroups in flight for small matrices (256 x 4096 fp32 x, Q4_0: 9.1 ->
// 5.9 us) and by loads in flight per lane for large ones (11008 x 4096
// Type 0: 15.3 -> 12.1 us); 1 row per wave was slower on three of four --
// all but Q4_0 with few rows, which takes it (256 x 4096 fp32 x: 5.9 ->
// 4.5 us; Type 0 there 4.6 -> 6.0 us, Q4_0 at 4096 rows 6.95 against 7.00).
constexpr int kRows = 2;

template <int FMT, int XT, int R>
hipError_t launch_tr(const void* blocks, int64_t m, int64_t k, const void* x, float* y,
                     hipStream_t s) {
  constexpr bool XH = XT == QBLK_F16;
  constexpr int KC = XH ? kChunkF16 : kChunkF32;
  const int64_t kc = k < KC ? k : KC;
  const size_t lds = (XH ? kc * 2 : kc * 4) + (kc / 32) * 4;
  const int64_t groups = (m + R - 1) / R;
  const unsigned grid = static_cast<unsigned>((groups + kWaves - 1) / kWaves);
  if (log_enabled())
    log_launch("gemv k_gemv fmt=%d x=%d rows/wave=%d m=%lld k=%lld grid=%u block=%d lds=%zu", FMT, XT, R,
               (long long)m, (long long)k, grid, kThreads, lds);
  hipLaunchKernelGGL((k_gemv<FMT, XT, R>), dim3(grid), dim3(kThreads), lds, s,
                     static_cast<const uint8_t*>(blocks), x, y, static_cast<int>(m),
                     static_cast<int>(k));
  return hipGetLastError();
}

template <int FMT, int XT>
hipError_t launch_t(const void* blocks, int64_t m, int64_t k, const void* x, float* y,
                    hipStream_t s) {
  if (FMT == QBLK_Q4_0 && m <= 1024) return launch_tr<FMT, XT, 1>(blocks, m, k, x, y, s);
  return launch_tr<FMT, XT, kRows>(blocks, m, k, x, y, s);
}

// What one launch of the fp16-x kernel multiplies: one matrix (items ==
// nullptr), or a batch of matrices of equal k.  m sets the tiling: the
// matrix's rows, or the batch's rows together.
struct GemvJob {
  const void* blocks;
  const void* x;
  float* y;
  int64_t m;
  const qblk_gemv_item_t* items;
  int count;
};

template <int FMT, int RMAX, int UPL, int KS, int WAVES, int XL = 0>
hipError_t launch_h_t(const GemvJob& j, int64_t k, int rows_per_wg, hipStream_t s) {
  if (j.items == nullptr) {
    const unsigned grid = static_cast<unsigned>((j.m + rows_per_wg - 1) / rows_per_wg);
    if (log_enabled())
      log_launch("gemv k_gemv_h fmt=%d row-slots/wave=%d units/lane=%d waves/row=%d waves=%d x-lds=%d m=%lld "
                 "k=%lld rows/wg=%d grid=%u", FMT, RMAX, UPL, KS, WAVES, XL, (long long)j.m, (long long)k,
                 rows_per_wg, grid);
    hipLaunchKernelGGL((k_gemv_h<FMT, RMAX, UPL, KS, WAVES, XL>), dim3(grid), dim3(WAVES * kWave), 0, s,
                       static_cast<const uint8_t*>(j.blocks), static_cast<const uint16_t*>(j.x), j.y,
                       static_cast<int>(j.m), static_cast<int>(k), rows_per_wg);
    return hipGetLastError();
  }
  GemvBatch b;
  unsigned grid = 0;
  for (int i = 0; i < j.count; i++) {
    b.blocks[i] = static_cast<const uint8_t*>(j.items[i].blocks);
    b.x[i] = static_cast<const uint16_t*>(j.items[i].x);
    b.y[i] = j.items[i].y;
    b.m[i] = static_cast<int>(j.items[i].m);
    grid += static_cast<unsigned>((j.items[i].m + rows_per_wg - 1) / rows_per_wg);
    b.wg_end[i] = grid;
  }
  b.count = j.count;
  if (log_enabled())
    log_launch("gemv k_gemv_hb fmt=%d row-slots/wave=%d units/lane=%d waves/row=%d waves=%d x-lds=%d matrices=%d "
               "rows=%lld k=%lld rows/wg=%d grid=%u", FMT, RMAX, UPL, KS, WAVES, XL, j.count, (long long)j.m,
               (long long)k, rows_per_wg, grid);
  hipLaunchKernelGGL((k_gemv_hb<FMT, RMAX, UPL, KS, WAVES, XL>), dim3(grid), dim3(WAVES * kWave), 0, s, b,
                     static_cast<int>(k), rows_per_wg);
  return hipGetLastError();
}

// Rows per workgroup: an even share of the rows over the CUs, between one and
// rmax_cap rounds of `slots` rows.  Where the share exceeds that cap, either
// the cap (even_rounds false: the last round of workgroups can run partly
// empty), or the share split into equal rounds of workgroups of at most the
// cap (even_rounds true: every CU gets the same rows in each round).
inline int rows_per_wg(int64_t m, int slots, int rmax_cap, bool even_rounds) {
  int64_t per = (m + cu_count() - 1) / cu_count();
  const int64_t cap = static_cast<int64_t>(slots) * rmax_cap;
  const int64_t rounds = (per + cap - 1) / cap;
  if (rounds > 1) per = even_rounds ? (per + rounds - 1) / rounds : cap;
  per = per < slots ? slots : per;
  return static_cast<int>(per);
}

// Row slots per wave: the smallest template count R >= rmax, up to RCAP.
template <int FMT, int UPL, int KS, int RCAP, int WAVES, int XL, int R = 1>
hipError_t launch_h_r(int rmax, const GemvJob& j, int64_t k, int rpw, hipStream_t s) {
  if constexpr (R < RCAP) {
    if (rmax > R) return launch_h_r<FMT, UPL, KS, RCAP, WAVES, XL, R + 1>(rmax, j, k, rpw, s);
  }
  return launch_h_t<FMT, R, UPL, KS, WAVES, XL>(j, k, rpw, s);
}

// Two workgroups per CU: 8 waves each, at most 128 registers per lane (the
// kernels' launch bounds ask for 4 waves per SIMD at 8 waves), rows shared
// evenly over 2 x CUs workgroup slots, in equal rounds of at most RCAP row
// slots per wave.
template <int FMT, int UPL, int KS, int RCAP, int XL = 0>
hipError_t launch_h_k2(const GemvJob& j, int64_t k, hipStream_t s) {
  constexpr int WAVES = 8, slots = WAVES / KS;
  int64_t per = (j.m + 2 * cu_count() - 1) / (2 * cu_count());
  const int64_t cap = static_cast<int64_t>(slots) * RCAP;
  const int64_t rounds = (per + cap - 1) / cap;
  if (rounds > 1) per = (per + rounds - 1) / rounds;
  per = per < slots ? slots : per;
  const int rpw = static_cast<int>(per);
  return launch_h_r<FMT, UPL, KS, RCAP, WAVES, XL>((rpw + slots - 1) / slots, j, k, rpw, s);
}

template <int FMT, int UPL, int KS, int RCAP, int WAVES = kWavesH, int XL = 0>
hipError_t launch_h_k(const GemvJob& j, int64_t k, hipStream_t s, bool even_rounds = true) {
  constexpr int slots = WAVES / KS;
  const int rpw = rows_per_wg(j.m, slots, RCAP, even_rounds);
  return launch_h_r<FMT, UPL, KS, RCAP, WAVES, XL>((rpw + slots - 1) / slots, j, k, rpw, s);
}

// fp16 x and at most 384 units (12288 weights) per row: the up-front kernel.
// Each wave loads x for every unit it covers and reuses it across its rows,
// so x is re-read once per wave; splitting a row over two waves halves the x
// each wave loads (it matters most when a CU holds few rows). By units per
// row S: up to 64 one wave per row and one unit per lane; up to 128 two
// waves per row with one unit per lane each, up to 8 rows per wave (at
// 4096 x 4096: 4.8-4.9 -> 4.3-4.5 us; at 11008 x 4096 Q4_0 8.0 -> 7.7,
// Type 1 7.6 -> 7.4, Q4_K 7.8 -> 7.5 us) -- except Type 0 and Q4_0 with
// more than 32 rows per CU: one wave per row, two units per lane, up to 4
// rows per wave of 16-wave workgroups, x staged once per workgroup through
// LDS before any weight load is issued (11008 x 4096 Type 0: 7.03 us with
// every wave loading its own x in 12-wave workgroups, 6.66 us with x staged,
// 6.60 us with x staged in 16-wave workgroups; Q4_0 7.42 -> 7.13 us; the
// affine formats staged so were slower, 7.18 -> 7.20 us and 7.28 -> 7.36
// us); up to 256 two waves per row with two units per lane; up to
// 384 three (Type 0 in 12-wave workgroups with up to 3 rows per wave: 4096 x
// 11008 7.98 against 8.20 us; the other formats gain 1.4% at most, and Q4_K
// runs out of registers; Type 0 with at most 16 rows per CU stages x through
// LDS before its loads, 4096 x 11008: 7.96 -> 7.00 us; for Type 1 and Q4_K,
// and Q4_0 at 4096 x 4096, staging so was slower: 7.71 -> 7.75, 7.27 -> 7.36,
// 4.00 -> 4.23 us).  With at most 16 rows per CU, x read by every wave
// outweighs the weights; x through LDS (one wave per row) is taken where it
// measured faster: Q4_0 up to 128 units (4096 x 4096: 4.44 -> 4.00 us) and
// Type 1 beyond 256 (4096 x 11008: 8.35 -> 7.68 us); for Type 0 and Q4_K it
// was not (4096 x 4096 within 2%, 4096 x 11008 Type 0 +9%).  These two keep
// the barrier after the weight loads (staging before them: 4.00 -> 4.09 and
// 7.71 -> 7.99 us).  Up to 128 units a workgroup takes up to 64 rows (4 slots
// of 16 or 8 of 8): from 49 to 64 rows per CU that is one round of workgroups
// where 48-row workgroups made 1.2-1.3 rounds (14336 x 4096: Type 0 10.7 ->
// 8.2 us, Q4_0 10.9 -> 8.7, Type 1 12.0 -> 8.9, Q4_K 12.3 -> 8.6).  With more
// rows per CU than a workgroup takes, rows of up to 256 units are split into
// equal rounds (16385 x 4096 Type 0 11.0 -> 10.3 us, Type 1 12.3 -> 11.0;
// 28672 x 4096 Type 0 16.8 -> 15.6, Q4_K 19.3 -> 16.5; 11008 x 8192 2-3% in
// every format); longer rows keep full workgroups and a partly empty last
// round (14336 x 11008 Q4_K: 29.5 us, 31.1 in equal rounds).  Past one round
// of 64-row workgroups the affine formats (up to 128 units) run two 8-wave
// workgroups per CU, so one workgroup's loads are in flight while the other
// finishes: Type 1 4-12% and Q4_K 1-15% faster from 16385 to 44032 rows
// (38400 x 4096 Type 1: 22.5 -> 21.0 us); for Type 0 and Q4_0 it was mixed
// (Type 0 +3-5% from 16385 to 22016 rows, -10% at 44032), so they keep one
// 16-wave workgroup per CU.
template <int FMT>
bool launch_h(const GemvJob& j, int64_t k, hipStream_t s, hipError_t* err) {
  const int64_t S = k / 32;
  if (S > 6 * 64) return false;
  const int64_t m = j.m;
  const int64_t per_cu = (m + cu_count() - 1) / cu_count();
  constexpr bool kSigned = FMT == QBLK_SB4 || FMT == QBLK_Q4_0;
  const bool few = per_cu <= kWavesH;  // one row per wave at most
  if (S <= 64) *err = launch_h_k<FMT, 1, 1, 3>(j, k, s);
  else if (S <= 128 && FMT == QBLK_Q4_0 && few)
    *err = launch_h_t<FMT, 1, 2, 1, kWavesH, 1>(j, k, rows_per_wg(m, kWavesH, 1, true), s);
  else if (S > 256 && FMT == QBLK_SB4_AFFINE && few)
    *err = launch_h_t<FMT, 1, 6, 1, kWavesH, 1>(j, k, rows_per_wg(m, kWavesH, 1, true), s);
  else if (S <= 128 && kSigned && per_cu > 32) *err = launch_h_k<FMT, 2, 1, 4, kWavesH, 2>(j, k, s);
  else if (S <= 128 && per_cu > 64) *err = launch_h_k2<FMT, 1, 2, 8>(j, k, s);
  else if (S <= 128) *err = launch_h_k<FMT, 1, 2, 8>(j, k, s);
  else if (S <= 256) *err = launch_h_k<FMT, 2, 2, 3>(j, k, s);
  else if (FMT == QBLK_SB4 && few) *err = launch_h_k<FMT, 3, 2, 2, kWavesH, 2>(j, k, s, false);
  else if (FMT == QBLK_SB4) *err = launch_h_k<FMT, 3, 2, 3, 12>(j, k, s, false);
  else *err = launch_h_k<FMT, 3, 2, 2>(j, k, s, false);
  return true;
}

template <int FMT>
hipError_t launch_fmt(const void* blocks, int64_t m, int64_t k, const void* x, int xt, float* y,
                      hipStream_t s) {
  hipError_t err = hipSuccess;
  if (xt == QBLK_F16 && launch_h<FMT>(GemvJob{blocks, x, y, m, nullptr, 0}, k, s, &err)) return err;
  if (xt == QBLK_F16) return launch_t<FMT, QBLK_F16>(blocks, m, k, x, y, s);
  if (xt == QBLK_F32) return launch_t<FMT, QBLK_F32>(blocks, m, k, x, y, s);
  return launch_t<FMT, QBLK_BF16>(blocks, m, k, x, y, s);
}

}  // namespace

namespace {
// One matrix in pieces of at most kGemvRowsPerLaunch rows (a piece starts
// at a row, so it is laid out like any other row start).
template <int FMT>
hipError_t launch_rows(const void* blocks, int64_t m, int64_t k, const void* x, int xt, float* y, hipStream_t s) {
  const int64_t rowbytes = (k / Fmt<FMT>::E) * Fmt<FMT>::B;
  for (int64_t r0 = 0; r0 < m; r0 += kGemvRowsPerLaunch) {
    const int64_t n = m - r0 < kGemvRowsPerLaunch ? m - r0 : kGemvRowsPerLaunch;
    const hipError_t e = launch_fmt<FMT>(static_cast<const uint8_t*>(blocks) + r0 * rowbytes, n, k, x, xt, y + r0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT>
hipError_t launch_batch_fmt(int64_t k, int xt, const qblk_gemv_item_t* items, int count, hipStream_t s) {
  int64_t rows = 0;
  for (int i = 0; i < count; i++) rows += items[i].m;
  hipError_t err = hipSuccess;
  if (xt == QBLK_F16 && rows <= kGemvRowsPerLaunch &&
      launch_h<FMT>(GemvJob{nullptr, nullptr, nullptr, rows, items, count}, k, s, &err))
    return err;
  // other x types, rows past 12288 weights or past one launch's rows: one
  // launch per matrix (or piece of one)
  for (int i = 0; i < count && err == hipSuccess; i++)
    err = launch_rows<FMT>(items[i].blocks, items[i].m, k, items[i].x, xt, items[i].y, s);
  return err;
}
}  // namespace

hipError_t launch_gemv_batch(int fmt, int64_t k, int xt, const qblk_gemv_item_t* items, int count,
                             hipStream_t s) {
  if (fmt == QBLK_Q4_0) return launch_batch_fmt<QBLK_Q4_0>(k, xt, items, count, s);
  if (fmt == QBLK_SB4) return launch_batch_fmt<QBLK_SB4>(k, xt, items, count, s);
  if (fmt == QBLK_Q4_K) return launch_batch_fmt<QBLK_Q4_K>(k, xt, items, count, s);
  return launch_batch_fmt<QBLK_SB4_AFFINE>(k, xt, items, count, s);
}

hipError_t launch_gemv(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       float* y, hipStream_t s) {
  if (fmt == QBLK_Q4_0) return launch_rows<QBLK_Q4_0>(blocks, m, k, x, xt, y, s);
  if (fmt == QBLK_SB4) return launch_rows<QBLK_SB4>(blocks, m, k, x, xt, y, s);
  if (fmt == QBLK_Q4_K) return launch_rows<QBLK_Q4_K>(blocks, m, k, x, xt, y, s);
  return launch_rows<QBLK_SB4_AFFINE>(blocks, m, k, x, xt, y, s);
}

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  // grid-stride over float4s: at most 8 workgroups per CU
  int64_t g = ((n >> 2) + 255) / 256;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
  g = g < 1 ? 1 : (g > cap ? cap : g);
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(g)), dim3(256), 0, s, y, n);
  return hipGetLastError();
}

}  // namespace qblk
