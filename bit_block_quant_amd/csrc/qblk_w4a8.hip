// qblk_w4a8.hip -- products of group-128 4-bit weights with 8-bit activations
// on gfx950 (the W4A8 scheme of the TurboQuant article, sections 2.1-2.2).
//
// What is computed: Y[t,i] = s_t * sum_g d[i,g] * sum_{k in g} (code-8) * xq[t,k]
// -- the product of the rebuilt weights d*(code-8) and the rebuilt activations
// s_t*xq.  The inner sums are integers, formed exactly in int32 (v_dot4_i32_i8
// for one token, int8 matrix ops -- 16x16x64 tiles up to 16 tokens, 32x32x32
// wide tiles beyond -- for several); each group's sum is then
// scaled by its fp16 weight scale in fp32, and the token scale is applied
// once at the end.  The codes enter the integer products as they are stored
// (0..15); the -8 offset is the integer -8 * sum(xq) over the same k range,
// formed once per token and k range and used as the starting value.
//
// Weight layout (planar): the code plane, k/2 bytes per row, byte j of group
// g holding weight 128g+j (low nibble) and 128g+64+j (high nibble), then the
// fp16 scale plane, k/128 entries per row.
#include "qblk_device.h"
#include "qblk_launch.h"

namespace qblk {
namespace {

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kOnes8 = 0x01010101u;

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}


// ===================================================================
// One token: every load of a wave issued up front.
//
// The rows are split evenly over workgroups of W = 16 (or 12) waves, one per
// CU; wave w takes rows w, w+W, w+2W, ... of its slice.  A code row is a run
// of 16-byte chunks of 32 weights; lane l takes chunks l, l+64, ... (UPL of
// them), so it sees the
// same activations in every row: chunk c (group c/4, quarter c%4) pairs its
// low nibbles with xq[128g+16q .. +16] and its high nibbles with the 16 bytes
// 64 further on.  Per chunk: 8 v_dot4 and 8 masks; per (chunk, row) one fp32
// multiply-add with the group's scale (four lanes share a group).
// ===================================================================
constexpr int kWavesV = 16;

template <int RMAX, int UPL, int WAVES = kWavesV>
__global__ __launch_bounds__(WAVES * kWave) void k_gemv_w4a8(const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ scales,
                                                              const int8_t* __restrict__ xq,
                                                              const float* __restrict__ xs,
                                                              float* __restrict__ y, int M, int K,
                                                              int rows_per_wg) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row0 = blockIdx.x * rows_per_wg;
  const int row_end = min(M, row0 + rows_per_wg);
  if (row0 + wave >= row_end) return;
  const int C = K >> 5;   // chunks per row
  const int NG = K >> 7;  // groups per row
  const int64_t rowbytes = K >> 1;

  // (1) the lane's activations: chunk 0's issued first, chunk i's just before
  // the weight groups of chunk i (so the first weight requests are not
  // queued behind every activation request of the CU's waves)
  uint4 xl[UPL], xh[UPL];
  int cc[UPL];
  bool live[UPL];
#pragma unroll
  for (int i = 0; i < UPL; i++) {
    const int c = lane + 64 * i;
    live[i] = c < C;
    cc[i] = min(c, C - 1);
  }
  auto load_x = [&](int i) {
    const int8_t* p = xq + 128 * (cc[i] >> 2) + 16 * (cc[i] & 3);
    xl[i] = *reinterpret_cast<const uint4*>(p);
    xh[i] = *reinterpret_cast<const uint4*>(p + 64);
  };
  load_x(0);
  __builtin_amdgcn_sched_barrier(0);

  // (2) codes and scales of every (chunk, row), chunk-major
  uint4 cw[RMAX][UPL];
  uint32_t sc[RMAX][UPL];
#pragma unroll
  for (int i = 0; i < UPL; i++) {
    if (i > 0) {
      load_x(i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < RMAX; r++) {
      const int row = min(row0 + wave + WAVES * r, row_end - 1);
      cw[r][i] = *reinterpret_cast<const uint4*>(codes + row * rowbytes + 16 * cc[i]);
      sc[r][i] = scales[static_cast<int64_t>(row) * NG + (cc[i] >> 2)];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // (3) -8 * sum(xq) over each chunk's 32 activations, formed for chunk i
  // just before its products, after an empty asm that "redefines" its
  // activation registers there (nothing may touch them before every weight
  // load is issued, and chunk i waits only for its own loads)
  int corr[UPL];
  auto chunk_corr = [&](int i) {
    asm volatile("" : "+v"(xl[i].x), "+v"(xl[i].y), "+v"(xl[i].z), "+v"(xl[i].w), "+v"(xh[i].x), "+v"(xh[i].y),
                 "+v"(xh[i].z), "+v"(xh[i].w)::"memory");
    int s = dot4(xl[i].x, kOnes8, 0);
    s = dot4(xl[i].y, kOnes8, s);
    s = dot4(xl[i].z, kOnes8, s);
    s = dot4(xl[i].w, kOnes8, s);
    s = dot4(xh[i].x, kOnes8, s);
    s = dot4(xh[i].y, kOnes8, s);
    s = dot4(xh[i].z, kOnes8, s);
    s = dot4(xh[i].w, kOnes8, s);
    corr[i] = -8 * s;
  };

  // (4) products
  float acc[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; r++) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < UPL; i++) {
    chunk_corr(i);
#pragma unroll
    for (int r = 0; r < RMAX; r++) {
      // one (chunk, row) group at a time: the accumulators and this group's
      // loaded registers are "redefined" here, in order, so the compiler can
      // neither hoist a later group's work nor sink an earlier group's, and
      // each group waits only for its own loads
#pragma unroll
      for (int q = 0; q < RMAX; q++) asm volatile("" : "+v"(acc[q]));
      asm volatile("" : "+v"(cw[r][i].x), "+v"(cw[r][i].y), "+v"(cw[r][i].z), "+v"(cw[r][i].w), "+v"(sc[r][i]));
      // a last row slot past the workgroup's rows repeats its last row: skip
      // the math (only after the pins, which keep its loads out of the branch)
      if (r == RMAX - 1 && row0 + wave + WAVES * r >= row_end) continue;
      const uint4 c = cw[r][i];
      int a = corr[i];
      a = dot4(c.x & kLo4, xl[i].x, a);
      a = dot4((c.x >> 4) & kLo4, xh[i].x, a);
      a = dot4(c.y & kLo4, xl[i].y, a);
      a = dot4((c.y >> 4) & kLo4, xh[i].y, a);
      a = dot4(c.z & kLo4, xl[i].z, a);
      a = dot4((c.z >> 4) & kLo4, xh[i].z, a);
      a = dot4(c.w & kLo4, xl[i].w, a);
      a = dot4((c.w >> 4) & kLo4, xh[i].w, a);
      const float d = live[i] ? f16_bits_to_f32(sc[r][i]) : 0.0f;
      acc[r] = __builtin_fmaf(d, static_cast<float>(a), acc[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float st = xs[0];
#pragma unroll
  for (int r = 0; r < RMAX; r++) {
    const float v = wave_sum_dpp(acc[r]);
    const int row = row0 + wave + WAVES * r;
    if (lane == kWave - 1 && row < row_end) y[row] = v * st;
  }
}

// ===================================================================
// Up to 16 tokens: v_mfma_i32_16x16x64_i8, weights loaded by whole units.
//
// Operand layout: lane l holds row (l % 16) of A and column (l % 16) of B,
// each with 16 int8 k values of its lane group (l / 16); lane l receives
// D[4*(l/16) + r][l % 16], r = 0..3.  Only A and B sharing the k assignment
// matters: for step s (0, 1) of a 128-weight group, lane group g takes code
// bytes j0..j0+7, j0 = 16g + 8s -- weights j0..j0+7 (low nibbles) and
// 64+j0..64+j0+7 (high nibbles) -- and the same 16 activations.  A = X
// (tokens), B = W^T (weight rows), so a lane's four outputs share one weight
// row and one scale per group.  The integer accumulator of a group starts at
// -8 * sum(xq) of its token over the group.
//
// Loading B straight from the code plane (16 rows per instruction) would ask
// for each cache line several times.  Instead a workgroup's tile -- 64 rows
// by NG groups -- is fetched as plain rows: lane after lane takes consecutive
// 16-byte units of a row (a group's 64 code bytes are 4 units), and the units
// go unchanged to LDS, each row padded by 16 bytes; with the contiguous k
// assignment above, one 16-byte LDS read per row and group feeds both steps
// (16 rows of a read phase: row stride = 4 mod 64 dwords, 64 different
// banks).  X is staged per group and token as 8 pieces of 16 bytes (piece p:
// activations 8p..8p+7 and 64+8p..64+8p+7), token rows 144 bytes apart, and
// a lane reads its pieces 2g and 2g+1.  KW waves share each 16 rows, each
// taking NG/KW of the groups, and add their sums in LDS at the end.  Every
// load is issued before the single barrier; the K range is split over the
// grid and the partial products are added into Y (zeroed first).
// ===================================================================
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreadsM = 256;
constexpr int kXRow = 144;  // bytes per staged token row

template <int NG, int KW, bool SPLIT>
__global__ __launch_bounds__(kThreadsM * KW) void k_gemm_w4a8_u(const uint8_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           const int8_t* __restrict__ xq,
                                                           const float* __restrict__ xs,
                                                           float* __restrict__ Y, int M, int K, int N) {
  constexpr int kT = kThreadsM * KW;             // KW waves per 16 rows, each a share of the groups
  constexpr int UR = 4 * NG;                      // units per row in the slice
  constexpr int kUPT = 64 * UR / kT;              // units per thread
  static_assert(64 * UR % kT == 0 && NG % KW == 0, "whole units per thread, whole groups per wave");
  constexpr int kCodeRow = 16 * UR + 16;          // bytes per staged code row
  constexpr int kPieces = NG * 16 * 8;            // 16-byte pieces of the X slice
  constexpr int kPer = (kPieces + kT - 1) / kT;
  constexpr int kSc = 64 * NG;                    // scales of the tile
  __shared__ uint4 xs4[NG * 16 * kXRow / 16];
  __shared__ uint4 cs4[64 * kCodeRow / 16];
  __shared__ float scs[kSc];
  __shared__ i32x4_t xcor4[NG * 4];               // -8 * sum(xq) per group and token
  __shared__ float4_t red[KW > 1 ? (KW - 1) * 4 * 64 : 1];
  int* const xcor = reinterpret_cast<int*>(xcor4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int ngr = K >> 7;
  const int64_t rowbytes = K >> 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int n0 = blockIdx.y * 16;
  const int b0 = blockIdx.z * NG;
  const int nb = min(NG, ngr - b0);  // groups in this piece of K (>= 1)

  // X first (L2-resident), then the units and scales of the tile.  Loads past
  // the slice's last group or past row M-1 re-read valid data that is never
  // used or never stored; tokens past N-1 read as zero.
  uint4 xv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int c = min(static_cast<int>(threadIdx.x) + i * kT, kPieces - 1);
    const int gi = c >> 7, tok = (c >> 3) & 15, cc = c & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n0 + tok < N)
      v = *reinterpret_cast<const uint4*>(xq + static_cast<int64_t>(n0 + tok) * K + 128 * (b0 + min(gi, nb - 1)) +
                                          16 * cc);
    xv[i] = v;
  }
  uint4 cu[kUPT];
#pragma unroll
  for (int i = 0; i < kUPT; i++) {
    const int U = static_cast<int>(threadIdx.x) + i * kT;
    const int r = U / UR, u = U % UR;
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    cu[i] = *reinterpret_cast<const uint4*>(codes + m * rowbytes + 64 * static_cast<int64_t>(b0 + min(u >> 2, nb - 1)) +
                                            16 * (u & 3));
  }
  uint32_t scv[(kSc + kT - 1) / kT];
#pragma unroll
  for (int i = 0; i < (kSc + kT - 1) / kT; i++) {
    const int c = min(static_cast<int>(threadIdx.x) + i * kT, kSc - 1);
    const int r = c / NG, gi = c % NG;
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    scv[i] = scales[m * ngr + b0 + min(gi, nb - 1)];
  }

  uint8_t* xsb = reinterpret_cast<uint8_t*>(xs4);
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int c = static_cast<int>(threadIdx.x) + i * kT;
    const int gi = c >> 7, tok = (c >> 3) & 15, cc = c & 7;
    if (kPieces % kT == 0 || c < kPieces) {
      // activations 16cc..16cc+15 of the group: pieces 2(cc&3) and 2(cc&3)+1,
      // first halves (cc < 4) or second halves (cc >= 4)
      uint8_t* row = xsb + (gi * 16 + tok) * kXRow + 32 * (cc & 3) + 8 * (cc >> 2);
      *reinterpret_cast<uint2*>(row) = make_uint2(xv[i].x, xv[i].y);
      *reinterpret_cast<uint2*>(row + 16) = make_uint2(xv[i].z, xv[i].w);
    }
    int sm = dot4(xv[i].x, kOnes8, 0);
    sm = dot4(xv[i].y, kOnes8, sm);
    sm = dot4(xv[i].z, kOnes8, sm);
    sm = dot4(xv[i].w, kOnes8, sm);
    // the 8 pieces of a token and group sit on 8 adjacent lanes
    sm += __shfl_xor(sm, 1, kWave);
    sm += __shfl_xor(sm, 2, kWave);
    sm += __shfl_xor(sm, 4, kWave);
    if ((kPieces % kT == 0 || c < kPieces) && cc == 0) xcor[gi * 16 + tok] = -8 * sm;
  }
  uint8_t* cs = reinterpret_cast<uint8_t*>(cs4);
#pragma unroll
  for (int i = 0; i < kUPT; i++) {
    const int U = static_cast<int>(threadIdx.x) + i * kT;
    const int r = U / UR, u = U % UR;
    *reinterpret_cast<uint4*>(cs + r * kCodeRow + 16 * u) = cu[i];
  }
#pragma unroll
  for (int i = 0; i < (kSc + kT - 1) / kT; i++) {
    const int c = static_cast<int>(threadIdx.x) + i * kT;
    if (kSc % kT == 0 || c < kSc) scs[c] = f16_bits_to_f32(scv[i]);
  }
  __syncthreads();

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int rl = (wave & 3) * 16 + l16, kw = wave >> 2;
#pragma unroll
  for (int gq = 0; gq < NG / KW; gq++) {
    const int gi = kw * (NG / KW) + gq;
    if (gi >= nb) break;
    const uint4 c = *reinterpret_cast<const uint4*>(cs + rl * kCodeRow + 64 * gi + 16 * g);
    const i32x4_t B0 = {static_cast<int>(c.x & kLo4), static_cast<int>(c.y & kLo4),
                        static_cast<int>((c.x >> 4) & kLo4), static_cast<int>((c.y >> 4) & kLo4)};
    const i32x4_t B1 = {static_cast<int>(c.z & kLo4), static_cast<int>(c.w & kLo4),
                        static_cast<int>((c.z >> 4) & kLo4), static_cast<int>((c.w >> 4) & kLo4)};
    const uint8_t* xr = xsb + (gi * 16 + l16) * kXRow + 32 * g;
    const i32x4_t A0 = *reinterpret_cast<const i32x4_t*>(xr);
    const i32x4_t A1 = *reinterpret_cast<const i32x4_t*>(xr + 16);
    const i32x4_t C0 = xcor4[gi * 4 + g];  // tokens 4g .. 4g+3
    i32x4_t D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, C0, 0, 0, 0);
    D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, D, 0, 0, 0);
    const float d = scs[rl * NG + gi];
    acc.x = __builtin_fmaf(d, static_cast<float>(D.x), acc.x);
    acc.y = __builtin_fmaf(d, static_cast<float>(D.y), acc.y);
    acc.z = __builtin_fmaf(d, static_cast<float>(D.z), acc.z);
    acc.w = __builtin_fmaf(d, static_cast<float>(D.w), acc.w);
  }

  if constexpr (KW > 1) {
    // the K shares of a row tile meet in LDS
    if (kw > 0) red[((kw - 1) * 4 + (wave & 3)) * 64 + lane] = acc;
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int q = 1; q < KW; q++) {
      const float4_t o = red[((q - 1) * 4 + wave) * 64 + lane];
      acc.x += o.x;
      acc.y += o.y;
      acc.z += o.z;
      acc.w += o.w;
    }
  }
  const int64_t m = m0 + rl;
  if (m < M) {
    const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int n = n0 + 4 * g + r;
      if (n < N) {
        float* dst = Y + static_cast<int64_t>(n) * M + m;
        if constexpr (SPLIT) atomicAdd(dst, v[r] * xs[n]);
        else *dst = v[r] * xs[n];
      }
    }
  }
}

// ===================================================================
// Many tokens: v_mfma_i32_32x32x32_i8, wide tiles.
//
// Operand layout: lane l holds row (l % 32) of A and column (l % 32) of B,
// each with 16 int8 k values of its half (l / 32); lane l receives
// D[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.  For step s (0..3) of a
// 128-weight group, half h takes code bytes j0..j0+7, j0 = 32h + 8s -- so a
// lane reads 32 contiguous code bytes per group -- i.e. weights j0..j0+7
// (low nibbles) and 64+j0..64+j0+7 (high nibbles), and the same activations.
// A = X (tokens), B = W^T, so all 16 outputs of a lane share one weight row
// and one scale per group; the integer accumulator starts at -8*sum(xq) of
// each output's token (16 values in output order: one 64-byte LDS read).
//
// A workgroup of 4 waves owns 128 weight rows (32 per wave) and 32*T32
// tokens.  X is staged SG groups at a time in LDS, double-buffered: per token
// and group 8 pieces of 16 bytes in operand order (piece 4h + s), token rows
// 128*SG + 16 bytes apart, so the 16 lanes of one read phase (16 consecutive
// tokens, one piece) hit 16 different 4-bank groups.  Within a stage the
// token tiles form a software pipeline.
// ===================================================================
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int T32, int SG, bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_gemm_w4a8_w(const uint8_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       const int8_t* __restrict__ xq,
                                                       const float* __restrict__ xs,
                                                       float* __restrict__ Y, int M, int K, int N,
                                                       int stages_per_split) {
  constexpr int NT = 32 * T32;
  constexpr int XROW = 128 * SG + 16;
  constexpr int XCH = NT * 8 * SG;
  constexpr int XPT = XCH / 256;
  static_assert(XCH % 256 == 0, "X chunks per thread");
  __shared__ uint4 xs4[2][NT * XROW / 16];
  __shared__ i32x4_t xcor4[2][SG][NT / 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int NG = K >> 7;
  const int NS = NG / SG;
  const int64_t rowbytes = K >> 1;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + l32;
  const int64_t rowc = row < M ? row : M - 1;
  const int n0 = blockIdx.y * NT;
  const int s_begin = SPLIT ? blockIdx.z * stages_per_split : 0;
  const int s_end = SPLIT ? min(NS, s_begin + stages_per_split) : NS;

  auto load_x = [&](int st, uint4 xv[XPT]) {
#pragma unroll
    for (int i = 0; i < XPT; i++) {
      const int c = threadIdx.x + i * 256;
      const int tok = c / (8 * SG), rem = c % (8 * SG);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n0 + tok < N)
        v = *reinterpret_cast<const uint4*>(xq + static_cast<int64_t>(n0 + tok) * K + 128 * SG * st + 16 * rem);
      xv[i] = v;
    }
  };
  auto store_x = [&](int buf, const uint4 xv[XPT]) {
    uint8_t* xsb = reinterpret_cast<uint8_t*>(xs4[buf]);
#pragma unroll
    for (int i = 0; i < XPT; i++) {
      const int c = threadIdx.x + i * 256;
      const int tok = c / (8 * SG), rem = c % (8 * SG);
      const int grp = rem >> 3, cc = rem & 7;
      // activations 16cc..16cc+15 (mod 64) of group grp: pieces p0 = 4h' + 2(cc&1)
      // and p0 + 1 with h' = (cc&3)/2; first halves for cc < 4, second halves after
      const int p0 = 4 * ((cc & 3) >> 1) + 2 * (cc & 1);
      uint8_t* r = xsb + tok * XROW + 128 * grp + 16 * p0 + 8 * (cc >> 2);
      *reinterpret_cast<uint2*>(r) = make_uint2(xv[i].x, xv[i].y);
      *reinterpret_cast<uint2*>(r + 16) = make_uint2(xv[i].z, xv[i].w);
      int s = dot4(xv[i].x, kOnes8, 0);
      s = dot4(xv[i].y, kOnes8, s);
      s = dot4(xv[i].z, kOnes8, s);
      s = dot4(xv[i].w, kOnes8, s);
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      s += __shfl_xor(s, 4, kWave);
      // stored in output order: the 16 starting values of lane (tile t, half h)
      // are slots 32t + 16h .. +15 (token 8(r/4) + 4h + r%4 of the tile at 16h + r)
      const int u = tok & 31;
      if (cc == 0) reinterpret_cast<int*>(xcor4[buf][grp])[(tok & ~31) + 16 * ((u >> 2) & 1) + 4 * (u >> 3) + (u & 3)] = -8 * s;
    }
  };
  auto load_w = [&](int st, uint4 raw[SG][2], uint32_t sc[SG]) {
#pragma unroll
    for (int grp = 0; grp < SG; grp++) {
      const int G = SG * st + grp;
      const uint4* p = reinterpret_cast<const uint4*>(codes + rowc * rowbytes + 64 * G + 32 * h);
      raw[grp][0] = p[0];
      raw[grp][1] = p[1];
      sc[grp] = scales[rowc * NG + G];
    }
  };

  f32x16_t acc[T32];
#pragma unroll
  for (int t = 0; t < T32; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;

  // codes and activations of the next stage are fetched during this one
  uint4 xv[XPT];
  uint4 raw[SG][2], n1[SG][2];
  uint32_t sc[SG], s1[SG];
  if (s_begin < s_end) {
    load_x(s_begin, xv);
    load_w(s_begin, raw, sc);
    store_x(0, xv);
  }
  for (int st = s_begin; st < s_end; st++) {
    const int buf = (st - s_begin) & 1;
    __syncthreads();
    const bool more = st + 1 < s_end;
    if (more) {
      load_x(st + 1, xv);
      load_w(st + 1, n1, s1);
    }
    const uint8_t* xsb = reinterpret_cast<const uint8_t*>(xs4[buf]);
#pragma unroll
    for (int grp = 0; grp < SG; grp++) {
      const float d = f16_bits_to_f32(sc[grp]);
      const uint32_t w[8] = {raw[grp][0].x, raw[grp][0].y, raw[grp][0].z, raw[grp][0].w,
                             raw[grp][1].x, raw[grp][1].y, raw[grp][1].z, raw[grp][1].w};
      i32x4_t B[4];
#pragma unroll
      for (int s = 0; s < 4; s++)
        B[s] = i32x4_t{static_cast<int>(w[2 * s] & kLo4), static_cast<int>(w[2 * s + 1] & kLo4),
                       static_cast<int>((w[2 * s] >> 4) & kLo4), static_cast<int>((w[2 * s + 1] >> 4) & kLo4)};
      // tiles in a software pipeline: tile t's matrix ops run while tile t+1's
      // operands are read and tile t-1's sums are scaled on the VALU
      const uint8_t* abase = xsb + l32 * XROW + 128 * grp + 64 * h;
      const int* cbase = reinterpret_cast<const int*>(xcor4[buf][grp]) + 16 * h;
      i32x4_t A[2][4];
      i32x16_t D[2];
#pragma unroll
      for (int s = 0; s < 4; s++) A[0][s] = *reinterpret_cast<const i32x4_t*>(abase + 16 * s);
      D[0] = *reinterpret_cast<const i32x16_t*>(cbase);
#pragma unroll
      for (int t = 0; t < T32; t++) {
        const int cur = t & 1, nxt = cur ^ 1;
        if (t + 1 < T32) {
#pragma unroll
          for (int s = 0; s < 4; s++)
            A[nxt][s] = *reinterpret_cast<const i32x4_t*>(abase + 32 * (t + 1) * XROW + 16 * s);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) D[cur] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[cur][s], B[s], D[cur], 0, 0, 0);
        if (t > 0) {
#pragma unroll
          for (int r = 0; r < 16; r++) acc[t - 1][r] = __builtin_fmaf(d, static_cast<float>(D[nxt][r]), acc[t - 1][r]);
        }
        if (t + 1 < T32) D[nxt] = *reinterpret_cast<const i32x16_t*>(cbase + 32 * (t + 1));
      }
#pragma unroll
      for (int r = 0; r < 16; r++)
        acc[T32 - 1][r] = __builtin_fmaf(d, static_cast<float>(D[(T32 - 1) & 1][r]), acc[T32 - 1][r]);
    }
    if (more) store_x(buf ^ 1, xv);
#pragma unroll
    for (int grp = 0; grp < SG; grp++) {
      raw[grp][0] = n1[grp][0];
      raw[grp][1] = n1[grp][1];
      sc[grp] = s1[grp];
    }
  }

  if (row >= M) return;
#pragma unroll
  for (int t = 0; t < T32; t++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int n = n0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
      if (n < N) {
        float* dst = Y + static_cast<int64_t>(n) * M + row;
        const float v = acc[t][r] * xs[n];
        if constexpr (SPLIT) atomicAdd(dst, v);
        else *dst = v;
      }
    }
  }
}

template <int RMAX, int UPL, int WAVES = kWavesV>
hipError_t launch_v_t(const uint8_t* codes, const uint16_t* scales, int64_t m, int64_t k, const int8_t* xq,
                      const float* xs, float* y, int rpw, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((m + rpw - 1) / rpw);
  if (log_enabled())
    log_launch("w4a8 k_gemv_w4a8 row-slots/wave=%d chunks/lane=%d waves=%d m=%lld k=%lld rows/wg=%d grid=%u", RMAX,
               UPL, WAVES, (long long)m, (long long)k, rpw, grid);
  hipLaunchKernelGGL((k_gemv_w4a8<RMAX, UPL, WAVES>), dim3(grid), dim3(WAVES * kWave), 0, s, codes, scales, xq, xs, y,
                     static_cast<int>(m), static_cast<int>(k), rpw);
  return hipGetLastError();
}

// chunks per lane (UPL) from k, then rows per wave (RMAX) from the rows per
// workgroup, capped so that a lane's loads fit its 128 registers (16 waves of
// a workgroup share a SIMD four at a time): RMAX * UPL <= 15, RMAX <= 3.
// Rows of 65 to 128 chunks with more than 32 rows per CU take 12-wave
// workgroups with up to 4 rows per wave instead, each lane's activations
// serving 4 rows (11008 x 4096: 6.05 against 6.18 us; with 16 rows per CU,
// 4096 x 11008, 12 waves lose: 6.75 against 6.36 us).
template <int UPL>
hipError_t launch_v_u(const uint8_t* codes, const uint16_t* scales, int64_t m, int64_t k, const int8_t* xq,
                      const float* xs, float* y, hipStream_t s) {
  constexpr int kRcap = UPL <= 5 ? 3 : (UPL == 6 ? 2 : 1);
  int64_t per = (m + cu_count() - 1) / cu_count();  // an even share of the rows over the CUs
  if (UPL == 2 && per > 32) {
    const int rpw = static_cast<int>(per > 48 ? 48 : per);
    if (rpw > 36) return launch_v_t<4, UPL, 12>(codes, scales, m, k, xq, xs, y, rpw, s);
    return launch_v_t<3, UPL, 12>(codes, scales, m, k, xq, xs, y, rpw, s);
  }
  per = per < kWavesV ? kWavesV : (per > kRcap * kWavesV ? kRcap * kWavesV : per);
  const int rpw = static_cast<int>(per);
  const int rmax = (rpw + kWavesV - 1) / kWavesV;
  if (rmax == 1 || kRcap == 1) return launch_v_t<1, UPL>(codes, scales, m, k, xq, xs, y, rpw, s);
  if (rmax == 2 || kRcap == 2) return launch_v_t<(kRcap >= 2 ? 2 : 1), UPL>(codes, scales, m, k, xq, xs, y, rpw, s);
  return launch_v_t<(kRcap >= 3 ? 3 : 1), UPL>(codes, scales, m, k, xq, xs, y, rpw, s);
}

hipError_t launch_v(const uint8_t* codes, const uint16_t* scales, int64_t m, int64_t k, const int8_t* xq,
                    const float* xs, float* y, hipStream_t s) {
  switch (static_cast<int>((k / 32 + 63) / 64)) {
    case 1: return launch_v_u<1>(codes, scales, m, k, xq, xs, y, s);
    case 2: return launch_v_u<2>(codes, scales, m, k, xq, xs, y, s);
    case 3: return launch_v_u<3>(codes, scales, m, k, xq, xs, y, s);
    case 4: return launch_v_u<4>(codes, scales, m, k, xq, xs, y, s);
    case 5: return launch_v_u<5>(codes, scales, m, k, xq, xs, y, s);
    case 6: return launch_v_u<6>(codes, scales, m, k, xq, xs, y, s);
    case 7: return launch_v_u<7>(codes, scales, m, k, xq, xs, y, s);
    default: return launch_v_u<8>(codes, scales, m, k, xq, xs, y, s);
  }
}

template <int NG, int KW>
hipError_t launch_mu(const uint8_t* codes, const uint16_t* scales, int64_t m, int64_t k, const int8_t* xq,
                     const float* xs, int64_t n, float* y, hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((m + 63) / 64);
  const unsigned gy = static_cast<unsigned>((n + 15) / 16);
  const unsigned gz = static_cast<unsigned>((k / 128 + NG - 1) / NG);
  if (log_enabled())
    log_launch("w4a8 k_gemm_w4a8_u tile=64x16 groups/piece=%d waves/tile=%d m=%lld k=%lld n=%lld grid=%ux%ux%u", NG,
               KW, (long long)m, (long long)k, (long long)n, gx, gy, gz);
  if (gz > 1) {
    const hipError_t e = launch_fill_zero(y, m * n, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_w4a8_u<NG, KW, true>), dim3(gx, gy, gz), dim3(kThreadsM * KW), 0, s, codes, scales, xq, xs, y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
  } else {
    hipLaunchKernelGGL((k_gemm_w4a8_u<NG, KW, false>), dim3(gx, gy, 1), dim3(kThreadsM * KW), 0, s, codes, scales, xq, xs, y,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
  }
  return hipGetLastError();
}

template <int T32, int SG>
hipError_t launch_w(const uint8_t* codes, const uint16_t* scales, int64_t m, int64_t k, const int8_t* xq,
                    const float* xs, int64_t n, float* y, int64_t want_tiles, hipStream_t s) {
  const unsigned gx = static_cast<unsigned>((m + 127) / 128);
  const unsigned gy = static_cast<unsigned>((n + 32 * T32 - 1) / (32 * T32));
  const int ns = static_cast<int>(k / 128 / SG);
  const int64_t tiles = static_cast<int64_t>(gx) * gy;
  if (tiles < want_tiles && ns > 1) {
    int split = static_cast<int>((want_tiles + tiles - 1) / tiles);
    split = split > ns ? ns : split;
    const int per = (ns + split - 1) / split;
    const unsigned gz = static_cast<unsigned>((ns + per - 1) / per);
    if (log_enabled())
      log_launch("w4a8 k_gemm_w4a8_w tile=128x%d groups/stage=%d m=%lld k=%lld n=%lld grid=%ux%ux%u stages/piece=%d",
                 32 * T32, SG, (long long)m, (long long)k, (long long)n, gx, gy, gz, per);
    const hipError_t e = launch_fill_zero(y, m * n, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_w4a8_w<T32, SG, true>), dim3(gx, gy, gz), dim3(kThreadsM), 0, s, codes, scales, xq,
                       xs, y, static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), per);
  } else {
    if (log_enabled())
      log_launch("w4a8 k_gemm_w4a8_w tile=128x%d groups/stage=%d m=%lld k=%lld n=%lld grid=%ux%ux1 stages/piece=%d",
                 32 * T32, SG, (long long)m, (long long)k, (long long)n, gx, gy, ns);
    hipLaunchKernelGGL((k_gemm_w4a8_w<T32, SG, false>), dim3(gx, gy, 1), dim3(kThreadsM), 0, s, codes, scales, xq,
                       xs, y, static_cast<int>(m), static_cast<int>(k), static_cast<int>(n), ns);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_w4a8(const void* blocks, int64_t m, int64_t k, const int8_t* xq, const float* xs,
                            int64_t n, float* y, hipStream_t s) {
  const uint8_t* codes = static_cast<const uint8_t*>(blocks);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(codes + m * k / 2);
  if (n == 1 && k <= 8 * 64 * 32) {
    // in pieces of at most kGemvRowsPerLaunch rows (codes and scales of a
    // piece start at its first row)
    for (int64_t r0 = 0; r0 < m; r0 += kGemvRowsPerLaunch) {
      const int64_t nr = m - r0 < kGemvRowsPerLaunch ? m - r0 : kGemvRowsPerLaunch;
      const hipError_t e = launch_v(codes + r0 * (k / 2), scales + r0 * (k / 128), nr, k, xq, xs, y + r0, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // tilings measured at 14336 x 4096 and 4096 x 14336: up to N = 32 the
  // unit-loaded kernel, 64 rows x 4 groups per workgroup of 8 waves (N = 2 /
  // 16: 12.0 / 14.8 us, against 16.4 / 17.9 us for operand-order loads with
  // K split three ways; 1, 2, 8 and 16 groups per workgroup and 4 or 16
  // waves were slower; N = 32: 20.5 us against 21.4-22.8 for the wide
  // kernel), then the wide kernel: 32 tokens (two groups per stage when the
  // group count is even) up to N = 64, 64 tokens up to
  // N = 256 (N = 200: 40 us against 61 for 128-token tiles, which leave CUs
  // idle at 14336 rows), 128 tokens beyond (N = 512: 69 us against 80; two
  // groups per stage spill at 128 tokens and lose at 64)
  // (reproducible products: no K split, the wide kernel from 2 tokens on)
  const bool det = deterministic();
  const int64_t cus = det ? 0 : cu_count();  // tiles wanted before K is split
  if (n <= 32 && !det) return launch_mu<4, 2>(codes, scales, m, k, xq, xs, n, y, s);
  if (n <= 64) {
    if ((k / 128) % 2 == 0) return launch_w<1, 2>(codes, scales, m, k, xq, xs, n, y, cus, s);
    return launch_w<1, 1>(codes, scales, m, k, xq, xs, n, y, cus, s);
  }
  if (n <= 256) return launch_w<2, 1>(codes, scales, m, k, xq, xs, n, y, cus, s);
  return launch_w<4, 1>(codes, scales, m, k, xq, xs, n, y, cus, s);
}

}  // namespace qblk
