// The C ABI's argument checks, built for the host alone under AddressSanitizer
// and UndefinedBehaviorSanitizer.  The ABI source is compiled here as plain
// C++ (it holds no device code); every kernel launcher, and the two HIP
// runtime queries it makes, are replaced below by stand-ins that record the
// call, so each entry point runs its checks on the CPU and the test sees
// exactly which launcher (if any) it reached, with which arguments.
#include "../bit_block_quant_amd/csrc/qblk_abi.hip"

#include <stdio.h>
#include <string.h>

#include <string>
#include <utility>
#include <vector>

namespace {

struct Call {
  std::string name;
  int64_t a = -1, b = -1, c = -1;  // sizes as passed (rows/m, k, n)
  int fmt = -1, type = -1;
  const void* p0 = nullptr;
  int count = 0;
};
Call g_call;
hipError_t g_ret = hipSuccess;

void rec(const char* name, const void* p0, int64_t a, int64_t b, int64_t c, int fmt, int type) {
  g_call.name = name;
  g_call.p0 = p0;
  g_call.a = a;
  g_call.b = b;
  g_call.c = c;
  g_call.fmt = fmt;
  g_call.type = type;
  g_call.count++;
}

}  // namespace

// ---------------------------------------------------------------- stand-ins
extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipErrorNoDevice;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 0;
  return hipErrorNoDevice;
}

namespace qblk {
hipError_t launch_quantize_q4_0(const void* w, int wt, int64_t rows, int64_t k, void*, hipStream_t) {
  rec("quantize_q4_0", w, rows, k, -1, QBLK_Q4_0, wt);
  return g_ret;
}
hipError_t launch_quantize_q4_0_ref(const float* w, int64_t rows, int64_t k, void*, hipStream_t) {
  rec("quantize_q4_0_ref", w, rows, k, -1, QBLK_Q4_0, QBLK_F32);
  return g_ret;
}
hipError_t launch_quantize_sb4(const void* w, int wt, int64_t rows, int64_t k, int affine, void*, hipStream_t) {
  rec("quantize_sb4", w, rows, k, -1, affine ? QBLK_SB4_AFFINE : QBLK_SB4, wt);
  return g_ret;
}
hipError_t launch_quantize_q4_k(const void* w, int wt, int64_t rows, int64_t k, void*, hipStream_t) {
  rec("quantize_q4_k", w, rows, k, -1, QBLK_Q4_K, wt);
  return g_ret;
}
hipError_t launch_quantize_w4g128(const void* w, int wt, int64_t rows, int64_t k, void*, hipStream_t) {
  rec("quantize_w4g128", w, rows, k, -1, QBLK_W4G128, wt);
  return g_ret;
}
hipError_t launch_quantize_act_i8(const void* x, int xt, int64_t n, int64_t k, int8_t*, float*, hipStream_t) {
  rec("quantize_act_i8", x, n, k, -1, -1, xt);
  return g_ret;
}
hipError_t launch_gemm_w4a8(const void* blocks, int64_t m, int64_t k, const int8_t*, const float*, int64_t n,
                            float*, hipStream_t) {
  rec("gemm_w4a8", blocks, m, k, n, QBLK_W4G128, -1);
  return g_ret;
}
hipError_t launch_gemv_batch(int fmt, int64_t k, int xt, const qblk_gemv_item_t* items, int count, hipStream_t) {
  int64_t rows = 0;
  for (int i = 0; i < count; i++) rows += items[i].m;  // reads every item it is given
  rec("gemv_batch", items[0].blocks, rows, k, count, fmt, xt);
  return g_ret;
}
hipError_t launch_dequant(int fmt, const void* blocks, int64_t rows, int64_t k, void*, int ot, hipStream_t) {
  rec("dequant", blocks, rows, k, -1, fmt, ot);
  return g_ret;
}
hipError_t launch_gemv(int fmt, const void* blocks, int64_t m, int64_t k, const void*, int xt, float*,
                       hipStream_t) {
  rec("gemv", blocks, m, k, 1, fmt, xt);
  return g_ret;
}
hipError_t launch_gemm(int fmt, const void* blocks, int64_t m, int64_t k, const void*, int xt, int64_t n, float*,
                       hipStream_t) {
  rec("gemm", blocks, m, k, n, fmt, xt);
  return g_ret;
}
hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t) {
  rec("fill_zero", y, n, -1, -1, -1, -1);
  return g_ret;
}
}  // namespace qblk

// -------------------------------------------------------------------- checks
static int g_fail = 0;

#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      g_fail++;                                                           \
    }                                                                     \
  } while (0)

// status st and no launcher reached
#define REJECTS(expr, st)                       \
  do {                                          \
    const int before_ = g_call.count;           \
    EXPECT((expr) == (st));                     \
    EXPECT(g_call.count == before_);            \
  } while (0)

// status QBLK_OK and exactly one launcher reached, the one named
#define LAUNCHES(expr, nm)                      \
  do {                                          \
    const int before_ = g_call.count;           \
    EXPECT((expr) == QBLK_OK);                  \
    EXPECT(g_call.count == before_ + 1);        \
    EXPECT(g_call.name == (nm));                \
  } while (0)

int main() {
  alignas(64) static unsigned char buf[4096];
  void* const A = buf;             // 16-byte aligned
  void* const B = buf + 1024;      // 16-byte aligned
  float* const Y = reinterpret_cast<float*>(buf + 2048);
  void* const MIS = buf + 8;       // 8-byte aligned only
  const int64_t kMax = (int64_t(1) << 31) - 1;
  const int64_t kHuge = int64_t(1) << 40;
  void* const s = nullptr;

  // geometry
  EXPECT(qblk_block_bytes(QBLK_Q4_0) == 18 && qblk_block_elems(QBLK_Q4_0) == 32);
  EXPECT(qblk_block_bytes(QBLK_SB4) == 138 && qblk_block_bytes(QBLK_SB4_AFFINE) == 148);
  EXPECT(qblk_block_bytes(QBLK_Q4_K) == 144 && qblk_block_bytes(QBLK_W4G128) == 66);
  EXPECT(qblk_block_bytes(static_cast<qblk_format_t>(9)) == 0);
  EXPECT(qblk_block_elems(static_cast<qblk_format_t>(-1)) == 0);
  EXPECT(qblk_packed_bytes(QBLK_SB4, 11008, 4096) == size_t(11008) * 16 * 138);
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, 0, 4096) == 0 && qblk_packed_bytes(QBLK_Q4_0, 3, 0) == 0);
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, 4, 33) == 0);    // k not a multiple of the block
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, -1, 32) == 0);
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, 4, -32) == 0);
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, kMax + 1, 32) == 0);  // a dimension past 2^31 - 1
  // both dimensions at the limit: the byte count (about 2^57) must be refused
  // without the product overflowing on the way
  EXPECT(qblk_packed_bytes(QBLK_Q4_0, kMax, (kMax / 32) * 32) == 0);
  EXPECT(qblk_packed_bytes(QBLK_SB4, INT64_MAX, 256) == 0);
  // each dimension in range, the packed size past 2^40 bytes
  EXPECT(qblk_packed_bytes(QBLK_SB4, int64_t(1) << 30, int64_t(1) << 14) == 0);
  EXPECT(qblk_packed_bytes(QBLK_SB4, int64_t(1) << 20, int64_t(1) << 14) < size_t(kHuge));
  EXPECT(qblk_packed_bytes(QBLK_SB4, INT64_MIN, 256) == 0);

  // quantizers: null, misaligned, bad type, bad shape, empty, and one valid call
  REJECTS(qblk_quantize_q4_0(nullptr, QBLK_F32, 2, 64, B, s), QBLK_ERR_NULL);
  REJECTS(qblk_quantize_q4_0(A, QBLK_F32, 2, 64, nullptr, s), QBLK_ERR_NULL);
  REJECTS(qblk_quantize_q4_0(MIS, QBLK_F32, 2, 64, B, s), QBLK_ERR_ALIGN);
  REJECTS(qblk_quantize_q4_0(A, static_cast<qblk_dtype_t>(3), 2, 64, B, s), QBLK_ERR_DTYPE);
  REJECTS(qblk_quantize_q4_0(A, QBLK_F32, 2, 48, B, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_quantize_q4_0(A, QBLK_F32, -2, 64, B, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_quantize_q4_0(nullptr, QBLK_F32, 0, 64, nullptr, s), QBLK_OK);  // empty: nothing to do
  LAUNCHES(qblk_quantize_q4_0(A, QBLK_BF16, 2, 64, B, s), "quantize_q4_0");
  EXPECT(g_call.a == 2 && g_call.b == 64 && g_call.type == QBLK_BF16 && g_call.p0 == A);

  REJECTS(qblk_quantize_q4_0_ref(A, QBLK_F16, 2, 64, B, s), QBLK_ERR_DTYPE);  // fp32 only
  LAUNCHES(qblk_quantize_q4_0_ref(A, QBLK_F32, 1, 32, B, s), "quantize_q4_0_ref");

  REJECTS(qblk_quantize_sb4(A, QBLK_F32, 1, 128, 0, B, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_quantize_sb4(A, QBLK_F32, 1, 256, 1, MIS, s), QBLK_ERR_ALIGN);
  REJECTS(qblk_quantize_sb4(A, QBLK_F32, kMax + 1, 256, 0, B, s), QBLK_ERR_SHAPE);
  LAUNCHES(qblk_quantize_sb4(A, QBLK_F16, 3, 512, 7, B, s), "quantize_sb4");  // any nonzero: affine
  EXPECT(g_call.fmt == QBLK_SB4_AFFINE && g_call.a == 3 && g_call.b == 512);
  LAUNCHES(qblk_quantize_sb4(A, QBLK_F32, 3, 512, 0, B, s), "quantize_sb4");
  EXPECT(g_call.fmt == QBLK_SB4);

  REJECTS(qblk_quantize_q4_k(A, QBLK_F32, 1, 255, B, s), QBLK_ERR_SHAPE);
  LAUNCHES(qblk_quantize_q4_k(A, QBLK_F32, 1, 256, B, s), "quantize_q4_k");
  REJECTS(qblk_quantize_w4g128(A, QBLK_F32, 1, 64, B, s), QBLK_ERR_SHAPE);
  LAUNCHES(qblk_quantize_w4g128(A, QBLK_F16, 1, 128, B, s), "quantize_w4g128");

  // activation quantizer: k a multiple of 8; scales 4-byte aligned suffices
  REJECTS(qblk_quantize_act_i8(A, QBLK_F16, 2, 12, static_cast<int8_t*>(B), Y, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_quantize_act_i8(A, QBLK_F16, 2, 16, static_cast<int8_t*>(B), nullptr, s), QBLK_ERR_NULL);
  REJECTS(qblk_quantize_act_i8(A, QBLK_F16, 2, 16, static_cast<int8_t*>(B),
                               reinterpret_cast<float*>(buf + 2050), s), QBLK_ERR_ALIGN);
  LAUNCHES(qblk_quantize_act_i8(A, QBLK_F16, 2, 16, static_cast<int8_t*>(B), reinterpret_cast<float*>(buf + 2052), s),
           "quantize_act_i8");
  REJECTS(qblk_quantize_act_i8(nullptr, QBLK_F16, 0, 16, nullptr, nullptr, s), QBLK_OK);

  // dequant
  REJECTS(qblk_dequant(static_cast<qblk_format_t>(5), A, 1, 32, B, QBLK_F32, s), QBLK_ERR_FORMAT);
  REJECTS(qblk_dequant(QBLK_SB4, A, 1, 256, B, static_cast<qblk_dtype_t>(-1), s), QBLK_ERR_DTYPE);
  LAUNCHES(qblk_dequant(QBLK_W4G128, A, 2, 256, B, QBLK_BF16, s), "dequant");
  EXPECT(g_call.fmt == QBLK_W4G128 && g_call.type == QBLK_BF16);

  // GEMV: k = 0 zero-fills y (m floats), m = 0 does nothing, W4G128 has no GEMV
  REJECTS(qblk_gemv(QBLK_W4G128, A, 1, 128, B, QBLK_F16, Y, s), QBLK_ERR_UNSUPPORTED);
  REJECTS(qblk_gemv(QBLK_SB4, A, 4, 256, B, QBLK_F16, nullptr, s), QBLK_ERR_NULL);
  REJECTS(qblk_gemv(QBLK_SB4, A, 4, 256, MIS, QBLK_F16, Y, s), QBLK_ERR_ALIGN);
  REJECTS(qblk_gemv(QBLK_SB4, nullptr, 0, 256, nullptr, QBLK_F16, nullptr, s), QBLK_OK);
  LAUNCHES(qblk_gemv(QBLK_SB4, nullptr, 5, 0, nullptr, QBLK_F16, Y, s), "fill_zero");
  EXPECT(g_call.a == 5 && g_call.p0 == Y);
  LAUNCHES(qblk_gemv(QBLK_Q4_K, A, 7, 512, B, QBLK_F32, Y, s), "gemv");
  EXPECT(g_call.fmt == QBLK_Q4_K && g_call.a == 7 && g_call.b == 512 && g_call.type == QBLK_F32);

  // GEMV batches: at most QBLK_GEMV_BATCH_MAX items, each checked before any
  // launch, items with m = 0 dropped
  {
    qblk_gemv_item_t it[QBLK_GEMV_BATCH_MAX + 1];
    for (auto& e : it) e = qblk_gemv_item_t{A, 4, B, Y};
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, -1, s), QBLK_ERR_SHAPE);
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, QBLK_GEMV_BATCH_MAX + 1, s), QBLK_ERR_SHAPE);
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, nullptr, 2, s), QBLK_ERR_NULL);
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, nullptr, 0, s), QBLK_OK);
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, static_cast<qblk_dtype_t>(9), it, 2, s), QBLK_ERR_DTYPE);
    REJECTS(qblk_gemv_batch(QBLK_W4G128, 256, QBLK_F16, it, 2, s), QBLK_ERR_UNSUPPORTED);
    REJECTS(qblk_gemv_batch(QBLK_SB4, 100, QBLK_F16, it, 2, s), QBLK_ERR_SHAPE);
    REJECTS(qblk_gemv_batch(static_cast<qblk_format_t>(9), 256, QBLK_F16, nullptr, 0, s), QBLK_ERR_FORMAT);
    REJECTS(qblk_gemv_batch(QBLK_SB4, -256, QBLK_F16, nullptr, 0, s), QBLK_ERR_SHAPE);
    it[2].x = MIS;  // a bad item anywhere stops the whole call
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, 3, s), QBLK_ERR_ALIGN);
    it[2].x = B;
    it[2].y = nullptr;
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, 3, s), QBLK_ERR_NULL);
    it[2].y = Y;
    it[1].m = -3;
    REJECTS(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, 3, s), QBLK_ERR_SHAPE);
    it[1] = qblk_gemv_item_t{nullptr, 0, nullptr, nullptr};
    LAUNCHES(qblk_gemv_batch(QBLK_SB4, 256, QBLK_F16, it, 3, s), "gemv_batch");
    EXPECT(g_call.a == 8 && g_call.b == 256 && g_call.c == 2 && g_call.p0 == A && g_call.type == QBLK_F16);
    LAUNCHES(qblk_gemv_batch(QBLK_SB4, 0, QBLK_F16, it, 2, s), "fill_zero");  // the m = 0 item has nothing to fill
    EXPECT(g_call.a == 4 && g_call.p0 == Y);
    LAUNCHES(qblk_gemv_batch(QBLK_Q4_K, 512, QBLK_F32, it + 2, QBLK_GEMV_BATCH_MAX - 1, s), "gemv_batch");
    EXPECT(g_call.c == QBLK_GEMV_BATCH_MAX - 1 && g_call.a == 4 * (QBLK_GEMV_BATCH_MAX - 1));
  }

  // GEMM: bf16 activations and k a multiple of 256 only; k = 0 zero-fills m * n
  REJECTS(qblk_gemm(QBLK_SB4, A, 4, 256, B, QBLK_F16, 2, Y, s), QBLK_ERR_UNSUPPORTED);
  REJECTS(qblk_gemm(QBLK_Q4_0, A, 4, 32, B, QBLK_BF16, 2, Y, s), QBLK_ERR_UNSUPPORTED);
  REJECTS(qblk_gemm(QBLK_W4G128, A, 4, 256, B, QBLK_BF16, 2, Y, s), QBLK_ERR_UNSUPPORTED);
  REJECTS(qblk_gemm(QBLK_SB4, A, 4, 256, B, QBLK_BF16, -1, Y, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_gemm(QBLK_SB4, A, 4, 256, B, QBLK_BF16, kMax + 1, Y, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_gemm(QBLK_SB4, A, 4, 256, B, QBLK_BF16, 0, nullptr, s), QBLK_OK);
  LAUNCHES(qblk_gemm(QBLK_SB4, nullptr, 3, 0, nullptr, QBLK_BF16, 5, Y, s), "fill_zero");
  EXPECT(g_call.a == 15);
  LAUNCHES(qblk_gemm(QBLK_SB4_AFFINE, A, 64, 4096, B, QBLK_BF16, 16, Y, s), "gemm");
  EXPECT(g_call.fmt == QBLK_SB4_AFFINE && g_call.a == 64 && g_call.b == 4096 && g_call.c == 16);

  // W4A8
  REJECTS(qblk_gemm_w4a8(A, 4, 100, static_cast<const int8_t*>(B), Y, 2, Y, s), QBLK_ERR_SHAPE);
  REJECTS(qblk_gemm_w4a8(A, 4, 128, static_cast<const int8_t*>(B), nullptr, 2, Y, s), QBLK_ERR_NULL);
  REJECTS(qblk_gemm_w4a8(A, 4, 128, static_cast<const int8_t*>(MIS), Y, 2, Y, s), QBLK_ERR_ALIGN);
  LAUNCHES(qblk_gemm_w4a8(nullptr, 4, 0, nullptr, nullptr, 2, Y, s), "fill_zero");
  EXPECT(g_call.a == 8);
  LAUNCHES(qblk_gemm_w4a8(A, 4, 128, static_cast<const int8_t*>(B), Y, 2, Y, s), "gemm_w4a8");
  EXPECT(g_call.c == 2);

  // at most 2^28 rows per product call
  const int64_t kGemmRows = int64_t(1) << 28;
  REJECTS(qblk_gemm(QBLK_SB4, A, kGemmRows + 1, 256, B, QBLK_BF16, 2, Y, s), QBLK_ERR_SHAPE);
  LAUNCHES(qblk_gemm(QBLK_SB4, A, kGemmRows, 256, B, QBLK_BF16, 2, Y, s), "gemm");
  REJECTS(qblk_gemm_w4a8(A, kGemmRows + 1, 128, static_cast<const int8_t*>(B), Y, 2, Y, s), QBLK_ERR_SHAPE);
  LAUNCHES(qblk_gemm_w4a8(A, kGemmRows, 128, static_cast<const int8_t*>(B), Y, 2, Y, s), "gemm_w4a8");

  // launches in pieces of whole workgroups: every unit once, in order
  {
    std::vector<std::pair<int64_t, int64_t>> got;
    auto rec = [&](int64_t u0, int64_t n) {
      got.emplace_back(u0, n);
      return hipSuccess;
    };
    auto covers = [&](int64_t units, int64_t per) {
      int64_t next = 0;
      bool ok = true;
      for (const auto& p : got) {
        ok = ok && p.first == next && p.second > 0 && p.second <= per && (p.first % per) == 0;
        next += p.second;
      }
      return ok && next == units;
    };
    // a limit of 10 workgroups of 256 threads, 8 units each: 80 units a launch
    EXPECT(qblk::in_pieces(1000, 8, 256, rec, 256 * 10) == hipSuccess);
    EXPECT(got.size() == 13 && covers(1000, 80));
    // the dispatch limit itself: (2^32 - 1) / 256 = 16777215 workgroups
    const int64_t wg_max = 16777215;
    got.clear();
    EXPECT(qblk::in_pieces(wg_max * 64, 64, 256, rec) == hipSuccess && got.size() == 1 && covers(wg_max * 64, wg_max * 64));
    got.clear();
    EXPECT(qblk::in_pieces(wg_max * 64 + 1, 64, 256, rec) == hipSuccess && got.size() == 2 &&
           covers(wg_max * 64 + 1, wg_max * 64) && got[1].second == 1);
    got.clear();
    EXPECT(qblk::in_pieces(wg_max + 5, 1, 256, rec) == hipSuccess && got.size() == 2 && covers(wg_max + 5, wg_max));
    // nothing to do: no launch; an error stops the sequence and is returned
    got.clear();
    EXPECT(qblk::in_pieces(0, 8, 256, rec) == hipSuccess && got.empty());
    int calls = 0;
    EXPECT(qblk::in_pieces(1000, 8, 256, [&](int64_t, int64_t) { return ++calls == 2 ? hipErrorInvalidValue : hipSuccess; },
                           256 * 10) == hipErrorInvalidValue &&
           calls == 2);
  }

  // a launcher's error becomes QBLK_ERR_LAUNCH
  g_ret = hipErrorInvalidValue;
  EXPECT(qblk_gemv(QBLK_SB4, A, 4, 256, B, QBLK_F16, Y, s) == QBLK_ERR_LAUNCH);
  EXPECT(qblk_quantize_q4_0(A, QBLK_F32, 1, 32, B, s) == QBLK_ERR_LAUNCH);
  g_ret = hipSuccess;

  // status strings: every code has its own text; unknown codes one of their own
  for (int st = 0; st <= 7; ++st) EXPECT(strlen(qblk_status_string(static_cast<qblk_status_t>(st))) > 0);
  EXPECT(strcmp(qblk_status_string(static_cast<qblk_status_t>(99)), "unknown status") == 0);
  EXPECT(strlen(qblk_version()) > 0);
  // the reproducible-products switch: off at load, set and cleared
  EXPECT(qblk_deterministic() == 0);
  EXPECT(qblk_set_deterministic(7) == QBLK_OK && qblk_deterministic() == 1);
  EXPECT(qblk_set_deterministic(0) == QBLK_OK && qblk_deterministic() == 0);

  // device queries that fail fall back to 256 compute units
  EXPECT(qblk::cu_count() == 256);
  // launch log: off unless QBLK_LOG=1 (the driver of this test sets it), and
  // a line longer than its buffer is cut, not overrun
  EXPECT(qblk::log_enabled());
  std::string longname(2000, 'x');
  qblk::log_launch("gemv %s m=%lld", longname.c_str(), 11008LL);

  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("clean\n");
  return 0;
}
