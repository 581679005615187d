// qblk_abi.hip -- the C ABI of libqblk (declared in include/qblk.h): argument
// checks on the host, then one kernel launch on the caller's stream.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/qblk.h"
#include "qblk_launch.h"

namespace qblk {

// per device ordinal; 0 = not queried yet.  Concurrent first calls may both
// query and store the same value.
static std::atomic<int> g_cus[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>& slot = g_cus[dev < 64 ? dev : 63];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) slot.store(n, std::memory_order_relaxed);
  return n;
}

// qblk_set_deterministic: 0 off (the default), 1 on
static std::atomic<int> g_det{0};

bool deterministic() { return g_det.load(std::memory_order_relaxed) != 0; }

// -1 unknown, 0 off, 1 on
static std::atomic<int> g_log{-1};

bool log_enabled() {
  int v = g_log.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("QBLK_LOG");
    v = (e && e[0] == '1') ? 1 : 0;
    g_log.store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

void log_launch(const char* fmt, ...) {
  if (!log_enabled()) return;
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "qblk: %s\n", line);
}

}  // namespace qblk

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Rows of one qblk_gemm / qblk_gemm_w4a8 call: the product kernels run up to
// 8 threads per row in one launch, which holds at most 2^32 - 1 threads.
constexpr int64_t kMaxGemmRows = int64_t(1) << 28;
constexpr int64_t kMaxBytes = int64_t(1) << 40;

int elems_of(int fmt) {
  switch (fmt) {
    case QBLK_Q4_0: return 32;
    case QBLK_W4G128: return 128;
    case QBLK_SB4:
    case QBLK_SB4_AFFINE:
    case QBLK_Q4_K: return 256;
    default: return 0;
  }
}

size_t bytes_of(int fmt) {
  switch (fmt) {
    case QBLK_Q4_0: return 18;
    case QBLK_SB4: return 138;
    case QBLK_SB4_AFFINE: return 148;
    case QBLK_Q4_K: return 144;
    case QBLK_W4G128: return 66;  // 64 code bytes + a 2-byte scale, in two planes
    default: return 0;
  }
}

bool dtype_ok(int t) { return t == QBLK_F32 || t == QBLK_F16 || t == QBLK_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape of a packed rows x k matrix: sizes in range, k a multiple of the block.
qblk_status_t check_shape(int fmt, int64_t rows, int64_t k) {
  const int e = elems_of(fmt);
  if (e == 0) return QBLK_ERR_FORMAT;
  if (rows < 0 || k < 0 || rows > kMaxDim || k > kMaxDim || k % e != 0) return QBLK_ERR_SHAPE;
  if (rows > 0 && k > 0 && rows * (k / e) > kMaxBytes / static_cast<int64_t>(bytes_of(fmt)))
    return QBLK_ERR_SHAPE;
  return QBLK_OK;
}

qblk_status_t check_ptr(const void* p, bool needed) {
  if (!needed) return QBLK_OK;
  if (!p) return QBLK_ERR_NULL;
  if (!aligned16(p)) return QBLK_ERR_ALIGN;
  return QBLK_OK;
}

// fp32 scale arrays (one per token) are read element by element: 4-byte
// alignment, so that a slice of them starting at any token is accepted
qblk_status_t check_ptr4(const void* p, bool needed) {
  if (!needed) return QBLK_OK;
  if (!p) return QBLK_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return QBLK_ERR_ALIGN;
  return QBLK_OK;
}

qblk_status_t from_hip(hipError_t e) { return e == hipSuccess ? QBLK_OK : QBLK_ERR_LAUNCH; }

#define QBLK_TRY(expr)                 \
  do {                                 \
    const qblk_status_t st_ = (expr);  \
    if (st_ != QBLK_OK) return st_;    \
  } while (0)

}  // namespace

extern "C" {

size_t qblk_block_bytes(qblk_format_t fmt) { return bytes_of(fmt); }

int qblk_block_elems(qblk_format_t fmt) { return elems_of(fmt); }

size_t qblk_packed_bytes(qblk_format_t fmt, int64_t rows, int64_t k) {
  if (check_shape(fmt, rows, k) != QBLK_OK) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(k / elems_of(fmt)) * bytes_of(fmt);
}

qblk_status_t qblk_quantize_q4_0(const void* w, qblk_dtype_t wt, int64_t rows, int64_t k,
                                 void* blocks, qblk_stream_t stream) {
  QBLK_TRY(check_shape(QBLK_Q4_0, rows, k));
  if (!dtype_ok(wt)) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(w, work));
  QBLK_TRY(check_ptr(blocks, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_quantize_q4_0(w, wt, rows, k, blocks,
                                             static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_quantize_q4_0_ref(const void* w, qblk_dtype_t wt, int64_t rows, int64_t k,
                                     void* blocks, qblk_stream_t stream) {
  QBLK_TRY(check_shape(QBLK_Q4_0, rows, k));
  if (wt != QBLK_F32) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(w, work));
  QBLK_TRY(check_ptr(blocks, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_quantize_q4_0_ref(static_cast<const float*>(w), rows, k, blocks,
                                                 static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_quantize_sb4(const void* w, qblk_dtype_t wt, int64_t rows, int64_t k,
                                int affine, void* blocks, qblk_stream_t stream) {
  const int fmt = affine ? QBLK_SB4_AFFINE : QBLK_SB4;
  QBLK_TRY(check_shape(fmt, rows, k));
  if (!dtype_ok(wt)) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(w, work));
  QBLK_TRY(check_ptr(blocks, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_quantize_sb4(w, wt, rows, k, affine ? 1 : 0, blocks,
                                            static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_quantize_q4_k(const void* w, qblk_dtype_t wt, int64_t rows, int64_t k,
                                 void* blocks, qblk_stream_t stream) {
  QBLK_TRY(check_shape(QBLK_Q4_K, rows, k));
  if (!dtype_ok(wt)) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(w, work));
  QBLK_TRY(check_ptr(blocks, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_quantize_q4_k(w, wt, rows, k, blocks,
                                             static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_quantize_w4g128(const void* w, qblk_dtype_t wt, int64_t rows, int64_t k,
                                   void* blocks, qblk_stream_t stream) {
  QBLK_TRY(check_shape(QBLK_W4G128, rows, k));
  if (!dtype_ok(wt)) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(w, work));
  QBLK_TRY(check_ptr(blocks, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_quantize_w4g128(w, wt, rows, k, blocks,
                                               static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_quantize_act_i8(const void* x, qblk_dtype_t xt, int64_t n, int64_t k,
                                   int8_t* xq, float* scale, qblk_stream_t stream) {
  if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % 8 != 0) return QBLK_ERR_SHAPE;
  if (!dtype_ok(xt)) return QBLK_ERR_DTYPE;
  QBLK_TRY(check_ptr(x, n > 0 && k > 0));
  QBLK_TRY(check_ptr(xq, n > 0 && k > 0));
  QBLK_TRY(check_ptr4(scale, n > 0));
  if (n == 0) return QBLK_OK;
  return from_hip(qblk::launch_quantize_act_i8(x, xt, n, k, xq, scale,
                                               static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_gemm_w4a8(const void* blocks, int64_t m, int64_t k, const int8_t* xq,
                             const float* scale, int64_t n, float* y, qblk_stream_t stream) {
  QBLK_TRY(check_shape(QBLK_W4G128, m, k));
  if (m > kMaxGemmRows) return QBLK_ERR_SHAPE;
  if (n < 0 || n > kMaxDim) return QBLK_ERR_SHAPE;
  const bool out = m > 0 && n > 0;
  QBLK_TRY(check_ptr(blocks, out && k > 0));
  QBLK_TRY(check_ptr(xq, out && k > 0));
  QBLK_TRY(check_ptr4(scale, out && k > 0));
  QBLK_TRY(check_ptr(y, out));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!out) return QBLK_OK;
  if (k == 0) return from_hip(qblk::launch_fill_zero(y, m * n, s));
  return from_hip(qblk::launch_gemm_w4a8(blocks, m, k, xq, scale, n, y, s));
}

qblk_status_t qblk_dequant(qblk_format_t fmt, const void* blocks, int64_t rows, int64_t k,
                           void* out, qblk_dtype_t ot, qblk_stream_t stream) {
  QBLK_TRY(check_shape(fmt, rows, k));
  if (!dtype_ok(ot)) return QBLK_ERR_DTYPE;
  const bool work = rows > 0 && k > 0;
  QBLK_TRY(check_ptr(blocks, work));
  QBLK_TRY(check_ptr(out, work));
  if (!work) return QBLK_OK;
  return from_hip(qblk::launch_dequant(fmt, blocks, rows, k, out, ot,
                                       static_cast<hipStream_t>(stream)));
}

qblk_status_t qblk_gemv(qblk_format_t fmt, const void* blocks, int64_t m, int64_t k,
                        const void* x, qblk_dtype_t xt, float* y, qblk_stream_t stream) {
  QBLK_TRY(check_shape(fmt, m, k));
  if (!dtype_ok(xt)) return QBLK_ERR_DTYPE;
  if (fmt == QBLK_W4G128) return QBLK_ERR_UNSUPPORTED;  // its product is qblk_gemm_w4a8
  QBLK_TRY(check_ptr(blocks, m > 0 && k > 0));
  QBLK_TRY(check_ptr(x, m > 0 && k > 0));
  QBLK_TRY(check_ptr(y, m > 0));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (m == 0) return QBLK_OK;
  if (k == 0) return from_hip(qblk::launch_fill_zero(y, m, s));
  return from_hip(qblk::launch_gemv(fmt, blocks, m, k, x, xt, y, s));
}

qblk_status_t qblk_gemv_batch(qblk_format_t fmt, int64_t k, qblk_dtype_t xt,
                              const qblk_gemv_item_t* items, int count, qblk_stream_t stream) {
  // the checks of qblk_gemv, in its order, then every item's
  QBLK_TRY(check_shape(fmt, 0, k));
  if (!dtype_ok(xt)) return QBLK_ERR_DTYPE;
  if (fmt == QBLK_W4G128) return QBLK_ERR_UNSUPPORTED;  // its product is qblk_gemm_w4a8
  if (count < 0 || count > QBLK_GEMV_BATCH_MAX) return QBLK_ERR_SHAPE;
  if (count > 0 && items == nullptr) return QBLK_ERR_NULL;
  for (int i = 0; i < count; i++) {
    const qblk_gemv_item_t& it = items[i];
    QBLK_TRY(check_shape(fmt, it.m, k));
    QBLK_TRY(check_ptr(it.blocks, it.m > 0 && k > 0));
    QBLK_TRY(check_ptr(it.x, it.m > 0 && k > 0));
    QBLK_TRY(check_ptr(it.y, it.m > 0));
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (k == 0) {
    for (int i = 0; i < count; i++)
      if (items[i].m > 0) QBLK_TRY(from_hip(qblk::launch_fill_zero(items[i].y, items[i].m, s)));
    return QBLK_OK;
  }
  // the items that have rows, in order
  qblk_gemv_item_t live[QBLK_GEMV_BATCH_MAX];
  int n = 0;
  for (int i = 0; i < count; i++)
    if (items[i].m > 0) live[n++] = items[i];
  if (n == 0) return QBLK_OK;
  return from_hip(qblk::launch_gemv_batch(fmt, k, xt, live, n, s));
}

qblk_status_t qblk_gemm(qblk_format_t fmt, const void* blocks, int64_t m, int64_t k,
                        const void* x, qblk_dtype_t xt, int64_t n, float* y,
                        qblk_stream_t stream) {
  QBLK_TRY(check_shape(fmt, m, k));
  if (m > kMaxGemmRows) return QBLK_ERR_SHAPE;
  if (!dtype_ok(xt)) return QBLK_ERR_DTYPE;
  if (n < 0 || n > kMaxDim) return QBLK_ERR_SHAPE;
  // the matrix-core kernels take bf16 activations and whole 256-weight groups
  if (xt != QBLK_BF16 || k % 256 != 0 || fmt == QBLK_W4G128) return QBLK_ERR_UNSUPPORTED;
  const bool out = m > 0 && n > 0;
  QBLK_TRY(check_ptr(blocks, out && k > 0));
  QBLK_TRY(check_ptr(x, out && k > 0));
  QBLK_TRY(check_ptr(y, out));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!out) return QBLK_OK;
  if (k == 0) return from_hip(qblk::launch_fill_zero(y, m * n, s));
  return from_hip(qblk::launch_gemm(fmt, blocks, m, k, x, xt, n, y, s));
}

const char* qblk_status_string(qblk_status_t st) {
  switch (st) {
    case QBLK_OK: return "ok";
    case QBLK_ERR_NULL: return "a required pointer is NULL";
    case QBLK_ERR_SHAPE: return "invalid size (negative, too large, or k not a multiple of the block size)";
    case QBLK_ERR_DTYPE: return "element type not accepted by this call";
    case QBLK_ERR_ALIGN: return "a data pointer is not 16-byte aligned";
    case QBLK_ERR_UNSUPPORTED: return "format/type combination not implemented";
    case QBLK_ERR_LAUNCH: return "kernel launch failed";
    case QBLK_ERR_FORMAT: return "unknown block format";
  }
  return "unknown status";
}

qblk_status_t qblk_set_deterministic(int on) {
  qblk::g_det.store(on != 0 ? 1 : 0, std::memory_order_relaxed);
  return QBLK_OK;
}

int qblk_deterministic(void) { return qblk::deterministic() ? 1 : 0; }

const char* qblk_version(void) { return "0.1.0"; }

}  // extern "C"
