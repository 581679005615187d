// qblk_launch.h -- host-side launchers of the gfx950 kernels (internal).
// Arguments are validated by the C ABI layer (qblk_abi.hip) before any of
// these is called; the launchers assume shapes, types and alignment are valid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qblk.h"

namespace qblk {

hipError_t launch_quantize_q4_0(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                hipStream_t s);
hipError_t launch_quantize_q4_0_ref(const float* w, int64_t rows, int64_t k, void* blocks,
                                    hipStream_t s);
hipError_t launch_quantize_sb4(const void* w, int wt, int64_t rows, int64_t k, int affine,
                               void* blocks, hipStream_t s);
hipError_t launch_quantize_q4_k(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                hipStream_t s);
hipError_t launch_quantize_w4g128(const void* w, int wt, int64_t rows, int64_t k, void* blocks,
                                  hipStream_t s);
hipError_t launch_quantize_act_i8(const void* x, int xt, int64_t n, int64_t k, int8_t* xq, float* scale,
                                  hipStream_t s);
hipError_t launch_gemm_w4a8(const void* blocks, int64_t m, int64_t k, const int8_t* xq, const float* xs,
                            int64_t n, float* y, hipStream_t s);
hipError_t launch_dequant(int fmt, const void* blocks, int64_t rows, int64_t k, void* out, int ot,
                          hipStream_t s);
hipError_t launch_gemv(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       float* y, hipStream_t s);
// items: 1..QBLK_GEMV_BATCH_MAX products with m > 0, validated
hipError_t launch_gemv_batch(int fmt, int64_t k, int xt, const qblk_gemv_item_t* items, int count,
                             hipStream_t s);
hipError_t launch_gemm(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       int64_t n, float* y, hipStream_t s);
hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s);

// A dispatch packet counts its work-items in 32 bits per grid dimension, so
// one launch covers at most 2^32 - 1 threads along x.  Launchers whose grid
// grows with the data run it in pieces of whole workgroups:
// launch(first, count) for consecutive ranges of `units` work units, at most
// (max_threads / threads) * per_wg units each, stopping at the first error.
constexpr int64_t kMaxDispatchThreads = 0xFFFFFFFFLL;

template <class Launch>
hipError_t in_pieces(int64_t units, int64_t per_wg, int64_t threads, Launch&& launch,
                     int64_t max_threads = kMaxDispatchThreads) {
  const int64_t per = (max_threads / threads) * per_wg;
  for (int64_t u0 = 0; u0 < units; u0 += per) {
    const hipError_t e = launch(u0, units - u0 < per ? units - u0 : per);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Rows of one GEMV launch: every GEMV kernel runs at most 128 threads per
// row (two waves per row, one row per wave), so 2^24 rows stay far below
// the dispatch limit; longer matrices are multiplied in pieces of rows.
constexpr int64_t kGemvRowsPerLaunch = int64_t(1) << 24;

// Compute units of the current device (queried once per device, then cached;
// 256 if the query fails).  Every launcher sizes its grid from this.
int cu_count();

// qblk_set_deterministic: when on, the product launchers never split the k
// range over workgroups (no atomic sums).
bool deterministic();

// QBLK_LOG=1 in the environment: every launch writes one line to stderr
// naming the kernel and the tiling it picked (read once per process).
bool log_enabled();
void log_launch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace qblk
