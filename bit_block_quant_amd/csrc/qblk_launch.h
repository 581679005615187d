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
hipError_t launch_gemm(int fmt, const void* blocks, int64_t m, int64_t k, const void* x, int xt,
                       int64_t n, float* y, hipStream_t s);
hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s);

}  // namespace qblk
