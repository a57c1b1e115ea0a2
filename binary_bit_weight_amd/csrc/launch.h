// Kernel launchers: host functions that enqueue the HIP kernels.  Arguments
// are validated by the C-ABI layer before any launcher is called; launchers
// only pick the kernel variant and grid, and return hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace llk {

hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, int8_t* xq, float* xs,
                           hipStream_t stream);

// fp32-activation decode product, formats i2_s (fmt 1) and TQ2_0 (fmt 2),
// 1 <= M <= 16.  Two kernels: the activation split into bf16 planes laid out
// as MFMA operands (into `ws`), then the packed-weight product.
size_t gemv_f32_workspace(int64_t M, int64_t K);
hipError_t launch_gemv_f32(int fmt, const void* codes, const void* scales, int64_t N, int64_t K,
                           const float* x, int64_t M, const float* bias, float* y, void* ws,
                           hipStream_t stream);

// int8-activation prefill product, format i2_s.
hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq,
                              const float* xs, int64_t M, const float* bias, float* y,
                              int32_t* acc_out, hipStream_t stream);

}  // namespace llk
