// Per-token absmax activation quantization (binary-gemm card, "API":
// quantize_activation; "Correctness": per-token absmax).  For each token
// row: a = max |x|; if a == 0 the scale and every code are 0; otherwise
// inv = 127/a (IEEE fp32 division), q = round-half-even(x * inv) clamped to
// [-127, 127], and the scale is a/127.
//
// One workgroup of 256 threads per token: pass 1 reduces |x| to the row
// max (wave butterflies, then 4 partial maxima through LDS), pass 2 re-reads
// the row (L2-resident) and writes the codes, and (when xsum is given) sums
// them into xsum[m] = sum_k q[m,k], the per-token term of the offset form
// sum_k w q = sum_k (w + 1) q - sum_k q.  16-byte loads when the row stride
// allows it.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

template <bool BF16>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
    if (BF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[i]) << 16);
    return static_cast<const float*>(x)[i];
}

__device__ __forceinline__ int8_t quant_one(float v, float inv) {
    float r = __builtin_rintf(__fmul_rn(v, inv));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return int8_t(int(r));
}

template <bool BF16, bool VEC>
__global__ void __launch_bounds__(256) quant_kernel(const void* __restrict__ x, int64_t K,
                                                     int8_t* __restrict__ xq, float* __restrict__ xs,
                                                     int32_t* __restrict__ xsum) {
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ float part[4];
    __shared__ int32_t qpart[4];
    int32_t qs = 0;
    // elements per 16-byte vector: 4 fp32 or 8 bf16
    constexpr int E = BF16 ? 8 : 4;
    const size_t esz = BF16 ? 2 : 4;
    const char* row = static_cast<const char*>(x) + size_t(m) * size_t(K) * esz;

    float a = 0.0f;
    if (VEC) {
        for (int64_t v = tid; v < K / E; v += 256) {
            i32x4 d = ld16(row + size_t(v) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t u = uint32_t(d[j]);
                if (BF16) {
                    a = fmaxf(a, fabsf(__uint_as_float(u << 16)));
                    a = fmaxf(a, fabsf(__uint_as_float(u & 0xffff0000u)));
                } else {
                    a = fmaxf(a, fabsf(__uint_as_float(u)));
                }
            }
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) a = fmaxf(a, fabsf(load_x<BF16>(row, k)));
    }
    a = wave_max(a);
    if ((tid & 63) == 0) part[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));

    const float inv = (a == 0.0f) ? 0.0f : __fdiv_rn(127.0f, a);
    if (tid == 0) xs[m] = (a == 0.0f) ? 0.0f : __fdiv_rn(a, 127.0f);
    int8_t* qrow = xq + size_t(m) * size_t(K);
    if (VEC) {
        for (int64_t v = tid; v < K / E; v += 256) {
            i32x4 d = ld16(row + size_t(v) * 16);
            if (BF16) {
                uint32_t o0 = 0, o1 = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t u = uint32_t(d[j]);
                    const int8_t ql = quant_one(__uint_as_float(u << 16), inv);
                    const int8_t qh = quant_one(__uint_as_float(u & 0xffff0000u), inv);
                    qs += int32_t(ql) + int32_t(qh);
                    uint32_t lo = uint8_t(ql);
                    uint32_t hi = uint8_t(qh);
                    uint32_t pair = lo | (hi << 8);
                    if (j < 2) o0 |= pair << (16 * j);
                    else o1 |= pair << (16 * (j - 2));
                }
                uint2 o = make_uint2(o0, o1);
                *reinterpret_cast<uint2*>(qrow + size_t(v) * 8) = o;
            } else {
                uint32_t o = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int8_t q = quant_one(__uint_as_float(uint32_t(d[j])), inv);
                    qs += int32_t(q);
                    o |= uint32_t(uint8_t(q)) << (8 * j);
                }
                *reinterpret_cast<uint32_t*>(qrow + size_t(v) * 4) = o;
            }
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) {
            const int8_t q = quant_one(load_x<BF16>(row, k), inv);
            qs += int32_t(q);
            qrow[k] = q;
        }
    }
    if (xsum) {
        int v[1] = {qs};
        wave_sum_n<1>(v);
        if ((tid & 63) == 0) qpart[tid >> 6] = v[0];
        __syncthreads();
        if (tid == 0) xsum[m] = qpart[0] + qpart[1] + qpart[2] + qpart[3];
    }
}

}  // namespace

namespace llk {

hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, int8_t* xq, float* xs, int32_t* xsum,
                           hipStream_t stream) {
    const size_t esz = bf16 ? 2 : 4;
    // the vector path needs every row to start on a 16-byte boundary and the
    // int8 output rows on an 8-byte (bf16) / 4-byte (fp32) boundary
    const bool vec = (size_t(K) * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0 &&
                     (reinterpret_cast<uintptr_t>(xq) % 8) == 0;
    const dim3 grid{unsigned(M)}, block{256};
    if (bf16) {
        if (vec) hipLaunchKernelGGL((quant_kernel<true, true>), grid, block, 0, stream, x, K, xq, xs, xsum);
        else hipLaunchKernelGGL((quant_kernel<true, false>), grid, block, 0, stream, x, K, xq, xs, xsum);
    } else {
        if (vec) hipLaunchKernelGGL((quant_kernel<false, true>), grid, block, 0, stream, x, K, xq, xs, xsum);
        else hipLaunchKernelGGL((quant_kernel<false, false>), grid, block, 0, stream, x, K, xq, xs, xsum);
    }
    return hipGetLastError();
}

}  // namespace llk
