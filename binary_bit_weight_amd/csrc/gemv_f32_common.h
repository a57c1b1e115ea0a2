// Activation-operand helpers shared by the fp32-activation GEMV kernels:
// the k order inside a 256-k segment, the exact three-plane bf16 split of
// fp32 activations and the operand ("fragment") layout built from them.
#pragma once
#include "common.h"

namespace llk {

// Actual k of the value held in A/B slot (t, q, e) of segment s: t = MFMA
// index within the segment (0..7), q = lane quarter (lane / 16), e = bf16
// element of the lane's operand (0..7).  B slot e of MFMA t takes code
// j = 4*(t%2) + e/2 + 8*(e%2) of dword t/2 of the lane's 16-byte chunk.
template <int FMT>
__host__ __device__ __forceinline__ int64_t slot_k(int64_t s, int t, int q, int e) {
    const int j = 4 * (t & 1) + (e >> 1) + 8 * (e & 1);
    const int v = t >> 1;
    if (FMT == 1)  // i2_s: byte (16q + 4v + j/4) of the segment, shift 2*(j%4)
        return 256 * s + 128 * (q >> 1) + 32 * (3 - (j & 3)) + 16 * (q & 1) + 4 * v + (j >> 2);
    // TQ2_0: element 4*byte + j%4 of the 256-element block s
    return 256 * s + 64 * q + 16 * v + j;
}

__device__ __forceinline__ uint32_t bf16_plane(float v, int p) {
    uint32_t h = __float_as_uint(v) & 0xffff0000u;
    if (p == 0) return h >> 16;
    float r = __fsub_rn(v, __uint_as_float(h));
    uint32_t mbits = __float_as_uint(r) & 0xffff0000u;
    if (p == 1) return mbits >> 16;
    float l = __fsub_rn(r, __uint_as_float(mbits));
    return __float_as_uint(l) >> 16;
}

// Activation operand layout ("fragments").  For segment s, MFMA t, plane
// row r = 3*m + p (token m, plane p, r < 3M) and lane quarter q, 16 bytes
// at index ((s*8 + t) * 3M + r) * 4 + q hold the 8 bf16 values of plane p
// of x[m, slot_k(s, t, q, 0..7)] (zero past K).  Lane (i = lane%16, q) of
// row tile tau reads entry r = 16*tau + i when r < 3M.
__device__ __forceinline__ i32x4 prep_value(const float* __restrict__ x, int M, int64_t K, int fmt, int64_t e) {
    const int q = int(e & 3);
    const int64_t rr = e >> 2;
    const int R = 3 * M;
    const int r = int(rr % R);
    const int64_t st = rr / R;
    const int t = int(st & 7);
    const int64_t s = st >> 3;
    const int m = r / 3, p = r % 3;
    const float* xr = x + int64_t(m) * K;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t k = fmt == 1 ? slot_k<1>(s, t, q, i) : slot_k<2>(s, t, q, i);
        const float v = (k < K) ? xr[k] : 0.0f;
        o[i >> 1] |= bf16_plane(v, p) << (16 * (i & 1));
    }
    return i32x4{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
}

__device__ __forceinline__ void prep_one(const float* __restrict__ x, int M, int64_t K, int fmt, int64_t e,
                                         i32x4* __restrict__ afrag) {
    afrag[e] = prep_value(x, M, K, fmt, e);
}

}  // namespace llk
