// Decode-size BitLinear product with fp32 activations, reading i2_s or TQ2_0
// codes directly (Hesper "BitLinear": "Fused BitLinear Kernel (i2_s
// format)", "M=1 Warp-Cooperative BitLinear Kernel"; Hesper "TQ2_0":
// "TQ2_0 Format").  y[m,n] = scale * sum_k w[n,k] x[m,k] (i2_s), or
// sum_b s[n,b] * sum_{k in b} w x over the 256-element blocks b (TQ2_0).
//
// MI355X design.  The multiply-accumulate runs on the bf16 matrix cores:
//   * x is split exactly into three bf16 planes, x = h + m + l (h = x with
//     its low 16 bits cleared, m likewise from x - h, l = x - h - m; each
//     step is an exact fp32 subtraction and l has at most 8 significant
//     bits), so every product plane * weight is exact and only the fp32
//     accumulation rounds;
//   * a 2-bit code becomes a bf16 value 2w in two VALU ops per pair of
//     weights: shifted into bits 14..15 of a 16-bit half, the two code bits
//     are the sign and the top exponent bit, which spell -2.0 (0xC000),
//     -0.0 (0x8000) or +2.0 (0x4000).  i2_s codes (w+1) are complemented
//     first; TQ2_0 codes (two's complement w) are used as they are.
// The planes of the M tokens are the rows of the 16 x K MFMA operand A (3M
// rows, up to three 16-row tiles); 16 weight rows are the 16 columns of B.
// One 16-byte load per lane covers 64 codes; four lanes cover 256
// consecutive k of one row (a "segment"), which feed eight
// v_mfma_f32_16x16x32_bf16.  The k-order inside a segment is a fixed
// permutation (slot_k below) that the activation-prep kernel applies to x,
// so A and B agree.  Four waves of a workgroup split the segments of one
// 16-row tile and meet in LDS at the end.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int kW = 4;  // waves per workgroup

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

// A operand fragments: frag f = (s*8 + t)*MT + tau holds, for each lane
// (row i = lane%16 of tile tau, quarter q = lane/16), the 8 bf16 values of
// plane (16*tau + i) % 3 of token (16*tau + i) / 3 at k = slot_k(s,t,q,0..7)
// (zero past K).  Rows >= 3M are never written nor read.
template <int FMT>
__global__ void __launch_bounds__(256) prep_f32_kernel(const float* __restrict__ x, int M, int64_t K, int MT,
                                                        int64_t nfrag, i32x4* __restrict__ afrag) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int lane = int(gid & 63);
    const int64_t f = gid >> 6;
    if (f >= nfrag) return;
    const int tau = int(f % MT);
    const int64_t st = f / MT;
    const int t = int(st & 7);
    const int64_t s = st >> 3;
    const int i = lane & 15, q = lane >> 4;
    const int r = 16 * tau + i;
    if (r >= 3 * M) return;
    const int m = r / 3, p = r % 3;
    const float* xr = x + int64_t(m) * K;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t k = slot_k<FMT>(s, t, q, e);
        const float v = (k < K) ? xr[k] : 0.0f;
        o[e >> 1] |= bf16_plane(v, p) << (16 * (e & 1));
    }
    i32x4 out = {int(o[0]), int(o[1]), int(o[2]), int(o[3])};
    afrag[f * 64 + lane] = out;
}

template <int FMT, int MT>
__global__ void __launch_bounds__(64 * kW) gemv_f32_kernel(const uint8_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales,
                                                            int64_t N, int64_t K,
                                                            const i32x4* __restrict__ afrag, int M,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ y) {
    __shared__ float red[kW][MT][4][64];
    __shared__ float csum[MT * 16][17];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nl = lane & 15, q = lane >> 4;
    const int64_t n0 = int64_t(blockIdx.x) * 16;
    const int64_t row = (n0 + nl < N) ? (n0 + nl) : (N - 1);
    const int64_t rowbytes = K / 4;
    const uint8_t* rowp = codes + row * rowbytes;
    const int64_t S = (K + 255) / 256;
    const bool arow = (16 * 0 + nl) < 3 * M;  // row of tile 0 in use (tiles > 0 checked below)

    f32x4 acc[MT];
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) acc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t s = wave; s < S; s += kW) {
        const int64_t off = 64 * s + 16 * q;
        i32x4 u = {0, 0, 0, 0};
        if (off < rowbytes) {
            u = ld16_stream(rowp + off);
            if (FMT == 1) u = ~u;
        }
        f32x4 blk[MT];
#pragma unroll
        for (int tau = 0; tau < MT; ++tau) blk[tau] = (FMT == 2) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[tau];
        const i32x4* af = afrag + (s * 8) * MT * 64 + lane;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t wv = uint32_t(u[t >> 1]);
            i32x4 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 4 * (t & 1) + e;
                b[e] = int((wv << (14 - 2 * jj)) & 0xC000C000u);
            }
#pragma unroll
            for (int tau = 0; tau < MT; ++tau) {
                i32x4 a = {0, 0, 0, 0};
                if ((tau == 0 ? arow : (16 * tau + nl) < 3 * M)) a = af[(t * MT + tau) * 64];
                blk[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                   __builtin_bit_cast(bf16x8, b), blk[tau], 0, 0, 0);
            }
        }
        if (FMT == 2) {
            const float sc = half_bits_to_float(scales[row * (K / 256) + s]);
#pragma unroll
            for (int tau = 0; tau < MT; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[tau][r] = __builtin_fmaf(sc, blk[tau][r], acc[tau][r]);
        } else {
#pragma unroll
            for (int tau = 0; tau < MT; ++tau) acc[tau] = blk[tau];
        }
    }

#pragma unroll
    for (int tau = 0; tau < MT; ++tau)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][tau][r][lane] = acc[tau][r];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int tau = 0; tau < MT; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = red[0][tau][r][lane];
#pragma unroll
                for (int w = 1; w < kW; ++w) v += red[w][tau][r][lane];
                // C layout: lane holds column lane%16, rows 4*(lane/16) + r of tile tau
                csum[16 * tau + 4 * q + r][nl] = v;
            }
    }
    __syncthreads();
    float factor = 0.5f;  // B holds 2w
    if (FMT == 1) {
        const float sc = *reinterpret_cast<const float*>(codes + N * rowbytes);
        factor = 0.5f * sc;
    }
    for (int o = threadIdx.x; o < M * 16; o += 64 * kW) {
        const int m = o >> 4, n = o & 15;
        if (n0 + n >= N) continue;
        float v = (csum[3 * m][n] + csum[3 * m + 1][n]) + csum[3 * m + 2][n];
        v = __fmul_rn(v, factor);
        if (bias) v = __fadd_rn(v, bias[n0 + n]);
        y[int64_t(m) * N + n0 + n] = v;
    }
}

template <int FMT>
hipError_t launch_fmt(const void* codes, const void* scales, int64_t N, int64_t K, const float* x, int M,
                      const float* bias, float* y, void* ws, hipStream_t stream) {
    const int MT = (3 * M + 15) / 16;
    const int64_t S = (K + 255) / 256;
    const int64_t nfrag = S * 8 * MT;
    i32x4* afrag = static_cast<i32x4*>(ws);
    const int64_t threads = nfrag * 64;
    hipLaunchKernelGGL(prep_f32_kernel<FMT>, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, x, M, K, MT,
                       nfrag, afrag);
    const dim3 grid{unsigned((N + 15) / 16)}, block{64 * kW};
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    const uint16_t* s = static_cast<const uint16_t*>(scales);
    switch (MT) {
    case 1: hipLaunchKernelGGL((gemv_f32_kernel<FMT, 1>), grid, block, 0, stream, c, s, N, K, afrag, M, bias, y); break;
    case 2: hipLaunchKernelGGL((gemv_f32_kernel<FMT, 2>), grid, block, 0, stream, c, s, N, K, afrag, M, bias, y); break;
    default: hipLaunchKernelGGL((gemv_f32_kernel<FMT, 3>), grid, block, 0, stream, c, s, N, K, afrag, M, bias, y); break;
    }
    return hipGetLastError();
}

}  // namespace

namespace llk {

size_t gemv_f32_workspace(int64_t M, int64_t K) {
    const int64_t MT = (3 * M + 15) / 16;
    const int64_t S = (K + 255) / 256;
    return size_t(S * 8 * MT * 64 * 16);
}

hipError_t launch_gemv_f32(int fmt, const void* codes, const void* scales, int64_t N, int64_t K, const float* x,
                           int64_t M, const float* bias, float* y, void* ws, hipStream_t stream) {
    if (fmt == 1) return launch_fmt<1>(codes, scales, N, K, x, int(M), bias, y, ws, stream);
    return launch_fmt<2>(codes, scales, N, K, x, int(M), bias, y, ws, stream);
}

}  // namespace llk
