// Prefill-size BitLinear product with int8 activations and i2_s weights on
// the int8 matrix cores (Hesper "BitLinear": "Subgroup-Matrix Multi-row
// BitLinear Kernel" computes Y = X W^T per output tile; binary-gemm card,
// "Requirements and limits": prefill needs a different kernel than the
// decode GEMV).  acc[m,n] = sum_k w[n,k] q[m,k] exactly in int32, and
// y = ((float)acc * s_tok[m]) * s_w.
//
// MI355X design: v_mfma_i32_32x32x32_i8.  Its B operand gives each lane 16
// consecutive k of one column; one 16-byte load of i2_s codes at byte
// 32g + 16h of a row holds, in its four shift planes, exactly the 16-k runs
// 128g + 32t + 16h + [0,16) for t = 0..3.  So lane (column n = lane%32,
// h = lane/32) feeds four MFMAs (t = 0..3) from one load, in natural k
// order, and the activations need no reordering.  A plane is decoded to
// int8 {-1,0,+1} in three ops per four weights: shift, mask to one code per
// byte, and a byte permute through the table {0xFF, 0x00, 0x01}.
// Workgroup tile 128 x 128 (four waves of 64 x 64); the int8 activation
// tile of each 128-k group is staged in LDS (rows padded to 144 bytes so
// the 32 rows read by one MFMA operand fall on distinct banks).
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int BM = 128, BN = 128, LDA = 144;

__device__ __forceinline__ i32x4 decode_plane_i8(i32x4 u, int t) {
    const int sh = 6 - 2 * t;
    i32x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t c = (uint32_t(u[j]) >> sh) & 0x03030303u;
        b[j] = int(__builtin_amdgcn_perm(0u, 0x000100FFu, c));
    }
    return b;
}

__global__ void __launch_bounds__(256) gemm_i8_i2s_kernel(const uint8_t* __restrict__ codes, int64_t N, int64_t K,
                                                           const int8_t* __restrict__ xq,
                                                           const float* __restrict__ xs, int64_t M,
                                                           const float* __restrict__ bias, float* __restrict__ y,
                                                           int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDA];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, h = lane >> 5;
    const int64_t m0 = int64_t(blockIdx.y) * BM, n0 = int64_t(blockIdx.x) * BN;
    const int64_t rowbytes = K / 4;

    // B rows of this lane (clamped to the last row; results of clamped rows are not stored)
    const uint8_t* brow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        int64_t n = n0 + wn * 64 + nb * 32 + li;
        n = n < N ? n : N - 1;
        brow[nb] = codes + n * rowbytes + 16 * h;
    }

    i32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    for (int64_t g = 0; g < K / 128; ++g) {
        // stage the 128 x 128 activation tile (1024 chunks of 16 bytes)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = tid + 256 * c;
            const int r = idx >> 3, col = idx & 7;
            int64_t m = m0 + r;
            m = m < M ? m : M - 1;
            const i32x4 v = ld16(xq + m * K + 128 * g + 16 * col);
            *reinterpret_cast<i32x4*>(As + r * LDA + 16 * col) = v;
        }
        i32x4 bc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bc[nb] = ld16_stream(brow[nb] + 32 * g);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            i32x4 bop[2], aop[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) bop[nb] = decode_plane_i8(bc[nb], t);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                aop[mb] = *reinterpret_cast<const i32x4*>(As + (wm * 64 + mb * 32 + li) * LDA + 32 * t + 16 * h);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[mb], bop[nb], acc[mb][nb], 0, 0, 0);
        }
        __syncthreads();
    }

    const float sw = *reinterpret_cast<const float*>(codes + N * rowbytes);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t n = n0 + wn * 64 + nb * 32 + li;
            if (n >= N) continue;
            const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m >= M) continue;
                const int32_t a = acc[mb][nb][r];
                float v = __fmul_rn(__fmul_rn(float(a), xs[m]), sw);
                if (bias) v = __fadd_rn(v, bn);
                y[m * N + n] = v;
                if (acc_out) acc_out[m * N + n] = a;
            }
        }
}

}  // namespace

namespace llk {

hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq, const float* xs,
                              int64_t M, const float* bias, float* y, int32_t* acc_out, hipStream_t stream) {
    const dim3 grid{unsigned((N + BN - 1) / BN), unsigned((M + BM - 1) / BM)}, block{256};
    hipLaunchKernelGGL(gemm_i8_i2s_kernel, grid, block, 0, stream, codes, N, K, xq, xs, M, bias, y, acc_out);
    return hipGetLastError();
}

}  // namespace llk
