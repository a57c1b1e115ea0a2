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
//
// Workgroup tile 128 x 128 (four waves of 64 x 64), one 128-k group per
// step.  The int8 activation tile of a step sits in one of four LDS
// buffers (rows padded to 144 bytes so the 32 rows of an MFMA operand fall
// on distinct banks); the activation and code loads of step g + 3 are
// issued into one of four register stages before step g multiplies (a
// scheduling barrier keeps them there), every load unconditionally from a
// clamped address so the compiler can count its waits.  One workgroup
// barrier per step.
//
// Split K.  With few output tiles (N = 2560 at M = 512 gives 80) the
// workgroups of a tile split its groups S ways.  Each split writes its exact
// int32 partial tile to the workspace and increments the tile's counter; the
// split that arrives last adds the others' partials to its own and runs the
// epilogue, then resets the counter (so the counters stay zero between
// calls).  Integer addition makes the result independent of the order.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int BM = 128, BN = 128, LDA = 144;
constexpr int kTileInts = BM * BN;                       // one partial tile
constexpr int kStages = 4;                               // LDS buffers / register stages
constexpr size_t kGemmLds = size_t(kStages) * BM * LDA;

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
                                                           int32_t* __restrict__ acc_out, int S,
                                                           int32_t* __restrict__ part, int32_t* __restrict__ counters) {
    extern __shared__ __attribute__((aligned(16))) int8_t As_raw[];
    int8_t (*As)[BM * LDA] = reinterpret_cast<int8_t (*)[BM * LDA]>(As_raw);   // [kStages][BM * LDA]
    __shared__ int last_flag;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, h = lane >> 5;
    const int64_t TM = (M + BM - 1) / BM;
    const int64_t tile = int64_t(blockIdx.x) / S;
    const int split = int(blockIdx.x % S);
    const int64_t m0 = (tile % TM) * BM, n0 = (tile / TM) * BN;
    const int64_t rowbytes = K / 4;
    const int64_t ng = K / 128;
    const int64_t g0 = ng * split / S, g1 = ng * (split + 1) / S;

    // B rows of this lane (clamped to the last row; results of clamped rows are not stored)
    const uint8_t* brow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        int64_t n = n0 + wn * 64 + nb * 32 + li;
        n = n < N ? n : N - 1;
        brow[nb] = codes + n * rowbytes + 16 * h;
    }
    // A rows of this thread's four 16-byte chunks per step (clamped likewise)
    const int8_t* arow[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int idx = tid + 256 * c;
        int64_t m = m0 + (idx >> 3);
        m = m < M ? m : M - 1;
        arow[c] = xq + m * K + 16 * (idx & 7);
    }

    struct Stage {
        i32x4 a[4];
        i32x4 b[2];
    };
    auto load = [&](int64_t g, Stage& s) {
        const int64_t gc = g < g1 ? g : g1 - 1;            // past the range: reload the last group (cached, unused)
#pragma unroll
        for (int c = 0; c < 4; ++c) s.a[c] = ld16(arow[c] + 128 * gc);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) s.b[nb] = ld16_stream(brow[nb] + 32 * gc);
    };
    auto store_a = [&](int buf, const Stage& s) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = tid + 256 * c;
            *reinterpret_cast<i32x4*>(&As[buf][(idx >> 3) * LDA + 16 * (idx & 7)]) = s.a[c];
        }
    };

    i32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    auto compute = [&](int buf, const Stage& s) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            i32x4 bop[2], aop[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) bop[nb] = decode_plane_i8(s.b[nb], t);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                aop[mb] = *reinterpret_cast<const i32x4*>(&As[buf][(wm * 64 + mb * 32 + li) * LDA + 32 * t + 16 * h]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[mb], bop[nb], acc[mb][nb], 0, 0, 0);
        }
    };

    // Step g multiplies from LDS buffer g%4 and register stage g%4; the loads
    // of step g + 3 go to stage (g+3)%4 (free since step g - 1) before the
    // multiply.  The main loop runs whole quadruples of steps with no early
    // exit (an exit between a load and its use would let the compiler sink
    // the load past the multiply); the last one to three steps follow it.
    Stage st0, st1, st2, st3;
    load(g0, st0);
    load(g0 + 1, st1);
    load(g0 + 2, st2);
    store_a(0, st0);
    __syncthreads();
    const int64_t nsteps = g1 - g0;
    int64_t g = g0;
    for (; g + 4 <= g1; g += 4) {
        load(g + 3, st3);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, st0);
        store_a(1, st1);
        __syncthreads();
        load(g + 4, st0);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, st1);
        store_a(2, st2);
        __syncthreads();
        load(g + 5, st1);
        __builtin_amdgcn_sched_barrier(0);
        compute(2, st2);
        store_a(3, st3);
        __syncthreads();
        load(g + 6, st2);
        __builtin_amdgcn_sched_barrier(0);
        compute(3, st3);
        store_a(0, st0);
        __syncthreads();
    }
    const int64_t rem = nsteps % 4;
    if (rem >= 1) compute(0, st0);
    if (rem >= 2) {
        store_a(1, st1);
        __syncthreads();
        compute(1, st1);
    }
    if (rem >= 3) {
        store_a(2, st2);
        __syncthreads();
        compute(2, st2);
    }

    if (S > 1) {
        // Publish this split's partial tile with device-coherent stores, wait for
        // them to complete, then count the split in; the split that arrives last
        // reads the others' partials (device-coherent loads) and finishes the tile.
        int32_t* mine = part + (tile * S + split) * int64_t(kTileInts);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) st_coherent(mine + ((mb * 2 + nb) * 16 + r) * 256 + tid, acc[mb][nb][r]);
        wait_vmem();
        __syncthreads();
        if (tid == 0) last_flag = atomicAdd(counters + tile, 1) == S - 1;
        __syncthreads();
        if (!last_flag) return;
        for (int s = 0; s < S; ++s) {
            if (s == split) continue;
            const int32_t* other = part + (tile * S + s) * int64_t(kTileInts);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mb][nb][r] += ld_coherent(other + ((mb * 2 + nb) * 16 + r) * 256 + tid);
        }
        if (tid == 0) st_coherent(counters + tile, 0);    // ready for the next call
    }

    // Epilogue.  The token scales and biases of this lane's rows and columns are
    // loaded up front from clamped indices (a load under a per-element branch
    // would be waited on one at a time); only the stores are guarded.
    const float sw = *reinterpret_cast<const float*>(codes + N * rowbytes);
    float xsv[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            xsv[mb][r] = xs[m < M ? m : M - 1];
        }
    float bnv[2] = {0.0f, 0.0f};
    if (bias)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t n = n0 + wn * 64 + nb * 32 + li;
            bnv[nb] = bias[n < N ? n : N - 1];
        }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t n = n0 + wn * 64 + nb * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const int32_t a = acc[mb][nb][r];
                float v = __fmul_rn(__fmul_rn(float(a), xsv[mb][r]), sw);
                if (bias) v = __fadd_rn(v, bnv[nb]);
                if (m < M && n < N) {
                    y[m * N + n] = v;
                    if (acc_out) acc_out[m * N + n] = a;
                }
            }
        }
}

#ifndef LL_GEMM_SLOTS
#define LL_GEMM_SLOTS 256
#endif
// Split count: enough workgroups to cover the chip (LL_GEMM_SLOTS resident
// workgroups) without leaving a split fewer than four groups.
int gemm_splits(int64_t M, int64_t N, int64_t K, bool allow = true) {
    if (!allow) return 1;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t ng = K / 128;
    int64_t s = 1;
    while (tiles * (s + 1) <= LL_GEMM_SLOTS && ng / (s + 1) >= 4) ++s;
    return int(s);
}

}  // namespace

namespace llk {

size_t gemm_i8_workspace(int64_t M, int64_t N, int64_t K) {
    const int S = gemm_splits(M, N, K);
    if (S == 1) return 0;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return size_t(tiles) * S * kTileInts * 4 + size_t(tiles) * 4;
}

hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq, const float* xs,
                              int64_t M, const float* bias, float* y, int32_t* acc_out, void* ws, hipStream_t stream) {
    const int S = gemm_splits(M, N, K, ws != nullptr);
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int32_t* part = static_cast<int32_t*>(ws);
    int32_t* counters = S > 1 ? part + tiles * S * int64_t(kTileInts) : nullptr;
    const dim3 grid{unsigned(tiles * S)}, block{256};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gemm_i8_i2s_kernel), kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_i8_i2s_kernel, grid, block, kGemmLds, stream, codes, N, K, xq, xs, M, bias, y, acc_out, S,
                       part, counters);
    return hipGetLastError();
}

}  // namespace llk
