// Prefill-size BitLinear product with int8 activations and i2_s weights on
// the int8 matrix cores (Hesper "BitLinear": "Subgroup-Matrix Multi-row
// BitLinear Kernel" computes Y = X W^T per output tile; binary-gemm card,
// "Requirements and limits": prefill needs a different kernel than the
// decode GEMV).  acc[m,n] = sum_k w[n,k] q[m,k] exactly in int32, and
// y = ((float)acc * s_tok[m]) * s_w.
//
// MI355X design: v_mfma_i32_32x32x32_i8; lane l holds 16 consecutive k of
// row (or column) l % 32 at k offset 16 (l / 32) of a 32-k step.  The 32
// bytes of one 128-k group of an i2_s row hold, in their four 2-bit fields,
// the k runs 32t + [0, 32) for t = 0..3 (byte j of the group, field t:
// element 32t + j), so the weights decode in natural k order and the
// activations need no reordering.
//
// Workgroup tile 128 x 128, eight waves of 32 x 64 (two waves per SIMD, so
// one wave's operand reads and barrier waits overlap the other's
// multiplies).  Per 128-k group the workgroup stores the int8 activation
// tile and the weight tile, decoded once to int8 {-1, 0, +1} (shift, mask,
// byte permute through {0xFF, 0x00, 0x01}), into one of two LDS buffers;
// rows are padded to 144 bytes so an MFMA operand's 32 rows fall on distinct
// banks.  Inside a group the operand reads of step t + 1 are issued before
// the multiplies of step t.  Global loads run three groups ahead in four
// register stages, every load from a clamped in-bounds address so the
// compiler can count its waits; one barrier per group.
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

constexpr int BM = 128, BN = 128, LDA = 144, LDB = 144;
constexpr int kThreads = 512;                            // eight waves
constexpr int kTileInts = BM * BN;                       // one partial tile
constexpr int kBuf = BM * LDA + BN * LDB;                // one LDS buffer: activation tile, then weight tile
constexpr size_t kGemmLds = size_t(2) * kBuf;


__global__ void __launch_bounds__(kThreads) gemm_i8_i2s_kernel(const uint8_t* __restrict__ codes, int64_t N,
                                                                int64_t K, const int8_t* __restrict__ xq,
                                                                const float* __restrict__ xs, int64_t M,
                                                                const float* __restrict__ bias, float* __restrict__ y,
                                                                int32_t* __restrict__ acc_out, int S,
                                                                int32_t* __restrict__ part,
                                                                int32_t* __restrict__ counters) {
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    __shared__ int last_flag;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;               // rows 32 wm, columns 64 wn of the tile
    const int li = lane & 31, h = lane >> 5;
    const int64_t TM = (M + BM - 1) / BM;
    const int64_t tile = int64_t(blockIdx.x) / S;
    const int split = int(blockIdx.x % S);
    const int64_t m0 = (tile % TM) * BM, n0 = (tile / TM) * BN;
    const int64_t rowbytes = K / 4;
    const int64_t ng = K / 128;
    const int64_t g0 = ng * split / S, g1 = ng * (split + 1) / S;

    // Loads of one group: two 16-byte activation chunks (row idx / 8, chunk
    // idx % 8 for idx = tid, tid + 512) and 8 code bytes (column tid / 4,
    // quarter tid % 4 of the 32-byte group); rows and columns are clamped
    // (results of clamped ones are not stored).
    const int8_t* arow[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int idx = tid + kThreads * c;
        int64_t m = m0 + (idx >> 3);
        m = m < M ? m : M - 1;
        arow[c] = xq + m * K + 16 * (idx & 7);
    }
    const int bcol = tid >> 2, bq = tid & 3;
    int64_t ncl = n0 + bcol;
    ncl = ncl < N ? ncl : N - 1;
    const uint8_t* bptr = codes + ncl * rowbytes + 8 * bq;

    struct Stage {
        i32x4 a[2];
        uint32_t b[2];
    };
    auto load = [&](int64_t g, Stage& s) {
        const int64_t gc = g < g1 ? g : g1 - 1;            // past the range: reload the last group (unused)
#pragma unroll
        for (int c = 0; c < 2; ++c) s.a[c] = ld16(arow[c] + 128 * gc);
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
        const u32x2 b2 = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x2*)(bptr + 32 * gc));
        s.b[0] = b2[0];
        s.b[1] = b2[1];
    };
    // Byte j of quarter bq is group byte 8 bq + j; its field t is element
    // 32 t + 8 bq + j, so each field gives 8 consecutive k of step t.
    auto store = [&](int buf, const Stage& s) {
        int8_t* A = lds + buf * kBuf;
        int8_t* B = A + BM * LDA;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int idx = tid + kThreads * c;
            *reinterpret_cast<i32x4*>(&A[(idx >> 3) * LDA + 16 * (idx & 7)]) = s.a[c];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int sh = 6 - 2 * t;
            uint2 v;
            v.x = __builtin_amdgcn_perm(0u, 0x000100FFu, (s.b[0] >> sh) & 0x03030303u);
            v.y = __builtin_amdgcn_perm(0u, 0x000100FFu, (s.b[1] >> sh) & 0x03030303u);
            *reinterpret_cast<uint2*>(&B[bcol * LDB + 32 * t + 8 * bq]) = v;
        }
    };

    i32x16 acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0;

    auto compute = [&](int buf) {
        const int8_t* A = lds + buf * kBuf + (wm * 32 + li) * LDA + 16 * h;
        const int8_t* B = lds + buf * kBuf + BM * LDA + (wn * 64 + li) * LDB + 16 * h;
        i32x4 ao[2], bo[2][2];
        ao[0] = *reinterpret_cast<const i32x4*>(A);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bo[0][nb] = *reinterpret_cast<const i32x4*>(B + nb * 32 * LDB);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < 3) {                                   // operands of step t + 1 first
                ao[nxt] = *reinterpret_cast<const i32x4*>(A + 32 * (t + 1));
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    bo[nxt][nb] = *reinterpret_cast<const i32x4*>(B + nb * 32 * LDB + 32 * (t + 1));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                acc[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[cur], bo[cur][nb], acc[nb], 0, 0, 0);
        }
    };

    // Group g + i is multiplied from LDS buffer i % 2; register stage i % 4
    // holds group g + i from its load (three groups earlier) to its store
    // (one group earlier).  The main loop runs whole quadruples of groups with
    // no early exit; the last one to three groups follow it.
    Stage st0, st1, st2, st3;
    load(g0, st0);
    load(g0 + 1, st1);
    load(g0 + 2, st2);
    load(g0 + 3, st3);
    store(0, st0);
    __syncthreads();
    const int64_t nsteps = g1 - g0;
    int64_t g = g0;
    for (; g + 4 <= g1; g += 4) {
        // loads first (kept there by the scheduling barrier); the store of the
        // next group and the multiplies of this one may interleave
        load(g + 4, st0);
        __builtin_amdgcn_sched_barrier(0);
        store(1, st1);
        compute(0);
        __syncthreads();
        load(g + 5, st1);
        __builtin_amdgcn_sched_barrier(0);
        store(0, st2);
        compute(1);
        __syncthreads();
        load(g + 6, st2);
        __builtin_amdgcn_sched_barrier(0);
        store(1, st3);
        compute(0);
        __syncthreads();
        load(g + 7, st3);
        __builtin_amdgcn_sched_barrier(0);
        store(0, st0);
        compute(1);
        __syncthreads();
    }
    const int64_t rem = nsteps % 4;
    if (rem >= 1) compute(0);
    if (rem >= 2) {
        store(1, st1);
        __syncthreads();
        compute(1);
    }
    if (rem >= 3) {
        store(0, st2);
        __syncthreads();
        compute(0);
    }

    if (S > 1) {
        // Publish this split's partial tile with device-coherent stores, wait for
        // them to complete, then count the split in; the split that arrives last
        // reads the others' partials (device-coherent loads) and finishes the tile.
        int32_t* mine = part + (tile * S + split) * int64_t(kTileInts);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st_coherent(mine + (nb * 16 + r) * kThreads + tid, acc[nb][r]);
        wait_vmem();
        __syncthreads();
        if (tid == 0) last_flag = atomicAdd(counters + tile, 1) == S - 1;
        __syncthreads();
        if (!last_flag) return;
        for (int s = 0; s < S; ++s) {
            if (s == split) continue;
            const int32_t* other = part + (tile * S + s) * int64_t(kTileInts);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][r] += ld_coherent(other + (nb * 16 + r) * kThreads + tid);
        }
        if (tid == 0) st_coherent(counters + tile, 0);    // ready for the next call
    }

    // Epilogue.  The token scales and biases of this lane's rows and columns are
    // loaded up front from clamped indices (a load under a per-element branch
    // would be waited on one at a time); only the stores are guarded.
    const float sw = *reinterpret_cast<const float*>(codes + N * rowbytes);
    float xsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        xsv[r] = xs[m < M ? m : M - 1];
    }
    float bnv[2] = {0.0f, 0.0f};
    if (bias)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t n = n0 + wn * 64 + nb * 32 + li;
            bnv[nb] = bias[n < N ? n : N - 1];
        }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n0 + wn * 64 + nb * 32 + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const int32_t a = acc[nb][r];
            float v = __fmul_rn(__fmul_rn(float(a), xsv[r]), sw);
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
    const dim3 grid{unsigned(tiles * S)}, block{unsigned(kThreads)};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gemm_i8_i2s_kernel), kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_i8_i2s_kernel, grid, block, kGemmLds, stream, codes, N, K, xq, xs, M, bias, y, acc_out, S,
                       part, counters);
    return hipGetLastError();
}

}  // namespace llk
