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
// The planes of the M tokens are the rows of the MFMA operand A (3M rows,
// up to three 16-row tiles); 16 weight rows are the 16 columns of B.  One
// 16-byte load per lane covers 64 codes; four lanes cover 256 consecutive
// k of one row (a "segment"), which feed eight v_mfma_f32_16x16x32_bf16.
// The k-order inside a segment is a fixed permutation (slot_k below) that
// the activation-prep kernel applies when it lays the planes out as MFMA
// operands, so A and B agree.
//
// Two product kernels share the per-tile loop:
//   * single product: four waves of a workgroup split the segments of one
//     16-row tile and meet in LDS (enough waves even for N = 2560);
//   * prepared batch: a device-resident table of independent products (all
//     GEMVs of a decode step) is walked by one launch, one wave per 16-row
//     tile over all of K, so the whole step costs two launches.
#include "common.h"
#include "gemv_f32_common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int kW = 4;  // waves per workgroup

__global__ void __launch_bounds__(256) prep_f32_kernel(const float* __restrict__ x, int M, int64_t K, int fmt,
                                                        int64_t nent, i32x4* __restrict__ afrag) {
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (e < nent) prep_one(x, M, K, fmt, e, afrag);
}

// Accumulates segments s = s0, s0 + ds, ... of one 16-row tile.  rowp:
// this lane's weight row; srow: its TQ2_0 block scales.
template <int FMT, int MT>
__device__ __forceinline__ void tile_segments(const uint8_t* __restrict__ rowp, int64_t rowbytes,
                                              const uint16_t* __restrict__ srow, int64_t S, int64_t s0, int64_t ds,
                                              const i32x4* __restrict__ afrag, int M, int lane, f32x4 (&acc)[MT]) {
    const int nl = lane & 15, q = lane >> 4;
    const int R = 3 * M;
    bool act[MT];
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) act[tau] = (16 * tau + nl) < R;

    auto load_codes = [&](int64_t s) -> i32x4 {
        const int64_t off = 64 * s + 16 * q;
        i32x4 u = {0, 0, 0, 0};
        if (s < S && off < rowbytes) {
            u = ld16_stream(rowp + off);
            if (FMT == 1) u = ~u;
        }
        return u;
    };

    i32x4 unext = load_codes(s0);
    for (int64_t s = s0; s < S; s += ds) {
        const i32x4 u = unext;
        unext = load_codes(s + ds);
        f32x4 blk[MT];
#pragma unroll
        for (int tau = 0; tau < MT; ++tau) blk[tau] = (FMT == 2) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[tau];
        const i32x4* af = afrag + ((s * 8) * R + nl) * 4 + q;
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
                if (act[tau]) a = af[(t * R + 16 * tau) * 4];
                blk[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                   __builtin_bit_cast(bf16x8, b), blk[tau], 0, 0, 0);
            }
        }
        if (FMT == 2) {
            const float sc = half_bits_to_float(srow[s]);
#pragma unroll
            for (int tau = 0; tau < MT; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[tau][r] = __builtin_fmaf(sc, blk[tau][r], acc[tau][r]);
        } else {
#pragma unroll
            for (int tau = 0; tau < MT; ++tau) acc[tau] = blk[tau];
        }
    }
}

// Writes y for one tile from the summed accumulators in LDS (cs[row][col],
// rows = plane rows 3m+p).  factor folds the 2w encoding and the i2_s scale.
__device__ __forceinline__ void store_tile(const float (*cs)[17], int M, int64_t n0, int64_t N, float factor,
                                           const float* __restrict__ bias, float* __restrict__ y, int tid, int nthr) {
    for (int o = tid; o < M * 16; o += nthr) {
        const int m = o >> 4, n = o & 15;
        if (n0 + n >= N) continue;
        float v = (cs[3 * m][n] + cs[3 * m + 1][n]) + cs[3 * m + 2][n];
        v = __fmul_rn(v, factor);
        if (bias) v = __fadd_rn(v, bias[n0 + n]);
        y[int64_t(m) * N + n0 + n] = v;
    }
}

template <int FMT>
__device__ __forceinline__ float out_factor(const uint8_t* codes, int64_t N, int64_t K) {
    if (FMT == 1) return 0.5f * *reinterpret_cast<const float*>(codes + N * (K / 4));
    return 0.5f;
}

template <int FMT, int MT>
__global__ void __launch_bounds__(64 * kW) gemv_f32_kernel(const uint8_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                            const i32x4* __restrict__ afrag, int M,
                                                            const float* __restrict__ bias, float* __restrict__ y) {
    __shared__ float red[kW][MT][4][64];
    __shared__ float csum[MT * 16][17];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nl = lane & 15, q = lane >> 4;
    const int64_t n0 = int64_t(blockIdx.x) * 16;
    const int64_t row = (n0 + nl < N) ? (n0 + nl) : (N - 1);
    const int64_t rowbytes = K / 4;
    f32x4 acc[MT];
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) acc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_segments<FMT, MT>(codes + row * rowbytes, rowbytes, FMT == 2 ? scales + row * (K / 256) : nullptr,
                           (K + 255) / 256, wave, kW, afrag, M, lane, acc);
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
    store_tile(csum, M, n0, N, out_factor<FMT>(codes, N, K), bias, y, threadIdx.x, 64 * kW);
}

// ---------------------------------------------------------------- prepared batch
struct BatchProb {            // one product of the batch (device table entry)
    const uint8_t* codes;
    const uint16_t* scales;
    const float* bias;
    float* y;
    const i32x4* afrag;
    int64_t N, K;
    int64_t tile0;            // first 16-row tile of this product in the launch
};
struct BatchPrep {            // one distinct activation matrix of the batch
    const float* x;
    i32x4* afrag;
    int64_t K;
    int64_t ent0;             // first fragment entry of this activation in the launch
};

template <typename T>
__device__ __forceinline__ int find_entry(const T* __restrict__ tab, int count, int64_t key, int64_t T::*field) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid].*field <= key) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ void __launch_bounds__(256) prep_batch_kernel(const BatchPrep* __restrict__ tab, int count, int M, int fmt,
                                                          int64_t total) {
    const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (g >= total) return;
    const int i = find_entry(tab, count, g, &BatchPrep::ent0);
    const BatchPrep& p = tab[i];
    prep_one(p.x, M, p.K, fmt, g - p.ent0, p.afrag);
}

template <int FMT, int MT>
__global__ void __launch_bounds__(64 * kW) gemv_f32_batch_kernel(const BatchProb* __restrict__ tab, int count, int M,
                                                                  int64_t tiles) {
    __shared__ float cs[kW][MT * 16][17];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nl = lane & 15, q = lane >> 4;
    const int64_t tile = int64_t(blockIdx.x) * kW + wave;
    const bool live = tile < tiles;
    const int pi = find_entry(tab, count, live ? tile : tiles - 1, &BatchProb::tile0);
    const BatchProb& P = tab[pi];
    const int64_t n0 = (tile - P.tile0) * 16;
    const int64_t row = (n0 + nl < P.N) ? (n0 + nl) : (P.N - 1);
    const int64_t rowbytes = P.K / 4;
    f32x4 acc[MT];
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) acc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live)
        tile_segments<FMT, MT>(P.codes + row * rowbytes, rowbytes, FMT == 2 ? P.scales + row * (P.K / 256) : nullptr,
                               (P.K + 255) / 256, 0, 1, P.afrag, M, lane, acc);
#pragma unroll
    for (int tau = 0; tau < MT; ++tau)
#pragma unroll
        for (int r = 0; r < 4; ++r) cs[wave][16 * tau + 4 * q + r][nl] = acc[tau][r];
    __syncthreads();
    if (live) store_tile(cs[wave], M, n0, P.N, out_factor<FMT>(P.codes, P.N, P.K), P.bias, P.y, lane, 64);
}

template <int FMT>
hipError_t launch_fmt(const void* codes, const void* scales, int64_t N, int64_t K, const float* x, int M,
                      const float* bias, float* y, void* ws, hipStream_t stream) {
    const int MT = (3 * M + 15) / 16;
    const int64_t S = (K + 255) / 256;
    const int64_t nent = S * 8 * (3 * M) * 4;
    i32x4* afrag = static_cast<i32x4*>(ws);
    hipLaunchKernelGGL(prep_f32_kernel, dim3(unsigned((nent + 255) / 256)), dim3(256), 0, stream, x, M, K, FMT, nent,
                       afrag);
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

template <int FMT>
void launch_batch_product(const void* table, int count, int M, int64_t tiles, hipStream_t stream) {
    const int MT = (3 * M + 15) / 16;
    const dim3 grid{unsigned((tiles + kW - 1) / kW)}, block{64 * kW};
    const BatchProb* tab = static_cast<const BatchProb*>(table);
    switch (MT) {
    case 1: hipLaunchKernelGGL((gemv_f32_batch_kernel<FMT, 1>), grid, block, 0, stream, tab, count, M, tiles); break;
    case 2: hipLaunchKernelGGL((gemv_f32_batch_kernel<FMT, 2>), grid, block, 0, stream, tab, count, M, tiles); break;
    default: hipLaunchKernelGGL((gemv_f32_batch_kernel<FMT, 3>), grid, block, 0, stream, tab, count, M, tiles); break;
    }
}

}  // namespace

namespace llk {

size_t gemv_f32_workspace(int64_t M, int64_t K) {
    const int64_t S = (K + 255) / 256;
    return size_t(S * 8 * (3 * M) * 4 * 16);
}

hipError_t launch_gemv_f32(int fmt, const void* codes, const void* scales, int64_t N, int64_t K, const float* x,
                           int64_t M, const float* bias, float* y, void* ws, hipStream_t stream) {
    if (fmt == 1) return launch_fmt<1>(codes, scales, N, K, x, int(M), bias, y, ws, stream);
    return launch_fmt<2>(codes, scales, N, K, x, int(M), bias, y, ws, stream);
}

size_t batch_prob_bytes() { return sizeof(BatchProb); }
size_t batch_prep_bytes() { return sizeof(BatchPrep); }

void fill_batch_prob(void* dst, const void* codes, const void* scales, const float* bias, float* y, const void* afrag,
                     int64_t N, int64_t K, int64_t tile0) {
    BatchProb p;
    p.codes = static_cast<const uint8_t*>(codes);
    p.scales = static_cast<const uint16_t*>(scales);
    p.bias = bias;
    p.y = y;
    p.afrag = static_cast<const i32x4*>(afrag);
    p.N = N;
    p.K = K;
    p.tile0 = tile0;
    *static_cast<BatchProb*>(dst) = p;
}

void fill_batch_prep(void* dst, const float* x, void* afrag, int64_t K, int64_t ent0) {
    BatchPrep p;
    p.x = x;
    p.afrag = static_cast<i32x4*>(afrag);
    p.K = K;
    p.ent0 = ent0;
    *static_cast<BatchPrep*>(dst) = p;
}

hipError_t launch_gemv_f32_batch_prep(const void* prep_table, int nprep, int fmt, int64_t M, int64_t entries,
                                      hipStream_t stream) {
    if (entries > 0)
        hipLaunchKernelGGL(prep_batch_kernel, dim3(unsigned((entries + 255) / 256)), dim3(256), 0, stream,
                           static_cast<const BatchPrep*>(prep_table), nprep, int(M), fmt, entries);
    return hipGetLastError();
}

hipError_t launch_gemv_f32_batch_product(const void* prob_table, int count, int fmt, int64_t M, int64_t tiles,
                                         hipStream_t stream) {
    if (fmt == 1) launch_batch_product<1>(prob_table, count, int(M), tiles, stream);
    else launch_batch_product<2>(prob_table, count, int(M), tiles, stream);
    return hipGetLastError();
}

}  // namespace llk
