// Decode product with fp32 activations, 1 <= M <= 3, i2_s or TQ2_0, on the
// int8 matrix cores with exact integer accumulation.
//
// Activation split.  Each token row x is written as
//     x = 2^(E-6) * sum_{p=0..4} q_p * 128^-p  +  r,
// where 2^(E-1) <= max|x| < 2^E, q_p are int8 (|q_p| <= 64) and
// |r| <= 2^(E-41): r0 = x * 2^(6-E), q_p = rint(r_p), r_(p+1) = 128 (r_p - q_p),
// every step exact in fp32.  The planes are rows of the MFMA operand A.
// Weights.  Codes are fed as int8 c = w + 1 in {0, 1, 2} (i2_s codes as they
// are; TQ2_0 codes c' = w mod 4 remapped by c = ((b0 ^ b1) << 1) | !b0 on the
// packed word), so sum w*q = sum c*q - sum q, with the plane sums sum q
// computed once per token.  Every product and sum is an exact integer in
// int32; the epilogue forms
//     y = scale * 2^(E-6) * sum_p 128^-p (acc_p - xsum_p)
// in fp64 (exact up to the final roundings), so the only deviation from the
// exact product is the plane truncation r: |y - y_exact| <=
// scale * K * 2^-41 * max|x|, far inside 1e-5 * scale * sum|x|.
//
// Memory.  v_mfma_i32_16x16x64_i8: a lane's 16 code bytes hold, in each of
// their four 2-bit fields, 16 codes that are consecutive in k for i2_s (the
// group layout puts elements r..r+15 of one shift plane in consecutive
// bytes), so the activation operand is 16 consecutive plane bytes; for
// TQ2_0 the preparation kernel stores the planes in the matching permuted
// order.  Weight rows are fetched per 1024-k window with loads of 4 rows x
// 256 contiguous bytes (long runs the memory system serves at full speed,
// unlike the 16-rows-by-64-bytes shape of the operand) and transposed
// through padded LDS rows; the window's activation planes are staged in LDS
// too.  Loads run two windows ahead of the multiply (registers hold the
// next-but-one window, LDS the next one).  A prepared batch runs many
// products per launch.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int kP = 5;                     // activation planes
constexpr int kWaves = 4;                 // 16-row tiles per workgroup
constexpr int kRows = 16 * kWaves;
constexpr int kWinK = 1024;               // k per window
constexpr int kWinB = kWinK / 4;          // code bytes per row per window
constexpr int kWStride = kWinB + 16;      // padded LDS weight row
constexpr int kWTile = 16 * kWStride;
constexpr int kAStride = kWinK + 16;      // padded LDS plane row
constexpr int kAChunks = 4;               // 16-byte plane chunks per thread per window (<= 1024 / 256)

__host__ __device__ inline int lds_bytes(int M) { return 2 * kWaves * kWTile + 2 * kP * M * kAStride + 64; }

// Position of element k inside its 256-element TQ2_0 block in the plane
// layout: field f = k%4 of byte 16q + 4v + b (k = 64q + 16v + 4b + f) goes to
// 64f + 16q + 4v + b, so one MFMA (one field) reads 16 consecutive bytes.
__device__ __forceinline__ int tq2_pos(int e) { return 64 * (e & 3) + 16 * (e >> 6) + 4 * ((e >> 4) & 3) + ((e >> 2) & 3); }

// Workspace layout of one activation: planes [5M][K] | xsum [5M][nblk] | E [M].
struct PlaneView {
    int8_t* planes;
    int32_t* xsum;
    int32_t* ex;
};
__host__ __device__ inline size_t planes_bytes(int64_t M, int64_t K) {
    const int64_t nblk = (K + 255) / 256;
    return size_t((kP * M * K + 15) / 16 * 16 + kP * M * nblk * 4 + M * 4 + 15) / 16 * 16;
}
__host__ __device__ inline PlaneView plane_view(void* base, int64_t M, int64_t K) {
    const int64_t nblk = (K + 255) / 256;
    char* p = static_cast<char*>(base);
    PlaneView v;
    v.planes = reinterpret_cast<int8_t*>(p);
    v.xsum = reinterpret_cast<int32_t*>(p + (kP * M * K + 15) / 16 * 16);
    v.ex = v.xsum + kP * M * nblk;
    return v;
}

// ---------------------------------------------------------------- activation preparation
// One workgroup of 256 threads per (256-k block, token): the row maximum
// (every workgroup of the token reads the whole row, from L2), then the five
// planes of its block and their sums.
template <int FMT>
__device__ __forceinline__ void prep_block(const float* __restrict__ xr, int64_t K, int M, int m, int64_t b,
                                           void* __restrict__ ws) {
    __shared__ float smax[4];
    __shared__ int ssum[4][kP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const PlaneView v = plane_view(ws, M, K);
    const int64_t nblk = (K + 255) / 256;
    float a = 0.0f;
    for (int64_t k = tid; k < K; k += 256) a = fmaxf(a, fabsf(xr[k]));
    a = wave_max(a);
    if (lane == 0) smax[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    int E = 0;
    if (a > 0.0f) (void)frexpf(a, &E);            // 2^(E-1) <= a < 2^E
    if (b == 0 && tid == 0) v.ex[m] = E;
    const int64_t k = 256 * b + tid;
    float r = (k < K && a > 0.0f) ? ldexpf(xr[k], 6 - E) : 0.0f;
    int q[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
        const float qp = __builtin_rintf(r);
        q[p] = int(qp);
        r = __fmul_rn(__fsub_rn(r, qp), 128.0f);
    }
    if (k < K) {
        const int64_t pos = FMT == 2 ? 256 * b + tq2_pos(tid) : k;
#pragma unroll
        for (int p = 0; p < kP; ++p) v.planes[int64_t(m * kP + p) * K + pos] = int8_t(q[p]);
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) {
        int s = q[p];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (lane == 0) ssum[wave][p] = s;
    }
    __syncthreads();
    if (tid < kP) v.xsum[int64_t(m * kP + tid) * nblk + b] = ssum[0][tid] + ssum[1][tid] + ssum[2][tid] + ssum[3][tid];
}

template <int FMT>
__global__ void __launch_bounds__(256) prep_planes_kernel(const float* __restrict__ x, int64_t K, int M,
                                                          void* __restrict__ ws) {
    const int64_t b = blockIdx.x;
    const int m = blockIdx.y;
    prep_block<FMT>(x + int64_t(m) * K, K, M, m, b, ws);
}

// ---------------------------------------------------------------- product
template <int FMT>
__device__ __forceinline__ void planes_rows(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                            int64_t N, int64_t K, const void* __restrict__ ws, int M,
                                            const float* __restrict__ bias, float* __restrict__ y, int64_t n0,
                                            char* __restrict__ lds) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nl = lane & 15, q = lane >> 4;
    const int RR = kP * M;                              // plane rows in use (<= 15)
    const uint32_t rowbytes = uint32_t(K / 4);
    const int nwin = int((K + kWinK - 1) / kWinK);
    const int nblk = int((K + 255) / 256);
    const PlaneView pv = plane_view(const_cast<void*>(ws), M, K);
    char* wbuf = lds;
    int8_t* abuf = reinterpret_cast<int8_t*>(lds + 2 * kWaves * kWTile);
    const int abytes = RR * kAStride;
    int* xtot = reinterpret_cast<int*>(abuf + 2 * abytes);   // [RR] total plane sums (i2_s)

    // loads of this lane: row 4i + q of the wave's tile, 16-byte chunk nl of each window
    const uint8_t* lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t n = n0 + 16 * wave + 4 * i + q;
        n = n < N ? n : N - 1;
        lrow[i] = codes + n * int64_t(rowbytes) + 16 * nl;
    }
    int64_t orow = n0 + 16 * wave + nl;
    orow = orow < N ? orow : N - 1;
    const uint16_t* srow = FMT == 2 ? scales + orow * (K / 256) : nullptr;

    struct Regs {
        i32x4 w[4];
        i32x4 a[kAChunks];
    };
    auto load = [&](int w, Regs& r) {
        const uint32_t off = uint32_t(w) * kWinB + 16 * nl;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.w[i] = (off < rowbytes) ? ld16_stream(lrow[i] + uint32_t(w) * kWinB) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 6, col = c & 63;
            const int64_t k = int64_t(w) * kWinK + 16 * col;
            r.a[i] = (row < RR && k < K) ? ld16(pv.planes + int64_t(row) * K + k) : i32x4{0, 0, 0, 0};
        }
    };
    auto store = [&](int buf, const Regs& r) {
        char* base = wbuf + (buf * kWaves + wave) * kWTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(base + (4 * i + q) * kWStride + 16 * nl) = r.w[i];
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 6, col = c & 63;
            if (row < RR) *reinterpret_cast<i32x4*>(abuf + buf * abytes + row * kAStride + 16 * col) = r.a[i];
        }
    };

    i32x4 acc = {0, 0, 0, 0};
    double dacc[4] = {0.0, 0.0, 0.0, 0.0};               // TQ2_0: block-scaled sums per plane row

    auto compute = [&](int w) {
        const int cur = w & 1;
        const char* wb = wbuf + (cur * kWaves + wave) * kWTile + nl * kWStride + 16 * q;
        const int8_t* ab = abuf + cur * abytes + nl * kAStride;
#pragma unroll
        for (int seg = 0; seg < 4; ++seg) {
            const int s = 4 * w + seg;                     // 256-k segment (= TQ2_0 block)
            if (uint32_t(64 * s) >= rowbytes) break;
            i32x4 u = *reinterpret_cast<const i32x4*>(wb + 64 * seg);
            if (FMT == 2) {
                // c = ((b0 ^ b1) << 1) | !b0 turns the two's-complement field w into w + 1
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t v = uint32_t(u[j]);
                    u[j] = int((v ^ ((v & 0x55555555u) << 1)) ^ 0x55555555u);
                }
            }
            i32x4 bacc = (FMT == 2) ? i32x4{0, 0, 0, 0} : acc;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // i2_s: MFMA t takes shift 6-2t (elements 32t..32t+31 of each group);
                // TQ2_0: field t; the operand offsets follow the plane layout.
                const int sh = FMT == 1 ? 6 - 2 * t : 2 * t;
                i32x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = int((uint32_t(u[j]) >> sh) & 0x03030303u);
                i32x4 a = {0, 0, 0, 0};
                const int aoff = FMT == 1 ? 256 * seg + 128 * (q >> 1) + 32 * t + 16 * (q & 1)
                                          : 256 * seg + 64 * t + 16 * q;
                if (nl < RR) a = *reinterpret_cast<const i32x4*>(ab + aoff);
                bacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, bacc, 0, 0, 0);
            }
            if (FMT == 2) {
                // C lane (column nl, quarter q) holds plane rows 4q..4q+3
                const double sc = double(half_bits_to_float(srow[s]));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * q + r;
                    const int xs = row < RR ? ld32(pv.xsum + row * nblk + s) : 0;
                    dacc[r] = __builtin_fma(sc, double(bacc[r] - xs), dacc[r]);
                }
            } else {
                acc = bacc;
            }
        }
    };

    // total plane sums for i2_s, once per workgroup
    if (FMT == 1 && tid < RR) {
        int s = 0;
        for (int b = 0; b < nblk; ++b) s += ld32(pv.xsum + tid * nblk + b);
        xtot[tid] = s;
    }

    Regs r0, r1;
    load(0, r0);
    if (nwin > 1) load(1, r1);
    store(0, r0);
    __syncthreads();
    // window w is multiplied from LDS buffer w%2 while window w+1 waits in
    // registers and window w+2 is being fetched
    for (int w = 0; w < nwin; w += 2) {
        if (w + 2 < nwin) load(w + 2, r0);
        compute(w);
        if (w + 1 < nwin) store((w + 1) & 1, r1);
        __syncthreads();
        if (w + 1 >= nwin) break;
        if (w + 3 < nwin) load(w + 3, r1);
        compute(w + 1);
        if (w + 2 < nwin) store((w + 2) & 1, r0);
        __syncthreads();
    }

    // per plane row: D_row = (i2_s) acc - total plane sum, or (TQ2_0) the
    // block-scaled sum; then y = f * 2^(E-6) * sum_p 128^-p D_(5m+p)
    double d[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (FMT == 1) d[r] = double(acc[r] - (row < RR ? xtot[row] : 0));
        else d[r] = dacc[r];
    }
    const double f = FMT == 1 ? double(*(const __attribute__((address_space(1))) float*)(
                                    codes + N * int64_t(rowbytes)))
                              : 1.0;
    const int64_t n = n0 + 16 * wave + nl;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        if (m >= M) break;
        double v = 0.0;
#pragma unroll
        for (int p = kP - 1; p >= 0; --p) {
            const int row = kP * m + p;
            const double part = __shfl(d[row & 3], nl + 16 * (row >> 2), 64);
            v = __builtin_fma(v, 1.0 / 128.0, part);     // Horner in 1/128: exact for these integers
        }
        if (q == 0 && n < N) {
            const int E = ld32(pv.ex + m);
            float out = float(f * ldexp(v, E - 6));
            if (bias) out = __fadd_rn(out, bias[n]);
            y[int64_t(m) * N + n] = out;
        }
    }
}

template <int FMT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_kernel(const uint8_t* __restrict__ codes,
                                                                   const uint16_t* __restrict__ scales, int64_t N,
                                                                   int64_t K, const void* __restrict__ ws, int M,
                                                                   const float* __restrict__ bias,
                                                                   float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    planes_rows<FMT>(codes, scales, N, K, ws, M, bias, y, int64_t(blockIdx.x) * kRows, lds);
}

struct PlanesProb {          // product of a prepared batch
    const uint8_t* codes;
    const uint16_t* scales;
    const void* ws;          // prepared planes of its activation
    const float* bias;
    float* y;
    int64_t N, K;
    int64_t wg0;             // first workgroup
};
struct PlanesPrep {          // distinct activation of a prepared batch
    const float* x;
    void* ws;
    int64_t K;
    int64_t wg0;             // first preparation workgroup (one per 256-k block and token)
};

template <typename T>
__device__ __forceinline__ int find_wg(const T* __restrict__ tab, int count, int64_t wg) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid].wg0 <= wg) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int FMT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_batch_kernel(const PlanesProb* __restrict__ tab, int count,
                                                                         int M) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t wg = blockIdx.x;
    const PlanesProb& P = tab[find_wg(tab, count, wg)];
    planes_rows<FMT>(P.codes, P.scales, P.N, P.K, P.ws, M, P.bias, P.y, (wg - P.wg0) * kRows, lds);
}

template <int FMT>
__global__ void __launch_bounds__(256) prep_planes_batch_kernel(const PlanesPrep* __restrict__ tab, int count, int M) {
    const int64_t wg = blockIdx.x;
    const PlanesPrep& P = tab[find_wg(tab, count, wg)];
    const int64_t nblk = (P.K + 255) / 256;
    const int64_t local = wg - P.wg0;
    const int m = int(local / nblk);
    prep_block<FMT>(P.x + int64_t(m) * P.K, P.K, M, m, local % nblk, P.ws);
}

template <typename F>
hipError_t allow_lds(F* kernel, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

}  // namespace

namespace llk {

size_t planes_workspace(int64_t M, int64_t K) { return planes_bytes(M, K); }
int64_t planes_batch_rows() { return kRows; }
size_t planes_prob_bytes() { return sizeof(PlanesProb); }
size_t planes_prep_bytes() { return sizeof(PlanesPrep); }
int64_t planes_prep_wgs(int64_t M, int64_t K) { return M * ((K + 255) / 256); }

void fill_planes_prob(void* dst, const void* codes, const void* scales, const void* ws, const float* bias, float* y,
                      int64_t N, int64_t K, int64_t wg0) {
    PlanesProb p;
    p.codes = static_cast<const uint8_t*>(codes);
    p.scales = static_cast<const uint16_t*>(scales);
    p.ws = ws;
    p.bias = bias;
    p.y = y;
    p.N = N;
    p.K = K;
    p.wg0 = wg0;
    *static_cast<PlanesProb*>(dst) = p;
}

void fill_planes_prep(void* dst, const float* x, void* ws, int64_t K, int64_t wg0) {
    PlanesPrep p;
    p.x = x;
    p.ws = ws;
    p.K = K;
    p.wg0 = wg0;
    *static_cast<PlanesPrep*>(dst) = p;
}

hipError_t launch_gemv_planes(int fmt, const void* codes, const void* scales, int64_t N, int64_t K, const float* x,
                              int64_t M, const float* bias, float* y, void* ws, hipStream_t stream) {
    const dim3 pgrid{unsigned((K + 255) / 256), unsigned(M)}, pblock{256};
    const dim3 grid{unsigned((N + kRows - 1) / kRows)}, block{64 * kWaves};
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    const uint16_t* s = static_cast<const uint16_t*>(scales);
    const size_t lds = size_t(lds_bytes(int(M)));
    hipError_t e;
    if (fmt == 1) {
        hipLaunchKernelGGL(prep_planes_kernel<1>, pgrid, pblock, 0, stream, x, K, int(M), ws);
        if ((e = allow_lds(gemv_planes_kernel<1>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(gemv_planes_kernel<1>, grid, block, lds, stream, c, s, N, K, ws, int(M), bias, y);
    } else {
        hipLaunchKernelGGL(prep_planes_kernel<2>, pgrid, pblock, 0, stream, x, K, int(M), ws);
        if ((e = allow_lds(gemv_planes_kernel<2>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(gemv_planes_kernel<2>, grid, block, lds, stream, c, s, N, K, ws, int(M), bias, y);
    }
    return hipGetLastError();
}

hipError_t launch_planes_batch_prep(const void* prep_table, int nprep, int fmt, int64_t M, int64_t wgs,
                                    hipStream_t stream) {
    const dim3 grid{unsigned(wgs)}, block{256};
    const PlanesPrep* tab = static_cast<const PlanesPrep*>(prep_table);
    if (fmt == 1) hipLaunchKernelGGL(prep_planes_batch_kernel<1>, grid, block, 0, stream, tab, nprep, int(M));
    else hipLaunchKernelGGL(prep_planes_batch_kernel<2>, grid, block, 0, stream, tab, nprep, int(M));
    return hipGetLastError();
}

hipError_t launch_planes_batch_product(const void* prob_table, int count, int fmt, int64_t M, int64_t wgs,
                                       hipStream_t stream) {
    const dim3 grid{unsigned(wgs)}, block{64 * kWaves};
    const PlanesProb* tab = static_cast<const PlanesProb*>(prob_table);
    const size_t lds = size_t(lds_bytes(int(M)));
    hipError_t e;
    if (fmt == 1) {
        if ((e = allow_lds(gemv_planes_batch_kernel<1>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(gemv_planes_batch_kernel<1>, grid, block, lds, stream, tab, count, int(M));
    } else {
        if ((e = allow_lds(gemv_planes_batch_kernel<2>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(gemv_planes_batch_kernel<2>, grid, block, lds, stream, tab, count, int(M));
    }
    return hipGetLastError();
}

}  // namespace llk
