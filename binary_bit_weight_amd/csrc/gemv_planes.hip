// Decode product with fp32 activations, 1 <= M <= 16 (passes of up to three
// tokens), i2_s or TQ2_0, on the int8 matrix cores with exact integer
// accumulation.  Single calls and M >= 2; a prepared batch of one token runs
// on the fp4 digit-plane engine instead.  The same product serves int8
// activations (one plane per token, all M <= 16 tokens in one pass, see
// kInt8 below).
//
// Activation split.  Each token row x is written as
//     x = 2^(E-6) * sum_{p=0..4} q_p * 128^-p  +  r,
// where 2^(E-1) <= max|x| < 2^E, q_p are int8 (|q_p| <= 64) and
// |r| <= 2^(E-41): r0 = x * 2^(6-E), q_p = rint(r_p), r_(p+1) = 128 (r_p - q_p),
// every step exact in fp32.  The planes are rows of the MFMA operand A.
// Weights.  Codes are fed as c = w + 1 in {0, 1, 2} (i2_s codes as they are;
// TQ2_0 codes c' = w mod 4 remapped by c = ((b0 ^ b1) << 1) | !b0 on the
// packed word), so sum w*q = sum c*q - sum q.  i2_s: the plane sums sum q
// come once per token from the preparation; a code is not shifted down to
// bit 0 of its byte: masked in place it is the int8 value c * 4^j (j < 3), so
// three of the four fields of a word cost one AND each; the MFMAs of each
// field accumulate separately over the row and are divided by their exact
// power of two at the end.  TQ2_0: every field is moved to bits 4..5 (the
// value 16 c), so the four MFMAs of a 256-k block chain into one
// accumulator, and the block's plane sums come from four more MFMAs against
// an all-ones operand; the fp64 block scale takes the factor 1/16.  Every
// product and sum is an exact integer in int32; the epilogue forms
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
// through a padded LDS tile private to the wave; the window's activation
// planes are staged in a shared, double-buffered LDS window, the only thing
// the workgroup synchronises on.  Loads run two windows ahead of the
// multiply.  A prepared batch runs many products per launch.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

#ifndef LL_PLANES_WAVES
#define LL_PLANES_WAVES 4
#endif
#ifndef LL_PLANES_WINK
#define LL_PLANES_WINK 1024
#endif
#ifndef LL_PLANES_NT
#define LL_PLANES_NT 1
#endif
#ifndef LL_PLANES_DUMMY
#define LL_PLANES_DUMMY 0
#endif

constexpr int kP = 5;                     // activation planes
constexpr int kWaves = LL_PLANES_WAVES;   // 16-row tiles per workgroup
constexpr int kRows = 16 * kWaves;
constexpr int kWinK = LL_PLANES_WINK;     // k per window
constexpr int kWinB = kWinK / 4;          // code bytes per row per window
constexpr int kWStride = kWinB + 16;      // padded LDS weight row
constexpr int kWTile = 16 * kWStride;     // one wave's weight tile
constexpr int kAStride = kWinK + 16;      // padded LDS plane row

__host__ __device__ inline int lds_bytes(int M) { return kWaves * kWTile + 2 * kP * M * kAStride; }

// Fused form of a single product (M = 1, K <= kFusedMaxK): every workgroup
// builds the planes of the whole row in its LDS (no preparation launch), then
// multiplies with no workgroup barrier.  It halves the latency of one call;
// in a prepared batch the repeated preparation and the larger LDS cost more
// than the launch it saves, so batches keep the preparation kernel.
// LDS: weight tiles | planes [5][astride] | sums | max.
#ifndef LL_PLANES_FUSED
#define LL_PLANES_FUSED 1
#endif
constexpr int kThreads = 64 * kWaves;
constexpr int64_t kFusedMaxK = LL_PLANES_FUSED ? 8192 : 0;
constexpr int kXIt = 8192 / (4 * kThreads);          // float4 of x per thread
__host__ __device__ inline int fused_astride(int64_t K) { return int((K + 255) / 256 * 256 + 16); }
// i2_s: each wave's plane sums (TQ2_0 forms its block sums in the product)
__host__ __device__ inline int fused_sums(int64_t K) {
    (void)K;
    return kWaves * kP;
}
__host__ __device__ inline int fused_lds_bytes(int64_t K) {
    return kWaves * kWTile + kP * fused_astride(K) + 4 * fused_sums(K) + 4 * kWaves;
}

// TQ2_0 plane layout: element 4m + f of a 256-element block (field f of
// code byte m) goes to byte 64 f + m of the block, so one MFMA (one field)
// reads 16 consecutive bytes.

// The product multiplies up to kPassM tokens at a time (5 x 3 = 15 plane
// rows fill one 16-row MFMA operand); larger M runs several passes.
constexpr int kPassM = 3;
__host__ __device__ inline int64_t npass(int64_t M) { return (M + kPassM - 1) / kPassM; }

// Workspace layout of one activation:
//     planes [5M][K] | E [M] | xtot [5M] (i2_s: each plane row's sum over
// the row).  TQ2_0's per-block plane sums are formed by the product itself
// (MFMAs against an all-ones operand).
struct PlaneView {
    int8_t* planes;
    int32_t* ex;
    int32_t* xtot;
};
__host__ __device__ inline size_t planes_bytes(int64_t M, int64_t K) {
    return size_t((kP * M * K + 15) / 16 * 16 + M * 4 + kP * M * 4 + 15) / 16 * 16;
}
__host__ __device__ inline PlaneView plane_view(const void* base, int64_t M, int64_t K) {
    char* p = static_cast<char*>(const_cast<void*>(base));
    PlaneView v;
    v.planes = reinterpret_cast<int8_t*>(p);
    v.ex = reinterpret_cast<int32_t*>(p + (kP * M * K + 15) / 16 * 16);
    v.xtot = v.ex + M;
    return v;
}
// The view of pass `pass` (tokens 3 pass .. 3 pass + 2) of a full view.
__host__ __device__ inline PlaneView pass_view(const PlaneView& v, int pass, int64_t K) {
    PlaneView u;
    u.planes = v.planes + int64_t(kP * kPassM) * pass * K;
    u.ex = v.ex + kPassM * pass;
    u.xtot = v.xtot + kP * kPassM * pass;
    return u;
}

// ---------------------------------------------------------------- activation preparation
// One workgroup of 256 threads per token; float4 loads, all issued before
// any use.  i2_s: thread t holds elements 4t + 1024i + [0, 4) and sums its
// digits per plane (one wave reduction per plane at the end).  TQ2_0: each
// thread holds 16 consecutive elements per four float4s, so its digits of
// one field are four consecutive bytes of the block's transposed layout (one
// dword store per plane and field).  The row maximum costs one barrier.
// Rows are processed in chunks of kPrepK elements (registers), the maximum
// over all chunks first.
constexpr int kPrepIt = 8;                           // float4 per thread per chunk
constexpr int kPrepK = 1024 * kPrepIt;               // elements per chunk

template <int FMT>
__device__ __forceinline__ void prep_token(const float* __restrict__ xr, int64_t K, int M, int m,
                                           void* __restrict__ ws) {
    __shared__ float smax[4];
    __shared__ int stot[4][kP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const PlaneView v = plane_view(ws, M, K);
    int tot[kP] = {0, 0, 0, 0, 0};                   // i2_s: this thread's share of the row's plane sums
    // first element of float4 i of a chunk
    auto kof = [&](int64_t k0, int i) -> int64_t {
        return FMT == 1 ? k0 + 1024 * i + 4 * tid : k0 + 4096 * (i / 4) + 16 * tid + 4 * (i % 4);
    };
    // K % 128 == 0 (both formats; TQ2_0: % 256), so k < K implies k + 3 < K.
    // (A scalar fallback here would turn these into FLAT loads, each waiting
    // for the previous one.)
    auto load_chunk = [&](int64_t k0, f32x4 (&x4)[kPrepIt]) {
#pragma unroll
        for (int i = 0; i < kPrepIt; ++i) {
            const int64_t k = kof(k0, i);
            x4[i] = k < K ? ld16f(xr + k) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    float a = 0.0f;
    f32x4 xfirst[kPrepIt];                           // the first chunk stays in registers
    for (int64_t k0 = 0; k0 < K; k0 += kPrepK) {
        f32x4 x4[kPrepIt];
        load_chunk(k0, x4);
#pragma unroll
        for (int i = 0; i < kPrepIt; ++i) {
            a = fmaxf(fmaxf(a, fmaxf(fabsf(x4[i].x), fabsf(x4[i].y))), fmaxf(fabsf(x4[i].z), fabsf(x4[i].w)));
            if (k0 == 0) xfirst[i] = x4[i];
        }
    }
    a = wave_max(a);
    if (lane == 0) smax[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    int E = 0;
    if (a > 0.0f) (void)frexpf(a, &E);            // 2^(E-1) <= a < 2^E
    if (tid == 0) v.ex[m] = E;
    for (int64_t k0 = 0; k0 < K; k0 += kPrepK) {
        f32x4 x4[kPrepIt];
        if (k0 == 0) {
#pragma unroll
            for (int i = 0; i < kPrepIt; ++i) x4[i] = xfirst[i];
        } else {
            load_chunk(k0, x4);                      // L2-resident re-read
        }
        if constexpr (FMT == 2) {
            // element 4m + f of a 256-k block goes to byte 64 f + m of its plane row
#pragma unroll
            for (int g = 0; g < kPrepIt / 4; ++g) {
                const int64_t kg = kof(k0, 4 * g);
                if (kg >= K) break;
                uint32_t d[kP][4] = {};              // plane p, field f: four digits
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv[4] = {x4[4 * g + i].x, x4[4 * g + i].y, x4[4 * g + i].z, x4[4 * g + i].w};
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        float r = a > 0.0f ? ldexpf(xv[f], 6 - E) : 0.0f;
#pragma unroll
                        for (int p = 0; p < kP; ++p) {
                            const float qp = __builtin_rintf(r);
                            d[p][f] |= uint32_t(uint8_t(int(qp))) << (8 * i);
                            r = __fmul_rn(__fsub_rn(r, qp), 128.0f);
                        }
                    }
                }
                const int64_t base = kg - (kg & 255) + ((kg & 255) >> 2);
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    int8_t* row = v.planes + int64_t(m * kP + p) * K;
#pragma unroll
                    for (int f = 0; f < 4; ++f) *reinterpret_cast<uint32_t*>(row + base + 64 * f) = d[p][f];
                }
            }
            continue;
        }
#pragma unroll
        for (int i = 0; i < kPrepIt; ++i) {
            const int64_t kb = k0 + 1024 * i;
            if (kb >= K) break;
            const int64_t k = kb + 4 * tid;
            const float xv[4] = {x4[i].x, x4[i].y, x4[i].z, x4[i].w};
            int q[4][kP];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float r = a > 0.0f ? ldexpf(xv[j], 6 - E) : 0.0f;
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    const float qp = __builtin_rintf(r);
                    q[j][p] = int(qp);
                    r = __fmul_rn(__fsub_rn(r, qp), 128.0f);
                }
            }
            if (k < K) {
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    int8_t* row = v.planes + int64_t(m * kP + p) * K;
                    const uint32_t packed = uint32_t(uint8_t(q[0][p])) | uint32_t(uint8_t(q[1][p])) << 8 |
                                            uint32_t(uint8_t(q[2][p])) << 16 | uint32_t(uint8_t(q[3][p])) << 24;
                    *reinterpret_cast<uint32_t*>(row + k) = packed;
                }
            }
#pragma unroll
            for (int p = 0; p < kP; ++p) tot[p] += (q[0][p] + q[1][p]) + (q[2][p] + q[3][p]);
        }
    }
    if constexpr (FMT == 1) {
        wave_sum_n(tot);
        if (lane == 0)
#pragma unroll
            for (int p = 0; p < kP; ++p) stot[wave][p] = tot[p];
        __syncthreads();
        if (tid < kP) v.xtot[m * kP + tid] = stot[0][tid] + stot[1][tid] + stot[2][tid] + stot[3][tid];
    }
}

template <int FMT>
__global__ void __launch_bounds__(256) prep_planes_kernel(const float* __restrict__ x, int64_t K, int M,
                                                          void* __restrict__ ws) {
    const int m = blockIdx.x;
    prep_token<FMT>(x + int64_t(m) * K, K, M, m, ws);
}

// Fused preparation of one token row inside the product workgroup (same
// split as above).  With T threads, thread t holds x[4t + 4Ti + (0..3)], so
// 256-k block (T/64)i + wave belongs to one wave.  Writes planes [5][astride]
// into A and the plane sums into sums: TQ2_0 per block [5][nblk], i2_s per
// wave [waves][5].
// Returns E; contains one workgroup barrier (the row maximum); the caller's
// next barrier publishes A and sums.
template <int FMT>
__device__ __forceinline__ int fused_prep(const float* __restrict__ x, int64_t K, int8_t* __restrict__ A, int astride,
                                          int* __restrict__ sums, float* __restrict__ smax) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // float4 i of this thread: elements k(i) .. k(i) + 3; i2_s: k(i) = 1024 i
    // + 4 tid; TQ2_0: 16 consecutive elements per thread and four float4s,
    // k(i) = 4096 (i / 4) + 16 tid + 4 (i % 4), so a thread's digits of one
    // field are four consecutive bytes of the block's transposed layout
    auto kof = [&](int i) -> int64_t {
        return FMT == 1 ? int64_t(4 * kThreads * i + 4 * tid) : int64_t(16 * kThreads * (i / 4) + 16 * tid + 4 * (i % 4));
    };
    f32x4 xv[kXIt];
#pragma unroll
    for (int i = 0; i < kXIt; ++i) {
        const int64_t k = kof(i);                      // K % 128 == 0: k < K implies k + 3 < K
        xv[i] = k < K ? ld16f(x + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kXIt; ++i)
        a = fmaxf(fmaxf(a, fmaxf(fabsf(xv[i].x), fabsf(xv[i].y))), fmaxf(fabsf(xv[i].z), fabsf(xv[i].w)));
    a = wave_max(a);
    if (lane == 0) smax[wave] = a;
    __syncthreads();
    a = smax[0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) a = fmaxf(a, smax[v]);
    int E = 0;
    if (a > 0.0f) (void)frexpf(a, &E);                // 2^(E-1) <= a < 2^E
    if constexpr (FMT == 2) {
        // element 4m + f of a 256-k block goes to byte 64 f + m of its plane
        // row; the block sums of the planes are formed by the product
#pragma unroll
        for (int g = 0; g < kXIt / 4; ++g) {
            const int64_t k0 = kof(4 * g);
            if (k0 >= K) break;
            uint32_t d[kP][4] = {};                    // plane p, field f: four digits
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xe[4] = {xv[4 * g + i].x, xv[4 * g + i].y, xv[4 * g + i].z, xv[4 * g + i].w};
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    float r = a > 0.0f ? ldexpf(xe[f], 6 - E) : 0.0f;
#pragma unroll
                    for (int p = 0; p < kP; ++p) {
                        const float qp = __builtin_rintf(r);
                        d[p][f] |= uint32_t(uint8_t(int(qp))) << (8 * i);
                        r = __fmul_rn(__fsub_rn(r, qp), 128.0f);
                    }
                }
            }
            const int m0 = int(k0 & 255) >> 2;            // 4-element index of the thread's first element
#pragma unroll
            for (int p = 0; p < kP; ++p)
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    *reinterpret_cast<uint32_t*>(A + p * astride + (k0 & ~int64_t(255)) + 64 * f + m0) = d[p][f];
        }
        (void)sums;
        return E;
    }
    int tot[kP] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kXIt; ++i) {
        const int64_t kb = 4 * kThreads * i;
        if (kb >= K) break;
        const int k = int(kb) + 4 * tid;
        const float xe[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        int q[4][kP];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = a > 0.0f ? ldexpf(xe[j], 6 - E) : 0.0f;
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                const float qp = __builtin_rintf(r);
                q[j][p] = int(qp);
                r = __fmul_rn(__fsub_rn(r, qp), 128.0f);
            }
        }
        if (k < K) {
#pragma unroll
            for (int p = 0; p < kP; ++p)
                *reinterpret_cast<uint32_t*>(A + p * astride + k) =
                    uint32_t(uint8_t(q[0][p])) | uint32_t(uint8_t(q[1][p])) << 8 |
                    uint32_t(uint8_t(q[2][p])) << 16 | uint32_t(uint8_t(q[3][p])) << 24;
        }
#pragma unroll
        for (int p = 0; p < kP; ++p) tot[p] += (q[0][p] + q[1][p]) + (q[2][p] + q[3][p]);
    }
    wave_sum_n(tot);
#pragma unroll
    for (int p = 0; p < kP; ++p)
        if (lane == 0) sums[wave * kP + p] = tot[p];
    return E;
}

// ---------------------------------------------------------------- product
// Field j of a code byte, masked in place: its int8 value is c * kFieldMul[j].
// i2_s MFMA t reads the field at bits 6-2t (elements 32t.. of each group);
// TQ2_0 MFMA t reads field t (bits 2t).
template <int FMT>
__device__ __forceinline__ uint32_t field(uint32_t u, int t) {
    const int bit = FMT == 1 ? 6 - 2 * t : 2 * t;
    if (bit == 6) return (u >> 2) & 0x30303030u;   // c * 16
    if (bit == 4) return u & 0x30303030u;          // c * 16
    if (bit == 2) return u & 0x0C0C0C0Cu;          // c * 4
    return u & 0x03030303u;                        // c
}
// TQ2_0 field t (bits 2t) moved to bits 4..5 of every byte: 16 c for all t,
// so the four steps of a 256-k block chain into one accumulator
__device__ __forceinline__ uint32_t field16(uint32_t u, int t) {
    if (t == 0) return (u << 4) & 0x30303030u;
    if (t == 1) return (u << 2) & 0x30303030u;
    if (t == 2) return u & 0x30303030u;
    return (u >> 2) & 0x30303030u;
}
template <int FMT>
__host__ __device__ constexpr int field_mul(int t) {
    return (FMT == 1 ? 6 - 2 * t : 2 * t) >= 4 ? 16 : ((FMT == 1 ? 6 - 2 * t : 2 * t) == 2 ? 4 : 1);
}

// Where the activation operand comes from.
//   kWindowed: prepared workspace, staged per window through a shared,
//              double-buffered LDS window (one workgroup barrier per window);
//   kFused:    the fp32 row x (M == 1), split into planes by the workgroup,
//              whole row in LDS, no barrier in the main loop.
//   kInt8:     int8 activations q with per-token scales (1 <= M <= 16): one
//              plane per token, read straight from the caller's [M][K] rows
//              and staged per window like kWindowed (TQ2_0 rows reordered
//              into the plane layout while being stored to LDS); the
//              per-token sums sum q come from extra MFMAs against an all-ones
//              operand, so nothing is prepared and there is one launch.
// (Copying a prepared row whole into LDS instead of windowing it was
// measured slower in batches: the larger LDS lowers occupancy more than
// the barriers cost.)
enum { kWindowed = 0, kFused = 1, kInt8 = 2 };

// ws: the fp32 token row (kFused); pvw: the prepared operands of these M <= 3
// tokens (kWindowed), or pvw.planes = the int8 rows [mrun][K] (kInt8, M the
// row capacity >= mrun, xs_tok the per-token scales).
template <int FMT, int M, int MODE>
__device__ __forceinline__ void planes_rows(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                            int64_t N, int64_t K, const void* __restrict__ ws, const PlaneView& pvw,
                                            const float* __restrict__ bias, float* __restrict__ y, int64_t n0,
                                            char* __restrict__ lds, const float* __restrict__ xs_tok = nullptr,
                                            int mrun = 0) {
    constexpr bool FUSED = MODE == kFused;
    constexpr bool INT8 = MODE == kInt8;
    constexpr bool WHOLE = FUSED;                      // whole plane row in LDS
    static_assert(!WHOLE || M == 1, "whole-row forms handle one token");
    constexpr int RR = (INT8 ? 1 : kP) * M;             // plane rows in use (<= 16)
    static_assert(RR <= 16, "one 16-row operand");
    const int rlast = (INT8 ? mrun : RR) - 1;           // last row present in memory
    constexpr int kAChunks = WHOLE ? 1 : (RR * (kWinK / 16) + 64 * kWaves - 1) / (64 * kWaves);   // plane chunks per thread
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nl = lane & 15, q = lane >> 4;
    const int arow = nl < RR ? nl : RR - 1;             // rows >= RR of the operand are never used
    const uint32_t rowbytes = uint32_t(K / 4);
    const int nwin = int((K + kWinK - 1) / kWinK);
    const int nblk = int((K + 255) / 256);
    const PlaneView pv = pvw;
    char* wtile = lds + wave * kWTile;                  // private to this wave
    int8_t* abuf = reinterpret_cast<int8_t*>(lds + kWaves * kWTile);
    constexpr int abytes = RR * kAStride;                // one window of plane rows
    const int astride = WHOLE ? fused_astride(K) : kAStride;
    int* fsums = reinterpret_cast<int*>(abuf + kP * fused_astride(K));           // fused only
    float* fsmax = reinterpret_cast<float*>(fsums + fused_sums(K));

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

    // Per window a wave loads its 16 rows x kWinB bytes as kLPR loads of
    // 4 rows x 256 bytes per row group; lane (q, nl) takes row 4i + q,
    // bytes 256j + 16nl of the window.
    constexpr int kLPR = kWinB / 256;
    constexpr int kAPerRow = kWinK / 16;                   // 16-byte plane chunks per plane row
    struct Regs {
        i32x4 w[4 * kLPR];
        i32x4 a[kAChunks];
        uint16_t sc[kWinK / 256];                          // TQ2_0: scales of this lane's row
    };
    uint16_t csc[kWinK / 256];                             // scales of the window being multiplied
    // Every load of a window is issued by every lane from an in-bounds
    // (clamped) address; chunks past the end of a row are zeroed when stored
    // to LDS.  (Lane-divergent branches around the loads made the compiler
    // wait for all outstanding loads before each LDS store.)  The prefetch of
    // a window past the last one is skipped with a uniform branch; issuing it
    // anyway on a few hot bytes (LL_PLANES_DUMMY=1) gives the compiler exact
    // wait counts, i.e. a full two-window prefetch, but measured slower on
    // the decode step (more requests in flight, no gain in bandwidth).
    // (kInt8: the first 16 bytes of the int8 rows, the only bytes every shape has)
    const uint8_t* dummy = INT8 ? reinterpret_cast<const uint8_t*>(pv.planes)
                                : (FUSED ? static_cast<const uint8_t*>(ws) : reinterpret_cast<const uint8_t*>(pv.planes)) + 16 * nl;
    auto load = [&](int w, Regs& r) {
        const bool live = w < nwin;
#pragma unroll
        for (int j = 0; j < kLPR; ++j) {
            const uint32_t off = uint32_t(w) * kWinB + 256 * j + 16 * nl;
            const uint32_t offc = off < rowbytes ? off : rowbytes - 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t* p = live ? lrow[i] - 16 * nl + offc : dummy;
                r.w[4 * j + i] = LL_PLANES_NT ? ld16_stream(p) : ld16(p);
            }
        }
        if constexpr (!WHOLE) {
#pragma unroll
            for (int i = 0; i < kAChunks; ++i) {
                const int c = tid + 64 * kWaves * i;
                const int row = c / kAPerRow, col = c % kAPerRow;
                const int64_t k = int64_t(w) * kWinK + 16 * col;
                r.a[i] = ld16(pv.planes + int64_t(row < rlast ? row : rlast) * K + (k < K ? k : K - 16));
            }
        }
        if (FMT == 2) {
#pragma unroll
            for (int t = 0; t < kWinK / 256; ++t) {
                const int b = (kWinK / 256) * w + t;
                r.sc[t] = ld2(srow + (b < nblk ? b : nblk - 1));
            }
        }
    };
    auto store_w = [&](int w, const Regs& r) {
        if (FMT == 2)
#pragma unroll
            for (int t = 0; t < kWinK / 256; ++t) csc[t] = r.sc[t];
#pragma unroll
        for (int j = 0; j < kLPR; ++j) {
            const bool ok = uint32_t(w) * kWinB + 256 * j + 16 * nl < rowbytes;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<i32x4*>(wtile + (4 * i + q) * kWStride + 256 * j + 16 * nl) =
                    ok ? r.w[4 * j + i] : i32x4{0, 0, 0, 0};
        }
    };
    auto store_a = [&](int w, const Regs& r) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + 64 * kWaves * i;
            const int row = c / kAPerRow, col = c % kAPerRow;
            const bool ok = int64_t(w) * kWinK + 16 * col < K;
            if (row >= RR) continue;
            const i32x4 v = ok ? r.a[i] : i32x4{0, 0, 0, 0};
            int8_t* dst = abuf + (w & 1) * abytes + row * kAStride;
            if (INT8 && FMT == 2) {
                // elements 16c + 4b + f of 256-k block (c = col % 16) go to the plane
                // layout's 64f + 4c + b: dword f gathers byte f of the chunk's four dwords
                const int base = 256 * (col >> 4) + 4 * (col & 15);
                const uint32_t d0 = uint32_t(v[0]), d1 = uint32_t(v[1]), d2 = uint32_t(v[2]), d3 = uint32_t(v[3]);
                const uint32_t x01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0.b0 d1.b0 d0.b1 d1.b1
                const uint32_t y01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0.b2 d1.b2 d0.b3 d1.b3
                const uint32_t x23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
                const uint32_t y23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
                *reinterpret_cast<uint32_t*>(dst + base) = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
                *reinterpret_cast<uint32_t*>(dst + base + 64) = __builtin_amdgcn_perm(x23, x01, 0x07060302u);
                *reinterpret_cast<uint32_t*>(dst + base + 128) = __builtin_amdgcn_perm(y23, y01, 0x05040100u);
                *reinterpret_cast<uint32_t*>(dst + base + 192) = __builtin_amdgcn_perm(y23, y01, 0x07060302u);
            } else {
                *reinterpret_cast<i32x4*>(dst + 16 * col) = v;
            }
        }
    };

    i32x4 acc[4];                                        // i2_s: one accumulator per field
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = i32x4{0, 0, 0, 0};
    i32x4 qsum = i32x4{0, 0, 0, 0};                      // kInt8, i2_s: sum q per row so far
    double dacc[4] = {0.0, 0.0, 0.0, 0.0};               // TQ2_0: block-scaled sums per plane row

    auto compute = [&](int w) {
        const char* wb = wtile + nl * kWStride + 16 * q;
        const int8_t* ab = WHOLE ? abuf + arow * astride + w * kWinK : abuf + (w & 1) * abytes + arow * kAStride;
#pragma unroll
        for (int seg = 0; seg < kWinK / 256; ++seg) {
            const int s = (kWinK / 256) * w + seg;         // 256-k segment (= TQ2_0 block)
            if (uint32_t(64 * s) >= rowbytes) break;
            i32x4 u = *reinterpret_cast<const i32x4*>(wb + 64 * seg);
            i32x4 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int aoff = FMT == 1 ? 256 * seg + 128 * (q >> 1) + 32 * t + 16 * (q & 1)
                                          : 256 * seg + 64 * t + 16 * q;
                a[t] = *reinterpret_cast<const i32x4*>(ab + aoff);
            }
            if (FMT == 2) {
                // c = ((b0 ^ b1) << 1) | !b0 turns the two's-complement field w into w + 1
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t v = uint32_t(u[j]);
                    u[j] = int((v ^ ((v & 0x55555555u) << 1)) ^ 0x55555555u);
                }
            }
            // i2_s: four accumulators (fields weighted 16, 16, 4, 1) over the
            // whole row; TQ2_0: one accumulator per block, 16 times the dot
            i32x4 bacc[FMT == 2 ? 1 : 4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                i32x4 b;
                if constexpr (FMT == 2) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) b[j] = int(field16(uint32_t(u[j]), t));
                    bacc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b, t == 0 ? i32x4{0, 0, 0, 0} : bacc[0], 0, 0, 0);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) b[j] = int(field<FMT>(uint32_t(u[j]), t));
                    bacc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b, acc[t], 0, 0, 0);
                }
            }
            i32x4 bsum = i32x4{0, 0, 0, 0};               // kInt8: sum q of this segment (TQ2_0) or so far (i2_s);
                                                          // TQ2_0: each plane row's sum over this segment
            if constexpr (INT8 || FMT == 2) {
                const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
                bsum = FMT == 2 ? bsum : qsum;
#pragma unroll
                for (int t = 0; t < 4; ++t) bsum = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], ones, bsum, 0, 0, 0);
                if (FMT == 1) qsum = bsum;
            }
            if constexpr (FMT == 2) {
                // C lane (column nl, quarter q) holds plane rows 4q..4q+3;
                // (s / 16) (16 dot - 16 xs) = s (dot - xs) exactly
                const double sc = double(half_bits_to_float(csc[seg])) * 0.0625;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * q + r;
                    const int xs = row >= RR ? 0 : bsum[r];
                    dacc[r] = __builtin_fma(sc, double(bacc[0][r] - 16 * xs), dacc[r]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[t] = bacc[t];
            }
        }
    };

    Regs r0, r1;
    load(0, r0);
    load(1, r1);
    int Ef = 0;
    if constexpr (FUSED) Ef = fused_prep<FMT>(static_cast<const float*>(ws), K, abuf, astride, fsums, fsmax);
    store_w(0, r0);
    if constexpr (!WHOLE) store_a(0, r0);
    __syncthreads();
    // Window w is multiplied from LDS while window w+1 waits in registers and
    // window w+2 is being fetched.  The weight tile is private to the wave:
    // its LDS accesses execute in program order, so rewriting it after the
    // multiply needs no workgroup barrier; the barrier orders the shared
    // activation window (the fused form holds the whole row: no barrier).
    for (int w = 0; w < nwin; w += 2) {
        if (LL_PLANES_DUMMY || w + 2 < nwin) load(w + 2, r0);
        compute(w);
        if (w + 1 < nwin) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            store_w(w + 1, r1);
            if constexpr (!WHOLE) store_a(w + 1, r1);
        }
        if constexpr (!WHOLE) __syncthreads();
        if (w + 1 >= nwin) break;
        if (LL_PLANES_DUMMY || w + 3 < nwin) load(w + 3, r1);
        compute(w + 1);
        if (w + 2 < nwin) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            store_w(w + 2, r0);
            if constexpr (!WHOLE) store_a(w + 2, r0);
        }
        if constexpr (!WHOLE) __syncthreads();
    }

    if constexpr (INT8) {
        // lane (nl, q) holds tokens 4q .. 4q + 3 of column n: i2_s
        // y = ((float)(sum_t acc_t / mul_t - sum q) * s_tok) * s_w, TQ2_0
        // y = s_tok * (block-scaled sum), then + bias
        const int64_t n = n0 + 16 * wave + nl;
        if (n >= N) return;
        const float sw = FMT == 1 ? *(const __attribute__((address_space(1))) float*)(codes + N * int64_t(rowbytes)) : 1.0f;
        const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * q + r;
            if (m >= mrun) break;
            const float st = xs_tok[m];
            float out;
            if (FMT == 1) {
                int dot = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) dot += acc[t][r] / field_mul<FMT>(t);
                out = __fmul_rn(__fmul_rn(float(dot - qsum[r]), st), sw);
            } else {
                out = float(double(st) * dacc[r]);
            }
            y[int64_t(m) * N + n] = bias ? __fadd_rn(out, bn) : out;
        }
        return;
    }
    // per plane row: D_row = (i2_s) sum_t acc_t / mul_t - total plane sum, or
    // (TQ2_0) the block-scaled sum; then y = f * 2^(E-6) * sum_p 128^-p D_(5m+p)
    double d[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (FMT == 1) {
            int dot = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) dot += acc[t][r] / field_mul<FMT>(t);
            int xt = 0;
            if (row < RR) {
                if constexpr (FUSED) {
#pragma unroll
                    for (int v = 0; v < kWaves; ++v) xt += fsums[v * kP + row];
                } else {
                    xt = ld32(pv.xtot + row);
                }
            }
            d[r] = double(dot - xt);
        } else {
            d[r] = dacc[r];
        }
    }
    const double f = FMT == 1 ? double(*(const __attribute__((address_space(1))) float*)(codes + N * int64_t(rowbytes)))
                              : 1.0;
    const int64_t n = n0 + 16 * wave + nl;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        double v = 0.0;
#pragma unroll
        for (int p = kP - 1; p >= 0; --p) {
            const int row = kP * m + p;
            const double part = __shfl(d[row & 3], nl + 16 * (row >> 2), 64);
            v = __builtin_fma(v, 1.0 / 128.0, part);     // Horner in 1/128: exact for these integers
        }
        if (q == 0 && n < N) {
            const int E = FUSED ? Ef : ld32(pv.ex + m);
            float out = float(f * ldexp(v, E - 6));
            if (bias) out = __fadd_rn(out, bias[n]);
            y[int64_t(m) * N + n] = out;
        }
    }
}

template <int FMT, int M>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_kernel(const uint8_t* __restrict__ codes,
                                                                   const uint16_t* __restrict__ scales, int64_t N,
                                                                   int64_t K, const void* __restrict__ ws,
                                                                   const float* __restrict__ bias,
                                                                   float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const PlaneView pv = plane_view(ws, M, K);
    planes_rows<FMT, M, kWindowed>(codes, scales, N, K, ws, pv, bias, y, int64_t(blockIdx.x) * kRows, lds);
}

// Mt > 3 tokens: passes of up to three tokens.  The passes of one row tile
// are consecutive logical workgroups, and logical runs are mapped onto one
// XCD (hardware workgroup w runs on XCD w % 8 and takes logical index
// (w % 8) * ceil(T / 8) + w / 8), so the passes of a tile run together and
// read its weights through one L2.
__device__ __forceinline__ int64_t xcd_logical(int64_t w, int64_t T) {
    const int64_t T8 = (T + 7) / 8;
    return (w % 8) * T8 + w / 8;
}
template <int FMT>
__device__ __forceinline__ void planes_pass(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                            int64_t N, int64_t K, const void* __restrict__ ws, int Mt, int pass,
                                            const float* __restrict__ bias, float* __restrict__ y, int64_t n0,
                                            char* __restrict__ lds) {
    const PlaneView pv = pass_view(plane_view(ws, Mt, K), pass, K);
    float* yp = y + int64_t(kPassM * pass) * N;
    switch (Mt - kPassM * pass) {
    case 1: planes_rows<FMT, 1, kWindowed>(codes, scales, N, K, ws, pv, bias, yp, n0, lds); break;
    case 2: planes_rows<FMT, 2, kWindowed>(codes, scales, N, K, ws, pv, bias, yp, n0, lds); break;
    default: planes_rows<FMT, 3, kWindowed>(codes, scales, N, K, ws, pv, bias, yp, n0, lds); break;
    }
}

template <int FMT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_multi_kernel(const uint8_t* __restrict__ codes,
                                                                         const uint16_t* __restrict__ scales, int64_t N,
                                                                         int64_t K, const void* __restrict__ ws, int Mt,
                                                                         const float* __restrict__ bias,
                                                                         float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t np = npass(Mt), T = (N + kRows - 1) / kRows * np;
    const int64_t L = xcd_logical(blockIdx.x, T);
    if (L >= T) return;                                    // whole workgroup
    planes_pass<FMT>(codes, scales, N, K, ws, Mt, int(L % np), bias, y, (L / np) * kRows, lds);
}

template <int FMT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_fused_kernel(const uint8_t* __restrict__ codes,
                                                                         const uint16_t* __restrict__ scales, int64_t N,
                                                                         int64_t K, const float* __restrict__ x,
                                                                         const float* __restrict__ bias,
                                                                         float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    planes_rows<FMT, 1, kFused>(codes, scales, N, K, x, PlaneView{}, bias, y, int64_t(blockIdx.x) * kRows, lds);
}

template <int FMT, int MT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_i8_kernel(const uint8_t* __restrict__ codes,
                                                                      const uint16_t* __restrict__ scales, int64_t N,
                                                                      int64_t K, const int8_t* __restrict__ xq,
                                                                      const float* __restrict__ xs, int M,
                                                                      const float* __restrict__ bias,
                                                                      float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const PlaneView pv{const_cast<int8_t*>(xq), nullptr, nullptr};
    planes_rows<FMT, MT, kInt8>(codes, scales, N, K, xq, pv, bias, y, int64_t(blockIdx.x) * kRows, lds, xs, M);
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
};


// Workgroup wg of a batch runs product map[wg] (one table load instead of a
// search: a workgroup's first weight fetch waits on this lookup).
template <int FMT, int M, int MODE>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_batch_kernel(const PlanesProb* __restrict__ tab,
                                                                         const int32_t* __restrict__ map) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t wg = blockIdx.x;
    const PlanesProb& P = tab[ld32(map + wg)];
    const PlaneView pv = plane_view(P.ws, M, P.K);
    planes_rows<FMT, M, MODE>(P.codes, P.scales, P.N, P.K, P.ws, pv, P.bias, P.y, (wg - P.wg0) * kRows, lds);
}

template <int FMT>
__global__ void __launch_bounds__(64 * kWaves) gemv_planes_batch_multi_kernel(const PlanesProb* __restrict__ tab,
                                                                               const int32_t* __restrict__ map,
                                                                               int Mt, int64_t wgs) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t np = npass(Mt), T = wgs * np;
    const int64_t L = xcd_logical(blockIdx.x, T);
    if (L >= T) return;                                    // whole workgroup
    const int64_t wg = L / np;
    const PlanesProb& P = tab[ld32(map + wg)];
    planes_pass<FMT>(P.codes, P.scales, P.N, P.K, P.ws, Mt, int(L % np), P.bias, P.y, (wg - P.wg0) * kRows, lds);
}

template <int FMT>
__global__ void __launch_bounds__(256) prep_planes_batch_kernel(const PlanesPrep* __restrict__ tab, int M) {
    const int wg = int(blockIdx.x);                  // activation wg / M, token wg % M
    const PlanesPrep& P = tab[wg / M];
    const int m = wg % M;
    prep_token<FMT>(P.x + int64_t(m) * P.K, P.K, M, m, P.ws);
}

template <typename F>
hipError_t allow_lds(F* kernel, size_t bytes) {
    return allow_dynamic_lds(reinterpret_cast<const void*>(kernel), bytes);
}

template <int FMT, int M>
hipError_t launch_single(const uint8_t* c, const uint16_t* s, int64_t N, int64_t K, void* ws, const float* bias,
                         float* y, hipStream_t stream) {
    const dim3 grid{unsigned((N + kRows - 1) / kRows)}, block{64 * kWaves};
    const size_t lds = size_t(lds_bytes(M));
    hipError_t e = allow_lds(gemv_planes_kernel<FMT, M>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_kernel<FMT, M>), grid, block, lds, stream, c, s, N, K, ws, bias, y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fused_single(const uint8_t* c, const uint16_t* s, int64_t N, int64_t K, const float* x,
                               const float* bias, float* y, hipStream_t stream) {
    const dim3 grid{unsigned((N + kRows - 1) / kRows)}, block{64 * kWaves};
    const size_t lds = size_t(fused_lds_bytes(K));
    hipError_t e = allow_lds(gemv_planes_fused_kernel<FMT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_fused_kernel<FMT>), grid, block, lds, stream, c, s, N, K, x, bias, y);
    return hipGetLastError();
}

template <int FMT, int MT>
hipError_t launch_i8(const uint8_t* c, const uint16_t* s, int64_t N, int64_t K, const int8_t* xq, const float* xs,
                     int M, const float* bias, float* y, hipStream_t stream) {
    const dim3 grid{unsigned((N + kRows - 1) / kRows)}, block{64 * kWaves};
    const size_t lds = size_t(kWaves * kWTile + 2 * MT * kAStride);
    hipError_t e = allow_lds(gemv_planes_i8_kernel<FMT, MT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_i8_kernel<FMT, MT>), grid, block, lds, stream, c, s, N, K, xq, xs, M, bias, y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_multi(const uint8_t* c, const uint16_t* s, int64_t N, int64_t K, void* ws, int Mt,
                        const float* bias, float* y, hipStream_t stream) {
    const int64_t T = (N + kRows - 1) / kRows * npass(Mt);
    const dim3 grid{unsigned((T + 7) / 8 * 8)}, block{64 * kWaves};
    const size_t lds = size_t(lds_bytes(kPassM));
    hipError_t e = allow_lds(gemv_planes_multi_kernel<FMT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_multi_kernel<FMT>), grid, block, lds, stream, c, s, N, K, ws, Mt, bias, y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_batch_multi(const PlanesProb* tab, const int32_t* map, int64_t wgs, int Mt, hipStream_t stream) {
    const int64_t T = wgs * npass(Mt);
    const dim3 grid{unsigned((T + 7) / 8 * 8)}, block{64 * kWaves};
    const size_t lds = size_t(lds_bytes(kPassM));
    hipError_t e = allow_lds(gemv_planes_batch_multi_kernel<FMT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_batch_multi_kernel<FMT>), grid, block, lds, stream, tab, map, Mt, wgs);
    return hipGetLastError();
}

template <int FMT, int M>
hipError_t launch_batch(const PlanesProb* tab, const int32_t* map, int64_t wgs, hipStream_t stream) {
    const dim3 grid{unsigned(wgs)}, block{64 * kWaves};
    const size_t lds = size_t(lds_bytes(M));
    hipError_t e = allow_lds(gemv_planes_batch_kernel<FMT, M, kWindowed>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_planes_batch_kernel<FMT, M, kWindowed>), grid, block, lds, stream, tab, map);
    return hipGetLastError();
}

}  // namespace

namespace llk {

bool planes_fused(int64_t M, int64_t K) { return M == 1 && K <= kFusedMaxK; }
size_t planes_workspace(int64_t M, int64_t K) { return planes_fused(M, K) ? 0 : planes_bytes(M, K); }
size_t planes_operand_bytes(int64_t M, int64_t K) { return planes_bytes(M, K); }
int64_t planes_batch_rows() { return kRows; }
size_t planes_prob_bytes() { return sizeof(PlanesProb); }
size_t planes_prep_bytes() { return sizeof(PlanesPrep); }

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

void fill_planes_prep(void* dst, const float* x, void* ws, int64_t K) {
    PlanesPrep p;
    p.x = x;
    p.ws = ws;
    p.K = K;
    *static_cast<PlanesPrep*>(dst) = p;
}

hipError_t launch_gemv_planes(int fmt, const void* codes, const void* scales, int64_t N, int64_t K, const float* x,
                              int64_t M, const float* bias, float* y, void* ws, hipStream_t stream) {
    const dim3 pgrid{unsigned(M)}, pblock{256};
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    const uint16_t* s = static_cast<const uint16_t*>(scales);
    if (planes_fused(M, K))
        return fmt == 1 ? launch_fused_single<1>(c, s, N, K, x, bias, y, stream)
                        : launch_fused_single<2>(c, s, N, K, x, bias, y, stream);
    if (fmt == 1) hipLaunchKernelGGL(prep_planes_kernel<1>, pgrid, pblock, 0, stream, x, K, int(M), ws);
    else hipLaunchKernelGGL(prep_planes_kernel<2>, pgrid, pblock, 0, stream, x, K, int(M), ws);
    if (M > kPassM)
        return fmt == 1 ? launch_multi<1>(c, s, N, K, ws, int(M), bias, y, stream)
                        : launch_multi<2>(c, s, N, K, ws, int(M), bias, y, stream);
    switch (fmt * 4 + int(M)) {
    case 5: return launch_single<1, 1>(c, s, N, K, ws, bias, y, stream);
    case 6: return launch_single<1, 2>(c, s, N, K, ws, bias, y, stream);
    case 7: return launch_single<1, 3>(c, s, N, K, ws, bias, y, stream);
    case 9: return launch_single<2, 1>(c, s, N, K, ws, bias, y, stream);
    case 10: return launch_single<2, 2>(c, s, N, K, ws, bias, y, stream);
    default: return launch_single<2, 3>(c, s, N, K, ws, bias, y, stream);
    }
}

hipError_t launch_gemv_i8_planes(int fmt, const void* codes, const void* scales, int64_t N, int64_t K,
                                 const int8_t* xq, const float* xs, int64_t M, const float* bias, float* y,
                                 hipStream_t stream) {
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    const uint16_t* s = static_cast<const uint16_t*>(scales);
    const int m = int(M), mt = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16;
    switch (fmt * 32 + mt) {
    case 33: return launch_i8<1, 1>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 34: return launch_i8<1, 2>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 36: return launch_i8<1, 4>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 40: return launch_i8<1, 8>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 48: return launch_i8<1, 16>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 65: return launch_i8<2, 1>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 66: return launch_i8<2, 2>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 68: return launch_i8<2, 4>(c, s, N, K, xq, xs, m, bias, y, stream);
    case 72: return launch_i8<2, 8>(c, s, N, K, xq, xs, m, bias, y, stream);
    default: return launch_i8<2, 16>(c, s, N, K, xq, xs, m, bias, y, stream);
    }
}

hipError_t launch_planes_batch_prep(const void* prep_table, int nprep, int fmt, int64_t M, hipStream_t stream) {
    const dim3 grid{unsigned(int64_t(nprep) * M)}, block{256};
    const PlanesPrep* tab = static_cast<const PlanesPrep*>(prep_table);
    if (fmt == 1) hipLaunchKernelGGL(prep_planes_batch_kernel<1>, grid, block, 0, stream, tab, int(M));
    else hipLaunchKernelGGL(prep_planes_batch_kernel<2>, grid, block, 0, stream, tab, int(M));
    return hipGetLastError();
}

hipError_t launch_planes_batch_product(const void* prob_table, const void* map, int fmt, int64_t M, int64_t wgs,
                                       hipStream_t stream) {
    const PlanesProb* tab = static_cast<const PlanesProb*>(prob_table);
    const int32_t* mp = static_cast<const int32_t*>(map);
    if (M > kPassM)
        return fmt == 1 ? launch_batch_multi<1>(tab, mp, wgs, int(M), stream)
                        : launch_batch_multi<2>(tab, mp, wgs, int(M), stream);
    switch (fmt * 4 + int(M)) {
    case 5: return launch_batch<1, 1>(tab, mp, wgs, stream);
    case 6: return launch_batch<1, 2>(tab, mp, wgs, stream);
    case 7: return launch_batch<1, 3>(tab, mp, wgs, stream);
    case 9: return launch_batch<2, 1>(tab, mp, wgs, stream);
    case 10: return launch_batch<2, 2>(tab, mp, wgs, stream);
    default: return launch_batch<2, 3>(tab, mp, wgs, stream);
    }
}

}  // namespace llk
