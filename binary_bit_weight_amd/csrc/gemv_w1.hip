// W1A8 product: binary weights (one sign bit each, one fp16 scale per group of
// G weights), int8 activations with a per-token scale, 1 <= M <= 16.
//
// [BG "Method"] With the stored bit b = (w + 1) / 2 the group dot product is
//     d = sum w*q = 2 * sum_{b=1} q - sum q,
// so only sum_{b=1} q has to be formed from the bits.  It runs on the fp8 x fp4
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales):
//   B (weights): a 32-bit word of bits masked in place is eight fp4 (e2m1)
//       values: word & (0x11111111 << j) for j = 0, 1, 2 leaves bit 4i + j at
//       bit j of nibble i (value b * 2^(j-1)), and (word >> 1) & 0x44444444
//       moves bit 4i + 3 (the nibble's sign position) to bit 2 (value b * 2):
//       five operations per 32 weights;
//   A (activations): q = 16 * hi + lo with hi, lo in [-8, 8], one MFMA row
//       each; rows are (token, group slot, digit).  The digit meeting nibble
//       position j is stored times 2^(2 - min(j, 2)), so every product is
//       2 b d whatever j is (integers of at most 3 significant bits below 2^6,
//       exact in fp8 e4m3).
// Every product is an integer below 2^5 in magnitude and every sum stays below
// 2^13, so the fp32 accumulation is exact: sum_{b=1} q = (16 D_hi + D_lo) / 2.
// The epilogue forms S = sum_g s_g * d_g with fp64 fmas of exact products in
// group order and y = (float)((double)xs * S) (+ bias), bit for bit the
// oracle's result.
//
// Operand layout.  For the 16x16x128 f8f6f4 MFMA with fp8 A and fp4 B the
// hardware pairs A element (lane quarter q, byte e) with B element (lane
// quarter q' = 2(e/16) + q/2, nibble e' = 16(q%2) + e%16) of the same
// column/row lane index (measured on the device).  B lane quarter q' holds
// word q' of the 128-k chunk of its row, its nibble e' = 8j + i being bit
// 4i + j, i.e. chunk-local weight 32q' + 4(e'%8) + e'/8.  The preparation
// kernel writes each A row in the matching order.
//
// Memory.  A workgroup is 4 waves x 32 rows (two 16-column MFMA blocks per
// wave).  Per 1024-k window each wave loads its rows as 8 rows x 128
// contiguous bytes per instruction into a padded LDS tile private to the
// wave, together with the window's group scales; the prepared A rows and
// group sums of the window are staged in a shared, double-buffered LDS
// window.  Loads run two windows ahead of the multiply.
#include "common.h"
#include "launch.h"

#include <mutex>
#include <type_traits>
#include <tuple>
#include <vector>

namespace {

using namespace llk;

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kW1Waves = 4;
constexpr int kW1RowsPerWave = 32;
constexpr int kW1Rows = kW1Waves * kW1RowsPerWave;   // 128 rows per workgroup
constexpr int kWinK1 = 1024;                          // k per window
constexpr int kWinB1 = kWinK1 / 8;                    // 128 code bytes per row per window
constexpr int kChunks = kWinK1 / 128;                 // 8 MFMA chunks per window
constexpr int kW1MaxSplits = 8;                       // K splits of a narrow matrix
#ifndef LL_W1_FUSE_WORK
#define LL_W1_FUSE_WORK 256                                // row blocks x A rows up to which the preparation is fused
#endif

// LDS row of a wave's tile: 128 code bytes | the window's scales (1024/G fp16) | pad to 16 mod 128.
__host__ __device__ inline int w1_stride(int G) {
    const int raw = kWinB1 + 2 * (kWinK1 / G);
    return (raw + 127) / 128 * 128 + 16;
}

// Rows of the A operand: (token m, group slot j, digit h) -> 2 (m S + j) + h,
// S = 128 / G slots per 128-k chunk (1 for G >= 128).
__host__ __device__ constexpr int w1_slots(int G) { return G >= 128 ? 1 : 128 / G; }
__host__ __device__ inline int w1_arows(int M, int G) { return 2 * M * w1_slots(G); }
// Units (a group of G >= 128, else a 128-k chunk) packed into one MFMA
// accumulator: the largest power of two with PK R <= 16, at most the units of
// a 1024-k window.
inline int w1_pack(int M, int G) {
    const int R = w1_arows(M, G);
    const int units = G >= 128 ? 8 / (G / 128) : 8;
    int pk = 1;
    while (pk * 2 * R <= 16 && pk * 2 <= units) pk *= 2;
    return pk;
}

// Workspace of one activation: A [K/128 chunks][R rows][128 B] | qs [M][K/G] int32.
__host__ __device__ inline size_t w1_a_bytes(int64_t M, int64_t K, int G) {
    return size_t(K / 128) * size_t(w1_arows(int(M), G)) * 128;
}
__host__ __device__ inline size_t w1_ws_bytes(int64_t M, int64_t K, int G) {
    return (w1_a_bytes(M, K, G) + 15) / 16 * 16 + size_t(M) * size_t(K / G) * 4;
}

// A window in LDS: [chunk 8][R rows][128 B] | zero row [128 B] | qs [M][1024/G] int32.
__host__ __device__ inline int w1_abuf_bytes(int M, int G) {
    return kChunks * w1_arows(M, G) * 128 + 128 + M * (kWinK1 / G) * 4;
}
__host__ __device__ inline int w1_lds_bytes(int M, int G) {
    return kW1Waves * kW1RowsPerWave * w1_stride(G) + 2 * ((w1_abuf_bytes(M, G) + 15) / 16 * 16);
}

// One 16-byte piece u of an A row of digit h (0: hi, 1: lo) from the 32
// source bytes (lo4, hi4) at 32 qp of its 128-k chunk, qp = 2 (u % 2) + u / 4.
// Piece u holds A bytes 16u + i of lane quarter q = u / 2; byte i pairs with B
// quarter qp, nibble e = 16 (q % 2) + i, i.e. B word j = e / 8 and the
// chunk-local weight 32 qp + 4 (i % 8) + j: source byte j of source dword
// i % 8.  The digit is stored times 2^(2 - min(j, 2)) through the hardware's
// fp32 -> fp8 (OCP e4m3) conversion, exact for these values.
// sum: the sixteen source values (0 outside the slot).
__device__ __forceinline__ i32x4 w1_piece(const i32x4& lo4, const i32x4& hi4, int u, int h, bool in_slot, int& sum) {
    const uint32_t dw[8] = {uint32_t(lo4[0]), uint32_t(lo4[1]), uint32_t(lo4[2]), uint32_t(lo4[3]),
                            uint32_t(hi4[0]), uint32_t(hi4[1]), uint32_t(hi4[2]), uint32_t(hi4[3])};
    const int b0 = 2 * ((u >> 1) & 1);
    uint32_t out[4];
    sum = 0;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        const int j = b0 + (w4 >> 1);                      // B word of output bytes 4 w4 .. 4 w4 + 3
        const float scale = float(1 << (2 - (j < 2 ? j : 2)));
        float f[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int v = in_slot ? int(int8_t(dw[4 * (w4 & 1) + bb] >> (8 * j))) : 0;
            sum += v;
            const int hi = (v + 8) >> 4;                    // floor((v + 8) / 16): v = 16 hi + lo, lo in [-8, 7]
            const int d = h == 0 ? hi : v - 16 * hi;
            f[bb] = float(d) * scale;
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], word, true);
        out[w4] = uint32_t(word);
    }
    return i32x4{int(out[0]), int(out[1]), int(out[2]), int(out[3])};
}

// The B operand of one 128-k chunk of a row from its 32-bit word of bits.
__device__ __forceinline__ i32x8 w1_bv(uint32_t word) {
    return i32x8{int(word & 0x11111111u), int(word & 0x22222222u), int(word & 0x44444444u),
                 int((word >> 1) & 0x44444444u), 0, 0, 0, 0};
}

// fp8 (A) x fp4 (B) product with the A block scales taken from byte `byte`
// (a constant after unrolling) of sa; B block scales 1.
template <int BYTE>
__device__ __forceinline__ f32x4 w1_mfma_b(const i32x8& a, const i32x8& b, const f32x4& c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, BYTE, sa, 0, 127);
}
__device__ __forceinline__ f32x4 w1_mfma_unit(int byte, const i32x8& a, const i32x8& b, const f32x4& c, int sa) {
    switch (byte) {
    case 0: return w1_mfma_b<0>(a, b, c, sa);
    case 1: return w1_mfma_b<1>(a, b, c, sa);
    case 2: return w1_mfma_b<2>(a, b, c, sa);
    default: return w1_mfma_b<3>(a, b, c, sa);
    }
}

// ---------------------------------------------------------------- preparation
// One thread per 16-byte piece of an A row (chunk c, row r, piece u), plus the
// group sums.  Grid: (ceil(chunks * R * 8 / 256), 1) and a second pass over
// groups.  Reads xq [M][K] int8.
__device__ void w1_qsum(const int8_t* __restrict__ xq, int64_t M, int64_t K, int G, void* __restrict__ ws,
                        int64_t block);

// Block `block` of the preparation of one activation (prep_blocks piece
// blocks, then the group-sum blocks).
__device__ __forceinline__ void w1_prep_body(const int8_t* __restrict__ xq, int64_t M, int64_t K, int G,
                                             void* __restrict__ ws, int64_t prep_blocks, int64_t block) {
    if (block >= prep_blocks) {                            // the group sums, in the same launch
        w1_qsum(xq, M, K, G, ws, block - prep_blocks);
        return;
    }
    const int S = w1_slots(G), R = w1_arows(int(M), G);
    const int64_t pieces = (K / 128) * R * 8;
    const int64_t id = block * 256 + threadIdx.x;
    int8_t* A = static_cast<int8_t*>(ws);
    if (id < pieces) {
        const int u = int(id % 8);
        const int r = int((id / 8) % R);
        const int64_t c = id / (8 * int64_t(R));
        const int h = r & 1, pm = r >> 1;
        const int m = pm / S, j = pm % S;
        const int8_t* xr = xq + int64_t(m) * K + 128 * c;
        const int qp = 2 * (u & 1) + (u >> 2);
        const bool in_slot = G >= 128 || (32 * qp) / G == j;   // the whole piece is in slot j or not
        const i32x4 lo4 = ld16(xr + 32 * qp), hi4 = ld16(xr + 32 * qp + 16);
        int sum;
        st16(A + (c * R + r) * 128 + 16 * u, w1_piece(lo4, hi4, u, h, in_slot, sum));
    }
}

__global__ void __launch_bounds__(256) w1_prep_kernel(const int8_t* __restrict__ xq, int64_t M, int64_t K, int G,
                                                      void* __restrict__ ws, int64_t prep_blocks) {
    w1_prep_body(xq, M, K, G, ws, prep_blocks, blockIdx.x);
}

// Group sums qs[m][g] = sum_{k in g} q: one wave per (token, group).
__device__ void w1_qsum(const int8_t* __restrict__ xq, int64_t M, int64_t K, int G, void* __restrict__ ws,
                        int64_t block) {
    const int lane = threadIdx.x & 63;
    const int64_t ng = K / G;
    const int64_t item = block * 4 + (threadIdx.x >> 6);
    if (item >= M * ng) return;
    const int64_t m = item / ng, g = item % ng;
    int s = 0;
    for (int i = lane; i < G; i += 64) s += xq[m * K + g * G + i];
    int v[1] = {s};
    wave_sum_n(v);
    int32_t* qs = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + (w1_a_bytes(M, K, G) + 15) / 16 * 16);
    if (lane == 0) qs[m * ng + g] = v[0];
}

// ---------------------------------------------------------------- product
// G: group size; MT: A row blocks of 16 (R = 2 M S <= 16 MT rows); NP: pairs
// (token, slot) per lane and row block that can be live (1 when R <= 2, else
// 2); PK: units packed into one accumulator (MT = 1, NP = 2 when PK > 1).
// Split K.  With few row blocks (a narrow matrix) the workgroups of a row
// block split its windows nsplit ways; each writes its partial sums S (exact
// in fp64, so their sum is too, in any order) to part and counts itself in;
// the last to arrive adds the partials and writes y, then resets the counter
// (counters start zero and every call leaves them zero).
// FUSED (G == 128, one row block of A rows): ws is the int8 activations
// xq [M][K] themselves; every workgroup forms its windows' digit rows and
// group sums while staging them (no preparation launch).
template <int G, int MT, int NP, int PK, bool FUSED>
__global__ void __launch_bounds__(64 * kW1Waves) __attribute__((amdgpu_waves_per_eu(G >= 128 && PK * (G / 128) == 8 && !FUSED ? 3 : 1))) w1_gemv_kernel(const uint32_t* __restrict__ bits,
                                                                 const uint16_t* __restrict__ scales, int64_t N,
                                                                 int64_t K, int M, const void* __restrict__ ws,
                                                                 const float* __restrict__ xs,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ y, int nsplit,
                                                                 double* __restrict__ part,
                                                                 int32_t* __restrict__ counters,
                                                                 uint16_t* __restrict__ y16) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ int last_flag;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t rb = int64_t(blockIdx.x) / nsplit;      // row block
    const int split = int(blockIdx.x % nsplit);
    const int nl = lane & 15, q = lane >> 4;
    constexpr int S = G >= 128 ? 1 : 128 / G;
    const int R = w1_arows(M, G);
    constexpr int stride = (kWinB1 + 2 * (kWinK1 / G) + 127) / 128 * 128 + 16;
    constexpr int ngw = kWinK1 / G;                        // groups per window
    const int64_t ng = K / G;
    const uint32_t rowbytes = uint32_t(K / 8);
    const int nwall = int((K + kWinK1 - 1) / kWinK1);
    const int w0 = int(int64_t(nwall) * split / nsplit);  // windows [w0, nwin) of this split
    const int nwin = int(int64_t(nwall) * (split + 1) / nsplit);
    const int64_t n0 = rb * kW1Rows + kW1RowsPerWave * wave;
    char* wtile = lds + wave * kW1RowsPerWave * stride;
    const int abytes = (w1_abuf_bytes(M, G) + 15) / 16 * 16;
    char* abase = lds + kW1Waves * kW1RowsPerWave * stride;
    const int8_t* Ag = static_cast<const int8_t*>(ws);
    const int32_t* qsg = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + (w1_a_bytes(M, K, G) + 15) / 16 * 16);

    // weight loads: 8 rows x 128 B per instruction, lane -> row 8i + lane/8, bytes 16 (lane%8)
    const int lr = lane >> 3, lc = lane & 7;
    const uint8_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t n = n0 + 8 * i + lr;
        n = n < N ? n : N - 1;
        wrow[i] = reinterpret_cast<const uint8_t*>(bits) + n * int64_t(rowbytes) + 16 * lc;
    }
    // scale loads: 32 rows x ngw scales per window, one fp16 per lane and load
    constexpr int kScMax = (kW1RowsPerWave * ngw + 63) / 64;
    constexpr int nsc = kScMax;
    // A window loads: R rows x 8 chunks x 128 B = 64 R pieces of 16 B; qs: M x ngw ints
    const int apieces = 64 * R;
    constexpr int kAMax = NP == 1 ? 1 : (16 * MT * 64 / PK + 255) / 256;   // R <= 16 MT / PK
    static_assert(!FUSED || (G == 128 && MT == 1), "fused preparation: G = 128, one row block");
    struct Regs {
        i32x4 w[4];
        uint16_t sc[kScMax];
        i32x4 a[kAMax * (FUSED ? 2 : 1)];                  // fused: the 32 source bytes of each piece
        int32_t qs[2];
    };
    const int8_t* xq = static_cast<const int8_t*>(ws);
    auto load = [&](int w, Regs& r) {
        const uint32_t off = uint32_t(w) * kWinB1 + 16 * lc;
        const uint32_t offc = off < rowbytes ? off : rowbytes - 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.w[i] = ld16_stream(wrow[i] - 16 * lc + offc);
#pragma unroll
        for (int u = 0; u < kScMax; ++u) {
            if (u < nsc) {
                const int e = lane + 64 * u;
                const int row = e / ngw, gi = e % ngw;
                int64_t n = n0 + (row < kW1RowsPerWave ? row : kW1RowsPerWave - 1);
                n = n < N ? n : N - 1;
                int64_t g = int64_t(w) * ngw + gi;
                g = g < ng ? g : ng - 1;
                r.sc[u] = ld2(scales + n * ng + g);
            }
        }
#pragma unroll
        for (int i = 0; i < kAMax; ++i) {
            if (i * 256 < apieces) {
                const int p = tid + 256 * i;
                const int pc = p < apieces ? p : apieces - 1;
                const int c = pc / (8 * R), rem = pc % (8 * R);
                int64_t cg = int64_t(w) * kChunks + c;
                const int64_t nchunk = K / 128;
                cg = cg < nchunk ? cg : nchunk - 1;
                if constexpr (FUSED) {
                    // piece u of row (token m, digit h): the 32 source bytes at 32 qp
                    const int u = rem & 7, m = rem >> 4, qp = 2 * (u & 1) + (u >> 2);
                    const int8_t* src = xq + int64_t(m) * K + 128 * cg + 32 * qp;
                    r.a[2 * i] = ld16(src);
                    r.a[2 * i + 1] = ld16(src + 16);
                } else {
                    r.a[i] = ld16(Ag + (cg * R) * 128 + 16 * rem);
                }
            }
        }
        if constexpr (!FUSED) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int e = tid + 256 * i;
                const int m = e / ngw, gi = e % ngw;
                int64_t g = int64_t(w) * ngw + gi;
                g = g < ng ? g : ng - 1;
                r.qs[i] = ld32(qsg + int64_t(m < M ? m : M - 1) * ng + g);
            }
        }
    };
    auto store_w = [&](int w, const Regs& r) {
        const bool ok = uint32_t(w) * kWinB1 + 16 * lc < rowbytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<i32x4*>(wtile + (8 * i + lr) * stride + 16 * lc) = ok ? r.w[i] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kScMax; ++u) {
            if (u < nsc) {
                const int e = lane + 64 * u;
                const int row = e / ngw, gi = e % ngw;
                if (row < kW1RowsPerWave)
                    *reinterpret_cast<uint16_t*>(wtile + row * stride + kWinB1 + 2 * gi) = r.sc[u];
            }
        }
    };
    auto store_a = [&](int w, const Regs& r) {
        char* ab = abase + (w & 1) * abytes;
        int32_t* qsl = reinterpret_cast<int32_t*>(ab + kChunks * R * 128 + 128);
        if constexpr (FUSED) {
            // digit rows converted here; the hi-digit pieces of a (chunk, token)
            // are 8 aligned lanes, whose source sums add up to the group sum
#pragma unroll
            for (int i = 0; i < kAMax; ++i) {
                if (i * 256 < apieces) {
                    const int p = tid + 256 * i;
                    const int pc = p < apieces ? p : apieces - 1;
                    const int c = pc / (8 * R), rem = pc % (8 * R);
                    const int u = rem & 7, h = (rem >> 3) & 1, m = rem >> 4;
                    int sum;
                    const i32x4 d = w1_piece(r.a[2 * i], r.a[2 * i + 1], u, h, true, sum);
                    sum += __shfl_xor(sum, 1, 64);
                    sum += __shfl_xor(sum, 2, 64);
                    sum += __shfl_xor(sum, 4, 64);
                    if (p < apieces) {
                        *reinterpret_cast<i32x4*>(ab + 16 * p) = d;
                        if (u == 0 && h == 0) qsl[m * ngw + c] = sum;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kAMax; ++i) {
                const int p = tid + 256 * i;
                if (i * 256 < apieces && p < apieces) *reinterpret_cast<i32x4*>(ab + 16 * p) = r.a[i];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int e = tid + 256 * i;
                if (e < M * ngw) qsl[e] = r.qs[i];
            }
        }
    };

    // zero rows (read by lanes whose A row is >= R) in both buffers
    if (tid < 16) {
        *reinterpret_cast<i32x4*>(abase + kChunks * R * 128 + 16 * (tid & 7) + 0 * abytes) = i32x4{0, 0, 0, 0};
        *reinterpret_cast<i32x4*>(abase + kChunks * R * 128 + 16 * (tid & 7) + 1 * abytes) = i32x4{0, 0, 0, 0};
    }

    f32x4 acc[2][MT];
    double sacc[2][MT][NP];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int b = 0; b < MT; ++b) {
            acc[cb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < NP; ++t) sacc[cb][b][t] = 0.0;
        }

    constexpr int cpg = G >= 128 ? G / 128 : 1;            // chunks per unit (a group, or one chunk of S groups)
    // Packing: the PK units of a set put their R rows at row offsets R s of
    // one accumulator, so one epilogue serves PK units.  Lane row nl carries
    // slot sl = nl / R, row rl = nl % R (no slot if nl >= PK R).
    constexpr int kSet = cpg * PK;                          // chunks per set (divides the window's 8)
    const int sl = PK == 1 ? 0 : (nl < PK * R ? nl / R : PK), rl = PK == 1 ? nl : nl % R;
    const int64_t nchunk = K / 128;
    auto compute = [&](int w) {
        const char* ab = abase + (w & 1) * abytes;
        const int32_t* qsl = reinterpret_cast<const int32_t*>(ab + kChunks * R * 128 + 128);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int64_t cg = int64_t(w) * kChunks + c;   // global chunk
            if (cg >= nchunk) break;
            // A operands (32 bytes per lane and row block)
            i32x8 av[MT];
#pragma unroll
            for (int b = 0; b < MT; ++b) {
                const char* ap;
                if (PK == 1) {
                    const int r = 16 * b + nl;
                    ap = r < R ? ab + (c * R + r) * 128 + 32 * q : ab + kChunks * R * 128;   // zero row
                } else {
                    ap = sl == (c / cpg) % PK ? ab + (c * R + rl) * 128 + 32 * q : ab + kChunks * R * 128;
                }
                const i32x4 lo = *reinterpret_cast<const i32x4*>(ap);
                const i32x4 hi = *reinterpret_cast<const i32x4*>(ap + 16);
                av[b] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
            const bool first = (c % kSet) == 0;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const uint32_t word = *reinterpret_cast<const uint32_t*>(wtile + (16 * cb + nl) * stride + 16 * c + 4 * q);
                const i32x8 bv = w1_bv(word);
#pragma unroll
                for (int b = 0; b < MT; ++b)
                    acc[cb][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av[b], bv, first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[cb][b], 0, 4, 0, 127, 0, 127);
            }
            if ((c % kSet) == kSet - 1 || cg + 1 == nchunk) {
                // epilogue of the set ending with this chunk
                const int u0 = (c / kSet) * PK;               // first unit of the set within the window
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const char* srow = wtile + (16 * cb + nl) * stride + kWinB1;
#pragma unroll
                    for (int b = 0; b < MT; ++b) {
#pragma unroll
                        for (int t = 0; t < NP; ++t) {
                            const int pp = 8 * b + 2 * q + t;         // pair of rows: slot s, (token, group slot) p
                            const int s = PK == 1 ? 0 : pp / (M * S);
                            const int p = PK == 1 ? pp : pp % (M * S);
                            const int m = p / S, j = p % S;
                            const int gi = G >= 128 ? u0 + s : (u0 + s) * S + j;   // group within the window
                            const bool ok = PK == 1 || (s < PK && int64_t(w) * ngw + gi < ng);
                            const float v = __builtin_fmaf(16.0f, acc[cb][b][2 * t], acc[cb][b][2 * t + 1]);
                            const int gic = ok ? gi : 0;
                            const int qsv = qsl[(m < M ? m : 0) * ngw + gic];
                            const int d = int(v) - qsv;
                            const double sc = double(half_bits_to_float(*reinterpret_cast<const uint16_t*>(srow + 2 * gic)));
                            const double nv = __builtin_fma(sc, double(d), sacc[cb][b][t]);
                            sacc[cb][b][t] = ok ? nv : sacc[cb][b][t];
                        }
                    }
                }
            }
        }
    };

    // Window w is multiplied from LDS while window w + 1 waits in registers
    // and window w + 2 is being fetched.  Every load is issued (windows past
    // the range reload in-bounds bytes that are never multiplied) and the
    // loop has no exit between a load and its use, so the compiler's waits
    // count exactly and the prefetch overlaps the multiply.
    Regs r0, r1;
    load(w0, r0);
    load(w0 + 1, r1);
    store_w(w0, r0);
    store_a(w0, r0);
    __syncthreads();
    int w = w0;
    for (; w + 2 <= nwin; w += 2) {
        load(w + 2, r0);
        compute(w);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store_w(w + 1, r1);
        store_a(w + 1, r1);
        __syncthreads();
        load(w + 3, r1);
        compute(w + 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store_w(w + 2, r0);
        store_a(w + 2, r0);
        __syncthreads();
    }
    if (w < nwin) compute(w);                              // odd window count: the last one is in LDS

    // y[m][n] = (float)((double)xs[m] * S[m][n]) (+ bias).  Pair
    // p = (k M + m) S + j (pack slot k) of row block b lives in lane quarter
    // (p % 8) / 2, slot t = p % 2; the pack slots and group slots of one token
    // are added through LDS (every partial sum is exact, so the order of
    // groups does not matter).
    __syncthreads();
    double* red = reinterpret_cast<double*>(lds);      // [2 cb][16 col][pairs up to 8 MT]
    const int npairs = 8 * MT;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int b = 0; b < MT; ++b)
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                const int p = 8 * b + 2 * q + t;
                red[(wave * 2 * 16 + cb * 16 + nl) * npairs + p] = sacc[cb][b][t];
            }
    __syncthreads();
    for (int e = tid; e < kW1Waves * 2 * 16 * M; e += 64 * kW1Waves) {
        const int m = e % M;
        const int col = e / M;                             // wave * 32 + cb * 16 + nl
        const int64_t n = rb * kW1Rows + col;
        double s = 0.0;
        for (int k = 0; k < PK; ++k)
            for (int j = 0; j < S; ++j) s += red[col * npairs + (k * M + m) * S + j];
        if (nsplit > 1) {
            st_coherent64(part + (int64_t(blockIdx.x) * kW1Rows + col) * M + m, s);
        } else if (n < N) {
            float out = float(double(xs[m]) * s);
            if (bias) out = __fadd_rn(out, bias[n]);
            if (y16)
                y16[int64_t(m) * N + n] = f32_to_bf16_rne(out);
            else
                y[int64_t(m) * N + n] = out;
        }
    }
    if (nsplit == 1) return;
    wait_vmem();
    __syncthreads();
    if (tid == 0) last_flag = arrive_release(counters + rb) == nsplit - 1;
    __syncthreads();
    if (!last_flag) return;
    acquire_agent();
    for (int e = tid; e < kW1Waves * 2 * 16 * M; e += 64 * kW1Waves) {
        const int m = e % M;
        const int col = e / M;
        const int64_t n = rb * kW1Rows + col;
        if (n >= N) continue;
        // every split's partial requested at once (nsplit <= kW1MaxSplits), added in split order
        double pv[kW1MaxSplits];
#pragma unroll
        for (int sp = 0; sp < kW1MaxSplits; ++sp) {
            const int spc = sp < nsplit ? sp : nsplit - 1;
            pv[sp] = ld_coherent64(part + ((rb * nsplit + spc) * kW1Rows + col) * M + m);
        }
        double s = 0.0;
#pragma unroll
        for (int sp = 0; sp < kW1MaxSplits; ++sp)
            if (sp < nsplit) s += pv[sp];
        float out = float(double(xs[m]) * s);
        if (bias) out = __fadd_rn(out, bias[n]);
        if (y16)
            y16[int64_t(m) * N + n] = f32_to_bf16_rne(out);
        else
            y[int64_t(m) * N + n] = out;
    }
    if (tid == 0) st_coherent(counters + rb, 0);          // ready for the next call
}

// ---------------------------------------------------------------- streaming product
// Tall matrices (no K split, few tokens).  Every workgroup first stages the A
// operand of the whole K range (digit rows, group sums) and the token scales
// in LDS, once.  Its waves then work alone: wave i of W streams the 32-row
// blocks i, i + W, i + 2W, ... window after window, its loads running two
// windows ahead straight across block boundaries, so no wave drains its
// pipeline or waits for another.  A block's epilogue adds its pack and group
// slots through the wave's own weight tile, which is free between the
// block's last window and the next block's first.
// LDS: [4 waves][32 rows][stride] tiles | [4 waves][32] fp32 biases |
// A [K/128][R][kARow] | qs [M][ngp] fp32 (group sums, exact; rows padded to
// ngp = K/G rounded up to a multiple of 4, 16-byte aligned) | padding | xs [M]
// fp32.  An A row
// holds 128 bytes padded to 144, so the 16 rows one MFMA operand read
// touches start 36 banks apart instead of all on the same bank.
constexpr int kARow = 144;
// A tile row: 128 code bytes | the window's scales, padded to 16 mod 128
// bytes (rows of one 8-row store then start 4 banks apart).
__host__ __device__ constexpr int w1_stream_stride(int G) {
    return (kWinB1 + 2 * (kWinK1 / G) - 16 + 127) / 128 * 128 + 16;
}
__host__ __device__ constexpr int64_t w1_qs_stride(int64_t K, int G) { return (K / G + 3) / 4 * 4; }
__host__ __device__ inline int w1_stream_a_bytes(int M, int64_t K, int G) {
    return int((K / 128) * w1_arows(M, G) * kARow + (M * w1_qs_stride(K, G) + 4) * 4 + 16 * 4);
}
__host__ __device__ inline int w1_stream_lds_bytes(int M, int64_t K, int G, int waves) {
    return waves * kW1RowsPerWave * (w1_stream_stride(G) + 4) + w1_stream_a_bytes(M, K, G);
}

#ifndef LL_W1_STREAM_WPE
#define LL_W1_STREAM_WPE 2                                 // waves per SIMD the register budget is cut for
#endif
#ifndef LL_W1_STREAM_FUSE
#define LL_W1_STREAM_FUSE 1                                // G = 128: every workgroup forms the A digits itself
#endif
// ... up to this many tokens.  Every workgroup converts the whole A operand,
// work that grows with the tokens; above two tokens the preparation launch
// (A formed once, copied into each workgroup's LDS) costs less.  Measured
// (us, fused / prepared): 7168 x 5120 at M = 1 7.3 / 8.6, M = 4 11.1 / 10.3,
// M = 8 15.6 / 11.7; 248320 x 5120 at M = 8 54.1 / 51.0.
#ifndef LL_W1_STREAM_FUSE_MAXM
#define LL_W1_STREAM_FUSE_MAXM 2
#endif
#ifndef LL_W1_STREAM_DEPTH
#define LL_W1_STREAM_DEPTH 3                               // windows of weights in flight per wave
#endif
// SCV (G >= 128, K a multiple of 1024): a window's scales of one row are one
// aligned 16- or 8-byte vector, loaded by lanes 0..31 in one instruction
// (else one fp16 per lane and load).
// KSPLIT (a matrix with fewer 32-row blocks than half the resident waves):
// each block is one wave's only work, and ks consecutive waves of a
// workgroup (ks a power of two dividing WV) split its windows, so a wave
// waits on fewer windows in a row.  Each wave leaves its per-row sums in its
// own tile; after a workgroup barrier the block's first wave adds the ks
// shares in order and writes y.  The fp64 sums of s_g d_g terms are exact
// (see the windowed product), so the split does not change a bit.
constexpr int kRedBytes = 2 * 16 * 8 * 8;                 // [2 cb][16 rows][8 pairs] fp64 epilogue sums
// The product of workgroup wg of nwg working on one matrix (lds: the
// workgroup's dynamic LDS).
template <int G, int PK, bool FUSED, int WV, bool SCV, bool KSPLIT>
__device__ __forceinline__ void w1_stream_body(const uint32_t* __restrict__ bits, const uint16_t* __restrict__ scales,
                                               int64_t N, int64_t K, int M, const void* __restrict__ ws,
                                               const float* __restrict__ xs, const float* __restrict__ bias,
                                               float* __restrict__ y, uint16_t* __restrict__ y16, int ks, int64_t wg,
                                               int64_t nwg, char* __restrict__ lds) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nl = lane & 15, q = lane >> 4;
    constexpr int S = G >= 128 ? 1 : 128 / G;
    const int R = w1_arows(M, G);
    constexpr int stride = w1_stream_stride(G);
    constexpr int ngw = kWinK1 / G;
    const int64_t ng = K / G, nchunk = K / 128;
    const uint32_t rowbytes = uint32_t(K / 8);
    const int nwin = int((K + kWinK1 - 1) / kWinK1);
    char* wtile = lds + wave * kW1RowsPerWave * stride;
    float* wbias = reinterpret_cast<float*>(lds + WV * kW1RowsPerWave * stride) + wave * kW1RowsPerWave;
    char* abase = lds + WV * kW1RowsPerWave * (stride + 4);
    const int64_t ngp = w1_qs_stride(K, G);                // group sums per token row (padded)
    float* qs_all = reinterpret_cast<float*>(abase + nchunk * R * kARow);
    float* xs_l = qs_all + M * ngp + 4;

    // The wave's share: 32-row blocks wid, wid + W, ...; T windows in all.
    // Its first windows are requested before the A operand is staged, so the
    // two latencies overlap.
    const int64_t nwb = (N + kW1RowsPerWave - 1) / kW1RowsPerWave;
    const int64_t W = nwg * WV;
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // uniform: scalar cursors
    // KSPLIT: wave wv works on block wv / ks of the workgroup, windows [wlo, whi)
    const int kss = KSPLIT ? wv % ks : 0;
    const int64_t wid = KSPLIT ? wg * (WV / ks) + wv / ks : wg * WV + wv;
    const int wlo = KSPLIT ? int(int64_t(nwin) * kss / ks) : 0;
    const int whi = KSPLIT ? int(int64_t(nwin) * (kss + 1) / ks) : nwin;
    const int64_t T = KSPLIT ? (wid < nwb ? whi - wlo : 0) : (wid < nwb ? (nwb - wid + W - 1) / W : 0) * nwin;

    // Loads are buffer loads whose resource starts at the window's first byte
    // (row n0, window w) and ends with the array: a lane offset past the end
    // (rows beyond N, the last row's bytes beyond K) reads zeros, and every
    // per-window address is scalar.  The lanes' offsets are fixed.
    const int lr = lane >> 3, lc = lane & 7;               // weight loads: 8 rows x 128 B, lane -> row 8i + lr, bytes 16 lc
    constexpr int kSc = kW1RowsPerWave * ngw / 64;          // scale loads per lane and window (one fp16 each)
    static_assert(kW1RowsPerWave * ngw % 64 == 0 && 64 % ngw == 0, "a window's scales fill whole loads");
    uint32_t woff[4], soff[kSc];
#pragma unroll
    for (int i = 0; i < 4; ++i) woff[i] = uint32_t(8 * i + lr) * rowbytes + 16 * lc;
#pragma unroll
    for (int u = 0; u < kSc; ++u) {
        const int e = lane + 64 * u;
        soff[u] = uint32_t((int64_t(e / ngw) * ng + e % ngw) * 2);
    }
    static_assert(!SCV || G >= 128, "row-vector scale loads: at most 8 scales per row and window");
    const uint32_t svoff = uint32_t(lane) * uint32_t(ng) * 2;   // SCV: row lane's scales of the window
    const uint32_t boff = 4 * uint32_t(lane & 31);
    const uint8_t* bits8 = reinterpret_cast<const uint8_t*>(bits);
    const uint8_t* sc8 = reinterpret_cast<const uint8_t*>(scales);
    const int64_t wbytes = N * int64_t(rowbytes), sbytes = N * ng * 2;
    struct Regs {
        i32x4 w[4];
        uint16_t sc[SCV ? 1 : kSc];
        i32x4 s4;                                          // SCV
        float b;                                           // the block's bias (its first window only)
    };
    // The wave's windows in order: window w of the block starting at row n0.
    // Loads, stores to the tile and multiplies each walk them with a cursor
    // of their own; loads past the last window repeat it (never multiplied).
    int64_t ln0 = wid * kW1RowsPerWave, lt = 0;
    int lw = wlo, sw = wlo, cw = wlo;
    int64_t cn0 = wid * kW1RowsPerWave;
    auto load = [&](Regs& r) {
        const int64_t n0 = ln0;
        const int w = lw;
        if (++lt < T && ++lw == nwin) {
            lw = 0;
            ln0 += W * kW1RowsPerWave;
        }
        const int64_t w0 = n0 * int64_t(rowbytes) + int64_t(w) * kWinB1;
        const auto wr = buffer_rsrc(bits8 + w0, wbytes - w0);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.w[i] = buffer_ld16_stream(wr, woff[i]);
        const int64_t s0 = (n0 * ng + int64_t(w) * ngw) * 2;
        const auto sr = buffer_rsrc(sc8 + s0, sbytes - s0);
        if constexpr (SCV) {
            if (lane < kW1RowsPerWave) {
                if constexpr (ngw == 8)
                    r.s4 = buffer_ld16(sr, svoff);
                else
                    r.s4 = buffer_ld8(sr, svoff);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSc; ++u) r.sc[u] = buffer_ld2(sr, soff[u]);
        }
        if (w == 0 && lane < kW1RowsPerWave) {                 // the bias rides with a block's first window
            const auto br = buffer_rsrc(bias ? bias + n0 : xs, bias ? (N - n0) * 4 : 0);
            r.b = __builtin_bit_cast(float, buffer_ld4(br, boff));
        }
    };
    constexpr int D = G >= 128 ? LL_W1_STREAM_DEPTH : 2;  // (small groups: many scale registers per window)
    Regs r[D];

    // A of the whole K range, once per workgroup.  FUSED: digit rows formed
    // here from xq [M][K]; the hi-digit pieces of a (chunk, token) are 8
    // aligned lanes whose source sums add up to the group sum (G = 128:
    // chunk = group).  The sources of the first pieces are requested before
    // the weights, so converting them waits on them alone.
    const int64_t apieces = nchunk * R * 8;
    const int8_t* xq = static_cast<const int8_t*>(ws);
    auto piece_src = [&](int64_t pc) {
        const int64_t c = pc / (8 * R);
        const int rem = int(pc % (8 * R));
        const int u = rem & 7, m = rem >> 4, qp = 2 * (u & 1) + (u >> 2);
        return xq + int64_t(m) * K + 128 * c + 32 * qp;
    };
    auto put_piece = [&](int64_t p, const i32x4& lo4, const i32x4& hi4) {
        const int64_t pc = p < apieces ? p : apieces - 1;
        const int64_t c = pc / (8 * R);
        const int rem = int(pc % (8 * R));
        const int u = rem & 7, h = (rem >> 3) & 1, m = rem >> 4;
        int sum;
        const i32x4 d = w1_piece(lo4, hi4, u, h, true, sum);
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        sum += __shfl_xor(sum, 4, 64);
        if (p < apieces) {
            *reinterpret_cast<i32x4*>(abase + (p >> 3) * kARow + 16 * (p & 7)) = d;
            if (u == 0 && h == 0) qs_all[int64_t(m) * ngp + c] = float(sum);
        }
    };
    constexpr int kPre = FUSED ? 3 : 0;                    // pieces per thread requested ahead of the weights
    i32x4 pre[kPre > 0 ? kPre : 1][2];
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int64_t p = tid + 64 * WV * i;
        const int8_t* src = piece_src(p < apieces ? p : apieces - 1);
        pre[i][0] = ld16(src);
        pre[i][1] = ld16(src + 16);
    }
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < D; ++i) load(r[i]);
    }
    if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < kPre; ++i) put_piece(tid + 64 * WV * i, pre[i][0], pre[i][1]);
        for (int64_t p0 = 64 * WV * kPre; p0 < apieces; p0 += 64 * WV) {
            const int64_t p = p0 + tid;
            const int8_t* src = piece_src(p < apieces ? p : apieces - 1);
            put_piece(p, ld16(src), ld16(src + 16));
        }
    } else {
        const int8_t* Ag = static_cast<const int8_t*>(ws);
        const int32_t* qsg = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + (w1_a_bytes(M, K, G) + 15) / 16 * 16);
        for (int64_t p = tid; p < apieces; p += 64 * WV)
            *reinterpret_cast<i32x4*>(abase + (p >> 3) * kARow + 16 * (p & 7)) = ld16(Ag + 16 * p);
        for (int64_t e = tid; e < M * ng; e += 64 * WV) qs_all[(e / ng) * ngp + e % ng] = float(ld32(qsg + e));
    }
    if (tid < M) xs_l[tid] = xs[tid];
    __syncthreads();
    if (!KSPLIT && T == 0) return;

    static_assert(kW1RowsPerWave * stride >= kRedBytes + 8 * kW1RowsPerWave * 8,
                  "a block's epilogue sums and (KSPLIT) its share for up to 8 tokens fit the tile");
    char* wt_lane = wtile + lr * stride + 16 * lc;          // + 8 i stride: this lane's 16 weight bytes of row 8i + lr
    char* st_lane = wtile + (lane / ngw) * stride + kWinB1 + 2 * (lane % ngw);   // + (64 u / ngw) stride: scale u
    auto store_w = [&](const Regs& r) {
        const int w = sw;
        sw = sw + 1 == nwin ? 0 : sw + 1;
        if (uint32_t(w + 1) * kWinB1 <= rowbytes) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(wt_lane + 8 * i * stride) = r.w[i];
        } else {
            const bool ok = uint32_t(w) * kWinB1 + 16 * lc < rowbytes;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<i32x4*>(wt_lane + 8 * i * stride) = ok ? r.w[i] : i32x4{0, 0, 0, 0};
        }
        if constexpr (SCV) {
            if (lane < kW1RowsPerWave) {
                if constexpr (ngw == 8)
                    *reinterpret_cast<i32x4*>(wtile + lane * stride + kWinB1) = r.s4;
                else
                    *reinterpret_cast<i32x2*>(wtile + lane * stride + kWinB1) = i32x2{r.s4[0], r.s4[1]};
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSc; ++u) *reinterpret_cast<uint16_t*>(st_lane + (64 * u / ngw) * stride) = r.sc[u];
        }
        if (w == 0 && lane < kW1RowsPerWave) wbias[lane] = r.b;
    };

    f32x4 acc[2];
    double sacc[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        sacc[cb][0] = sacc[cb][1] = 0.0;
    }
    constexpr int cpg = G >= 128 ? G / 128 : 1;             // chunks per unit (a group, or one chunk of S groups)
    constexpr int kSet = cpg * PK;                          // chunks per packed set
    constexpr int kSets = (kChunks + kSet - 1) / kSet;
    constexpr int kGStep = G >= 128 ? PK : PK * S;          // groups per set
    // Lane row nl of the A operand: PK == 1 row nl; else slot sl = nl / R,
    // row rl = nl % R (no slot: nl >= PK R).  A lane always holds its own
    // unit's A row.  Unit u of a packed set is multiplied with the A block
    // scale 1 (E8M0 127) on the rows of slot u and 2^-127 (E8M0 0) on all
    // others: a row of another slot then adds terms below 2^-121 (|digit| <=
    // 32, b <= 2) to sums that are integers, below 2^-110 in all, which the
    // fp32 sums round away (a row summing to 0 stays below 1 and int() gives
    // 0).  So one A read serves all PK units of a set and no zero rows are
    // read.
    const int sl = PK == 1 ? 0 : (nl < PK * R ? nl / R : PK), rl = PK == 1 ? nl : nl % R;
    const bool has_row = PK == 1 ? nl < R : sl < PK;
    const int own_sl = has_row ? sl : 0, own_rl = has_row ? rl : 0;    // rowless lanes read any A row
    const char* a_lane = abase + (own_sl * cpg * R + own_rl) * kARow + 32 * q;   // + (window chunk of unit 0) R kARow
    uint32_t sa[2] = {0u, 0u};                              // E8M0 block scale of unit u: byte u % 4 of sa[u / 4]
#pragma unroll
    for (int u = 0; u < PK; ++u)
        if (has_row && sl == u) sa[u / 4] |= 127u << (8 * (u % 4));
    const char* b_lane = wtile + nl * stride + 4 * q;       // + 16 cb stride + 16 c: word of chunk c
    // epilogue pairs: lane slot tt holds pair pp = 2 q + tt = (k M + m) S + j
    int g0[2], qb[2];
    bool sok[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int pp = 2 * q + tt;
        const int sp = PK == 1 ? 0 : pp / (M * S);
        const int p = PK == 1 ? pp : pp % (M * S);
        const int m = p / S, j = p % S;
        sok[tt] = PK == 1 || sp < PK;
        g0[tt] = sok[tt] ? (G >= 128 ? sp : sp * S + j) : 0;   // group within the set
        qb[tt] = sok[tt] ? (m < M ? m : 0) * int(ngp) + g0[tt] : 0;   // outside: not read
    }
    // One window's multiply.  FULL (every chunk of the window inside K): no
    // exit between chunks, so every LDS read of the window (A rows, weight
    // words, the epilogues' scales and group sums) is issued ahead of the
    // chain of matrix products.
    auto compute = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int w = cw;
        const char* a_w = a_lane + int64_t(w) * kChunks * R * kARow;
        uint32_t wd[kChunks][2];
        float scv[kSets][2][2];
        float qsv[kSets][2];
        bool okv[kSets][2];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) wd[c][cb] = *reinterpret_cast<const uint32_t*>(b_lane + 16 * cb * stride + 16 * c);
        }
        if constexpr (FULL && PK == 1 && ngw == 8 && kSets == 8) {
            // one token pair per lane slot, a whole window of eight groups:
            // a row's eight scales are one 16-byte read of its tile row, a
            // token's eight group sums two 16-byte reads (rows of ngp floats)
            i32x4 sv[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) sv[cb] = *reinterpret_cast<const i32x4*>(wtile + (16 * cb + nl) * stride + kWinB1);
            f32x4 qv[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const float* qp = qs_all + qb[tt] + int64_t(w) * ngw;
                qv[tt][0] = *reinterpret_cast<const f32x4*>(qp);
                qv[tt][1] = *reinterpret_cast<const f32x4*>(qp + 4);
            }
#pragma unroll
            for (int st = 0; st < kSets; ++st)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    okv[st][tt] = true;
                    qsv[st][tt] = qv[tt][st >> 2][st & 3];
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        scv[st][cb][tt] = half_bits_to_float(uint16_t(uint32_t(sv[cb][st >> 1]) >> (16 * (st & 1))));
                }
        } else
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                int gi = g0[tt] + st * kGStep;                      // group within the window
                bool ok = sok[tt];
                if (!FULL) {
                    ok = ok && int64_t(w) * ngw + gi < ng;
                    gi = ok ? gi : 0;
                }
                okv[st][tt] = ok;
                qsv[st][tt] = sok[tt] ? qs_all[qb[tt] + int64_t(w) * ngw + (gi - g0[tt])] : 0.0f;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    scv[st][cb][tt] = half_bits_to_float(
                        *reinterpret_cast<const uint16_t*>(wtile + (16 * cb + nl) * stride + kWinB1 + 2 * gi));
            }
        }
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
            // the lane's own A rows for this set: chunk st kSet + sl cpg + i
            i32x8 av[cpg];
#pragma unroll
            for (int i = 0; i < cpg; ++i) {
                const char* ap = a_w + (st * kSet + i) * R * kARow;
                if (!FULL && int64_t(w) * kChunks + st * kSet + own_sl * cpg + i >= nchunk) ap = a_lane;   // past K: any row
                const i32x4 lo = *reinterpret_cast<const i32x4*>(ap);
                const i32x4 hi = *reinterpret_cast<const i32x4*>(ap + 16);
                av[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int u = 0; u < PK; ++u) {
#pragma unroll
                for (int i = 0; i < cpg; ++i) {
                    const int c = st * kSet + u * cpg + i;
                    if (c >= kChunks) continue;
                    const int64_t cg = int64_t(w) * kChunks + c;
                    if (!FULL && cg >= nchunk) continue;
                    const bool first = u == 0 && i == 0;
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[cb] = w1_mfma_unit(u % 4, av[i], w1_bv(wd[c][cb]), first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[cb],
                                               int(sa[u / 4]));
                    if ((c % kSet) == kSet - 1 || (!FULL && cg + 1 == nchunk)) {
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                            for (int tt = 0; tt < 2; ++tt) {
                                const float v = __builtin_fmaf(16.0f, acc[cb][2 * tt], acc[cb][2 * tt + 1]);
                                // the group dot v - sum q, exact in fp32 (integers below 2^17); with
                                // packed slots a pair outside them has v below 1, truncated to 0, and
                                // a zero group sum: it adds 0; in a cut window a group past K adds 0 * d
                                const float d = __fsub_rn(PK == 1 ? v : __builtin_truncf(v), qsv[st][tt]);
                                const double sc = FULL || okv[st][tt] ? double(scv[st][cb][tt]) : 0.0;
                                sacc[cb][tt] = __builtin_fma(sc, double(d), sacc[cb][tt]);
                            }
                        }
                    }
                }
            }
        }
    };
    // y[m][n] = (float)((double)xs[m] * S[m][n]) (+ bias) for the block whose
    // last window was just multiplied: pair p = (k M + m) S + j (pack slot k)
    // of lane quarter p / 2, slot p % 2; lane (row col, token parity) adds its
    // token's pairs
    auto finish = [&]() {
        const int64_t n0 = cn0;
        double* red = reinterpret_cast<double*>(wtile);    // [2 cb][16 nl][8 pairs] (kRedBytes)
        const int col = lane & 31;
        const float bias_v = wbias[col];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                red[(cb * 16 + nl) * 8 + 2 * q + tt] = sacc[cb][tt];
                sacc[cb][tt] = 0.0;
            }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const int64_t n = n0 + col;
        for (int m = lane >> 5; m < M; m += 2) {
            double sum = 0.0;
            for (int k = 0; k < PK; ++k)
                for (int j = 0; j < S; ++j) sum += red[col * 8 + (k * M + m) * S + j];
            if (n < N) {
                float out = float(double(xs_l[m]) * sum);
                if (bias) out = __fadd_rn(out, bias_v);
                if (y16)
                    y16[int64_t(m) * N + n] = f32_to_bf16_rne(out);
                else
                    y[int64_t(m) * N + n] = out;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    // multiply the window in the tile; after a block's last window, its epilogue
    auto step = [&]() {
        if (int64_t(cw + 1) * kChunks <= nchunk)
            compute(std::true_type{});
        else
            compute(std::false_type{});
        if (!KSPLIT && cw + 1 == nwin) {
            finish();
            cw = 0;
            cn0 += W * kW1RowsPerWave;
        } else {
            ++cw;
        }
    };

    // Window t is multiplied from the tile while windows t + 1 ... t + D - 1
    // wait in registers and window t + D is being fetched into the
    // registers window t came in.
    if (T > 0) {
        store_w(r[0]);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        int64_t t = 0;
        for (; t + D <= T; t += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                load(r[i]);                                // window t + i + D
                step();                                    // window t + i
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                store_w(r[(i + 1) % D]);                   // window t + i + 1
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
        }
#pragma unroll
        for (int i = 0; i < D - 1; ++i) {                  // the last T - t < D windows, all loaded
            if (t + i < T) {
                step();
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                store_w(r[(i + 1) % D]);
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
        }
    }
    if constexpr (KSPLIT) {
        // this wave's share of its block (zero without windows): per row col
        // and token m, share[m][col] at kRedBytes in its own tile, which no
        // store of a window touches any more
        double* red = reinterpret_cast<double*>(wtile);
        double* share = reinterpret_cast<double*>(wtile + kRedBytes);
        const int col = lane & 31;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) red[(cb * 16 + nl) * 8 + 2 * q + tt] = sacc[cb][tt];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        for (int m = lane >> 5; m < M; m += 2) {
            double sum = 0.0;
            for (int k = 0; k < PK; ++k)
                for (int j = 0; j < S; ++j) sum += red[col * 8 + (k * M + m) * S + j];
            share[m * kW1RowsPerWave + col] = sum;
        }
        __syncthreads();
        if (kss == 0 && wid < nwb) {
            const int64_t n = wid * kW1RowsPerWave + col;
            for (int m = lane >> 5; m < M; m += 2) {
                double sum = 0.0;
                for (int k2 = 0; k2 < ks; ++k2)
                    sum += reinterpret_cast<const double*>(lds + (wv + k2) * kW1RowsPerWave * stride +
                                                           kRedBytes)[m * kW1RowsPerWave + col];
                if (n < N) {
                    float out = float(double(xs_l[m]) * sum);
                    if (bias) out = __fadd_rn(out, bias[n]);
                    if (y16)
                        y16[int64_t(m) * N + n] = f32_to_bf16_rne(out);
                    else
                        y[int64_t(m) * N + n] = out;
                }
            }
        }
    }
}

template <int G, int PK, bool FUSED, int WV, bool SCV, bool KSPLIT>
__global__ void __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(LL_W1_STREAM_WPE))) w1_stream_kernel(const uint32_t* __restrict__ bits,
                                                                 const uint16_t* __restrict__ scales, int64_t N,
                                                                 int64_t K, int M, const void* __restrict__ ws,
                                                                 const float* __restrict__ xs,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ y, uint16_t* __restrict__ y16,
                                                                 int ks) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    w1_stream_body<G, PK, FUSED, WV, SCV, KSPLIT>(bits, scales, N, K, M, ws, xs, bias, y, y16, ks, blockIdx.x, gridDim.x,
                                                  lds);
}

template <int G, int MT, int NP, int PK, bool FUSED = false>
hipError_t launch_w1(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                     const float* xs, const float* bias, float* y, int nsplit, double* part, int32_t* counters,
                     uint16_t* y16, hipStream_t stream) {
    const dim3 grid{unsigned((N + kW1Rows - 1) / kW1Rows * nsplit)}, block{64 * kW1Waves};
    size_t lds = size_t(w1_lds_bytes(M, G));
    const size_t red = size_t(kW1Waves) * 2 * 16 * 8 * MT * sizeof(double);
    lds = lds > red ? lds : red;
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(w1_gemv_kernel<G, MT, NP, PK, FUSED>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((w1_gemv_kernel<G, MT, NP, PK, FUSED>), grid, block, lds, stream, bits, sc, N, K, M, ws, xs, bias,
                       y, nsplit, part, counters, y16);
    return hipGetLastError();
}

#ifndef LL_W1_STREAM_A_MAX8
#define LL_W1_STREAM_A_MAX8 (112 * 1024)                   // A bytes up to which the streaming product runs
#endif

// Workgroups of a kernel resident on the whole device at once (cached per
// kernel, LDS size and device).
int resident_wgs(const void* kernel, int threads, size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::vector<std::tuple<const void*, size_t, int, int>> seen;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : seen)
        if (std::get<0>(e) == kernel && std::get<1>(e) == lds && std::get<2>(e) == dev) return std::get<3>(e);
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, lds) != hipSuccess) return 0;
    const int n = cus * per;
    seen.emplace_back(kernel, lds, dev, n);
    return n;
}

bool w1_streamed(int64_t N, int64_t K, int G, int64_t Mb);

#ifndef LL_W1_STREAM_KSPLIT
#define LL_W1_STREAM_KSPLIT 1                              // split the windows of short matrices over waves
#endif
template <int G, int PK, bool FUSED, int WV, bool SCV>
hipError_t launch_w1_stream_wv(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                               const float* xs, const float* bias, float* y, uint16_t* y16, hipStream_t stream) {
    const void* kern = reinterpret_cast<const void*>(w1_stream_kernel<G, PK, FUSED, WV, SCV, false>);
    const size_t lds = size_t(w1_stream_lds_bytes(M, K, G, WV));
    hipError_t e = allow_dynamic_lds(kern, lds);
    if (e != hipSuccess) return e;
    const int slots = resident_wgs(kern, 64 * WV, lds);
    if (slots <= 0) return hipErrorInvalidConfiguration;
    const int64_t nwb = (N + kW1RowsPerWave - 1) / kW1RowsPerWave;
    const int64_t nwin = (K + kWinK1 - 1) / kWinK1;
    // KSPLIT: the split with the fewest windows per wave whose workgroups are
    // all resident at once (the smaller split on a tie)
    int ks = 1;
    if (LL_W1_STREAM_KSPLIT && nwb * 2 <= int64_t(slots) * WV)
        for (int k = 2; k <= WV; k *= 2)
            if ((nwb + WV / k - 1) / (WV / k) <= slots && (nwin + k - 1) / k < (nwin + ks - 1) / ks) ks = k;
    if (ks > 1) {
        const void* kk = reinterpret_cast<const void*>(w1_stream_kernel<G, PK, FUSED, WV, SCV, true>);
        e = allow_dynamic_lds(kk, lds);
        if (e != hipSuccess) return e;
        const int64_t grid = (nwb + WV / ks - 1) / (WV / ks);
        hipLaunchKernelGGL((w1_stream_kernel<G, PK, FUSED, WV, SCV, true>), dim3{unsigned(grid)}, dim3{64 * WV}, lds,
                           stream, bits, sc, N, K, M, ws, xs, bias, y, y16, ks);
        return hipGetLastError();
    }
    // as many blocks for every wave as the fullest one needs: the grid is the
    // fewest workgroups that still give each wave at most that many
    const int64_t per_wave = (nwb + int64_t(slots) * WV - 1) / (int64_t(slots) * WV);
    const int64_t grid = (nwb + WV * per_wave - 1) / (WV * per_wave);
    hipLaunchKernelGGL((w1_stream_kernel<G, PK, FUSED, WV, SCV, false>), dim3{unsigned(grid)}, dim3{64 * WV}, lds, stream,
                       bits, sc, N, K, M, ws, xs, bias, y, y16, 1);
    return hipGetLastError();
}
// Eight waves per workgroup: one workgroup per CU (the register budget
// allows two waves per SIMD) sharing one staged copy of A.  Measured against
// four-wave workgroups (two per CU, each staging its own A) on the LM head
// 248320 x 5120: M = 1 36.6 -> 36.1 us, M = 2 41.3 -> 38.9, M = 4 53.8 -> 49.2.
template <int G, int PK, bool FUSED>
hipError_t launch_w1_stream_k(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                              const float* xs, const float* bias, float* y, uint16_t* y16, hipStream_t stream) {
    if constexpr (G >= 128) {
        if (K % kWinK1 == 0) return launch_w1_stream_wv<G, PK, FUSED, 8, true>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    }
    return launch_w1_stream_wv<G, PK, FUSED, 8, false>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
}

template <int G, bool F>
hipError_t launch_w1_stream_f(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                              const float* xs, const float* bias, float* y, uint16_t* y16, hipStream_t stream) {
    constexpr int kUnits = G >= 128 ? kChunks / (G / 128) : kChunks;
    constexpr int kMaxPk = G >= 128 ? kUnits : 8 / w1_slots(G);
    constexpr int P8 = kMaxPk < 8 ? kMaxPk : 8, P4 = kMaxPk < 4 ? kMaxPk : 4;
    switch (w1_pack(M, G)) {
    case 8: return launch_w1_stream_k<G, P8, F>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    case 4: return launch_w1_stream_k<G, P4, F>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    case 2: return launch_w1_stream_k<G, 2, F>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    default: return launch_w1_stream_k<G, 1, F>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    }
}
// fused: ws is xq [M][K] and each workgroup forms the A digits itself (G =
// 128 only); else ws holds the prepared operands of w1_prep_kernel.
template <int G>
hipError_t launch_w1_stream(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                            const float* xs, const float* bias, float* y, uint16_t* y16, bool fused,
                            hipStream_t stream) {
    if constexpr (G == 128) {
        if (fused) return launch_w1_stream_f<G, true>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
    }
    return launch_w1_stream_f<G, false>(bits, sc, N, K, M, ws, xs, bias, y, y16, stream);
}

// The preparation is fused into the product for G = 128 when every
// workgroup forming its own windows' digits costs less than the separate
// launch: that work grows with row blocks x A rows, and the measured break
// even lies between 224 (7168 rows, two tokens: 12.9 -> 11.4 us) and 272
// (17408 rows, one token: 17.1 -> 18.4 us).
bool w1_fused(int64_t N, int G, int64_t Mb) {
    const int64_t rbs = (N + kW1Rows - 1) / kW1Rows;
    return G == 128 && w1_arows(int(Mb), G) <= 16 && rbs * w1_arows(int(Mb), G) <= LL_W1_FUSE_WORK;
}

template <int G>
hipError_t launch_w1_g(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int M, const void* ws,
                       const float* xs, const float* bias, float* y, int nsplit, double* part, int32_t* counters,
                       bool fused, uint16_t* y16, hipStream_t stream) {
    constexpr int kUnits = G >= 128 ? kChunks / (G / 128) : kChunks;   // units per window
    constexpr int kMaxPk = G >= 128 ? kUnits : 8 / w1_slots(G);          // R >= 2 S
    constexpr int P8 = kMaxPk < 8 ? kMaxPk : 8, P4 = kMaxPk < 4 ? kMaxPk : 4;
    if constexpr (G == 128) {
        if (fused) {
            switch (w1_pack(M, G)) {
            case 8: return launch_w1<G, 1, 2, 8, true>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
            case 4: return launch_w1<G, 1, 2, 4, true>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
            case 2: return launch_w1<G, 1, 2, 2, true>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
            default: return launch_w1<G, 1, 2, 1, true>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
            }
        }
    }
    switch (w1_pack(M, G)) {
    case 8: return launch_w1<G, 1, 2, P8>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
    case 4: return launch_w1<G, 1, 2, P4>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
    case 2: return launch_w1<G, 1, 2, 2>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
    default: break;
    }
    if (w1_arows(M, G) <= 16) return launch_w1<G, 1, 2, 1>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
    return launch_w1<G, 2, 2, 1>(bits, sc, N, K, M, ws, xs, bias, y, nsplit, part, counters, y16, stream);
}

// Tokens per pass: the A rows of a pass (2 x tokens x slots) fit two row blocks.
int64_t w1_tokens_per_pass_max(int G) { return 16 / w1_slots(G); }

#ifndef LL_W1_TARGET_WGS
#define LL_W1_TARGET_WGS 256
#endif

// K splits: enough workgroups to spread a narrow matrix over the chip, at
// most one split per 1024-k window.
int w1_splits(int64_t N, int64_t K) {
    const int64_t rbs = (N + kW1Rows - 1) / kW1Rows;
    if (rbs > kMaxCounters) return 1;                  // one counter per row block
    const int64_t nwin = (K + kWinK1 - 1) / kWinK1;
    int64_t s = (LL_W1_TARGET_WGS + rbs - 1) / rbs;
    s = s < nwin ? s : nwin;
    s = s < kW1MaxSplits ? s : kW1MaxSplits;
    return int(s < 1 ? 1 : s);
}
// The streaming product: a matrix tall enough to run unsplit, A rows in one
// row block, the A operand of the whole K range small enough for LDS.
#ifndef LL_W1_STREAM_NARROW
#define LL_W1_STREAM_NARROW 1                              // short matrices stream too (their windows split over waves)
#endif
bool w1_streamed(int64_t N, int64_t K, int G, int64_t Mb) {
    return (LL_W1_STREAM_NARROW || w1_splits(N, K) == 1) && w1_arows(int(Mb), G) <= 16 &&
           w1_stream_a_bytes(int(Mb), K, G) <= LL_W1_STREAM_A_MAX8;
}
// Tokens per pass: up to two row blocks of A rows; half that when only the
// half pass can stream (two streamed passes read the weights twice and still
// beat one pass of the windowed product).
int64_t w1_tokens_per_pass(int64_t N, int64_t K, int G, int64_t M) {
    const int64_t tb = w1_tokens_per_pass_max(G);
    if (M > tb / 2 && !w1_streamed(N, K, G, M < tb ? M : tb) && w1_streamed(N, K, G, tb / 2)) return tb / 2;
    return tb;
}
// Split-K scratch after the pass operands: partial sums [rbs x nsplit x 128 rows x tokens] fp64.
size_t w1_split_off(int64_t Mp, int64_t K, int G) { return (w1_ws_bytes(Mp, K, G) + 255) / 256 * 256; }

// ---------------------------------------------------------------- prepared batches
// Many W1 products (G = 128, 1 <= M <= 8, the A operand of each within the
// streaming product's LDS) in two launches.  The first forms the operands of
// every distinct activation into the plan memory (the layout of
// w1_prep_kernel); the second runs every product's streaming product from
// them, the workgroups of all products in one grid (a table maps each
// workgroup to its product).  The host gives each product a number of
// workgroups so that all of them are resident at once and the longest
// stream of windows any wave has is as short as it can be; each wave then
// streams its blocks back to back, as in a single product.
struct W1Prob {              // one product
    const uint32_t* bits;
    const uint16_t* scales;
    const void* ops;         // prepared operands of its activation
    const float* xs;         // token scales [M]
    const float* bias;
    float* y;
    int64_t N, K;
    int64_t wg0, wgs;        // its first workgroup and workgroup count
};
struct W1Prep {              // one distinct activation
    const int8_t* xq;        // [M][K]
    void* ops;
    int64_t K;
    int64_t blk0, pblocks;   // its first block of the preparation launch; its piece blocks
};
constexpr int kW1BatchWaves = 8;

__global__ void __launch_bounds__(256) w1_batch_prep_kernel(const W1Prep* __restrict__ tab, int nprep, int M) {
    // this block's activation: the last entry whose first block is <= blockIdx.x
    const int64_t b = blockIdx.x;
    int lo = 0, hi = nprep - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (tab[mid].blk0 <= b) lo = mid;
        else hi = mid - 1;
    }
    const W1Prep& P = tab[lo];
    w1_prep_body(P.xq, M, P.K, 128, P.ops, P.pblocks, b - P.blk0);
}

template <int PK, bool SCV>
__global__ void __launch_bounds__(64 * kW1BatchWaves) __attribute__((amdgpu_waves_per_eu(LL_W1_STREAM_WPE)))
w1_batch_kernel(const W1Prob* __restrict__ tab, const int32_t* __restrict__ map, int M) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t wg = blockIdx.x;
    const W1Prob& P = tab[ld32(map + wg)];
    w1_stream_body<128, PK, false, kW1BatchWaves, SCV, false>(P.bits, P.scales, P.N, P.K, M, P.ops, P.xs, P.bias, P.y,
                                                              nullptr, 1, wg - P.wg0, P.wgs, lds);
}

template <int PK, bool SCV>
int w1_batch_resident(int M, int64_t kmax) {
    const size_t lds = size_t(w1_stream_lds_bytes(M, kmax, 128, kW1BatchWaves));
    const void* k = reinterpret_cast<const void*>(w1_batch_kernel<PK, SCV>);
    if (allow_dynamic_lds(k, lds) != hipSuccess) return 0;
    return resident_wgs(k, 64 * kW1BatchWaves, lds);
}

template <int PK, bool SCV>
hipError_t launch_w1_batch(const W1Prob* tab, const int32_t* map, int64_t wgs, int M, int64_t kmax, hipStream_t stream) {
    const size_t lds = size_t(w1_stream_lds_bytes(M, kmax, 128, kW1BatchWaves));
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(w1_batch_kernel<PK, SCV>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((w1_batch_kernel<PK, SCV>), dim3{unsigned(wgs)}, dim3{64 * kW1BatchWaves}, lds, stream, tab, map, M);
    return hipGetLastError();
}

}  // namespace

namespace llk {

size_t w1_workspace(int64_t M, int64_t N, int64_t K, int G) {
    const int64_t tb = w1_tokens_per_pass(N, K, G, M);
    const int64_t Mp = M < tb ? M : tb;
    const int ns = w1_splits(N, K);
    if (ns == 1) return w1_ws_bytes(Mp, K, G);
    const int64_t rbs = (N + kW1Rows - 1) / kW1Rows;
    return w1_split_off(Mp, K, G) + size_t(rbs) * ns * kW1Rows * Mp * 8;
}

hipError_t launch_w1_gemv(const uint32_t* bits, const uint16_t* scales, int64_t N, int64_t K, int G, const int8_t* xq,
                          const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                          hipStream_t stream, uint16_t* y16) {
    const int64_t tb = w1_tokens_per_pass(N, K, G, M);
    const int ns = w1_splits(N, K);
    const int64_t Mp = M < tb ? M : tb;
    double* part = ns > 1 ? reinterpret_cast<double*>(static_cast<char*>(ws) + w1_split_off(Mp, K, G)) : nullptr;
    for (int64_t m0 = 0; m0 < M; m0 += tb) {               // every pass reads the weights once
        const int64_t Mb = M - m0 < tb ? M - m0 : tb;
        const int8_t* xb = xq + m0 * K;
        const int R = w1_arows(int(Mb), G);
        const int64_t pieces = (K / 128) * R * 8;
        const int64_t pblocks = (pieces + 255) / 256;
        const int64_t items = Mb * (K / G);
        const bool streamed = w1_streamed(N, K, G, Mb);
        const bool fused = streamed ? G == 128 && LL_W1_STREAM_FUSE && Mb <= LL_W1_STREAM_FUSE_MAXM : w1_fused(N, G, Mb);
        if (!fused)
            hipLaunchKernelGGL(w1_prep_kernel, dim3{unsigned(pblocks + (items + 3) / 4)}, dim3{256}, 0, stream, xb, Mb,
                               K, G, ws, pblocks);
        const void* aop = fused ? static_cast<const void*>(xb) : static_cast<const void*>(ws);
        hipError_t e = hipSuccess;
        if (streamed) {
            float* yb = y16 ? nullptr : y + m0 * N;
            uint16_t* yb16 = y16 ? y16 + m0 * N : nullptr;
            switch (G) {
            case 32: e = launch_w1_stream<32>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, yb, yb16, fused, stream); break;
            case 64: e = launch_w1_stream<64>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, yb, yb16, fused, stream); break;
            case 128: e = launch_w1_stream<128>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, yb, yb16, fused, stream); break;
            default: e = launch_w1_stream<256>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, yb, yb16, fused, stream); break;
            }
            if (e != hipSuccess) return e;
            continue;
        }
        switch (G) {
        case 32:
            e = launch_w1_g<32>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, y + m0 * N, ns, part, counters, fused,
                                y16 ? y16 + m0 * N : nullptr, stream);
            break;
        case 64:
            e = launch_w1_g<64>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, y + m0 * N, ns, part, counters, fused,
                                y16 ? y16 + m0 * N : nullptr, stream);
            break;
        case 128:
            e = launch_w1_g<128>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, y + m0 * N, ns, part, counters, fused,
                                 y16 ? y16 + m0 * N : nullptr, stream);
            break;
        default:
            e = launch_w1_g<256>(bits, scales, N, K, int(Mb), aop, xs + m0, bias, y + m0 * N, ns, part, counters, fused,
                                 y16 ? y16 + m0 * N : nullptr, stream);
            break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool w1_batch_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= 8 && K % 128 == 0 && w1_stream_a_bytes(int(M), K, 128) <= LL_W1_STREAM_A_MAX8;
}
int64_t w1_batch_wgs(int64_t N) { return ((N + kW1RowsPerWave - 1) / kW1RowsPerWave + kW1BatchWaves - 1) / kW1BatchWaves; }
int64_t w1_batch_blocks(int64_t N) { return (N + kW1RowsPerWave - 1) / kW1RowsPerWave; }
int64_t w1_batch_prep_blocks(int64_t M, int64_t K) {
    const int64_t pieces = (K / 128) * w1_arows(int(M), 128) * 8;
    return (pieces + 255) / 256 + (M * (K / 128) + 3) / 4;
}
size_t w1_batch_operand_bytes(int64_t M, int64_t K) { return w1_ws_bytes(M, K, 128); }
size_t w1_batch_prob_bytes() { return sizeof(W1Prob); }
size_t w1_batch_prep_bytes() { return sizeof(W1Prep); }

int w1_batch_slots(int64_t M, int64_t kmax, bool scv) {
    const int m = int(M);
    switch (w1_pack(m, 128) * 2 + (scv ? 1 : 0)) {
    case 17: return w1_batch_resident<8, true>(m, kmax);
    case 16: return w1_batch_resident<8, false>(m, kmax);
    case 9: return w1_batch_resident<4, true>(m, kmax);
    case 8: return w1_batch_resident<4, false>(m, kmax);
    case 5: return w1_batch_resident<2, true>(m, kmax);
    case 4: return w1_batch_resident<2, false>(m, kmax);
    case 3: return w1_batch_resident<1, true>(m, kmax);
    default: return w1_batch_resident<1, false>(m, kmax);
    }
}

void fill_w1_prob(void* dst, const void* bits, const void* scales, const void* ops, const float* xs, const float* bias,
                  float* y, int64_t N, int64_t K, int64_t wg0, int64_t wgs) {
    W1Prob p;
    p.bits = static_cast<const uint32_t*>(bits);
    p.scales = static_cast<const uint16_t*>(scales);
    p.ops = ops;
    p.xs = xs;
    p.bias = bias;
    p.y = y;
    p.N = N;
    p.K = K;
    p.wg0 = wg0;
    p.wgs = wgs;
    *static_cast<W1Prob*>(dst) = p;
}

void fill_w1_prep(void* dst, const int8_t* xq, void* ops, int64_t M, int64_t K, int64_t blk0) {
    W1Prep p;
    p.xq = xq;
    p.ops = ops;
    p.K = K;
    p.blk0 = blk0;
    p.pblocks = ((K / 128) * w1_arows(int(M), 128) * 8 + 255) / 256;
    *static_cast<W1Prep*>(dst) = p;
}

hipError_t launch_w1_batch_prep(const void* prep_table, int nprep, int64_t blocks, int64_t M, hipStream_t stream) {
    hipLaunchKernelGGL(w1_batch_prep_kernel, dim3{unsigned(blocks)}, dim3{256}, 0, stream,
                       static_cast<const W1Prep*>(prep_table), nprep, int(M));
    return hipGetLastError();
}

hipError_t launch_w1_batch_product(const void* prob_table, const void* map, int64_t wgs, int64_t M, int64_t kmax,
                                   bool scv, hipStream_t stream) {
    const W1Prob* tab = static_cast<const W1Prob*>(prob_table);
    const int32_t* mp = static_cast<const int32_t*>(map);
    const int m = int(M);
    switch (w1_pack(m, 128) * 2 + (scv ? 1 : 0)) {
    case 17: return launch_w1_batch<8, true>(tab, mp, wgs, m, kmax, stream);
    case 16: return launch_w1_batch<8, false>(tab, mp, wgs, m, kmax, stream);
    case 9: return launch_w1_batch<4, true>(tab, mp, wgs, m, kmax, stream);
    case 8: return launch_w1_batch<4, false>(tab, mp, wgs, m, kmax, stream);
    case 5: return launch_w1_batch<2, true>(tab, mp, wgs, m, kmax, stream);
    case 4: return launch_w1_batch<2, false>(tab, mp, wgs, m, kmax, stream);
    case 3: return launch_w1_batch<1, true>(tab, mp, wgs, m, kmax, stream);
    default: return launch_w1_batch<1, false>(tab, mp, wgs, m, kmax, stream);
    }
}

}  // namespace llk
