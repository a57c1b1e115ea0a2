// Single-token decode product with fp32 activations (M = 1), i2_s or TQ2_0,
// on the fp4 x fp4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operands e2m1 and unit block scales).
//
// The product is y[n] = scale * sum_k w[n,k] x[k] with ternary w (BitNet
// b1.58 i2_s format: codes 00/01/10 for -1/0/+1, 128-element groups, one fp32
// tensor scale after the codes; llama.cpp TQ2_0: 256-element blocks of 2-bit
// two's-complement codes with an fp16 scale per block).
//
// Activation digits.  Let max|x| < 2^E.  Every element is rounded to the
// integer X = rint(x * 2^(34-E)), |X| < 2^34, and X is written with twelve
// balanced base-8 digits d_r in [-4, 3]:
//     X = sum_{r=0..11} d_r * 8^(11-r)
// (the digits of X + 4*(8^12-1)/7, each minus 4).  Every digit is an e2m1
// value, so the twelve digit planes are the rows of the fp4 operand A.  The
// rounding to X is the only approximation: |x - X 2^(E-34)| <= 2^(E-35) <=
// 2^-34 max|x|, so |y - y_exact| <= scale * K * 2^-34 * max|x|.  The bound
// the product promises is at least 1e-5 * scale * max|x| (sum|x| >= max|x|),
// so the engine takes K <= 2^17 (2^17 * 2^-34 = 7.6e-6); longer rows go to
// the int8-plane engine, whose truncation error is 2^-41 relative.
//
// Weights as fp4.  i2_s codes c = w + 1 in {0, 1, 2} are used as the e2m1
// bit patterns 0000 / 0001 / 0010, i.e. the values c/2; masking a code word
// with 0x33333333 (and the word shifted by 2) leaves two codes per byte in
// the low bits of two nibbles, so eight weights cost one or two operations.
// Then sum_k w x = 2 * sum_k (c/2) X - sum_k X, with sum_k X formed by the
// preparation.  TQ2_0 codes are turned into signed e2m1 halves (+-0.5 as
// 0001 / 1001) by moving the code's high bit to the nibble's sign bit, and
// each 256-k block's MFMA sum is multiplied by the block's fp16 scale (one
// token: into fp32 plane accumulators; several tokens: a lane first folds
// its four plane sums exactly, then adds the scaled fold in fp64).  Every
// MFMA sum is exact in fp32 (multiples of 1/2 below 2^23); the epilogue
// weights the planes by 8^(11-r) in fp64.
//
// Layout and parallelism.  MFMA lane l holds row (or column) l % 16 and the
// 32 k values 32 (l/16) + e of a 128-k step.  The 16 bytes of a weight row at
// byte 16 q of a 64-byte chunk (256 k: two i2_s groups, one TQ2_0 block)
// give lane quarter q the B operands of the chunk's two steps; the
// preparation writes the activation digits in exactly the k order this
// implies.  A wave owns 32 weight rows (two 16-row column blocks sharing each
// activation operand read) and fetches them per 1024 k with loads of 4 rows x
// 256 contiguous bytes (the shape the memory system streams fastest; a load
// in operand order touches 16 rows per 16 lanes), which go through a padded
// LDS tile private to the wave (a TQ2_0 row's block scales for the tile sit
// in its padding, one 2-byte load per lane and column block).  The workgroup's four waves share a
// double-buffered LDS window of activation digits, the only thing they
// synchronise on.  Loads run two tiles ahead of the multiply.  Workgroup ids
// are mapped so that the workgroups of one product run on one XCD and share
// its L2 copy of the activation digits.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int kPl = 12;                                // digit planes
constexpr int kPlRowBytes = 16;                        // 32 nibbles: one plane, one step, one lane quarter
constexpr int kQuarterBytes = kPl * kPlRowBytes;       // 192
constexpr int kStepBytes = 4 * kQuarterBytes;          // 768: one 128-k step
constexpr int kChunkBytes = 2 * kStepBytes;            // 1536: one 256-k chunk
constexpr int kSliceChunks = 8;                        // chunks per preparation workgroup
// 16-row column blocks per wave: two (one activation operand read feeds
// both), except for one token of i2_s, where one block per wave (64-row
// workgroups, twice as many) measured faster on the 30-layer decode step
// (5.62 -> 5.80 TB/s; the fused step 5.54 -> 5.66) while TQ2_0 and more
// tokens lost with it (TQ2_0 batch of 118 copies at M = 1: 6.15 -> 5.85 TB/s;
// M = 8: 2.32 -> 1.84).
#ifndef LL_F4_CB
#define LL_F4_CB 2
#endif
#ifndef LL_F4_CB_I2S1
#define LL_F4_CB_I2S1 1
#endif
__host__ __device__ constexpr int f4_cb(int FMT, int MT) { return FMT == 1 && MT == 1 ? LL_F4_CB_I2S1 : LL_F4_CB; }
#ifndef LL_F4_CUNROLL
#define LL_F4_CUNROLL 1                                // chunk loop of the multiply not unrolled (register use)
#endif
#ifndef LL_F4_NT
#define LL_F4_NT 1                                     // weights read with non-temporal loads
#endif
constexpr int kGroup = 4;                              // chunks per weight tile: 256 bytes of each row
#ifndef LL_F4_WAVES
#define LL_F4_WAVES 4
#endif
constexpr int kWaves = LL_F4_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kAWin = kGroup * kChunkBytes;            // activation digits of one tile's k range
constexpr int64_t kMaxK = int64_t(1) << 17;            // the rounding of x stays inside the tolerance (exact fp32 MFMA sums up to 2^20)

constexpr uint32_t kDigitNibbles = 0x5420ACDEu;        // nibble v: e2m1 code of the digit v - 4
constexpr uint32_t kBiasLo = 0x24924u, kBiasHi = 0x24924u;   // 4*(8^12-1)/7 split at bit 18

__host__ __device__ constexpr int64_t nchunks(int64_t K) { return (K + 255) / 256; }
__host__ __device__ constexpr int64_t nslices(int64_t K) { return (nchunks(K) + kSliceChunks - 1) / kSliceChunks; }
// After the digit planes: int32 E at meta + 0, the slices' int64 sums of X at meta + 8 + 8 s.
__host__ __device__ constexpr int64_t meta_off(int64_t K) { return nchunks(K) * kChunkBytes; }
__host__ __device__ constexpr int64_t op_bytes(int64_t K) { return meta_off(K) + 8 + 8 * nslices(K); }

struct F4Prep {
    const float* x;
    void* ops;
    int64_t K;
    // RMSNorm prologue [BL "Fused RMSNorm + BitLinear + Residual Add M=1
    // Kernel"], or NULL: the operand is xn = (x * rinv) * norm_w with
    // rinv = 1 / sqrt(sum x^2 / K + eps) (0 for a zero row with eps = 0).
    const float* norm_w;
    float eps;
};

struct F4Prob {
    const uint8_t* codes;
    const uint16_t* scales;       // TQ2_0 block scales, [N][K/256]
    const uint8_t* ops;           // prepared digits of its activation
    const float* bias;
    float* y;
    int64_t N, K;
    int64_t wg0;                  // first (logical) workgroup of this product
    // Gated pair [BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"]: codes/scales are
    // the gate, codes2/scales2 the up weights (same N, K, x);
    // y = (r * r) * u with r = max(0, gate), u = up.
    const uint8_t* codes2;
    const uint16_t* scales2;
    int32_t pair;
    int32_t M;                    // tokens (1 .. 16): token m's digits at ops + m opstride, y row m
    int64_t opstride;
};

// ---------------------------------------------------------------- digits
struct TokScale {
    int E;                        // max|x| < 2^E
    float f1, f2;                 // x * f1 * f2 = x * 2^(34 - E), both factors exact powers of two
};

// 1 / sqrt(sum x^2 / K + eps) of a token row, rounded once to fp32 (sum and
// root in fp64), by the 256 threads of a workgroup (barrier inside).
// The row is read in batches of kRowBatch 16-byte loads per thread, all
// requested before any is used (clamped to the row; the copies past it are
// not counted).  The first batch, the whole row up to 8192 elements, is
// straight-line code, so its loads overlap every load issued before it.
constexpr int kRowBatch = 8;

__device__ __forceinline__ float rms_inv(const float* x, int64_t K, float eps, int tid, double* sacc) {
    double ss = 0.0;
    const int64_t n4 = K / 4;
    auto batch = [&](int64_t i0) {
        f32x4 u[kRowBatch];
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            const int64_t i = i0 + 256 * b;
            u[b] = ld16f(x + 4 * (i < n4 ? i : n4 - 1));
        }
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b)
            if (i0 + 256 * b < n4)
                ss += (double(u[b][0]) * u[b][0] + double(u[b][1]) * u[b][1]) +
                      (double(u[b][2]) * u[b][2] + double(u[b][3]) * u[b][3]);
    };
    batch(tid);
    for (int64_t i0 = tid + 256 * kRowBatch; i0 < n4; i0 += 256 * kRowBatch) batch(i0);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    if ((tid & 63) == 0) sacc[tid >> 6] = ss;
    __syncthreads();
    const double d = (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
    const double den = d / double(K) + double(eps);
    return den > 0.0 ? float(1.0 / sqrt(den)) : 0.0f;
}

// max |x| (or |xn| with a norm: xn = (x * rinv) * w) over a token row, by the
// 256 threads of a workgroup (barrier inside).
__device__ __forceinline__ TokScale token_scale(const float* x, const float* w, float rinv, int64_t K, int tid,
                                                float* smax) {
    float mx = 0.0f;
    const int64_t n4 = K / 4;
    auto batch = [&](int64_t i0) {
        f32x4 u[kRowBatch], g[kRowBatch];
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            const int64_t i = i0 + 256 * b, ic = i < n4 ? i : n4 - 1;
            u[b] = ld16f(x + 4 * ic);
            if (w) g[b] = ld16f(w + 4 * ic);
        }
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            if (i0 + 256 * b >= n4) continue;              // a clamped copy
            if (w)
#pragma unroll
                for (int e = 0; e < 4; ++e) u[b][e] = __fmul_rn(__fmul_rn(u[b][e], rinv), g[b][e]);
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(u[b][0]), fabsf(u[b][1])), fmaxf(fabsf(u[b][2]), fabsf(u[b][3]))));
        }
    };
    batch(tid);
    for (int64_t i0 = tid + 256 * kRowBatch; i0 < n4; i0 += 256 * kRowBatch) batch(i0);
    mx = wave_max(mx);
    if ((tid & 63) == 0) smax[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    TokScale ts;
    ts.E = 0;
    (void)frexpf(mx, &ts.E);                               // E = 0 when mx == 0
    const int sh = 34 - ts.E;                              // in [-94, 183]
    const int sa = sh < 120 ? sh : 120;
    ts.f1 = ldexpf(1.0f, sa);
    ts.f2 = ldexpf(1.0f, sh - sa);
    return ts;
}

// Digits of NE elements: nibble e of out[r] = e2m1 code of digit r of element
// e (element e at bits 4e); xsum += their X.
template <int NE>
__device__ __forceinline__ void make_digits(const float (&v)[NE], const TokScale& ts, uint32_t (&out)[kPl],
                                            long long& xsum) {
#pragma unroll
    for (int r = 0; r < kPl; ++r) out[r] = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const float t = rintf((v[e] * ts.f1) * ts.f2);     // X, an integer-valued float, |X| < 2^34
        const float th = floorf(t * 0x1p-18f);             // X = th 2^18 + tl, 0 <= tl < 2^18 (both exact)
        const float tl = fmaf(th, -0x1p18f, t);
        const int hi = int(th), lo = int(tl);
        xsum += (long long)hi * (1 << 18) + lo;
        const uint32_t l2 = uint32_t(lo) + kBiasLo;        // X + bias = H 2^18 + L
        const uint32_t L = l2 & 0x3FFFFu;
        const uint32_t H = uint32_t(hi + int(kBiasHi) + int(l2 >> 18));
#pragma unroll
        for (int r = 0; r < kPl; ++r) {
            const uint32_t src = r < 6 ? H : L;
            const int o = 3 * (5 - (r % 6));
            const uint32_t d = (src >> o) & 7u;
            out[r] |= ((kDigitNibbles >> (4 * d)) & 15u) << (4 * e);
        }
    }
}

// ---------------------------------------------------------------- preparation
// Workgroup (token, slice): digits of chunks [8 slice, 8 slice + 8).  Thread
// t: chunk 8 slice + t/32, step s = (t/16) % 2, lane quarter q = (t/4) % 4,
// dword j = t % 4 of the quarter's 16-byte plane rows: eight elements, whose
// digits fill nibbles e = 2b + h (b = 0..3, h = 0..1) of twelve dwords.
template <int FMT>
__global__ void __launch_bounds__(256) f4_prep_kernel(const F4Prep* __restrict__ tab) {
    const F4Prep& P = tab[blockIdx.x];
    const int64_t K = P.K;
    const int slice = int(blockIdx.y);
    if (slice >= nslices(K)) return;                       // whole workgroup
    const float* x = P.x;
    const float* nw = P.norm_w;
    uint8_t* ops = static_cast<uint8_t*>(P.ops);
    __shared__ float smax[4];                              // four waves
    __shared__ long long ssum[4];
    __shared__ double sacc[4];
    const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6;

    const int lc = tid >> 5, s = (tid >> 4) & 1, q = (tid >> 2) & 3, j = tid & 3;
    const int64_t c = int64_t(slice) * kSliceChunks + lc;
    const bool live = c < nchunks(K);
    // This thread's elements are requested first and used only after the
    // row's max |x|, so the two sets of loads are in flight together.
    constexpr int NR = FMT == 1 ? 2 : 4;
    f32x4 raw[NR], rawn[NR];
    bool ok = live;
    if (FMT == 1) {
        // i2_s: byte 16 (q%2) + 4 j + b of group 2c + q/2 holds the elements
        // 128 g + 32 t + 16 (q%2) + 4 j + b at shifts 6 - 2t; nibble h of the
        // masked word takes t = 3 - 2h (step 0) or t = 2 - 2h (step 1).
        const int64_t g = 2 * c + (q >> 1);
        ok = live && g < K / 128;
        const int64_t gc = ok ? g : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = (s == 0 ? 3 : 2) - 2 * h;
            const int64_t k0 = 128 * gc + 32 * t + 16 * (q & 1) + 4 * j;
            raw[h] = ld16f(x + k0);
            if (nw) rawn[h] = ld16f(nw + k0);
        }
    } else {
        // TQ2_0: byte 16 q + 4 j + b of block c holds elements 4 (16 q + 4 j + b) + i
        // at bits 2 i; nibble h of step s takes i = 2h + s.
        const int64_t cc = live ? c : 0;
        const int64_t k0 = 256 * cc + 64 * q + 16 * j;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            raw[b] = ld16f(x + k0 + 4 * b);
            if (nw) rawn[b] = ld16f(nw + k0 + 4 * b);
        }
    }
    // RMSNorm prologue: the same two fp32 multiplies as in token_scale
    const float rinv = nw ? rms_inv(x, K, P.eps, tid, sacc) : 0.0f;
    // max |x| over the token
    const TokScale ts = token_scale(x, nw, rinv, K, tid, smax);
    const int E = ts.E;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // element e = 2b + h: i2_s word h, lane b; TQ2_0 word b, lane 2h + s
        const int b = e >> 1, h = e & 1;
        float xv = FMT == 1 ? raw[h][b] : raw[b][2 * h + s];
        if (nw) xv = __fmul_rn(__fmul_rn(xv, rinv), FMT == 1 ? rawn[h][b] : rawn[b][2 * h + s]);
        v[e] = ok ? xv : 0.0f;
    }
    uint32_t out[kPl];
    long long xsum = 0;
    make_digits<8>(v, ts, out, xsum);
    if (live) {
        uint8_t* dst = ops + c * kChunkBytes + s * kStepBytes + q * kQuarterBytes + 4 * j;
#pragma unroll
        for (int r = 0; r < kPl; ++r)
            *(__attribute__((address_space(1))) uint32_t*)(dst + r * kPlRowBytes) = out[r];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) xsum += __shfl_xor(xsum, o, kWave);
    if (lane == 0) ssum[wave] = xsum;
    __syncthreads();
    if (tid == 0) {
        const long long tot = ssum[0] + ssum[1] + ssum[2] + ssum[3];
        *(__attribute__((address_space(1))) long long*)(ops + meta_off(K) + 8 + 8 * slice) = tot;
        if (slice == 0) *(__attribute__((address_space(1))) int32_t*)(ops + meta_off(K)) = E;
    }
}

// ---------------------------------------------------------------- product
__device__ __forceinline__ f32x4 mfma_f4(i32x4 a, i32x4 b, f32x4 c) {
    const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, 127, 0, 127);
}

// Shapes per token count MT (1, 2, 4, 8): every token is its own 16-row
// MFMA block (twelve digit planes, four rows of weight 0), so one decoded
// weight tile feeds MT blocks.  KG chunks of 256 k per pipeline group: 4
// (weight loads of 4 rows x 256 bytes) while the activation windows of all
// tokens fit beside the tiles, else 2 (8 rows x 128 bytes).
// LDS: two activation windows, then one weight tile per wave.
template <int FMT, int MT>
struct F4Cfg {
    static constexpr int CB = f4_cb(FMT, MT);                    // 16-row column blocks per wave
    static constexpr int WaveRows = 16 * CB;
    static constexpr int WgRows = kWaves * WaveRows;
    static constexpr int KG = MT <= 2 ? 4 : MT <= 8 ? 2 : 1;
    static constexpr int WStride = KG * 64 + 16;                 // padded LDS tile row
    static constexpr int WTile = 16 * CB * WStride;              // one wave's tile
    static constexpr int AWin = MT * KG * kChunkBytes;           // one group's digits, all tokens
    static constexpr int APer = (AWin / 16 + kThreads - 1) / kThreads;   // 16-byte window pieces per thread
    static constexpr int LPR = KG * 4;                           // lanes per row in a weight load
    static constexpr int RPI = 64 / LPR;                         // rows per weight load
    static constexpr int NLD = WaveRows / RPI;                   // weight loads per wave and group
    static constexpr int64_t Lds = 2 * int64_t(AWin) + int64_t(kWaves) * WTile;
};
static_assert(F4Cfg<1, 1>::AWin == kAWin && F4Cfg<2, 1>::AWin == kAWin, "one-token shapes");

template <int FMT, int MT>
struct Regs {
    i32x4 w[F4Cfg<FMT, MT>::NLD];            // load i: row RPI i + lane / LPR, 16 bytes at 16 (lane % LPR)
    i32x4 a[F4Cfg<FMT, MT>::APer];           // pieces tid + kThreads p of the activation window
    uint16_t sc[F4Cfg<FMT, MT>::CB];         // TQ2_0: scale of row nl, chunk q % KG of the group, per column block
};

// out[m] = this lane's result for token m0 + m: lane l holds row row0 + l
// (column block l / 16, meaningful for l < 16 CB, rows < N and m0 + m <
// P.M), bias not added.  Token t's digits are at P.ops + t P.opstride.
template <int FMT, int MT>
__device__ __forceinline__ void f4_rows(const F4Prob& P, const uint8_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int64_t row0, int m0, int tid, char* abuf,
                                        char* wtile, float (&out)[MT]) {
    using C = F4Cfg<FMT, MT>;
    constexpr int kCB = C::CB;
    constexpr int KG = C::KG;
    const int lane = tid & 63, nl = lane & 15, q = lane >> 4;
    const int64_t N = P.N, K = P.K, nch = nchunks(K);
    const uint32_t rowbytes = uint32_t(K / 4);
    const int ngr = int((nch + KG - 1) / KG);
    const int64_t abytes = nch * kChunkBytes;
    const int lr = lane / C::LPR, lp = lane % C::LPR;
    // loads: lane takes row RPI i + lr, bytes KG 64 g + 16 lp of group g
    const uint8_t* lrow[C::NLD];
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) {
        int64_t r = row0 + C::RPI * j + lr;
        r = r < N ? r : N - 1;                             // clamped rows are not stored
        lrow[j] = codes + r * int64_t(rowbytes);
    }
    const uint16_t* srow[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
        int64_t r = row0 + 16 * cb + nl;
        r = r < N ? r : N - 1;
        srow[cb] = scales + r * nch;
    }
    // Several tokens: thread tid fetches pieces of one token, ttok = tid /
    // TPT, the pieces tin + TPT p (p < APer) of that token's KG chunks.
    constexpr int TPT = MT > 1 ? kThreads / MT : kThreads;
    constexpr int PPT = KG * (kChunkBytes / 16);           // 16-byte pieces per token and group
    static_assert(MT == 1 || (PPT % TPT == 0 && PPT / TPT == C::APer), "pieces per thread");
    const int ttok = MT > 1 ? tid / TPT : 0, tin = MT > 1 ? tid % TPT : 0;
    const uint8_t* tokops = P.ops + int64_t(m0 + ttok < P.M ? m0 + ttok : P.M - 1) * P.opstride;   // tokens past M: unused
    const uint32_t ab = uint32_t(abytes);
    // Every load is issued by every lane from an in-bounds (clamped) address;
    // bytes past the end of a row are zeroed when stored to LDS.
    auto load = [&](int g, Regs<FMT, MT>& r) {
        const int gc = g < ngr ? g : ngr - 1;
        const uint32_t off = uint32_t(gc) * (KG * 64) + 16 * lp;
        const uint32_t offc = off < rowbytes ? off : rowbytes - 16;
#pragma unroll
        for (int j = 0; j < C::NLD; ++j) r.w[j] = LL_F4_NT ? ld16_stream(lrow[j] + offc) : ld16(lrow[j] + offc);
#pragma unroll
        for (int p = 0; p < C::APer; ++p) {
            const int pc = tid + kThreads * p;             // piece of the window: token pc / (KG 96)
            if constexpr (MT == 1) {
                int64_t o = int64_t(gc) * C::AWin + 16 * pc;
                o = o < abytes ? o : abytes - 16;
                r.a[p] = ld16(P.ops + o);
            } else {
                const uint32_t o = uint32_t(gc) * (KG * kChunkBytes) + 16 * (tin + TPT * p);
                r.a[p] = ld16(tokops + __builtin_elementwise_min(o, ab - 16));   // both multiples of 16
            }
        }
        if (FMT == 2) {
            int64_t b = int64_t(gc) * KG + q % KG;
            b = b < nch ? b : nch - 1;
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) r.sc[cb] = ld2(srow[cb] + b);
        }
    };
    auto store = [&](int g, const Regs<FMT, MT>& r) {
        if constexpr (MT > 1) {
            // a group inside the row (every group but a partial last one) is stored as loaded
            char* win = abuf + (g & 1) * C::AWin + 16 * (ttok * PPT + tin);
            if (uint32_t(g + 1) * (KG * kChunkBytes) <= ab && uint32_t(g + 1) * (KG * 64) <= rowbytes) {
#pragma unroll
                for (int j = 0; j < C::NLD; ++j)
                    *reinterpret_cast<i32x4*>(wtile + (C::RPI * j + lr) * C::WStride + 16 * lp) = r.w[j];
#pragma unroll
                for (int p = 0; p < C::APer; ++p) *reinterpret_cast<i32x4*>(win + 16 * TPT * p) = r.a[p];
            } else {
                const bool ok = uint32_t(g) * (KG * 64) + 16 * lp < rowbytes;
#pragma unroll
                for (int j = 0; j < C::NLD; ++j)
                    *reinterpret_cast<i32x4*>(wtile + (C::RPI * j + lr) * C::WStride + 16 * lp) = ok ? r.w[j] : i32x4{0, 0, 0, 0};
#pragma unroll
                for (int p = 0; p < C::APer; ++p) {
                    const bool aok = uint32_t(g) * (KG * kChunkBytes) + 16 * (tin + TPT * p) < ab;
                    *reinterpret_cast<i32x4*>(win + 16 * TPT * p) = aok ? r.a[p] : i32x4{0, 0, 0, 0};
                }
            }
            if (FMT == 2 && q < KG)
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb)
                    *reinterpret_cast<uint16_t*>(wtile + (16 * cb + nl) * C::WStride + KG * 64 + 2 * q) = r.sc[cb];
            return;
        }
        const bool ok = uint32_t(g) * (KG * 64) + 16 * lp < rowbytes;
#pragma unroll
        for (int j = 0; j < C::NLD; ++j)
            *reinterpret_cast<i32x4*>(wtile + (C::RPI * j + lr) * C::WStride + 16 * lp) = ok ? r.w[j] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < C::APer; ++p) {
            const int pc = tid + kThreads * p;
            const int within = pc % (KG * (kChunkBytes / 16));
            const bool aok = int64_t(g) * (KG * kChunkBytes) + 16 * (MT == 1 ? pc : within) < abytes;   // digits past the row end are zero
            if (C::APer * kThreads * 16 == C::AWin || pc < C::AWin / 16)
                *reinterpret_cast<i32x4*>(abuf + (g & 1) * C::AWin + 16 * pc) = aok ? r.a[p] : i32x4{0, 0, 0, 0};
        }
        if (FMT == 2 && q < KG)                        // the group's block scales in the row padding
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb)
                *reinterpret_cast<uint16_t*>(wtile + (16 * cb + nl) * C::WStride + KG * 64 + 2 * q) = r.sc[cb];
    };
    // block scales of the group being multiplied: chunk c of column block cb
    // in bits 16 c of cscp[cb] (a runtime shift, not a runtime index)
    uint64_t cscp[kCB];
    auto scale_of = [&](int c, int cb) { return half_bits_to_float(uint16_t(cscp[cb] >> (16 * c))); };

    // TQ2_0 with several tokens: per block, a lane folds its four plane sums
    // (rows 4q + i, weighted 8^(3 - i); exact in fp32: multiples of 1/2
    // below 2^20) and adds the block-scaled fold into one fp64 accumulator
    // per token and column block (the product of an fp16 scale and the fold
    // is exact in fp64), so the result carries no rounding but that of x
    constexpr bool kFold = FMT == 2 && MT > 1;
    f32x4 acc[kFold ? 1 : MT][kCB];
    double facc[kFold ? MT : 1][kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
        for (int m = 0; m < (kFold ? 1 : MT); ++m) acc[m][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < (kFold ? MT : 1); ++m) facc[m][cb] = 0.0;
    }
    // rows kPl..15 of the operand are weighted 0 in the epilogue: they read
    // rows 0..3 of the quarter, so no two lanes of an 8-lane LDS phase share
    // an address
    const int arow = q * kQuarterBytes + (nl < kPl ? nl : nl - kPl) * kPlRowBytes;

    auto decode = [&](const i32x4& u4, i32x4& b0, i32x4& b1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = uint32_t(u4[i]);
            if (FMT == 1) {
                b0[i] = int(u & 0x33333333u);
                b1[i] = int((u >> 2) & 0x33333333u);
            } else {
                b0[i] = int((u & 0x11111111u) | ((u & 0x22222222u) << 2));
                b1[i] = int(((u >> 2) & 0x11111111u) | (u & 0x88888888u));
            }
        }
    };
    auto mma = [&](f32x4& a, const i32x4& a0, const i32x4& a1, const i32x4& b0, const i32x4& b1, float sb) {
        if (FMT == 1) {
            a = mfma_f4(a0, b0, a);
            a = mfma_f4(a1, b1, a);
        } else {
            f32x4 blk = mfma_f4(a0, b0, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            blk = mfma_f4(a1, b1, blk);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = fmaf(sb, blk[i], a[i]);
        }
    };
    auto compute = [&](int g) {
        const int cn = nch - int64_t(g) * KG < KG ? int(nch - int64_t(g) * KG) : KG;
        if (FMT == 2)
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
                const char* sp = wtile + (16 * cb + nl) * C::WStride + KG * 64;
                cscp[cb] = KG == 4 ? *reinterpret_cast<const uint64_t*>(sp) : uint64_t(*reinterpret_cast<const uint32_t*>(sp));
            }
#pragma unroll LL_F4_CUNROLL
        for (int c = 0; c < cn; ++c) {                  // the last group may hold fewer chunks
            const char* ap = abuf + (g & 1) * C::AWin + arow + c * kChunkBytes;
            if constexpr (MT == 1) {
                const i32x4 a0 = *reinterpret_cast<const i32x4*>(ap);
                const i32x4 a1 = *reinterpret_cast<const i32x4*>(ap + kStepBytes);
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb) {
                    const i32x4 u4 = *reinterpret_cast<const i32x4*>(wtile + (16 * cb + nl) * C::WStride + 64 * c + 16 * q);
                    i32x4 b0, b1;
                    decode(u4, b0, b1);
                    mma(acc[0][cb], a0, a1, b0, b1, FMT == 2 ? scale_of(c, cb) : 0.0f);
                }
            } else {
                // the weight tile is decoded once and multiplied by every
                // token's block; token m + 1's operands are read while token m
                // multiplies, and (TQ2_0) token m's block sums are folded
                // while token m + 1's products run
                i32x4 b0[kCB], b1[kCB];
                double sb[kCB];
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb) {
                    const i32x4 u4 = *reinterpret_cast<const i32x4*>(wtile + (16 * cb + nl) * C::WStride + 64 * c + 16 * q);
                    decode(u4, b0[cb], b1[cb]);
                    sb[cb] = FMT == 2 ? double(scale_of(c, cb)) : 0.0;
                }
                i32x4 a[2][2];
                f32x4 blk[2][kCB];
                auto read_tok = [&](int m, i32x4 (&o)[2]) {
                    const char* am = ap + m * (KG * kChunkBytes);
                    o[0] = *reinterpret_cast<const i32x4*>(am);
                    o[1] = *reinterpret_cast<const i32x4*>(am + kStepBytes);
                };
                auto fold = [&](int m, const f32x4 (&bk)[kCB]) {
#pragma unroll
                    for (int cb = 0; cb < kCB; ++cb) {
                        const float t = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(bk[cb][0], 8.0f, bk[cb][1]), 8.0f, bk[cb][2]), 8.0f, bk[cb][3]);
                        facc[m][cb] = __builtin_fma(sb[cb], double(t), facc[m][cb]);
                    }
                };
                read_tok(0, a[0]);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m + 1 < MT) read_tok(m + 1, a[(m + 1) & 1]);
#pragma unroll
                    for (int cb = 0; cb < kCB; ++cb) {
                        if constexpr (kFold) {
                            blk[m & 1][cb] = mfma_f4(a[m & 1][0], b0[cb], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                            blk[m & 1][cb] = mfma_f4(a[m & 1][1], b1[cb], blk[m & 1][cb]);
                        } else {
                            acc[m][cb] = mfma_f4(a[m & 1][0], b0[cb], acc[m][cb]);
                            acc[m][cb] = mfma_f4(a[m & 1][1], b1[cb], acc[m][cb]);
                        }
                    }
                    if constexpr (kFold)
                        if (m > 0) fold(m - 1, blk[(m - 1) & 1]);
                }
                if constexpr (kFold) fold(MT - 1, blk[(MT - 1) & 1]);
            }
        }
    };

    // Group g is multiplied from LDS (the wave's weight tile, the shared
    // activation window g % 2) while group g + 1 waits in registers and group
    // g + 2 is being fetched.  The weight tile is private to the wave and its
    // LDS accesses execute in program order, so it is rewritten after the
    // multiply without a barrier; the barrier orders the shared windows.  The
    // loop runs while both of its fetches are groups of the row; a tail
    // multiplies the last one to three.
    Regs<FMT, MT> r0, r1;
    load(0, r0);
    load(1, r1);                                       // past the row for a one-group row: in-bounds bytes, unused
    store(0, r0);
    __syncthreads();
    int g = 0;
    for (; g + 4 <= ngr; g += 2) {                     // no exit between a load and its use
        load(g + 2, r0);
        compute(g);
        __builtin_amdgcn_sched_barrier(0);             // a group's multiplies stay before its successor's
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store(g + 1, r1);
        __syncthreads();
        load(g + 3, r1);
        compute(g + 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store(g + 2, r0);
        __syncthreads();
    }
    // 1 .. 3 groups left (the same count in the whole workgroup): group g is
    // in the tile, group g + 1 in r1; only group g + 2 is still to be fetched
    const int left = ngr - g;
    if (left == 3) load(g + 2, r0);
    compute(g);
    if (left >= 2) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store(g + 1, r1);
        __syncthreads();
        compute(g + 1);
    }
    if (left == 3) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        store(g + 2, r0);
        __syncthreads();
        compute(g + 2);
    }

    // Epilogue per token: plane 4q + i of this lane's column weighted by
    // 2 * 8^(11 - r) (the 2 undoes the half-valued weights), summed over the
    // quarters.
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int mc = m0 + m < P.M ? m0 + m : P.M - 1;
        const uint8_t* meta = P.ops + int64_t(mc) * P.opstride + meta_off(K);
        const int E = ld32(meta);
        double tot[kCB];
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            double t = 0.0;
            if constexpr (kFold) {
                // the fold of quarter q (planes 4q .. 4q + 3) weighs 2 * 8^(8 - 4q); quarter 3 holds no plane
                t = q < 3 ? facc[m][cb] * ldexp(1.0, 25 - 12 * q) : 0.0;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * q + i;
                    const double wgt = r < kPl ? ldexp(1.0, 1 + 3 * (kPl - 1 - r)) : 0.0;
                    t = fma(double(acc[m][cb][i]), wgt, t);
                }
            }
            t += __shfl_xor(t, 16, kWave);
            t += __shfl_xor(t, 32, kWave);
            tot[cb] = t;
        }
        // lane l holds row row0 + l of column block l / 16
        double t = tot[0];
#pragma unroll
        for (int cb = 1; cb < kCB; ++cb)
            if (q == cb) t = tot[cb];
        const double unit = ldexp(1.0, E - 34);
        double yv;
        if (FMT == 1) {
            long long xs = 0;
            for (int64_t sl = 0; sl < nslices(K); ++sl)
                xs += *(__attribute__((address_space(1))) const long long*)(meta + 8 + 8 * sl);
            const float scale = *(const __attribute__((address_space(1))) float*)(codes + N * int64_t(rowbytes));
            yv = double(scale) * ((t - double(xs)) * unit);
        } else {
            yv = t * unit;                                  // block scales are inside t
        }
        out[m] = float(yv);
    }
}

// Waves per SIMD the register allocation aims at, per format and token count
// (the LDS of F4Cfg<MT> allows 3, 2, 3, 2 workgroups per CU).  TQ2_0 keeps
// each group's block scales in the LDS row padding, so one token fits three
// waves without spilling; with four tokens it would spill inside the main
// loop at three waves (measured 17% slower than two).
#ifndef LL_F4_OCC
#define LL_F4_OCC 3
#endif
#ifndef LL_F4_TQ2_MT16
#define LL_F4_TQ2_MT16 1                               // TQ2_0, 9 .. 16 tokens: one pass of sixteen
#endif
#ifndef LL_F4_OCC_TQ2
#define LL_F4_OCC_TQ2 3
#endif
#ifndef LL_F4_OCC_TQ2_MT4
#define LL_F4_OCC_TQ2_MT4 2
#endif
__host__ __device__ constexpr int f4_occ(int FMT, int MT) {
    return MT >= 8 || MT == 2 ? 2 : MT == 4 ? (FMT == 2 ? LL_F4_OCC_TQ2_MT4 : 3) : FMT == 2 ? LL_F4_OCC_TQ2 : LL_F4_OCC;
}

// grid: 8 * ceil(T / 8) workgroups for T logical ones; hardware workgroup w
// runs on XCD w % 8, and takes logical index (w % 8) * T8 + w / 8.
// passes > 1 (M > MT): logical workgroup L multiplies tile L / passes for the
// tokens [MT (L % passes), MT (L % passes + 1)); the passes of one tile are
// consecutive logical workgroups, so they run on one XCD and the later ones
// find the weights in its L2.
template <int FMT, bool PAIRS, int MT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(f4_occ(FMT, MT)))) f4_batch_kernel(
    const F4Prob* __restrict__ tab, const int32_t* __restrict__ map, int64_t T, int passes) {
    static_assert(!PAIRS || MT == 1, "gated pairs are one-token items");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t w = blockIdx.x, T8 = (T + 7) / 8;
    const int64_t LP = (w % 8) * T8 + w / 8;
    if (LP >= T) return;                                   // whole workgroup
    const int64_t L = MT == 1 ? LP : LP / passes;          // one token: one pass
    const int m0 = MT == 1 ? 0 : MT * int(LP % passes);
    const F4Prob& P = tab[ld32(map + L)];
    const int tid = int(threadIdx.x), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: selects stay scalar
    using C = F4Cfg<FMT, MT>;
    char* wtile = lds + 2 * C::AWin + wave * C::WTile;
    // Gated pair (only in launches whose table holds one): waves 0, 1
    // multiply 64 gate rows, waves 2, 3 the same rows of the up matrix, all
    // from one activation window.  Waves past the last row still take part
    // (clamped rows, nothing stored): the loop has barriers.
    const bool pair = PAIRS && P.pair != 0;
    const int half = pair ? wave >> 1 : 0;
    const int64_t row0 = pair ? (L - P.wg0) * (C::WgRows / 2) + (wave & 1) * C::WaveRows
                              : (L - P.wg0) * C::WgRows + wave * C::WaveRows;
    float v[MT];
    f4_rows<FMT, MT>(P, half ? P.codes2 : P.codes, half ? P.scales2 : P.scales, row0, m0, tid, lds, wtile, v);
    const int64_t row = row0 + lane;                       // = row0 + 16 cb + nl for cb = q
    if (!pair) {
        // [BL "Fused BitLinear + Residual Add Kernel"]: a residual passed as the bias is added last
        const float bv = P.bias ? P.bias[row < P.N ? row : P.N - 1] : 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float out = v[m];
            if (P.bias) out = __fadd_rn(out, bv);
            if (m0 + m < P.M && lane < C::WaveRows && row < P.N) P.y[int64_t(m0 + m) * P.N + row] = out;
        }
        return;
    }
    // the up results reach the gate waves through LDS
    __syncthreads();                                       // every wave is done with the operand buffers
    float* xch = reinterpret_cast<float*>(lds);
    if (half == 1 && lane < C::WaveRows) xch[(wave & 1) * C::WaveRows + lane] = v[0];
    __syncthreads();
    if (half == 0 && lane < C::WaveRows && row < P.N) {
        const float u = xch[(wave & 1) * C::WaveRows + lane];
        const float r = v[0] > 0.0f ? v[0] : 0.0f;
        P.y[row] = __fmul_rn(__fmul_rn(r, r), u);
    }
}

}  // namespace

namespace llk {

bool f4_engine(int64_t M, int64_t kmax) { return M >= 1 && M <= 16 && kmax <= kMaxK; }
int64_t f4_op_stride(int64_t K) { return (op_bytes(K) + 255) / 256 * 256; }
size_t f4_operand_bytes(int64_t M, int64_t K) { return size_t(M * f4_op_stride(K)); }
// the launch variant launch_f4_fmt picks for M tokens: its rows per workgroup
int64_t f4_batch_rows(bool pair, int fmt, int64_t M) {
    const int mt = M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : M <= 8 || fmt != 2 || !LL_F4_TQ2_MT16 ? 8 : 16;
    const int64_t rows = kWaves * 16 * f4_cb(fmt, mt);
    return pair ? rows / 2 : rows;
}
size_t f4_prob_bytes() { return sizeof(F4Prob); }
size_t f4_prep_bytes() { return sizeof(F4Prep); }
int64_t f4_grid(int64_t T) { return 8 * ((T + 7) / 8); }

void fill_f4_prob(void* dst, const void* codes, const void* scales, const void* ops, const float* bias, float* y,
                  int64_t N, int64_t K, int64_t wg0, const void* codes2, const void* scales2, int64_t M) {
    F4Prob p;
    p.codes2 = static_cast<const uint8_t*>(codes2);
    p.scales2 = static_cast<const uint16_t*>(scales2);
    p.pair = codes2 != nullptr;
    p.codes = static_cast<const uint8_t*>(codes);
    p.scales = static_cast<const uint16_t*>(scales);
    p.ops = static_cast<const uint8_t*>(ops);
    p.bias = bias;
    p.y = y;
    p.N = N;
    p.K = K;
    p.wg0 = wg0;
    p.M = int32_t(M);
    p.opstride = f4_op_stride(K);
    *static_cast<F4Prob*>(dst) = p;
}

void fill_f4_prep(void* dst, const float* x, void* ops, int64_t K, const float* norm_w, float eps) {
    F4Prep p;
    p.x = x;
    p.ops = ops;
    p.K = K;
    p.norm_w = norm_w;
    p.eps = eps;
    *static_cast<F4Prep*>(dst) = p;
}

hipError_t launch_f4_batch_prep(const void* prep_table, int nprep, int fmt, int64_t kmax, hipStream_t stream) {
    const dim3 grid{unsigned(nprep), unsigned(nslices(kmax))}, block{256};
    const F4Prep* t = static_cast<const F4Prep*>(prep_table);
    if (fmt == 1)
        hipLaunchKernelGGL(f4_prep_kernel<1>, grid, block, 0, stream, t);
    else
        hipLaunchKernelGGL(f4_prep_kernel<2>, grid, block, 0, stream, t);
    return hipGetLastError();
}

template <int FMT, bool PAIRS, int MT>
hipError_t launch_f4_product(const F4Prob* t, const int32_t* m, int64_t T, int passes, hipStream_t stream) {
    const dim3 grid{unsigned(f4_grid(T * passes))}, block{unsigned(kThreads)};
    const size_t lds = size_t(F4Cfg<FMT, MT>::Lds);
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(f4_batch_kernel<FMT, PAIRS, MT>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((f4_batch_kernel<FMT, PAIRS, MT>), grid, block, lds, stream, t, m, T * passes, passes);
    return hipGetLastError();
}

// M = 9 .. 16: i2_s runs two passes of eight tokens (sixteen f32x4 plane
// accumulators per column block would leave one wave per SIMD); TQ2_0, whose
// folded fp64 accumulators take two registers per token, one pass of sixteen
// with 256-k groups (6912 x 2560 batch at M = 16: 461 -> 431 us).
template <int FMT>
hipError_t launch_f4_fmt(const F4Prob* t, const int32_t* m, int64_t T, bool pairs, int64_t M, hipStream_t stream) {
    if (M == 1)
        return pairs ? launch_f4_product<FMT, true, 1>(t, m, T, 1, stream) : launch_f4_product<FMT, false, 1>(t, m, T, 1, stream);
    if (M == 2) return launch_f4_product<FMT, false, 2>(t, m, T, 1, stream);
    if (M <= 4) return launch_f4_product<FMT, false, 4>(t, m, T, 1, stream);
    if (FMT == 2 && LL_F4_TQ2_MT16 && M > 8) return launch_f4_product<FMT, false, 16>(t, m, T, 1, stream);
    return launch_f4_product<FMT, false, 8>(t, m, T, M <= 8 ? 1 : 2, stream);
}

hipError_t launch_f4_batch_product(const void* prob_table, const void* map, int fmt, int64_t T, int64_t kmax,
                                   bool pairs, int64_t M, hipStream_t stream) {
    (void)kmax;
    const F4Prob* t = static_cast<const F4Prob*>(prob_table);
    const int32_t* m = static_cast<const int32_t*>(map);
    return fmt == 1 ? launch_f4_fmt<1>(t, m, T, pairs, M, stream) : launch_f4_fmt<2>(t, m, T, pairs, M, stream);
}

}  // namespace llk
