// Prefill-size BitLinear product with int8 activations on the int8 matrix
// cores (Hesper "BitLinear": "Subgroup-Matrix Multi-row BitLinear Kernel"
// computes Y = X W^T per output tile; binary-gemm card, "Requirements and
// limits": prefill needs a different kernel than the decode GEMV).  For i2_s
// weights acc[m,n] = sum_k w[n,k] q[m,k] exactly in int32, and
// y = ((float)acc * s_tok[m]) * s_w.
//
// MI355X design: v_mfma_i32_32x32x32_i8; lane l holds 16 consecutive k of
// row (or column) l % 32 at k offset 16 (l / 32) of a 32-k step.  The 32
// bytes of one 128-k group of an i2_s row hold, in their four 2-bit fields,
// the k runs 32t + [0, 32) for t = 0..3 (byte j of the group, field t:
// element 32t + j), so a lane's 16 code bytes (bytes 16 (l / 32) .. + 15 of
// its column's group) are its B operand for all four 32-k steps, and the
// activations need no reordering.
//
// Workgroup tile 128 x 128, four waves (one per SIMD), each owning a 64 x 64
// wave tile (four 32 x 32 accumulators) over the whole of K.
//   - Activations: a 128-row x 128-k int8 tile per group, loaded from global
//     memory into registers D - 1 groups ahead, stored into one of two LDS
//     buffers (rows padded to 144 bytes, so the eight lanes of an LDS access
//     fall on distinct banks) and read back as MFMA operands.
//   - Weight codes never touch LDS: each lane loads its own 16 code bytes
//     per column block and group straight into registers (the two waves of a
//     column share them through the L1), decoded in registers per step
//     (shift, mask, byte permute).
//   - The loop is software-pipelined: while the four MFMAs of a 32-k step
//     run, the lane reads the next step's activation operands from LDS and
//     decodes the next step's weights; the next group's tile is stored into
//     the other LDS buffer during the first step; one barrier per group,
//     placed before the last step's MFMAs so that they overlap the wait, and
//     waiting on LDS traffic only (global prefetches stay in flight).
//
// TQ2_0 weights (llama.cpp TQ2_0 as described by the Hesper API doc: 2-bit
// two's-complement codes, four consecutive elements per byte, an fp16 scale
// per 256-element block; codes and scales in separate device arrays) use the
// same kernel.  Element k of a row is again in code byte k/4, so the code
// loads are the same; field t of byte j holds element 4j + t, so a step
// takes field t of its lane's 16 code bytes (elements 4 (16 h + j) + t) and
// the activation tile is stored as four planes of 32 bytes per 128-k group,
// plane t holding elements 4i + t (a 4 x 4 byte transpose of every 16-byte
// piece).  Each 256-k block's exact int32 sum is scaled by the block scale
// into fp32 accumulators (the block's first multiply starts from zero), and
// y = acc * s_tok (+ bias).  Split K keeps whole blocks and the last split
// adds the fp32 partials in split order, so the result does not depend on
// which split finishes last.
//
// W1 sign bits with fp16 scales per 128-weight group (binary-gemm card,
// "Method"; group size 128 only) use it too: bit k of a row is bit k % 8 of
// byte k / 8, so a 128-k group is 16 code bytes in natural k order and the
// activation tile is stored as for i2_s.  A lane's 16 weights of a step are
// 16 bits of code dword t; each nibble is spread to four bytes by one
// multiply and a mask and mapped to -1 / +1 by a byte permute.  Every group
// is a scale block.
//
// Narrow tiles.  Where 128 x 128 tiles would leave half the chip idle, an
// i2_s product runs 64 x 128 tiles (64 tokens, 128 weight rows; one wave
// along M).  Halves along K.  A narrow tile may run eight waves as two
// halves of four: half h multiplies the h-th half of the tile's groups from
// LDS buffers of its own, every barrier is met by both halves (equal group
// counts), and at the end half 1 hands its exact int32 sums to half 0
// through LDS, which adds them and writes the tile.
//
// Split K.  With few output tiles (N = 2560 at M = 512 gives 80) the
// workgroups of a tile split its groups S ways.  Each split writes its
// partial tile to the workspace and counts itself in at the tile's counter
// (an agent-scope release); the split that arrives last takes an acquire
// fence, adds the others' partials to its own and runs the epilogue, then
// resets the counter (so the counters stay zero between calls).  Integer
// addition makes the i2_s result independent of the order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

constexpr int BM = 128, BN = 128, LDA = 144;
#ifndef LL_GEMM_I2S_WAVES
#define LL_GEMM_I2S_WAVES 8                              // i2_s: eight waves, two per SIMD
#endif
#ifndef LL_GEMM_BLOCK_WAVES
#define LL_GEMM_BLOCK_WAVES 8                            // TQ2_0 and W1 (block-scaled sums)
#endif
constexpr int kBuf = BM * LDA;                           // one LDS buffer: the activation tile of a group
constexpr size_t kGemmLds = size_t(2) * kBuf;
#ifndef LL_GEMM_XCD
#define LL_GEMM_XCD 1                                    // XCD-grouped workgroup order
#endif
#ifndef LL_GEMM_I2S_SETS
#define LL_GEMM_I2S_SETS 1                               // i2_s accumulator sets: 1, or 3 (codes masked in place)
#endif
#ifndef LL_GEMM_DEPTH
#define LL_GEMM_DEPTH 3                                  // register stages (groups) of global loads
#endif
#ifndef LL_GEMM_DEPTH_TQ2
#define LL_GEMM_DEPTH_TQ2 2                              // TQ2_0: two stages (measured 4-6% faster than three)
#endif

// Waits for this wave's LDS operations, then meets the other waves of the
// workgroup.  Outstanding global loads (prefetches of later groups) stay in
// flight; the memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// FMT 1: i2_s, FMT 2: TQ2_0 (scales: fp16 [N][K/256]), FMT 3: W1 with
// G = 128 (codes: the sign-bit words, scales: fp16 [N][K/128]).  XSUM (i2_s):
// the per-token sums of q come in xsum (from the quantization) instead of
// being summed here.  y16: bf16 output written instead of y, or NULL.
template <int FMT, bool XSUM = false, int WV = 4, int BNT = BN, int KH = 1, int BMT = BM>
__device__ __forceinline__ void gemm_i8_body(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                             int64_t N, int64_t K, const int8_t* __restrict__ xq,
                                             const float* __restrict__ xs, int64_t M, const float* __restrict__ bias,
                                             float* __restrict__ y, int32_t* __restrict__ acc_out, int S,
                                             int32_t* __restrict__ part, int32_t* __restrict__ counters,
                                             const int32_t* __restrict__ xsum, uint16_t* __restrict__ y16) {
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    __shared__ int last_flag;
    __shared__ __attribute__((aligned(16))) float xs_tile[BMT];   // token scales of the tile's rows
    __shared__ __attribute__((aligned(16))) int32_t qsum_tile[KH][BMT];  // i2_s: sum_k q of the tile's rows (per half)
    // WV = 4: one wave per SIMD, wave tiles 64 x 64; WV = 8: two waves per
    // SIMD (one's vector work runs while the other's matrix products do),
    // wave tiles 64 x 32; KH = 2: two halves of WV / 2 waves along K
    static_assert(KH == 1 || (KH == 2 && FMT != 3 && LL_GEMM_I2S_SETS == 1), "halves along K: i2_s or TQ2_0");
    static_assert(BMT == 128 || (BMT == 64 && FMT != 3), "tile rows: 128, or 64 (i2_s, TQ2_0)");
    constexpr int TH = 64 * WV;                            // threads
    constexpr int THH = TH / KH;                           // threads of one half
    constexpr int WNW = WV / KH / (BMT / 64);              // waves along N (BMT / 64 along M)
    constexpr int kBufT = BMT * LDA;                       // one LDS buffer: the activation tile of a group
    constexpr int NB = BNT / (32 * WNW);                   // 32-column blocks per wave
    static_assert(NB >= 1 && NB * 32 * WNW == BNT, "tile width: whole 32-column blocks per wave");
    constexpr int64_t kPart = int64_t(BMT) * BNT;          // ints of one partial tile
    constexpr int CA = BMT * 8 / THH;                      // 16-byte activation chunks per thread and group
    constexpr int WC = 32 * NB;                            // columns per wave
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = KH == 1 ? 0 : w / (WV / KH);            // the half this wave belongs to
    const int htid = tid % THH;                            // thread index within the half
    const int wm = (w % (WV / KH)) / WNW, wn = (w % (WV / KH)) % WNW;   // rows 64 wm, columns WC wn of the tile
    const int li = lane & 31, h = lane >> 5;
    const int64_t TM = (M + BMT - 1) / BMT;
    // Hardware workgroup b runs on XCD b % 8; it takes logical index
    // (b % 8) T8 + b / 8, so consecutive logical workgroups (the splits and
    // row tiles of one column tile, which read the same weight codes) share
    // one XCD's L2.
    const int64_t T = ((N + BNT - 1) / BNT) * TM * S, T8 = (T + 7) / 8;
    const int64_t L = LL_GEMM_XCD ? (int64_t(blockIdx.x) % 8) * T8 + int64_t(blockIdx.x) / 8 : int64_t(blockIdx.x);
    if (L >= T) return;                                    // whole workgroup, before any barrier
    const int64_t tile = L / S;
    const int split = int(L % S);
    // Where the activation rows of all row tiles outgrow about three
    // quarters of an XCD's 4 MB L2, the row tiles form two groups and the
    // XCDs' runs of consecutive tiles take one group's rows of a run of
    // column tiles, so each L2 holds half the activations (2560 x 6912 at
    // M = 512: 16.9 -> 15.4 us; where the rows fit, one group measured
    // faster).
    // (tile counts stay far below 2^31: 32-bit index arithmetic)
    int64_t m0, n0;
    if (TM % 2 == 0 && TM * BMT * K > (int64_t(3) << 20)) {
        const uint32_t t = uint32_t(tile), tmg = uint32_t(TM / 2), grp = tmg * uint32_t((N + BNT - 1) / BNT);
        const uint32_t rg = t / grp, loc = t - rg * grp;
        m0 = int64_t(rg * tmg + loc % tmg) * BMT;
        n0 = int64_t(loc / tmg) * BNT;
    } else {
        m0 = (tile % TM) * BMT;
        n0 = (tile / TM) * BNT;
    }
    const int64_t rowbytes = FMT == 3 ? K / 8 : K / 4;
    const int64_t ng = K / 128;
    // TQ2_0: splits of whole 256-k blocks, so every split starts on an even group
    const int64_t nsplit_units = FMT != 2 ? ng : K / 256, per_unit = FMT != 2 ? 1 : 2;
    const int64_t gs0 = per_unit * (nsplit_units * split / S), gs1 = per_unit * (nsplit_units * (split + 1) / S);
    // This half's groups [g0, g1): halves of whole units (TQ2_0: blocks),
    // half 0 the shorter.  Both halves run the main loop for half 0's count
    // and the tail up to half 1's (gend), so they meet the same barriers; the
    // groups of half 0 past g1 load and synchronise but multiply nothing.
    // (i2_s: the launcher makes the halves equal.)
    const int64_t nunit = (gs1 - gs0) / per_unit, u0 = KH == 1 ? nunit : nunit / 2;
    const int64_t g0 = gs0 + kh * u0 * per_unit;
    const int64_t g1 = KH == 1 || kh == 0 ? g0 + u0 * per_unit : gs1;
    const int64_t gmain = gs0 + kh * u0 * per_unit + u0 * per_unit;   // end of the common main loop
    const int64_t gend = g0 + (nunit - u0 * (KH - 1)) * per_unit;       // end of the loop (half 1's count)

    // Activation loads of one group: CA 16-byte chunks per thread, chunk
    // idx = tid + TH c is row idx / 8, bytes 16 (idx % 8) of the group;
    // rows past M are clamped (their results are not stored).
    const int8_t* arow[CA];
#pragma unroll
    for (int c = 0; c < CA; ++c) {
        const int idx = htid + THH * c;
        int64_t m = m0 + (idx >> 3);
        m = m < M ? m : M - 1;
        arow[c] = xq + m * K + 16 * (idx & 7);
    }
    // Weight codes of this lane's NB columns (wn WC + nb 32 + li), clamped;
    // i2_s / TQ2_0: bytes 16 h .. 16 h + 15 of the 32-byte group; W1: the
    // group's 16 bytes (both halves of the wave load the same).
    const uint8_t* bptr[NB];
    const uint16_t* sptr[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        int64_t n = n0 + wn * WC + nb * 32 + li;
        n = n < N ? n : N - 1;
        bptr[nb] = codes + n * rowbytes + (FMT == 3 ? 0 : 16 * h);
        sptr[nb] = FMT == 2 ? scales + n * (K / 256) : FMT == 3 ? scales + n * (K / 128) : nullptr;
    }

    struct Stage {
        i32x4 a[CA];
        i32x4 b[NB];
        uint16_t sc[FMT == 1 ? 1 : NB];                     // TQ2_0 / W1: the group's block scales
    };
    auto load = [&](int64_t g, Stage& s) {
        // past the range: reload the last group (unused); an empty range
        // (never launched) stays on its first group, inside the rows
        const int64_t gc = g < g1 ? g : g1 > g0 ? g1 - 1 : g0;
#pragma unroll
        for (int c = 0; c < CA; ++c) s.a[c] = ld16(arow[c] + 128 * gc);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s.b[nb] = ld16(bptr[nb] + (FMT == 3 ? 16 : 32) * gc);
        if constexpr (FMT != 1)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s.sc[nb] = ld2(sptr[nb] + (FMT == 2 ? gc / 2 : gc));
    };
    // i2_s: this thread's share of sum_k q of its CA rows (idx / 8), summed
    // from the chunks it stores (v_dot4 against 1)
    int32_t qs[CA] = {};
    int8_t* const lds_h = lds + kh * 2 * kBufT;            // this half's two buffers
    auto store_a = [&](int buf, const Stage& s) {
        int8_t* A = lds_h + buf * kBufT;
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int idx = htid + THH * c;
            int8_t* arow_l = &A[(idx >> 3) * LDA];
            if constexpr (FMT == 1 && !XSUM)
#pragma unroll
                for (int e = 0; e < 4; ++e) qs[c] = __builtin_amdgcn_sdot4(s.a[c][e], 0x01010101, qs[c], false);
            if constexpr (FMT != 2) {
                *reinterpret_cast<i32x4*>(arow_l + 16 * (idx & 7)) = s.a[c];
            } else {
                // piece p (elements 16 p + 4 i + t in byte t of dword i) ->
                // dword t = elements 16 p + 4 i + t, i = 0..3: bytes 4p..4p+3 of plane t
                const uint32_t d0 = uint32_t(s.a[c][0]), d1 = uint32_t(s.a[c][1]);
                const uint32_t d2 = uint32_t(s.a[c][2]), d3 = uint32_t(s.a[c][3]);
                const uint32_t x01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0.b0 d1.b0 d0.b1 d1.b1
                const uint32_t y01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0.b2 d1.b2 d0.b3 d1.b3
                const uint32_t x23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
                const uint32_t y23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
                const int p = idx & 7;
                *reinterpret_cast<uint32_t*>(arow_l + 0 + 4 * p) = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
                *reinterpret_cast<uint32_t*>(arow_l + 32 + 4 * p) = __builtin_amdgcn_perm(x23, x01, 0x07060302u);
                *reinterpret_cast<uint32_t*>(arow_l + 64 + 4 * p) = __builtin_amdgcn_perm(y23, y01, 0x05040100u);
                *reinterpret_cast<uint32_t*>(arow_l + 96 + 4 * p) = __builtin_amdgcn_perm(y23, y01, 0x07060302u);
            }
        }
    };
    // activation operands of step t (rows wm 64 + mb 32 + li, k 32 t + 16 h)
    auto read_a = [&](int buf, int t, i32x4 (&ao)[2]) {
        const int8_t* A = lds_h + buf * kBufT + (wm * 64 + li) * LDA + 32 * t + 16 * h;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) ao[mb] = *reinterpret_cast<const i32x4*>(A + mb * 32 * LDA);
    };
    // weight operands of step t from the lane's code registers
    auto decode = [&](const i32x4 (&bq)[NB], int t, i32x4 (&bo)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (FMT == 3) {
                // bits 16 h .. 16 h + 15 of code dword t: k = 32 t + 16 h + j
                const uint32_t v = uint32_t(bq[nb][t]) >> (16 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t sp = (((v >> (4 * i)) & 0xFu) * 0x00204081u) & 0x01010101u;   // bit e -> byte e
                    bo[nb][i] = int(__builtin_amdgcn_perm(0u, 0x000001FFu, sp));                // 0 -> -1, 1 -> +1
                }
            } else if constexpr (FMT == 1 && LL_GEMM_I2S_SETS == 3) {
                // i2_s: the code c = w + 1 of field t (bits 6 - 2t) masked where
                // it sits: step 0 (shifted down two bits) and step 1 give 16 c,
                // step 2 gives 4 c, step 3 gives c; each step's accumulator set
                // carries that factor
                const uint32_t mask = t <= 1 ? 0x30303030u : t == 2 ? 0x0C0C0C0Cu : 0x03030303u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bo[nb][i] = int((t == 0 ? uint32_t(bq[nb][i]) >> 2 : uint32_t(bq[nb][i])) & mask);
            } else if constexpr (FMT == 1) {
                // i2_s, one accumulator set: the code c = w + 1 of field t
#pragma unroll
                for (int i = 0; i < 4; ++i) bo[nb][i] = int((uint32_t(bq[nb][i]) >> (6 - 2 * t)) & 0x03030303u);
            } else {
                // TQ2_0: field t at bits 2t, two's complement {0, +1, -2, -1}
                constexpr uint32_t table = 0xFFFE0100u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bo[nb][i] = int(__builtin_amdgcn_perm(0u, table, (uint32_t(bq[nb][i]) >> (2 * t)) & 0x03030303u));
            }
        }
    };

    // epilogue operands, requested before the main loop so their latency is
    // hidden: the token scales of the tile's rows (into LDS, read back after
    // the loop), the weight scale, the biases of this lane's columns
    if (tid < BMT) {
        const int64_t m = m0 + tid;
        xs_tile[tid] = xs[m < M ? m : M - 1];
        if constexpr (XSUM) qsum_tile[0][tid] = xsum[m < M ? m : M - 1];
    }
    const float sw = FMT == 1 ? *reinterpret_cast<const float*>(codes + N * rowbytes) : 1.0f;
    const float* bsrc = bias ? bias : xs;                 // always a valid address
    float bnv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t n = n0 + wn * WC + nb * 32 + li;
        bnv[nb] = bsrc[bias ? (n < N ? n : N - 1) : 0];
    }

    // acc: the exact integer sums (i2_s: of steps 0 and 1, times 16);
    // i2_s also acc4 (step 2, times 4) and acc1 (step 3)
    constexpr int NS = FMT == 1 && LL_GEMM_I2S_SETS == 3 ? 2 : 1;
    i32x16 acc[2][NB], acc4[NS][NB], acc1[NS][NB];
    f32x16 facc[FMT == 1 ? 1 : 2][NB];                     // TQ2_0 / W1: scaled block sums
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[mb][nb][r] = 0;
                if constexpr (FMT == 1) {
                    acc4[mb % NS][nb][r] = 0;
                    acc1[mb % NS][nb][r] = 0;
                } else {
                    facc[mb][nb][r] = 0.0f;
                }
            }

    // the four MFMAs of step t; `fresh`: the step starts a new scale block
    // (TQ2_0: first step of an even group; W1: first step of every group)
    auto mfma = [&](const i32x4 (&ao)[2], const i32x4 (&bo)[NB], int t, bool fresh) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (FMT == 1 && LL_GEMM_I2S_SETS == 3) {
                    if (t <= 1)
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[mb], bo[nb], acc[mb][nb], 0, 0, 0);
                    else if (t == 2)
                        acc4[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[mb], bo[nb], acc4[mb][nb], 0, 0, 0);
                    else
                        acc1[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[mb], bo[nb], acc1[mb][nb], 0, 0, 0);
                } else {
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[mb], bo[nb], fresh ? i32x16{} : acc[mb][nb], 0, 0, 0);
                }
            }
    };
    // TQ2_0 / W1: a finished scale block's exact sums into the fp32 accumulators
    auto scale_in = [&](const float (&sc)[NB]) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) facc[mb][nb][r] = __builtin_fmaf(float(acc[mb][nb][r]), sc[nb], facc[mb][nb][r]);
    };

    // Pipeline (one wave per SIMD, so any wait of the wave idles its matrix
    // core: every wait below targets operations issued at least a step
    // earlier).  Per group gi, multiplied from LDS buffer buf with its four
    // steps' activation operands already in registers (ac):
    //   step 0: MFMAs; decode step 1; store the next group's tile into the
    //           other buffer; load group gi + D into the freed register stage
    //   step 1: MFMAs; decode step 2
    //   barrier (the stores of step 0 are done by now)
    //   step 2: MFMAs; decode step 3; read all four steps' operands of the
    //           next group (an), used two steps later
    //   step 3: MFMAs; decode the next group's step 0
    // Register stage i % D holds group g0 + i from its load (D - 1 groups
    // ahead) until the step 0 that stores its tile and copies its codes.
    constexpr int D = FMT == 2 ? LL_GEMM_DEPTH_TQ2 : LL_GEMM_DEPTH;
    constexpr int U = D % 2 ? 2 * D : D;                // unroll: a multiple of D and of the buffer count
    static_assert(D >= 2, "register depth");
    Stage st[D];
    i32x4 bq[NB], bqn[NB], bo[2][NB], ac[4][2], an[4][2];
    float sc[NB] = {}, scn[NB] = {};
#pragma unroll
    for (int i = 0; i < D; ++i) load(g0 + i, st[i]);
    store_a(0, st[0]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        bq[nb] = st[0].b[nb];
        bqn[nb] = bq[nb];
        if constexpr (FMT != 1) sc[nb] = half_bits_to_float(st[0].sc[nb]);
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < 4; ++t) read_a(0, t, ac[t]);
    decode(bq, 0, bo[0]);

    // One group gi (register stage si, LDS buffer buf); `next`: a following
    // group exists.  `odd` (TQ2_0): gi ends a 256-k block.
    auto group = [&](int64_t gi, int si, int buf, bool next, bool odd, bool live) {
        const bool fresh0 = (FMT == 2 && !odd) || FMT == 3;
        __builtin_amdgcn_sched_barrier(0);
        // step 0
        if (live) mfma(ac[0], bo[0], 0, fresh0);
        decode(bq, 1, bo[1]);
        if (next) {
            const Stage& ns = st[(si + 1) % D];
            store_a(buf ^ 1, ns);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                bqn[nb] = ns.b[nb];
                if constexpr (FMT != 1) scn[nb] = half_bits_to_float(ns.sc[nb]);
            }
        }
        load(gi + D, st[si]);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // two global loads
        }
        __builtin_amdgcn_sched_barrier(0);
        // step 1
        if (live) mfma(ac[1], bo[1], 1, false);
        decode(bq, 2, bo[0]);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (next) lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // step 2
        if (live) mfma(ac[2], bo[0], 2, false);
        decode(bq, 3, bo[1]);
        if (next)
#pragma unroll
            for (int t = 0; t < 4; ++t) read_a(buf ^ 1, t, an[t]);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // step 3
        if (live) mfma(ac[3], bo[1], 3, false);
        if (next) decode(bqn, 0, bo[0]);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FMT == 3)
            if (live) scale_in(sc);
        if constexpr (FMT == 2)
            if (odd && live) scale_in(sc);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ac[t][0] = an[t][0];
            ac[t][1] = an[t][1];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            bq[nb] = bqn[nb];
            if constexpr (FMT == 2) {
                if (odd) sc[nb] = scn[nb];
            } else if constexpr (FMT == 3) {
                sc[nb] = scn[nb];
            }
        }
    };

    // (g0 is even (TQ2_0) and U is even, so group g0 + i is odd exactly when i is)
    int64_t g = g0;
    for (; g + U < gmain; g += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) group(g + i, i % D, i & 1, true, i & 1, true);
    }
    // the last 1 .. U groups (TQ2_0 halves: up to U + 2, half 0's last ones past g1)
    constexpr int TAIL = U + (KH == 2 && FMT == 2 ? 2 : 0);
    const int rem = int(gend - g);
#pragma unroll
    for (int j = 0; j < TAIL; ++j)
        if (j < rem) group(g + j, j % D, j & 1, j + 1 < rem, j & 1, g + j < g1);

    using E = std::conditional_t<FMT == 1, int32_t, float>;
    using V = std::conditional_t<FMT == 1, i32x16, f32x16>;
    if constexpr (FMT == 1) {
        // i2_s: sum_k w q = sum_k c q - sum_k q (w = c - 1); the row sums of q
        // over this split's groups, from the eight threads that stored each
        // row (with XSUM the whole rows' sums, subtracted once in the epilogue)
        if constexpr (!XSUM) {
#pragma unroll
            for (int c = 0; c < CA; ++c) {
#pragma unroll
                for (int o = 1; o < 8; o <<= 1) qs[c] += __shfl_xor(qs[c], o, kWave);
                if ((htid & 7) == 0) qsum_tile[kh][(htid >> 3) + (THH / 8) * c] = qs[c];
            }
        }
        if constexpr (KH == 2) {
            // every wave is past its last LDS operand read; half 1's sums go
            // through the (now free) activation buffers to half 0, which
            // finishes the tile alone (no barrier follows: S = 1)
            __syncthreads();
            int32_t* xch = reinterpret_cast<int32_t*>(lds) + (w % (WV / KH)) * (2 * NB * 16 * 64) + lane;
            if (kh == 1)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) xch[((mb * NB + nb) * 16 + r) * 64] = acc[mb][nb][r];
            __syncthreads();
            if (kh == 1) return;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mb][nb][r] += xch[((mb * NB + nb) * 16 + r) * 64];
        } else {
            __syncthreads();
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                i32x4 q4 = *reinterpret_cast<const i32x4*>(&qsum_tile[0][wm * 64 + mb * 32 + 8 * rq + 4 * h]);
                if constexpr (KH == 2 && !XSUM) q4 += *reinterpret_cast<const i32x4*>(&qsum_tile[1][wm * 64 + mb * 32 + 8 * rq + 4 * h]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * rq + e;
                        const int32_t qsub = XSUM ? 0 : q4[e];
                        if constexpr (LL_GEMM_I2S_SETS == 3)
                            acc[mb][nb][r] = (acc[mb][nb][r] >> 4) + (acc4[mb % NS][nb][r] >> 2) + acc1[mb % NS][nb][r] - qsub;
                        else
                            acc[mb][nb][r] = acc[mb][nb][r] - qsub;
                    }
            }
    }
    V fin[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (FMT == 1)
                fin[mb][nb] = acc[mb][nb];
            else
                fin[mb][nb] = facc[mb][nb];
        }
    if constexpr (KH == 2 && FMT != 1) {
        // TQ2_0 halves: half 1's fp32 block-scaled sums reach half 0 through
        // the activation buffers; half 0 adds them to its own (one fixed
        // order) and finishes the tile alone (no barrier follows: S = 1)
        __syncthreads();
        int32_t* xch = reinterpret_cast<int32_t*>(lds) + (w % (WV / KH)) * (2 * NB * 16 * 64) + lane;
        if (kh == 1)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float fv = fin[mb][nb][r];           // (a scalar copy: the element, not the vector, is cast)
                        xch[((mb * NB + nb) * 16 + r) * 64] = __builtin_bit_cast(int32_t, fv);
                    }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    fin[mb][nb][r] = __fadd_rn(fin[mb][nb][r], __builtin_bit_cast(float, xch[((mb * NB + nb) * 16 + r) * 64]));
    }

    if (S > 1) {
        // Publish this split's partial tile (device-coherent stores), wait for
        // them, count the split in; the split that arrives last reads the
        // others' partials (device-coherent loads) and finishes the tile.
        int32_t* mine = part + (tile * S + split) * kPart;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    st_coherent(mine + ((mb * NB + nb) * 16 + r) * TH + tid, __builtin_bit_cast(int32_t, E(fin[mb][nb][r])));
        wait_vmem();
        __syncthreads();
        if (tid == 0) last_flag = arrive_release(counters + tile) == S - 1;
        __syncthreads();
        if (!last_flag) return;
        acquire_agent();
        if constexpr (FMT == 1) {
            for (int s = 0; s < S; ++s) {
                if (s == split) continue;
                const int32_t* other = part + (tile * S + s) * kPart;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            fin[mb][nb][r] += ld_coherent(other + ((mb * NB + nb) * 16 + r) * TH + tid);
            }
        } else {
            // fp32 partials added in split order (this split's own from registers)
            V tot[2][NB];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) tot[mb][nb][r] = 0.0f;
            for (int s = 0; s < S; ++s) {
                const int32_t* other = part + (tile * S + s) * kPart;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            tot[mb][nb][r] += s == split ? fin[mb][nb][r]
                                                         : __builtin_bit_cast(float, ld_coherent(other + ((mb * NB + nb) * 16 + r) * TH + tid));
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) fin[mb][nb] = tot[mb][nb];
        }
        if (tid == 0) st_coherent(counters + tile, 0);    // ready for the next call
    }

    // Epilogue: i2_s y = ((float)acc * s_tok) * s_w (+ bias); TQ2_0 / W1
    // y = acc * s_tok (+ bias), written with non-temporal stores (the output,
    // 14 MB for 512 x 6912 in fp32, streams to memory in one burst as the
    // tiles end; 6912 x 2560 at M = 512: 14.8 -> 13.7 us).  Lane (li, h) holds column wn 64 + nb 32 + li
    // and rows wm 64 + mb 32 + 8 (r / 4) + 4 h + r % 4; its output pointer is
    // formed once, each store adds a uniform offset.  The stores of a full
    // tile run as one straight block (a branch between stores would make each
    // wait for the one before).
    float xsv[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&xs_tile[wm * 64 + mb * 32 + 8 * rq + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) xsv[mb][4 * rq + e] = v[e];
            if constexpr (FMT == 1 && XSUM) {
                const i32x4 q4 = *reinterpret_cast<const i32x4*>(&qsum_tile[0][wm * 64 + mb * 32 + 8 * rq + 4 * h]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) fin[mb][nb][4 * rq + e] -= q4[e];
            }
        }
    float out[2][NB][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v = FMT == 1 ? __fmul_rn(__fmul_rn(float(fin[mb][nb][r]), xsv[mb][r]), sw)
                                   : __fmul_rn(float(fin[mb][nb][r]), xsv[mb][r]);
                out[mb][nb][r] = bias ? __fadd_rn(v, bnv[nb]) : v;
            }
    const int64_t lrow = m0 + wm * 64 + 4 * h, lcol = n0 + wn * WC + li;
    if (y16) {
        uint16_t* yl16 = y16 + lrow * N + lcol;
        if (m0 + BMT <= M && n0 + BNT <= N) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __builtin_nontemporal_store(f32_to_bf16_rne(out[mb][nb][r]), &yl16[int64_t(mb * 32 + 8 * (r >> 2) + (r & 3)) * N + nb * 32]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int ml = mb * 32 + 8 * (r >> 2) + (r & 3);
                        if (lrow + ml < M && lcol + nb * 32 < N)
                            __builtin_nontemporal_store(f32_to_bf16_rne(out[mb][nb][r]), &yl16[int64_t(ml) * N + nb * 32]);
                    }
        }
        return;
    }
    float* yl = y + lrow * N + lcol;
    if (m0 + BMT <= M && n0 + BNT <= N) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __builtin_nontemporal_store(out[mb][nb][r], &yl[int64_t(mb * 32 + 8 * (r >> 2) + (r & 3)) * N + nb * 32]);
    } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = mb * 32 + 8 * (r >> 2) + (r & 3);
                    if (lrow + ml < M && lcol + nb * 32 < N) __builtin_nontemporal_store(out[mb][nb][r], &yl[int64_t(ml) * N + nb * 32]);
                }
    }
    if (FMT == 1 && acc_out) {
        int32_t* al = acc_out + lrow * N + lcol;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = mb * 32 + 8 * (r >> 2) + (r & 3);
                    if (lrow + ml < M && lcol + nb * 32 < N) al[int64_t(ml) * N + nb * 32] = int32_t(fin[mb][nb][r]);
                }
    }
}

// Register budgets: two waves per SIMD (eight-wave workgroups, or two
// four-wave workgroups on a CU once there are more tiles than CUs).

template <bool XSUM, int WV, int BNT, int KH = 1, int BMT = BM>
__global__ void __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2, 2))) gemm_i8_i2s_kernel(const uint8_t* __restrict__ codes, int64_t N, int64_t K, const int8_t* __restrict__ xq,
                                 const float* __restrict__ xs, int64_t M, const float* __restrict__ bias,
                                 float* __restrict__ y, int32_t* __restrict__ acc_out, int S,
                                 int32_t* __restrict__ part, int32_t* __restrict__ counters,
                                 const int32_t* __restrict__ xsum, uint16_t* __restrict__ y16) {
    gemm_i8_body<1, XSUM, WV, BNT, KH, BMT>(codes, nullptr, N, K, xq, xs, M, bias, y, acc_out, S, part, counters, xsum, y16);
}

template <int WV, int BNT>
__global__ void __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(WV / 4, WV / 4))) gemm_i8_w1_kernel(
    const uint8_t* __restrict__ bits, const uint16_t* __restrict__ scales, int64_t N, int64_t K,
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int64_t M, const float* __restrict__ bias,
    float* __restrict__ y, int S, int32_t* __restrict__ part, int32_t* __restrict__ counters, uint16_t* __restrict__ y16) {
    gemm_i8_body<3, false, WV, BNT>(bits, scales, N, K, xq, xs, M, bias, y, nullptr, S, part, counters, nullptr, y16);
}

template <int WV, int BNT, int KH = 1, int BMT = BM>
__global__ void __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(WV / 4, WV / 4))) gemm_i8_tq2_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int64_t N, int64_t K,
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int64_t M, const float* __restrict__ bias,
    float* __restrict__ y, int S, int32_t* __restrict__ part, int32_t* __restrict__ counters, uint16_t* __restrict__ y16) {
    gemm_i8_body<2, false, WV, BNT, KH, BMT>(codes, scales, N, K, xq, xs, M, bias, y, nullptr, S, part, counters, nullptr, y16);
}

#ifndef LL_GEMM_SLOTS
#define LL_GEMM_SLOTS 256
#endif
#ifndef LL_GEMM_NARROW
#define LL_GEMM_NARROW 1
#endif
#ifndef LL_GEMM_HALVES
#define LL_GEMM_HALVES 1
#endif
#ifndef LL_GEMM_MAX_SPLITS
#define LL_GEMM_MAX_SPLITS 4                             // the last split adds the others' partial tiles serially
#endif
#ifndef LL_GEMM_SPLIT_GROUPS
#define LL_GEMM_SPLIT_GROUPS 10                          // 128-k groups a split keeps at least
#endif
#ifndef LL_GEMM_TQ2_HALVES
#define LL_GEMM_TQ2_HALVES 1                             // TQ2_0: narrow tiles as two halves where unsplit
#endif
#ifndef LL_GEMM_NARROW_ROWS
#define LL_GEMM_NARROW_ROWS 64                           // narrow tiles: 64 x 128 (or 128 x 64)
#endif
// Tile shape: 128 x 128 tiles of eight waves, or, for an i2_s product
// whose 128 x 128 tiles would leave half the chip idle (K would be split),
// tiles of half the area: 64 tokens x 128 weight rows (four waves along N,
// the same 64 x 32 wave tiles), split further only where those still leave
// the chip half idle.  Against 128 x 128 split tiles: 2560 x 6912 at M = 512
// 23.7 -> 21.4 us with 128 x 64 tiles, 2560 x 2560 18.3 -> 10.9 us.  The 64
// x 128 shape reads half the activation bytes per group of the 128 x 64 one
// for the same products (and each wave loads its own codes): 2560 x 6912 at
// M = 512 19.8 -> 16.8 us, 2560 x 2560 11.2 -> 9.4 us.  The block-scaled
// formats keep the wide tiles: their extra vector work per group needs the
// second wave per SIMD (TQ2_0 2560 x 6912 at M = 512: 26.1 us wide, 30.8 us
// with 128 x 64 tiles).  A narrow i2_s tile with K unsplit and an even group
// count runs eight waves as two halves along K (21.4 -> 19.8 us with the
// 128 x 64 shape).
struct TileShape {
    int bm, bn;
};
TileShape gemm_shape(int64_t M, int64_t N, bool narrow_ok) {
    constexpr int nbm = LL_GEMM_NARROW_ROWS, nbn = BM * BN / 2 / LL_GEMM_NARROW_ROWS;
    const int64_t wide = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const bool narrow = LL_GEMM_NARROW && narrow_ok && wide * 2 <= LL_GEMM_SLOTS &&
                        ((M + nbm - 1) / nbm) * ((N + nbn - 1) / nbn) <= LL_GEMM_SLOTS;
    return narrow ? TileShape{nbm, nbn} : TileShape{BM, BN};
}
bool gemm_narrow(int64_t M, int64_t N, bool narrow_ok) {
    const TileShape t = gemm_shape(M, N, narrow_ok);
    return t.bm != BM || t.bn != BN;
}
int64_t gemm_tiles(int64_t M, int64_t N, bool narrow_ok) {
    const TileShape t = gemm_shape(M, N, narrow_ok);
    return ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
}
int gemm_splits(int64_t M, int64_t N, int64_t K, bool narrow_ok, bool allow);
// Narrow tiles: i2_s wherever they apply; TQ2_0 where they need no split and
// K holds two 256-k blocks or more (it always runs them as two halves along
// K, one block or more each, its block scaling wanting two waves per SIMD);
// W1 never.
bool narrow_for(int fmt, int64_t M, int64_t N, int64_t K) {
    if (fmt == 1) return true;
    if (fmt != 2 || !LL_GEMM_TQ2_HALVES || K / 256 < 2) return false;   // each half at least one 256-k block
    return gemm_narrow(M, N, true) && gemm_splits(M, N, K, true, true) == 1;
}
// Split count: enough workgroups to cover the chip (LL_GEMM_SLOTS resident
// workgroups), at most four splits (the last one adds the others' partial
// tiles one after another) of at least ten 128-k groups each (TQ2_0:
// splits keep whole blocks), and at most one counter per tile in the
// counter region.  Measured on 2560 x 6912 at M = 64: twelve splits 17.2
// us, six 12.6, four 11.2; on 2560 x 2560 at M = 64 two splits beat four
// (9.2 against 10.1 us).
int gemm_splits(int64_t M, int64_t N, int64_t K, bool narrow_ok, bool allow) {
    const int64_t tiles = gemm_tiles(M, N, narrow_ok);
    if (!allow || tiles > kMaxCounters) return 1;
    const int64_t ng = K / 128;
    int64_t s = 1;
    while (s < LL_GEMM_MAX_SPLITS && tiles * (s + 1) <= LL_GEMM_SLOTS && ng / (s + 1) >= LL_GEMM_SPLIT_GROUPS) ++s;
    return int(s);
}

template <typename Kern, typename... Args>
hipError_t launch_tiles_lds(Kern kernel, int64_t tiles, int S, int threads, size_t lds, hipStream_t stream, Args... args) {
    const int64_t T = tiles * S;
    const dim3 grid{unsigned(LL_GEMM_XCD ? (T + 7) / 8 * 8 : T)}, block{unsigned(threads)};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kernel), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    return hipGetLastError();
}
template <typename Kern, typename... Args>
hipError_t launch_tiles(Kern kernel, int64_t tiles, int S, int threads, hipStream_t stream, Args... args) {
    return launch_tiles_lds(kernel, tiles, S, threads, kGemmLds, stream, args...);
}

}  // namespace

namespace llk {

size_t gemm_i8_workspace(int64_t M, int64_t N, int64_t K, int fmt) {
    const bool narrow_ok = narrow_for(fmt, M, N, K);
    const int S = gemm_splits(M, N, K, narrow_ok, true);
    if (S == 1) return 0;
    const TileShape t = gemm_shape(M, N, narrow_ok);
    return size_t(gemm_tiles(M, N, narrow_ok)) * S * size_t(t.bm) * size_t(t.bn) * 4;
}

hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq, const float* xs,
                              int64_t M, const float* bias, float* y, int32_t* acc_out, int32_t* counters, void* ws,
                              hipStream_t stream, const int32_t* xsum, uint16_t* y16) {
    const int64_t tiles = gemm_tiles(M, N, true);
    const int S = gemm_splits(M, N, K, true, ws != nullptr && counters != nullptr);
    constexpr int WV = LL_GEMM_I2S_WAVES;
    int32_t* part = static_cast<int32_t*>(ws);
    if (gemm_narrow(M, N, true)) {
        // narrow tiles (half the area): eight waves as two halves along K
        // where the halves get equal group counts and K is not split over
        // workgroups, else four waves
        constexpr int NBM = LL_GEMM_NARROW_ROWS, NBN = BM * BN / 2 / LL_GEMM_NARROW_ROWS;
        if (LL_GEMM_HALVES && S == 1 && (K / 128) % 2 == 0) {
            if (xsum)
                return launch_tiles_lds(gemm_i8_i2s_kernel<true, 8, NBN, 2, NBM>, tiles, S, 512, 2 * kGemmLds, stream, codes,
                                        N, K, xq, xs, M, bias, y, acc_out, S, part, counters, xsum, y16);
            return launch_tiles_lds(gemm_i8_i2s_kernel<false, 8, NBN, 2, NBM>, tiles, S, 512, 2 * kGemmLds, stream, codes,
                                    N, K, xq, xs, M, bias, y, acc_out, S, part, counters, xsum, y16);
        }
        if (xsum)
            return launch_tiles(gemm_i8_i2s_kernel<true, 4, NBN, 1, NBM>, tiles, S, 256, stream, codes, N, K, xq, xs, M,
                                bias, y, acc_out, S, part, counters, xsum, y16);
        return launch_tiles(gemm_i8_i2s_kernel<false, 4, NBN, 1, NBM>, tiles, S, 256, stream, codes, N, K, xq, xs, M, bias,
                            y, acc_out, S, part, counters, xsum, y16);
    }
    if (xsum)
        return launch_tiles(gemm_i8_i2s_kernel<true, WV, BN>, tiles, S, 64 * WV, stream, codes, N, K, xq, xs, M, bias, y,
                            acc_out, S, part, counters, xsum, y16);
    return launch_tiles(gemm_i8_i2s_kernel<false, WV, BN>, tiles, S, 64 * WV, stream, codes, N, K, xq, xs, M, bias, y,
                        acc_out, S, part, counters, xsum, y16);
}

hipError_t launch_gemm_i8_w1(const uint32_t* bits, const uint16_t* scales, int64_t N, int64_t K, const int8_t* xq,
                             const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                             hipStream_t stream, uint16_t* y16) {
    const int64_t tiles = gemm_tiles(M, N, false);
    const int S = gemm_splits(M, N, K, false, ws != nullptr && counters != nullptr);
    constexpr int WV = LL_GEMM_BLOCK_WAVES;
    const uint8_t* b8 = reinterpret_cast<const uint8_t*>(bits);
    return launch_tiles(gemm_i8_w1_kernel<WV, BN>, tiles, S, 64 * WV, stream, b8, scales, N, K, xq, xs, M, bias, y, S,
                        static_cast<int32_t*>(ws), counters, y16);
}

hipError_t launch_gemm_i8_tq2(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, const int8_t* xq,
                              const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                              hipStream_t stream, uint16_t* y16) {
    const bool narrow = narrow_for(2, M, N, K);
    const int64_t tiles = gemm_tiles(M, N, narrow);
    const int S = gemm_splits(M, N, K, narrow, ws != nullptr && counters != nullptr);
    constexpr int WV = LL_GEMM_BLOCK_WAVES;
    if (narrow) {                                          // unsplit (S = 1): two halves along K
        if (S != 1) return hipErrorInvalidValue;           // half 1 leaves before a split's handoff
        constexpr int NBM = LL_GEMM_NARROW_ROWS, NBN = BM * BN / 2 / LL_GEMM_NARROW_ROWS;
        return launch_tiles_lds(gemm_i8_tq2_kernel<8, NBN, 2, NBM>, tiles, S, 512, 2 * kGemmLds, stream, codes, scales, N,
                                K, xq, xs, M, bias, y, S, static_cast<int32_t*>(ws), counters, y16);
    }
    return launch_tiles(gemm_i8_tq2_kernel<WV, BN>, tiles, S, 64 * WV, stream, codes, scales, N, K, xq, xs, M, bias, y, S,
                        static_cast<int32_t*>(ws), counters, y16);
}

}  // namespace llk
