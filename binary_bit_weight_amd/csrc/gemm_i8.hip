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
// Workgroup tile 128 x 128 as four 64 x 64 wave tiles, each owned by two
// waves (eight waves, two per SIMD): one multiplies the 32-k steps 0 and 1
// of every 128-k group, the other steps 2 and 3, and the pair adds its
// halves through LDS at the end.  A wave keeps four 32 x 32 accumulators,
// so every operand read from LDS feeds two multiplies, and while one wave of
// a SIMD waits (LDS, barrier) the other multiplies.  Per group the workgroup
// stores the int8 activation tile (rows padded to 144 bytes) and the weight
// codes still packed (32 bytes per column, padded to 48) into one of two LDS
// buffers.  A lane reads its column's 16 code bytes once per group and
// decodes its two steps in registers (shift, mask, byte permute through
// {0xFF, 0x00, 0x01}).  Both paddings put the 8 lanes of one LDS access on
// distinct banks.  Global loads run D - 1 groups ahead in D register
// stages, every load from a clamped in-bounds address so the compiler can
// count its waits; one barrier per group.
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
// 16 bits of its code dword; each nibble is spread to four bytes by one
// multiply and a mask and mapped to -1 / +1 (b * 0xFE ^ 0xFF).  Every group
// is a scale block; its scale is kept per LDS buffer, since the next group
// is stored before this one is multiplied.
//
// Split K.  With few output tiles (N = 2560 at M = 512 gives 80) the
// workgroups of a tile split its groups S ways.  Each split writes its exact
// int32 partial tile to the workspace and increments the tile's counter; the
// split that arrives last adds the others' partials to its own and runs the
// epilogue, then resets the counter (so the counters stay zero between
// calls).  Integer addition makes the result independent of the order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int BM = 128, BN = 128, LDA = 144, LDB = 48;
constexpr int kThreads = 512;                            // eight waves
constexpr int kTileInts = BM * BN;                       // one partial tile
constexpr int kBuf = BM * LDA + BN * LDB;                // one LDS buffer: activation tile, then packed codes
constexpr int kXchg = kTileInts * 4;                     // final exchange of half accumulators (bytes)
constexpr size_t kGemmLds = size_t(2) * kBuf > size_t(kXchg) ? size_t(2) * kBuf : size_t(kXchg);
#ifndef LL_GEMM_XCD
#define LL_GEMM_XCD 1                                    // XCD-grouped workgroup order
#endif
#ifndef LL_GEMM_DEPTH
#define LL_GEMM_DEPTH 4                                  // register stages of global loads
#endif
#ifndef LL_GEMM_DEPTH_TQ2
#define LL_GEMM_DEPTH_TQ2 2                              // TQ2_0: its fp32 block sums take the registers of two stages
#endif


// FMT 1: i2_s, FMT 2: TQ2_0 (scales: fp16 [N][K/256]), FMT 3: W1 with
// G = 128 (codes: the sign-bit words, scales: fp16 [N][K/128]).
template <int FMT>
__device__ __forceinline__ void gemm_i8_body(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                             int64_t N, int64_t K, const int8_t* __restrict__ xq,
                                             const float* __restrict__ xs, int64_t M, const float* __restrict__ bias,
                                             float* __restrict__ y, int32_t* __restrict__ acc_out, int S,
                                             int32_t* __restrict__ part, int32_t* __restrict__ counters) {
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    __shared__ int last_flag;
    const int tid = threadIdx.x, lane = tid & 63;
    const int kh = __builtin_amdgcn_readfirstlane(tid >> 8);   // k half: steps 2 kh, 2 kh + 1
    const int wq = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    const int wm = wq >> 1, wn = wq & 1;                   // rows 64 wm, columns 64 wn of the tile
    const int li = lane & 31, h = lane >> 5;
    const int64_t TM = (M + BM - 1) / BM;
    // Hardware workgroup w runs on XCD w % 8; it takes logical index
    // (w % 8) T8 + w / 8, so consecutive logical workgroups (the splits and
    // row tiles of one column tile, which read the same weight codes) share
    // one XCD's L2.
    const int64_t T = ((N + BN - 1) / BN) * TM * S, T8 = (T + 7) / 8;
    const int64_t L = LL_GEMM_XCD ? (int64_t(blockIdx.x) % 8) * T8 + int64_t(blockIdx.x) / 8 : int64_t(blockIdx.x);
    if (L >= T) return;                                    // whole workgroup, before any barrier
    const int64_t tile = L / S;
    const int split = int(L % S);
    const int64_t m0 = (tile % TM) * BM, n0 = (tile / TM) * BN;
    const int64_t rowbytes = FMT == 3 ? K / 8 : K / 4;
    const int64_t ng = K / 128;
    // TQ2_0: splits of whole 256-k blocks, so every split starts on an even group
    const int64_t nsplit_units = FMT != 2 ? ng : K / 256, per_unit = FMT != 2 ? 1 : 2;
    const int64_t g0 = per_unit * (nsplit_units * split / S), g1 = per_unit * (nsplit_units * (split + 1) / S);

    // Loads of one group: two 16-byte activation chunks (row idx / 8, chunk
    // idx % 8 for idx = tid + 512 c) and 8 code bytes (column tid / 4,
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
    const int bcol = tid >> 2, bqt = tid & 3;
    int64_t ncl = n0 + bcol;
    ncl = ncl < N ? ncl : N - 1;
    const uint8_t* bptr = codes + ncl * rowbytes + (FMT == 3 ? 4 : 8) * bqt;
    // TQ2_0 / W1: block scales of this lane's two columns
    const uint16_t* sptr[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        int64_t n = n0 + wn * 64 + nb * 32 + li;
        n = n < N ? n : N - 1;
        sptr[nb] = FMT == 2 ? scales + n * (K / 256) : FMT == 3 ? scales + n * (K / 128) : nullptr;
    }

    struct Stage {
        i32x4 a[2];
        u32x2 b;
        uint16_t sc[FMT == 1 ? 1 : 2];                      // TQ2_0 / W1: the group's block scales
    };
    auto load = [&](int64_t g, Stage& s) {
        const int64_t gc = g < g1 ? g : g1 - 1;            // past the range: reload the last group (unused)
#pragma unroll
        for (int c = 0; c < 2; ++c) s.a[c] = ld16(arow[c] + 128 * gc);
        if constexpr (FMT == 3)
            s.b = u32x2{*(const __attribute__((address_space(1))) uint32_t*)(bptr + 16 * gc), 0u};
        else
            s.b = *(const __attribute__((address_space(1))) u32x2*)(bptr + 32 * gc);
        if constexpr (FMT != 1)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) s.sc[nb] = ld2(sptr[nb] + (FMT == 2 ? gc / 2 : gc));
    };
    // scales of the block being multiplied: TQ2_0 in curs[0], taken when the
    // block's second (odd) group is stored; W1 in curs[buf], the group in LDS
    // buffer buf
    float curs[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    auto store = [&](int buf, const Stage& s, bool odd) {
        int8_t* A = lds + buf * kBuf;
        int8_t* B = A + BM * LDA;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int idx = tid + kThreads * c;
            int8_t* arow_l = &A[(idx >> 3) * LDA];
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
        if constexpr (FMT == 3)
            *reinterpret_cast<uint32_t*>(&B[bcol * LDB + 4 * bqt]) = s.b[0];
        else
            *reinterpret_cast<u32x2*>(&B[bcol * LDB + 8 * bqt]) = s.b;
        if constexpr (FMT == 2) {
            if (odd)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) curs[0][nb] = half_bits_to_float(s.sc[nb]);
        } else if constexpr (FMT == 3) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) curs[buf][nb] = half_bits_to_float(s.sc[nb]);
        }
    };

    // epilogue operands, requested before the main loop so their latency is
    // hidden: token scales of this lane's rows (row half kh after the
    // exchange), the weight scale, the biases of its columns
    float xsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + kh * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        xsv[r] = xs[m < M ? m : M - 1];
    }
    const float sw = FMT == 1 ? *reinterpret_cast<const float*>(codes + N * rowbytes) : 1.0f;
    const float* bsrc = bias ? bias : xs;                 // always a valid address
    float bnv[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n0 + wn * 64 + nb * 32 + li;
        bnv[nb] = bsrc[bias ? (n < N ? n : N - 1) : 0];
    }

    i32x16 acc[2][2];
    f32x16 facc[FMT == 1 ? 1 : 2][2];                      // TQ2_0 / W1: scaled block sums
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[mb][nb][r] = 0;
                if constexpr (FMT != 1) facc[mb][nb][r] = 0.0f;
            }

    // odd (TQ2_0): the group ends a 256-k block, whose sums are then scaled
    // into facc; the block's first multiply (even group, first step) starts
    // from zero
    auto compute = [&](int buf, bool odd) {
        const int8_t* A = lds + buf * kBuf + (wm * 64 + li) * LDA + 16 * h + 64 * kh;
        // (W1: all 16 code bytes of the column's group; the lane takes its half of each dword)
        const int8_t* B = lds + buf * kBuf + BM * LDA + (wn * 64 + li) * LDB + (FMT == 3 ? 0 : 16 * h);
        // i2_s: code byte j of this lane's 16 holds, in field t (bits 6 - 2t),
        // the weight of k = 32 t + 16 h + j: the B operand of step t.  TQ2_0:
        // field t (bits 2t) holds element 4 (16 h + j) + t, matching plane t.
        i32x4 bq[2], ao[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bq[nb] = *reinterpret_cast<const i32x4*>(B + nb * 32 * LDB);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                ao[tt][mb] = *reinterpret_cast<const i32x4*>(A + mb * 32 * LDA + 32 * tt);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int sh = FMT == 1 ? 6 - 4 * kh - 2 * tt : 4 * kh + 2 * tt;
            // code -> int8 by byte permute: i2_s {-1, 0, +1}, TQ2_0 {0, +1, -2, -1}
            constexpr uint32_t table = FMT == 1 ? 0x000100FFu : 0xFFFE0100u;
            i32x4 bo[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                if constexpr (FMT == 3) {
                    // bits 16 h .. 16 h + 15 of code dword t = 2 kh + tt: k = 32 t + 16 h + j
                    const uint32_t v = (uint32_t(bq[nb][2 * kh + tt]) >> (16 * h)) & 0xFFFFu;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t sp = (((v >> (4 * i)) & 0xFu) * 0x00204081u) & 0x01010101u;   // bit e -> byte e
                        bo[nb][i] = int((sp * 0xFEu) ^ 0xFFFFFFFFu);                                // 1 -> +1, 0 -> -1
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        bo[nb][i] = int(__builtin_amdgcn_perm(0u, table, (uint32_t(bq[nb][i]) >> sh) & 0x03030303u));
                }
            }
            const bool first = (FMT == 2 && !odd && tt == 0) || (FMT == 3 && tt == 0);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[tt][mb], bo[nb], first ? i32x16{} : acc[mb][nb],
                                                                        0, 0, 0);
        }
        if constexpr (FMT != 1)
            if (FMT == 3 || odd)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const float sc = FMT == 3 ? curs[buf][nb] : curs[0][nb];
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            facc[mb][nb][r] = __builtin_fmaf(float(acc[mb][nb][r]), sc, facc[mb][nb][r]);
                    }
    };

    // Group g + i is multiplied from LDS buffer i % 2; register stage i % D
    // holds group g + i from its load (D - 1 groups earlier) to its store
    // (one group earlier).  The main loop runs whole runs of D groups with no
    // early exit; the last 1 .. D - 1 groups follow it.
    constexpr int D = FMT == 1 ? LL_GEMM_DEPTH : LL_GEMM_DEPTH_TQ2;   // (W1 as TQ2_0)
    static_assert(D % 2 == 0 && D >= 2, "even register depth");
    // (g0 and D are even, so group g + i is odd exactly when i is)
    Stage st[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load(g0 + i, st[i]);
    store(0, st[0], false);
    __syncthreads();
    const int64_t nsteps = g1 - g0;
    int64_t g = g0;
    for (; g + D <= g1; g += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            // loads first (kept there by the scheduling barrier); the store of
            // the next group and the multiplies of this one may interleave
            load(g + D + i, st[i]);
            __builtin_amdgcn_sched_barrier(0);
            store((i + 1) & 1, st[(i + 1) % D], (i + 1) & 1);
            compute(i & 1, i & 1);
            __syncthreads();
        }
    }
    const int rem = int(nsteps % D);
#pragma unroll
    for (int j = 0; j < D - 1; ++j) {
        if (j < rem) {
            if (j > 0) {
                store(j & 1, st[j], j & 1);
                __syncthreads();
            }
            compute(j & 1, j & 1);
        }
    }

    // The two k halves of each wave tile meet: the wave of half kh keeps row
    // block mb = kh and hands the other to its partner through LDS.
    // (TQ2_0: the same with the fp32 block-scaled sums)
    using E = std::conditional_t<FMT == 1, int32_t, float>;
    using V = std::conditional_t<FMT == 1, i32x16, f32x16>;
    __syncthreads();                                       // every wave is done with the operand buffers
    E* xb = reinterpret_cast<E*>(lds);
    V fin[2];
    if constexpr (FMT == 1) {
        if (kh == 0) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                fin[nb] = acc[0][nb];
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[((0 * 4 + wq) * 32 + nb * 16 + r) * 64 + lane] = acc[1][nb][r];
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                fin[nb] = acc[1][nb];
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[((1 * 4 + wq) * 32 + nb * 16 + r) * 64 + lane] = acc[0][nb][r];
            }
        }
    } else {
        if (kh == 0) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                fin[nb] = facc[0][nb];
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[((0 * 4 + wq) * 32 + nb * 16 + r) * 64 + lane] = facc[1][nb][r];
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                fin[nb] = facc[1][nb];
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[((1 * 4 + wq) * 32 + nb * 16 + r) * 64 + lane] = facc[0][nb][r];
            }
        }
    }
    __syncthreads();
    {
        const E* pb = xb + ((1 - kh) * 4 + wq) * 32 * 64;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) fin[nb][r] += pb[(nb * 16 + r) * 64 + lane];
    }

    if (S > 1) {
        // Publish this split's partial tile with device-coherent stores, wait for
        // them to complete, then count the split in; the split that arrives last
        // reads the others' partials (device-coherent loads) and finishes the tile.
        int32_t* mine = part + (tile * S + split) * int64_t(kTileInts);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st_coherent(mine + (nb * 16 + r) * kThreads + tid, __builtin_bit_cast(int32_t, E(fin[nb][r])));
        wait_vmem();
        __syncthreads();
        if (tid == 0) last_flag = arrive_acq_rel(counters + tile) == S - 1;
        __syncthreads();
        if (!last_flag) return;
        if constexpr (FMT == 1) {
            for (int s = 0; s < S; ++s) {
                if (s == split) continue;
                const int32_t* other = part + (tile * S + s) * int64_t(kTileInts);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) fin[nb][r] += ld_coherent(other + (nb * 16 + r) * kThreads + tid);
            }
        } else {
            // fp32 partials added in split order (this split's own from registers)
            V tot[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) tot[nb][r] = 0.0f;
            for (int s = 0; s < S; ++s) {
                const int32_t* other = part + (tile * S + s) * int64_t(kTileInts);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        tot[nb][r] += s == split ? fin[nb][r]
                                                 : __builtin_bit_cast(float, ld_coherent(other + (nb * 16 + r) * kThreads + tid));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) fin[nb] = tot[nb];
        }
        if (tid == 0) st_coherent(counters + tile, 0);    // ready for the next call
    }

    // Epilogue: y = ((float)acc * s_tok) * s_w (+ bias); TQ2_0 y = acc * s_tok (+ bias).  Lane (li, h) of half
    // kh holds column wn 64 + nb 32 + li and rows wm 64 + kh 32 + 8 (r / 4) +
    // 4 h + r % 4; its output pointer is formed once, each store adds a
    // uniform row offset.  The stores of a full tile run as one straight block
    // (a branch between stores would make each wait for the one before).
    float out[2][16];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = FMT == 1 ? __fmul_rn(__fmul_rn(float(fin[nb][r]), xsv[r]), sw) : __fmul_rn(float(fin[nb][r]), xsv[r]);
            out[nb][r] = bias ? __fadd_rn(v, bnv[nb]) : v;
        }
    const int64_t lrow = m0 + wm * 64 + kh * 32 + 4 * h, lcol = n0 + wn * 64 + li;
    float* yl = y + lrow * N + lcol;
    if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) yl[int64_t(8 * (r >> 2) + (r & 3)) * N + nb * 32] = out[nb][r];
    } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = 8 * (r >> 2) + (r & 3);
                if (lrow + ml < M && lcol + nb * 32 < N) yl[int64_t(ml) * N + nb * 32] = out[nb][r];
            }
    }
    if (FMT == 1 && acc_out) {
        int32_t* al = acc_out + lrow * N + lcol;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = 8 * (r >> 2) + (r & 3);
                if (lrow + ml < M && lcol + nb * 32 < N) al[int64_t(ml) * N + nb * 32] = int32_t(fin[nb][r]);
            }
    }
}

__global__ void __launch_bounds__(kThreads) gemm_i8_i2s_kernel(const uint8_t* __restrict__ codes, int64_t N,
                                                                int64_t K, const int8_t* __restrict__ xq,
                                                                const float* __restrict__ xs, int64_t M,
                                                                const float* __restrict__ bias, float* __restrict__ y,
                                                                int32_t* __restrict__ acc_out, int S,
                                                                int32_t* __restrict__ part,
                                                                int32_t* __restrict__ counters) {
    gemm_i8_body<1>(codes, nullptr, N, K, xq, xs, M, bias, y, acc_out, S, part, counters);
}

__global__ void __launch_bounds__(kThreads) gemm_i8_w1_kernel(const uint8_t* __restrict__ bits,
                                                               const uint16_t* __restrict__ scales, int64_t N,
                                                               int64_t K, const int8_t* __restrict__ xq,
                                                               const float* __restrict__ xs, int64_t M,
                                                               const float* __restrict__ bias, float* __restrict__ y,
                                                               int S, int32_t* __restrict__ part,
                                                               int32_t* __restrict__ counters) {
    gemm_i8_body<3>(bits, scales, N, K, xq, xs, M, bias, y, nullptr, S, part, counters);
}

__global__ void __launch_bounds__(kThreads) gemm_i8_tq2_kernel(const uint8_t* __restrict__ codes,
                                                                const uint16_t* __restrict__ scales, int64_t N,
                                                                int64_t K, const int8_t* __restrict__ xq,
                                                                const float* __restrict__ xs, int64_t M,
                                                                const float* __restrict__ bias, float* __restrict__ y,
                                                                int S, int32_t* __restrict__ part,
                                                                int32_t* __restrict__ counters) {
    gemm_i8_body<2>(codes, scales, N, K, xq, xs, M, bias, y, nullptr, S, part, counters);
}

#ifndef LL_GEMM_SLOTS
#define LL_GEMM_SLOTS 256
#endif
// Split count: enough workgroups to cover the chip (LL_GEMM_SLOTS resident
// workgroups) without leaving a split fewer than four groups (two TQ2_0
// blocks: splits keep whole blocks).
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
    return size_t(tiles) * S * kTileInts * 4;
}

hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq, const float* xs,
                              int64_t M, const float* bias, float* y, int32_t* acc_out, int32_t* counters, void* ws, hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int S = gemm_splits(M, N, K, ws != nullptr && counters != nullptr && tiles <= kMaxCounters);
    int32_t* part = static_cast<int32_t*>(ws);
    const int64_t T = tiles * S;
    const dim3 grid{unsigned(LL_GEMM_XCD ? (T + 7) / 8 * 8 : T)}, block{unsigned(kThreads)};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gemm_i8_i2s_kernel), kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_i8_i2s_kernel, grid, block, kGemmLds, stream, codes, N, K, xq, xs, M, bias, y, acc_out, S,
                       part, counters);
    return hipGetLastError();
}

hipError_t launch_gemm_i8_w1(const uint32_t* bits, const uint16_t* scales, int64_t N, int64_t K, const int8_t* xq,
                             const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                             hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int S = gemm_splits(M, N, K, ws != nullptr && counters != nullptr && tiles <= kMaxCounters);
    int32_t* part = static_cast<int32_t*>(ws);
    const int64_t T = tiles * S;
    const dim3 grid{unsigned(LL_GEMM_XCD ? (T + 7) / 8 * 8 : T)}, block{unsigned(kThreads)};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gemm_i8_w1_kernel), kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_i8_w1_kernel, grid, block, kGemmLds, stream, reinterpret_cast<const uint8_t*>(bits), scales,
                       N, K, xq, xs, M, bias, y, S, part, counters);
    return hipGetLastError();
}

hipError_t launch_gemm_i8_tq2(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, const int8_t* xq,
                              const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                             hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int S = gemm_splits(M, N, K, ws != nullptr && counters != nullptr && tiles <= kMaxCounters);
    int32_t* part = static_cast<int32_t*>(ws);
    const int64_t T = tiles * S;
    const dim3 grid{unsigned(LL_GEMM_XCD ? (T + 7) / 8 * 8 : T)}, block{unsigned(kThreads)};
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gemm_i8_tq2_kernel), kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_i8_tq2_kernel, grid, block, kGemmLds, stream, codes, scales, N, K, xq, xs, M, bias, y, S,
                       part, counters);
    return hipGetLastError();
}

}  // namespace llk
