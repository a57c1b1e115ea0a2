/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for the packed low-bit
 * BitLinear product.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library; the product
 * library never links, calls or reads it, and it shares no code, header,
 * table or helper with the product library.
 *
 * Sources (the pages this follows):
 *   [BL]  Hesper API doc "Hesper/Layers/BitLinear": sections "i2_s Packing
 *         Format" (code table, layout, scale at the end of the tensor data),
 *         "BitLinear Mathematics" (the matrix-vector product), "High-Level
 *         API" (4-byte little-endian fp32 scale).
 *   [TQ]  Hesper API doc "Hesper/Quantization/TQ2_0": sections "TQ2_0 Format"
 *         (256-element blocks, 4 values per byte, fp16 scale, code table) and
 *         "Memory Layout Example" (64 packed bytes then scale_low, scale_high).
 *   [BG]  binary-gemm kernel card: sections "API" (pack_weights,
 *         quantize_activation, binary_gemm), "Method" (the stored bit
 *         b = (w+1)/2 and the dot identity), "Correctness" (zeros pack as -1,
 *         per-token absmax activations), "Usage" (from_dense: sign plus group
 *         mean-abs scale).
 *
 * Readings where the pages leave a step open are stated next to the code
 * that takes them.  Every accumulation is int64 (integer paths) or fp64
 * (floating-point paths); fp32 appears only where the method itself fixes
 * fp32 steps (activation quantization, the int8 epilogues).
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (no contraction, so every fp32 step below is one IEEE operation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Half and bfloat16 helpers, written from the IEEE 754 binary16 and   */
/* the bfloat16 (top half of binary32) definitions.                    */
/* ------------------------------------------------------------------ */

/* binary16 bits -> exact double. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* double -> binary16 bits, round to nearest, ties to even. */
uint16_t orc_f64_to_f16(double v)
{
    uint16_t sign = 0;
    if (isnan(v)) return 0x7e00;
    if (signbit(v)) { sign = 0x8000; v = -v; }
    if (v == 0.0) return sign;
    int E;
    frexp(v, &E);                 /* v = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                /* v in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: quantum 2^-24; rint rounds ties to even */
        double m = rint(ldexp(v, 24));
        return (uint16_t)(sign | (uint16_t)m);   /* m == 1024 is the smallest normal */
    }
    double m = rint(ldexp(v, 10 - e));            /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00); /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* bfloat16 bits are the upper 16 bits of a binary32. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to the even bf16 [BG "API":
   binary_linear returns bf16]: of the two bf16 values around f (f's bits
   cut to 16, and the next one away from zero) the nearer one, the one with
   an even last bit on a tie.  The next value past the largest finite bf16
   counts as 2^128 (so overflow rounds to infinity as in IEEE); NaN gives the
   quiet NaN 0x7FC0 with f's sign. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0) return lo;                 /* exactly representable (also +-inf) */
    uint16_t hi = (uint16_t)(lo + 1);
    double fv = fabs((double)f);
    double lv = fabs((double)orc_bf16_to_f32(lo));
    double hv = (hi & 0x7FFFu) == 0x7F80u ? ldexp(1.0, 128) : fabs((double)orc_bf16_to_f32(hi));
    double dl = fv - lv, dh = hv - fv;
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1u) ? hi : lo;
}

static void put_f32_le(uint8_t* p, float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    p[0] = (uint8_t)(u & 0xff);
    p[1] = (uint8_t)((u >> 8) & 0xff);
    p[2] = (uint8_t)((u >> 16) & 0xff);
    p[3] = (uint8_t)((u >> 24) & 0xff);
}

static float get_f32_le(const uint8_t* p)
{
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------ */
/* i2_s  [BL "i2_s Packing Format"]                                    */
/*                                                                     */
/* Code table: -1 -> 0b00, 0 -> 0b01, +1 -> 0b10; value = code - 1.    */
/* Each row holds K/4 bytes (rows contiguous; K a multiple of 128).    */
/* In each 128-element group of a row (32 bytes), element r sits in    */
/* byte r%32 of the group at shift 6 - 2*(r/32): elements 0..31 at     */
/* >>6, 32..63 at >>4, 64..95 at >>2, 96..127 at >>0.                  */
/* One fp32 scale, 4 bytes little-endian, right after the N*K/4 bytes. */
/* ------------------------------------------------------------------ */

static const uint8_t I2S_CODE_OF[3] = { 0x0 /* -1 */, 0x1 /* 0 */, 0x2 /* +1 */ };

static void i2s_locate(int64_t n, int64_t k, int64_t K, int64_t* byte, int* shift)
{
    int64_t g = k / 128, r = k % 128;
    *byte = n * (K / 4) + 32 * g + (r % 32);
    *shift = 6 - 2 * (int)(r / 32);
}

/* w: int8 [N,K] with values in {-1,0,1}.  out: N*K/4 + 4 bytes.
   Returns 0, or -1 for a bad shape, -4 for a weight outside {-1,0,1}. */
int orc_i2s_encode(const int8_t* w, int64_t N, int64_t K, float scale, uint8_t* out)
{
    if (N <= 0 || K <= 0 || K % 128) return -1;
    memset(out, 0, (size_t)(N * K / 4));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v = w[n * K + k];
            if (v < -1 || v > 1) return -4;
            int64_t b; int s;
            i2s_locate(n, k, K, &b, &s);
            out[b] |= (uint8_t)(I2S_CODE_OF[v + 1] << s);
        }
    put_f32_le(out + N * K / 4, scale);
    return 0;
}

/* Decodes every element (code - 1) and the tail scale.  Returns the
   number of invalid codes (0b11) seen; such elements decode as +2, the
   value the "code - 1" formula gives. */
int64_t orc_i2s_decode(const uint8_t* p, int64_t N, int64_t K, int8_t* w, float* scale)
{
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t b; int s;
            i2s_locate(n, k, K, &b, &s);
            int code = (p[b] >> s) & 3;
            if (code == 3) ++bad;
            w[n * K + k] = (int8_t)(code - 1);
        }
    if (scale) *scale = get_f32_le(p + N * K / 4);
    return bad;
}

/* Selected rows of y = scale * sum_k w[n,k] * x[m,k]  [BL "BitLinear
   Mathematics"], decoding each weight from the packed bytes, in fp64.
   x: fp32 [M,K].  rows: the nr row indices to evaluate (NULL = all N).
   y: fp64 [M, nr].  tsum (may be NULL): fp64 [M, nr] of
   scale * sum_k |x[m,k]|, the quantity the fp32 tolerance is relative to. */
void orc_i2s_gemv_f32(const uint8_t* p, int64_t N, int64_t K, const float* x, int64_t M,
                      const int64_t* rows, int64_t nr, double* y, double* tsum)
{
    double scale = (double)get_f32_le(p + N * K / 4);
    if (!rows) nr = N;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, ab = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t b; int s;
                i2s_locate(n, k, K, &b, &s);
                int w = ((p[b] >> s) & 3) - 1;
                acc += (double)w * (double)x[m * K + k];
                ab += fabs((double)x[m * K + k]);
            }
            y[m * nr + i] = scale * acc;
            if (tsum) tsum[m * nr + i] = fabs(scale) * ab;
        }
    }
}

/* int8 activations: acc = sum_k w*q exactly (int64); y = ((float)acc *
   s_tok) * s_w, two fp32 multiplies in that order.  acc_out (may be NULL)
   receives acc as int64 [M, nr]. */
void orc_i2s_gemm_i8(const uint8_t* p, int64_t N, int64_t K, const int8_t* q, const float* s_tok,
                     int64_t M, const int64_t* rows, int64_t nr, float* y, int64_t* acc_out)
{
    float s_w = get_f32_le(p + N * K / 4);
    if (!rows) nr = N;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t b; int s;
                i2s_locate(n, k, K, &b, &s);
                int w = ((p[b] >> s) & 3) - 1;
                acc += (int64_t)w * (int64_t)q[m * K + k];
            }
            volatile float t = (float)acc * s_tok[m];
            y[m * nr + i] = t * s_w;
            if (acc_out) acc_out[m * nr + i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* TQ2_0  [TQ "TQ2_0 Format", "Memory Layout Example"]                 */
/*                                                                     */
/* Blocks of 256 elements: 64 packed bytes (4 values per byte) then    */
/* the fp16 scale as scale_low, scale_high: 66 bytes per block.        */
/* Codes: 0 -> 0b00, +1 -> 0b01, -1 -> 0b11 (two's complement).        */
/* Readings: element e of a block sits in byte e/4 at bits 2*(e%4)     */
/* (four consecutive values per byte, least significant pair first);   */
/* blocks run along K inside a row, rows contiguous.  Code 0b10 is     */
/* never produced; read as two's complement it is -2.                  */
/* ------------------------------------------------------------------ */

static int tq2_code_of(int w) { return w == 0 ? 0x0 : (w == 1 ? 0x1 : 0x3); }

static int tq2_value_of(int code)
{
    switch (code) {
    case 0x0: return 0;
    case 0x1: return 1;
    case 0x3: return -1;
    default:  return -2;   /* 0b10, two's complement of a 2-bit field */
    }
}

/* w: int8 [N,K]; sc: fp16 bits [N*K/256] (block order); out: 66*N*K/256 bytes. */
int orc_tq2_encode(const int8_t* w, const uint16_t* sc, int64_t N, int64_t K, uint8_t* out)
{
    if (N <= 0 || K <= 0 || K % 256) return -1;
    int64_t nb = K / 256;
    memset(out, 0, (size_t)(66 * N * nb));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int v = w[n * K + k];
            if (v < -1 || v > 1) return -4;
            int64_t blk = n * nb + k / 256;
            int e = (int)(k % 256);
            out[66 * blk + e / 4] |= (uint8_t)(tq2_code_of(v) << (2 * (e % 4)));
        }
    for (int64_t blk = 0; blk < N * nb; ++blk) {
        out[66 * blk + 64] = (uint8_t)(sc[blk] & 0xff);        /* scale_low */
        out[66 * blk + 65] = (uint8_t)((sc[blk] >> 8) & 0xff); /* scale_high */
    }
    return 0;
}

/* Returns the number of 0b10 codes seen. */
int64_t orc_tq2_decode(const uint8_t* blocks, int64_t N, int64_t K, int8_t* w, uint16_t* sc)
{
    int64_t nb = K / 256, bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t blk = n * nb + k / 256;
            int e = (int)(k % 256);
            int code = (blocks[66 * blk + e / 4] >> (2 * (e % 4))) & 3;
            if (code == 2) ++bad;
            w[n * K + k] = (int8_t)tq2_value_of(code);
        }
    if (sc)
        for (int64_t blk = 0; blk < N * nb; ++blk)
            sc[blk] = (uint16_t)(blocks[66 * blk + 64] | (blocks[66 * blk + 65] << 8));
    return bad;
}

/* y = sum over blocks b of the row of s_b * sum_{k in b} w*x, fp64.
   tsum = sum_b |s_b| * sum_{k in b} |x|.  Same row/ output conventions as
   orc_i2s_gemv_f32. */
void orc_tq2_gemv_f32(const uint8_t* blocks, int64_t N, int64_t K, const float* x, int64_t M,
                      const int64_t* rows, int64_t nr, double* y, double* tsum)
{
    int64_t nb = K / 256;
    if (!rows) nr = N;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, ab = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* blk = blocks + 66 * (n * nb + b);
                double s = orc_f16_to_f64((uint16_t)(blk[64] | (blk[65] << 8)));
                double part = 0.0, pab = 0.0;
                for (int e = 0; e < 256; ++e) {
                    int w = tq2_value_of((blk[e / 4] >> (2 * (e % 4))) & 3);
                    double xv = (double)x[m * K + b * 256 + e];
                    part += (double)w * xv;
                    pab += fabs(xv);
                }
                acc += s * part;
                ab += fabs(s) * pab;
            }
            y[m * nr + i] = acc;
            if (tsum) tsum[m * nr + i] = ab;
        }
    }
}

/* int8 activations with TQ2_0 weights (the int8 reading of the block   */
/* product above, with x replaced by its quantization q, s_tok):        */
/* y = s_tok * sum_b s_b * d_b, d_b = sum_{k in b} w*q exactly (int64), */
/* every product and the sum in fp64.  tsum = s_tok * sum_b |s_b| *     */
/* sum_{k in b} |q|.  y, tsum: fp64 [M, nr]; same row conventions as    */
/* orc_i2s_gemv_f32.                                                    */
void orc_tq2_gemm_i8(const uint8_t* blocks, int64_t N, int64_t K, const int8_t* q, const float* s_tok,
                     int64_t M, const int64_t* rows, int64_t nr, double* y, double* tsum)
{
    int64_t nb = K / 256;
    if (!rows) nr = N;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, ab = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* blk = blocks + 66 * (n * nb + b);
                double s = orc_f16_to_f64((uint16_t)(blk[64] | (blk[65] << 8)));
                int64_t d = 0, da = 0;
                for (int e = 0; e < 256; ++e) {
                    int w = tq2_value_of((blk[e / 4] >> (2 * (e % 4))) & 3);
                    int64_t qv = q[m * K + b * 256 + e];
                    d += (int64_t)w * qv;
                    da += qv < 0 ? -qv : qv;
                }
                acc += s * (double)d;
                ab += fabs(s) * (double)da;
            }
            y[m * nr + i] = (double)s_tok[m] * acc;
            if (tsum) tsum[m * nr + i] = (double)s_tok[m] * ab;
        }
    }
}

/* ------------------------------------------------------------------ */
/* W1 sign bits  [BG "API", "Method", "Correctness"]                   */
/*                                                                     */
/* Stored bit b = (w+1)/2: +1 -> 1, -1 -> 0; zeros are packed as -1.   */
/* Reading: weight k of row n is bit k%32 of 32-bit word n*(K/32)+k/32 */
/* (least significant bit first).  One fp16 scale per G weights:       */
/* scales [N, K/G].                                                    */
/* ------------------------------------------------------------------ */

int orc_w1_encode(const int8_t* w, int64_t N, int64_t K, uint32_t* out)
{
    if (N <= 0 || K <= 0 || K % 32) return -1;
    memset(out, 0, (size_t)(N * (K / 32)) * 4);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int b = w[n * K + k] > 0 ? 1 : 0;     /* 0 and -1 both store 0 */
            out[n * (K / 32) + k / 32] |= (uint32_t)b << (k % 32);
        }
    return 0;
}

void orc_w1_decode(const uint32_t* bits, int64_t N, int64_t K, int8_t* w)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int b = (bits[n * (K / 32) + k / 32] >> (k % 32)) & 1;
            w[n * K + k] = (int8_t)(2 * b - 1);   /* w = 2b - 1 */
        }
}

/* from_dense [BG "Usage": sign + group mean-abs scale].  Readings: the
   sign bit is 1 where W > 0 (W == 0 stores -1, as zeros do in packing);
   the scale of a group is the mean of |W| over its G entries, summed in
   fp64 and rounded once to fp16 (nearest, ties to even).
   Rows [n0, n0+nrows) of a dense fp32 matrix with K columns; W points at
   row n0. */
int orc_w1_from_dense(const float* W, int64_t nrows, int64_t K, int32_t G, uint32_t* bits, uint16_t* sc)
{
    if (nrows <= 0 || K <= 0 || G <= 0 || K % 32 || K % G) return -1;
    memset(bits, 0, (size_t)(nrows * (K / 32)) * 4);
    for (int64_t n = 0; n < nrows; ++n) {
        for (int64_t k = 0; k < K; ++k)
            if (W[n * K + k] > 0.0f)
                bits[n * (K / 32) + k / 32] |= 1u << (k % 32);
        for (int64_t g = 0; g < K / G; ++g) {
            double s = 0.0;
            for (int64_t j = 0; j < G; ++j) s += fabs((double)W[n * K + g * G + j]);
            sc[n * (K / G) + g] = orc_f64_to_f16(s / (double)G);
        }
    }
    return 0;
}

/* W1A8 product.  For token m, row n, group g:
     d[g]  = sum_{k in g} w*q            (int64)
     dd[g] = 2 * sum_{k in g, b=1} q - sum_{k in g} q   (the card's identity)
   The two must agree; the return value counts disagreements (always 0 for
   a correct decode).  S = sum_g s[n,g] * d[g] in fp64, g ascending.
   y = (float)((double)s_tok[m] * S), then + bias[n] in fp32 when bias is
   given.  s_out (may be NULL) receives S. */
int64_t orc_w1a8_gemm(const uint32_t* bits, const uint16_t* sc, int64_t N, int64_t K, int32_t G,
                      const int8_t* q, const float* s_tok, int64_t M, const float* bias,
                      const int64_t* rows, int64_t nr, float* y, double* s_out)
{
    int64_t mism = 0;
    if (!rows) nr = N;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            double S = 0.0;
            for (int64_t g = 0; g < K / G; ++g) {
                int64_t d = 0, pos = 0, tot = 0;
                for (int64_t j = 0; j < G; ++j) {
                    int64_t k = g * G + j;
                    int b = (bits[n * (K / 32) + k / 32] >> (k % 32)) & 1;
                    int64_t qv = q[m * K + k];
                    d += (int64_t)(2 * b - 1) * qv;
                    if (b) pos += qv;
                    tot += qv;
                }
                if (d != 2 * pos - tot) ++mism;
                S += orc_f16_to_f64(sc[n * (K / G) + g]) * (double)d;
            }
            float v = (float)((double)s_tok[m] * S);
            if (bias) v = v + bias[n];
            y[m * nr + i] = v;
            if (s_out) s_out[m * nr + i] = S;
        }
    }
    return mism;
}

/* ------------------------------------------------------------------ */
/* Per-token absmax activation quantization [BG "API":                 */
/* quantize_activation; "Correctness": per-token absmax].              */
/* Readings (constants are not on the page): a = max_k |x|; a == 0     */
/* gives s = 0 and q = 0; otherwise inv = 127/a (one fp32 division),   */
/* q = round-half-even(x * inv) (one fp32 multiply) clamped to         */
/* [-127, 127], and s = a/127 (one fp32 division).                     */
/* ------------------------------------------------------------------ */

void orc_quantize_f32(const float* x, int64_t M, int64_t K, int8_t* q, float* s)
{
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(x[m * K + k]);
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
            s[m] = 0.0f;
            continue;
        }
        volatile float inv = 127.0f / a;
        for (int64_t k = 0; k < K; ++k) {
            volatile float v = x[m * K + k] * inv;
            float r = rintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
        volatile float sv = a / 127.0f;
        s[m] = sv;
    }
}

/* Same, from bfloat16 bits (bf16 -> fp32 is exact). */
void orc_quantize_bf16(const uint16_t* xb, int64_t M, int64_t K, int8_t* q, float* s)
{
    float* x = (float*)malloc((size_t)(M * K) * sizeof(float));
    for (int64_t i = 0; i < M * K; ++i) x[i] = orc_bf16_to_f32(xb[i]);
    orc_quantize_f32(x, M, K, q, s);
    free(x);
}
