// Host-side packing, unpacking and validation of the three packed weight
// formats (declared in lowbit.h).  Pure CPU code; these run once per weight
// tensor, offline, so they favour clarity over speed but stay O(N*K).
//
// i2_s   -- Hesper "BitLinear", section "i2_s Packing Format".
// TQ2_0  -- Hesper "TQ2_0", sections "TQ2_0 Format", "Memory Layout Example".
// W1     -- binary-gemm card, sections "API" and "Method".
#include <cmath>
#include <cstring>

#include "internal.h"

namespace {

// Builds each i2_s output byte from the four elements it holds: byte j of
// group g carries elements 128g + j + 32t at shift 6 - 2t (t = 0..3), with
// code = value + 1.
ll_status pack_i2s_row(const int8_t* w, int64_t K, uint8_t* out) {
    for (int64_t g = 0; g < K / 128; ++g) {
        const int8_t* src = w + 128 * g;
        for (int j = 0; j < 32; ++j) {
            unsigned byte = 0;
            for (int t = 0; t < 4; ++t) {
                int v = src[j + 32 * t];
                if (v < -1 || v > 1) return LL_ECODE;
                byte |= unsigned(v + 1) << (6 - 2 * t);
            }
            out[32 * g + j] = uint8_t(byte);
        }
    }
    return LL_OK;
}

// TQ2_0 code of a ternary value: 0 -> 0b00, +1 -> 0b01, -1 -> 0b11, i.e. the
// low two bits of the value in two's complement.
inline unsigned tq2_code(int v) { return unsigned(v) & 3u; }
// Two's-complement reading of a 2-bit field (0b10 reads as -2).
inline int tq2_value(unsigned c) { return int(c ^ 2u) - 2; }

uint16_t f16_from_double_rne(double v) {
    // IEEE binary16, round to nearest even; inputs here are finite.
    uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (a == 0.0) return sign;
    if (a >= 65520.0) return uint16_t(sign | 0x7c00);
    int e;
    (void)std::frexp(a, &e);          // a = f * 2^e, f in [0.5, 1)
    int exp = e - 1;                  // a in [2^exp, 2^(exp+1))
    if (exp < -14) exp = -14;         // subnormals share the quantum 2^-24
    double q = std::ldexp(a, 10 - exp);
    double r = std::nearbyint(q);     // default rounding mode: ties to even
    uint32_t m = uint32_t(r);
    // m in [0, 2048]; the exponent field is exp + 15 for m >= 1024 (normal),
    // and a carry to 2048 bumps the exponent.
    uint32_t bits;
    if (m >= 1024) {
        if (m == 2048) { m = 1024; ++exp; }
        bits = (uint32_t(exp + 15) << 10) | (m - 1024);
    } else {
        bits = m;                     // subnormal (exp == -14)
    }
    if (bits >= 0x7c00) bits = 0x7c00;
    return uint16_t(sign | bits);
}

}  // namespace

extern "C" {

size_t ll_packed_size(int32_t fmt, int64_t N, int64_t K, int32_t group, size_t* scales_bytes) {
    size_t sb = 0, cb = 0;
    if (N <= 0 || K <= 0) return 0;
    switch (fmt) {
    case LL_FMT_I2S:
        if (K % 128) return 0;
        cb = size_t(N) * size_t(K) / 4 + 4;
        break;
    case LL_FMT_TQ2_0:
        if (K % 256) return 0;
        cb = size_t(N) * size_t(K / 256) * 66;
        sb = size_t(N) * size_t(K / 256) * 2;
        break;
    case LL_FMT_W1:
        if (K % 32 || group <= 0 || group % 32 || K % group) return 0;
        cb = size_t(N) * size_t(K) / 8;
        sb = size_t(N) * size_t(K / group) * 2;
        break;
    default:
        return 0;
    }
    if (scales_bytes) *scales_bytes = sb;
    return cb;
}

ll_status ll_pack_i2s(const int8_t* w, int64_t N, int64_t K, float scale, uint8_t* out) {
    if (!w || !out || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_pack_i2s: null pointer or non-positive size");
    if (K % 128) return ll::fail(LL_ESHAPE, "ll_pack_i2s: K must be a multiple of 128");
    // validate first so that an error leaves `out` untouched
    for (int64_t i = 0; i < N * K; ++i)
        if (w[i] < -1 || w[i] > 1) return ll::fail(LL_ECODE, "ll_pack_i2s: weight outside {-1,0,+1}");
    for (int64_t n = 0; n < N; ++n) pack_i2s_row(w + n * K, K, out + n * (K / 4));
    uint32_t u;
    std::memcpy(&u, &scale, 4);
    uint8_t* tail = out + N * (K / 4);
    for (int b = 0; b < 4; ++b) tail[b] = uint8_t(u >> (8 * b));
    return LL_OK;
}

ll_status ll_unpack_i2s(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, float* scale) {
    if (!packed || !w || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_unpack_i2s: null pointer or non-positive size");
    if (K % 128) return ll::fail(LL_ESHAPE, "ll_unpack_i2s: K must be a multiple of 128");
    bool bad = false;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < K / 128; ++g)
            for (int j = 0; j < 32; ++j) {
                unsigned byte = packed[n * (K / 4) + 32 * g + j];
                for (int t = 0; t < 4; ++t) {
                    unsigned c = (byte >> (6 - 2 * t)) & 3u;
                    bad |= (c == 3);
                    w[n * K + 128 * g + 32 * t + j] = int8_t(int(c) - 1);
                }
            }
    if (scale) {
        const uint8_t* tail = packed + N * (K / 4);
        uint32_t u = uint32_t(tail[0]) | uint32_t(tail[1]) << 8 | uint32_t(tail[2]) << 16 | uint32_t(tail[3]) << 24;
        std::memcpy(scale, &u, 4);
    }
    return bad ? ll::fail(LL_ECODE, "ll_unpack_i2s: code 0b11 present") : LL_OK;
}

ll_status ll_pack_tq2(const int8_t* w, const uint16_t* scales, int64_t N, int64_t K, uint8_t* out) {
    if (!w || !scales || !out || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_pack_tq2: null pointer or non-positive size");
    if (K % 256) return ll::fail(LL_ESHAPE, "ll_pack_tq2: K must be a multiple of 256");
    for (int64_t i = 0; i < N * K; ++i)
        if (w[i] < -1 || w[i] > 1) return ll::fail(LL_ECODE, "ll_pack_tq2: weight outside {-1,0,+1}");
    const int64_t nb = N * (K / 256);
    for (int64_t b = 0; b < nb; ++b) {
        const int8_t* src = w + 256 * b;     // blocks run along K, rows contiguous
        uint8_t* dst = out + 66 * b;
        for (int j = 0; j < 64; ++j) {
            unsigned byte = 0;
            for (int f = 0; f < 4; ++f) byte |= tq2_code(src[4 * j + f]) << (2 * f);
            dst[j] = uint8_t(byte);
        }
        dst[64] = uint8_t(scales[b] & 0xff);
        dst[65] = uint8_t(scales[b] >> 8);
    }
    return LL_OK;
}

ll_status ll_unpack_tq2(const uint8_t* blocks, int64_t N, int64_t K, int8_t* w, uint16_t* scales) {
    if (!blocks || !w || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_unpack_tq2: null pointer or non-positive size");
    if (K % 256) return ll::fail(LL_ESHAPE, "ll_unpack_tq2: K must be a multiple of 256");
    bool bad = false;
    const int64_t nb = N * (K / 256);
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* src = blocks + 66 * b;
        for (int e = 0; e < 256; ++e) {
            unsigned c = (src[e >> 2] >> (2 * (e & 3))) & 3u;
            bad |= (c == 2);
            w[256 * b + e] = int8_t(tq2_value(c));
        }
        if (scales) scales[b] = uint16_t(src[64] | (src[65] << 8));
    }
    return bad ? ll::fail(LL_ECODE, "ll_unpack_tq2: code 0b10 present") : LL_OK;
}

ll_status ll_tq2_split(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    if (!blocks || !codes || !scales || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_tq2_split: null pointer or non-positive size");
    if (K % 256) return ll::fail(LL_ESHAPE, "ll_tq2_split: K must be a multiple of 256");
    const int64_t nb = N * (K / 256);
    for (int64_t b = 0; b < nb; ++b) {
        std::memcpy(codes + 64 * b, blocks + 66 * b, 64);
        scales[b] = uint16_t(blocks[66 * b + 64] | (blocks[66 * b + 65] << 8));
    }
    return LL_OK;
}

ll_status ll_pack_w1(const int8_t* w, int64_t N, int64_t K, uint32_t* out) {
    if (!w || !out || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_pack_w1: null pointer or non-positive size");
    if (K % 32) return ll::fail(LL_ESHAPE, "ll_pack_w1: K must be a multiple of 32");
    for (int64_t word = 0; word < N * (K / 32); ++word) {
        const int8_t* src = w + 32 * word;
        uint32_t v = 0;
        for (int i = 0; i < 32; ++i) v |= uint32_t(src[i] > 0) << i;
        out[word] = v;
    }
    return LL_OK;
}

ll_status ll_unpack_w1(const uint32_t* bits, int64_t N, int64_t K, int8_t* w) {
    if (!bits || !w || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_unpack_w1: null pointer or non-positive size");
    if (K % 32) return ll::fail(LL_ESHAPE, "ll_unpack_w1: K must be a multiple of 32");
    for (int64_t word = 0; word < N * (K / 32); ++word)
        for (int i = 0; i < 32; ++i) w[32 * word + i] = ((bits[word] >> i) & 1u) ? 1 : -1;
    return LL_OK;
}

ll_status ll_w1_from_dense(const float* W, int64_t N, int64_t K, int32_t group, uint32_t* bits, uint16_t* scales) {
    if (!W || !bits || !scales || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_w1_from_dense: null pointer or non-positive size");
    if (K % 32 || group <= 0 || group % 32 || K % group)
        return ll::fail(LL_ESHAPE, "ll_w1_from_dense: need K % 32 == 0, group a positive multiple of 32, K % group == 0");
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        for (int64_t word = 0; word < K / 32; ++word) {
            uint32_t v = 0;
            for (int i = 0; i < 32; ++i) v |= uint32_t(row[32 * word + i] > 0.0f) << i;
            bits[n * (K / 32) + word] = v;
        }
        for (int64_t g = 0; g < K / group; ++g) {
            double s = 0.0;
            for (int32_t j = 0; j < group; ++j) s += std::fabs(double(row[g * group + j]));
            scales[n * (K / group) + g] = f16_from_double_rne(s / double(group));
        }
    }
    return LL_OK;
}

ll_status ll_validate(int32_t fmt, const void* codes, int64_t N, int64_t K, int64_t* bad_index) {
    if (bad_index) *bad_index = -1;
    if (!codes || N <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_validate: null pointer or non-positive size");
    const uint8_t* p = static_cast<const uint8_t*>(codes);
    if (fmt == LL_FMT_I2S) {
        if (K % 128) return ll::fail(LL_ESHAPE, "ll_validate: i2_s needs K % 128 == 0");
        for (int64_t i = 0; i < N * K / 4; ++i) {
            unsigned b = p[i];
            for (int t = 0; t < 4; ++t)
                if (((b >> (6 - 2 * t)) & 3u) == 3u) {
                    int64_t n = i / (K / 4), r = i % (K / 4);
                    if (bad_index) *bad_index = n * K + 128 * (r / 32) + 32 * t + r % 32;
                    return ll::fail(LL_ECODE, "ll_validate: i2_s code 0b11");
                }
        }
        return LL_OK;
    }
    if (fmt == LL_FMT_TQ2_0) {
        if (K % 256) return ll::fail(LL_ESHAPE, "ll_validate: TQ2_0 needs K % 256 == 0");
        for (int64_t i = 0; i < N * K / 4; ++i) {
            unsigned b = p[i];
            for (int f = 0; f < 4; ++f)
                if (((b >> (2 * f)) & 3u) == 2u) {
                    if (bad_index) *bad_index = 4 * i + f;
                    return ll::fail(LL_ECODE, "ll_validate: TQ2_0 code 0b10");
                }
        }
        return LL_OK;
    }
    if (fmt == LL_FMT_W1) {
        if (K % 32) return ll::fail(LL_ESHAPE, "ll_validate: W1 needs K % 32 == 0");
        return LL_OK;
    }
    return ll::fail(LL_EINVAL, "ll_validate: unknown format");
}

}  // extern "C"
