"""Pure-Python brute-force restatements used to pin the C oracle on tiny inputs.

Each function follows a *different* statement on the pages from the one the
oracle's C code follows, so an index or shift slip in either shows up as a
disagreement:

* i2_s: the per-u32 unpacking statement of "Hesper/Layers/BitLinear",
  section "Fused BitLinear Kernel (i2_s format)" (group128 = u32 index / 8,
  base position = (u32 index % 8) * 4, element = group128*128 + base + byte
  + (3 - shift/2)*32), where the oracle uses the per-element layout list of
  section "i2_s Packing Format".
* TQ2_0: the per-byte helper shape of "Hesper/Quantization/TQ2_0", section
  "DSL Helper Functions" (value idx 0..3 of a byte at shift idx*2), with the
  code table of section "TQ2_0 Format".
* W1: element-wise sign products, while the oracle also evaluates the card's
  dot identity.

Products use Python integers and ``fractions.Fraction`` so they are exact.
Shapes must stay tiny (pure-Python loops).
"""
from fractions import Fraction
import struct

I2S_TABLE = {0b00: -1, 0b01: 0, 0b10: 1}          # BitLinear "i2_s Packing Format"
TQ2_TABLE = {0b00: 0, 0b01: 1, 0b11: -1}          # TQ2_0 "TQ2_0 Format"


def i2s_unpack(packed, N, K):
    w = [[None] * K for _ in range(N)]
    u32_per_row = K // 16
    for n in range(N):
        for u in range(u32_per_row):
            group128 = u // 8
            base = (u % 8) * 4
            for b in range(4):
                byte = packed[n * (K // 4) + u * 4 + b]
                for s in (6, 4, 2, 0):
                    elem = group128 * 128 + base + b + (3 - s // 2) * 32
                    w[n][elem] = I2S_TABLE[(byte >> s) & 3]
    scale = struct.unpack("<f", bytes(packed[N * K // 4:N * K // 4 + 4]))[0]
    return w, scale


def tq2_unpack(blocks, N, K):
    w = [[None] * K for _ in range(N)]
    scales = []
    nb = K // 256
    for n in range(N):
        for bi in range(nb):
            blk = blocks[66 * (n * nb + bi):66 * (n * nb + bi + 1)]
            for i in range(64):
                for idx in range(4):
                    w[n][bi * 256 + i * 4 + idx] = TQ2_TABLE[(blk[i] >> (idx * 2)) & 3]
            scales.append(blk[64] | (blk[65] << 8))
    return w, scales


def f16(bits):
    """Exact value of binary16 bits as a Fraction (struct's 'e' decoder)."""
    return Fraction(struct.unpack("<e", struct.pack("<H", bits))[0])


def ternary_gemv(w, scale, x):
    """Exact scale * sum_j w[i][j] * x[j] for every row, as Fractions."""
    s = Fraction(scale)
    return [s * sum(Fraction(wij) * Fraction(float(xj)) for wij, xj in zip(row, x)) for row in w]


def tq2_gemv(w, scales, x):
    K = len(x)
    out = []
    for n, row in enumerate(w):
        tot = Fraction(0)
        for bi in range(K // 256):
            s = f16(scales[n * (K // 256) + bi])
            tot += s * sum(Fraction(row[k]) * Fraction(float(x[k])) for k in range(bi * 256, bi * 256 + 256))
        out.append(tot)
    return out


def w1_unpack(words, N, K):
    return [[1 if (int(words[n][k // 32]) >> (k % 32)) & 1 else -1 for k in range(K)] for n in range(N)]


def w1a8(words, scales, K, G, q, s_tok):
    """Exact S[n] = sum_g s[n,g] * sum_{k in g} w*q and y = float32(float64(s_tok * S))."""
    N = len(words)
    w = w1_unpack(words, N, K)
    res = []
    for n in range(N):
        S = Fraction(0)
        for g in range(K // G):
            d = sum(w[n][k] * int(q[k]) for k in range(g * G, (g + 1) * G))
            S += f16(int(scales[n][g])) * d
        res.append(S)
    return res
