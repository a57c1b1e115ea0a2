"""Pins for the CPU oracle: every oracle function checked against facts that do
not come from the oracle itself -- the pages' code tables, layout statements
and printed footprint table (fixtures under tests/golden/), hand-derived
worked examples, closed forms, identities, numpy library routines on the
unpacked weights, and exact brute force on tiny shapes (tests/brute.py).

The W1 bit order inside a 32-bit word (least significant bit first) is
pinned to the only bit-order statements on the pages, those of the WHT
sign-table pull request (tests/golden/w1_bit_order.txt).  The TQ2_0 element
order inside a block (least significant pair first) is pinned to the TQ2_0
page's own helper shift (the value index in a byte times two, tests/brute.py);
no real TQ2_0 file is available to check it against.

Parity unpinned (internally consistent, not checkable against an outside
artefact because none is available): the activation-quantization constants
(/127, ties-to-even, multiply by 127/absmax).  It is one reading, stated in
oracle.c where it is used.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import brute
from conftest import read_golden
from binary_bit_weight_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _code(s):
    return int(s, 2)


# ------------------------------------------------------------------ fp16 / bf16
def test_f16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_encode_matches_numpy(orc):
    g = np.random.default_rng(5)
    vals = np.concatenate([
        g.standard_normal(4000) * 0.02,
        g.uniform(0.005, 0.05, 2000),
        g.uniform(-70000, 70000, 500),
        g.uniform(-1e-6, 1e-6, 1000),           # subnormal range
        np.arange(-2048, 2049) * 2.0 ** -24,     # exact subnormal grid + ties
        (np.arange(1024, 2048) + 0.5) * 2.0 ** -10,  # ties between normals
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -25 * 3],
    ])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f64_to_f16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_bf16_round_trip(orc):
    """Every bf16 value converts back to itself; NaNs stay NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = np.array([orc.bf16_to_f32(int(b)) for b in bits], np.float32)
    got = orc.f32_to_bf16(vals)
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], bits[~nan])
    assert np.isnan(np.array([orc.bf16_to_f32(int(b)) for b in got[nan]], np.float32)).all()


def test_f32_to_bf16_matches_integer_rounding(orc):
    """Against the integer form of round-to-nearest-even on the bit pattern
    (add 0x7FFF plus the lowest kept bit, cut 16 bits), a different
    formulation from the oracle's comparison of the two neighbours, on
    random finite floats of every magnitude."""
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    u = u[np.isfinite(f)]
    ref = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(u.view(np.float32)), ref)


def test_f32_to_bf16_worked_cases(orc):
    one = np.float32(1.0)
    cases = [(one, 0x3F80),
             (np.float32(1 + 2.0 ** -8), 0x3F80),                   # tie, even below
             (np.float32(1 + 3 * 2.0 ** -8), 0x3F82),               # tie, even above
             (np.float32(1 + 2.0 ** -8 + 2.0 ** -20), 0x3F81),      # past the tie
             (np.float32(-(1 + 2.0 ** -8 + 2.0 ** -20)), 0xBF81),
             (np.float32(np.finfo(np.float32).max), 0x7F80),        # past max bf16 + half ulp: infinity
             (np.float32(2.0 ** -133), 0x0001),                     # the least bf16 subnormal, exact
             (np.float32(2.0 ** -134), 0x0000)]                     # half of it: tie, even (zero)
    for v, b in cases:
        assert int(orc.f32_to_bf16(np.array([v]))[0]) == b, (v, b)


def test_bf16_decode(orc):
    g = np.random.default_rng(6)
    bits = g.integers(0, 65536, 5000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    got = np.array([orc.bf16_to_f32(int(b)) for b in bits], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ i2_s
def test_i2s_code_table(orc):
    table = {int(t): _code(c) for t, c in read_golden("i2s_code_table.txt")}
    assert table == {-1: 0, 0: 1, 1: 2}
    for v, code in table.items():
        w = np.full((2, 128), v, np.int8)
        p = orc.i2s_encode(w, 1.0)
        body = p[:64]
        for s in (6, 4, 2, 0):
            assert np.all((body >> s) & 3 == code)
    # decode: each code reads back as code - 1 (dequantization rule)
    for code in (0, 1, 2):
        byte = code * 0b01010101
        p = np.concatenate([np.full(32, byte, np.uint8), np.frombuffer(struct.pack("<f", 1.0), np.uint8)])
        w, s, bad = orc.i2s_decode(p, 1, 128)
        assert bad == 0 and s == 1.0 and np.all(w == code - 1)


def test_i2s_layout_list(orc):
    layout = [tuple(int(v) for v in r) for r in read_golden("i2s_layout.txt")]
    K = 256
    zero = orc.i2s_encode(np.zeros((1, K), np.int8), 1.0)[:K // 4]
    assert np.all(zero == 0x55)
    for g in range(K // 128):
        for e0, e1, b0, b1, shift in layout:
            for k in range(e0, e1 + 1):
                w = np.zeros((1, K), np.int8)
                w[0, 128 * g + k] = 1
                p = orc.i2s_encode(w, 1.0)[:K // 4]
                diff = np.nonzero(p != zero)[0]
                assert diff.tolist() == [32 * g + b0 + (k - e0)]
                byte = int(p[diff[0]])
                assert (byte >> shift) & 3 == 0b10
                assert byte & ~(3 << shift) & 0xFF == 0x55 & ~(3 << shift) & 0xFF


def test_i2s_two_page_statements_agree(orc):
    # layout list (oracle) vs per-u32 unpack statement (brute), every position
    for seed, (N, K) in enumerate([(3, 128), (2, 384), (1, 512)]):
        w = synth.ternary(100 + seed, N, K)
        p = orc.i2s_encode(w, 0.25)
        wb, s = brute.i2s_unpack(p.tolist(), N, K)
        assert np.array_equal(np.array(wb, np.int8), w) and s == 0.25
        wd, s2, bad = orc.i2s_decode(p, N, K)
        assert np.array_equal(wd, w) and s2 == 0.25 and bad == 0


def test_i2s_worked_example(orc):
    # 0x92 = 10 01 00 10: shift 6 -> +1, 4 -> 0, 2 -> -1, 0 -> +1
    p = np.concatenate([np.full(32, 0x92, np.uint8), np.frombuffer(struct.pack("<f", 0.0625), np.uint8)])
    w, s, bad = orc.i2s_decode(p, 1, 128)
    expect = np.array([1] * 32 + [0] * 32 + [-1] * 32 + [1] * 32, np.int8)
    assert np.array_equal(w[0], expect) and s == 0.0625 and bad == 0
    x = np.arange(128, dtype=np.float32)
    y, t = orc.i2s_gemv_f32(p, 1, 128, x)
    # sum(0..31) - sum(64..95) + sum(96..127) = 496 - 2544 + 3568 = 1520
    assert y[0, 0] == 95.0
    assert t[0, 0] == 0.0625 * 8128.0
    y1, _ = orc.i2s_gemv_f32(p, 1, 128, np.ones(128, np.float32))
    assert y1[0, 0] == 2.0


def test_i2s_scale_is_le_f32_at_tail(orc):
    w = synth.ternary(3, 4, 128)
    p = orc.i2s_encode(w, -3.5e-3)
    assert p.size == 4 * 128 // 4 + 4
    assert bytes(p[-4:]) == struct.pack("<f", np.float32(-3.5e-3))


@pytest.mark.parametrize("N,K,M", [(37, 384, 3), (256, 512, 1), (5, 128, 16)])
def test_i2s_gemv_vs_numpy_matmul(orc, N, K, M):
    w = synth.ternary(11 + N, N, K)
    x = synth.normal_f32(12 + N, M, K)
    scale = np.float32(0.0625)
    p = orc.i2s_encode(w, scale)
    y, t = orc.i2s_gemv_f32(p, N, K, x)
    ref = float(scale) * (x.astype(np.float64) @ w.astype(np.float64).T)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(t, float(scale) * np.abs(x.astype(np.float64)).sum(1, keepdims=True)
                               * np.ones((1, N)), rtol=1e-12)
    # BitLinear identity: scale * (sum over +1 weights - sum over -1 weights)
    pos = x.astype(np.float64) @ (w == 1).astype(np.float64).T
    neg = x.astype(np.float64) @ (w == -1).astype(np.float64).T
    np.testing.assert_allclose(y, float(scale) * (pos - neg), rtol=1e-12, atol=1e-12)


def test_i2s_gemv_exact_bruteforce(orc):
    N, K = 3, 256
    w = synth.ternary(21, N, K)
    x = synth.normal_f32(22, 1, K)[0]
    p = orc.i2s_encode(w, 0.03125)
    y, t = orc.i2s_gemv_f32(p, N, K, x)
    exact = brute.ternary_gemv(w.tolist(), 0.03125, x.tolist())
    bound = 0.03125 * K * 2.0 ** -52 * float(np.abs(x).sum())
    for i in range(N):
        assert abs(y[0, i] - float(exact[i])) <= bound


def test_i2s_closed_forms(orc):
    K = 384
    x = synth.normal_f32(31, 2, K)
    for k in (0, 31, 32, 127, 128, 200, 383):
        for v in (1, -1):
            w = np.zeros((1, K), np.int8)
            w[0, k] = v
            p = orc.i2s_encode(w, 0.5)
            y, _ = orc.i2s_gemv_f32(p, 1, K, x)
            assert np.array_equal(y[:, 0], v * 0.5 * x[:, k].astype(np.float64))
    p = orc.i2s_encode(np.ones((1, K), np.int8), 0.5)
    y, _ = orc.i2s_gemv_f32(p, 1, K, x)
    np.testing.assert_allclose(y[:, 0], 0.5 * x.astype(np.float64).sum(1), rtol=1e-13)
    p = orc.i2s_encode(np.zeros((1, K), np.int8), 0.5)
    y, _ = orc.i2s_gemv_f32(p, 1, K, x)
    assert np.all(y == 0.0)


def test_i2s_invalid_code_and_rejects(orc):
    p = np.concatenate([np.full(32, 0x55, np.uint8), np.frombuffer(struct.pack("<f", 1.0), np.uint8)])
    p[5] = 0x57                    # low field = 0b11
    _, _, bad = orc.i2s_decode(p, 1, 128)
    assert bad == 1
    with pytest.raises(ValueError):
        orc.i2s_encode(np.zeros((1, 100), np.int8), 1.0)
    with pytest.raises(ValueError):
        orc.i2s_encode(np.full((1, 128), 2, np.int8), 1.0)


def test_i2s_rows_subset(orc):
    N, K = 50, 256
    w = synth.ternary(41, N, K)
    x = synth.normal_f32(42, 2, K)
    p = orc.i2s_encode(w, 0.07)
    yall, _ = orc.i2s_gemv_f32(p, N, K, x)
    rows = np.array([0, 7, 49])
    ysub, _ = orc.i2s_gemv_f32(p, N, K, x, rows)
    assert np.array_equal(ysub, yall[:, rows])


def test_i2s_gemm_i8(orc):
    N, K, M = 19, 384, 5
    w = synth.ternary(51, N, K)
    q = synth.rng(52).integers(-127, 128, size=(M, K)).astype(np.int8)
    s_tok = synth.uniform_f32(53, M, 0.001, 0.05)
    s_w = np.float32(0.0421)
    p = orc.i2s_encode(w, s_w)
    y, acc = orc.i2s_gemm_i8(p, N, K, q, s_tok)
    ref_acc = q.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc, ref_acc)
    ref_y = (ref_acc.astype(np.float32) * s_tok[:, None]).astype(np.float32) * s_w
    assert np.array_equal(y.view(np.uint32), ref_y.astype(np.float32).view(np.uint32))
    # one-hot weight: acc is the activation itself
    w1 = np.zeros((1, K), np.int8)
    w1[0, 129] = -1
    y1, a1 = orc.i2s_gemm_i8(orc.i2s_encode(w1, 1.0), 1, K, q, np.ones(M, np.float32))
    assert np.array_equal(a1[:, 0], -q[:, 129].astype(np.int64))


# ------------------------------------------------------------------ TQ2_0
def test_tq2_code_table_and_constants(orc):
    table = {int(t): _code(c) for t, c in read_golden("tq2_code_table.txt")}
    assert table == {0: 0, 1: 1, -1: 3}
    const = {k: int(v) for k, v in read_golden("tq2_constants.txt")}
    assert const == {"blockSize": 256, "blockSizeBytes": 66, "valuesPerByte": 4}
    for v, code in table.items():
        w = np.full((1, 512), v, np.int8)
        sc = np.array([0x3C00, 0x3800], np.uint16)
        b = orc.tq2_encode(w, sc)
        assert b.size == 2 * const["blockSizeBytes"]
        for blk in range(2):
            body = b[66 * blk:66 * blk + 64]
            for idx in range(const["valuesPerByte"]):
                assert np.all((body >> (2 * idx)) & 3 == code)
            # scale_low then scale_high
            assert b[66 * blk + 64] == sc[blk] & 0xFF and b[66 * blk + 65] == sc[blk] >> 8
        wd, scd, bad = orc.tq2_decode(b, 1, 512)
        assert np.all(wd == v) and np.array_equal(scd, sc) and bad == 0


def test_tq2_worked_example(orc):
    # 0x71 = 01 11 00 01; least significant pair first: +1, 0, -1, +1
    blk = np.concatenate([np.full(64, 0x71, np.uint8), np.array([0x00, 0x38], np.uint8)])  # 0.5
    w, sc, bad = orc.tq2_decode(blk, 1, 256)
    assert np.array_equal(w[0], np.tile(np.array([1, 0, -1, 1], np.int8), 64)) and bad == 0
    x = np.arange(256, dtype=np.float32)
    y, t = orc.tq2_gemv_f32(blk, 1, 256, x)
    assert y[0, 0] == 0.5 * 8128.0
    assert t[0, 0] == 0.5 * 32640.0


def test_tq2_helper_form_agrees(orc):
    N, K = 3, 512
    w = synth.ternary(61, N, K)
    sc = synth.uniform_f16_bits(62, N * K // 256, 0.005, 0.05)
    b = orc.tq2_encode(w, sc)
    wb, scb = brute.tq2_unpack(b.tolist(), N, K)
    assert np.array_equal(np.array(wb, np.int8), w) and scb == sc.tolist()


@pytest.mark.parametrize("N,K,M", [(29, 512, 1), (8, 768, 8), (3, 256, 16)])
def test_tq2_gemv_vs_numpy(orc, N, K, M):
    w = synth.ternary(71 + N, N, K)
    sc = synth.uniform_f16_bits(72 + N, N * K // 256, 0.005, 0.05)
    x = synth.normal_f32(73 + N, M, K)
    b = orc.tq2_encode(w, sc)
    y, t = orc.tq2_gemv_f32(b, N, K, x)
    s = sc.view(np.float16).astype(np.float64).reshape(N, K // 256)
    x64 = x.astype(np.float64).reshape(M, K // 256, 256)
    w64 = w.astype(np.float64).reshape(N, K // 256, 256)
    ref = np.einsum("mbk,nbk,nb->mn", x64, w64, s)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    tref = np.einsum("mbk,nb->mn", np.abs(x64), np.abs(s))
    np.testing.assert_allclose(t, tref, rtol=1e-12)


def test_tq2_exact_bruteforce(orc):
    N, K = 2, 512
    w = synth.ternary(81, N, K)
    sc = synth.uniform_f16_bits(82, N * K // 256, 0.005, 0.05)
    x = synth.normal_f32(83, 1, K)[0]
    b = orc.tq2_encode(w, sc)
    y, t = orc.tq2_gemv_f32(b, N, K, x)
    exact = brute.tq2_gemv(w.tolist(), sc.tolist(), x.tolist())
    for i in range(N):
        assert abs(y[0, i] - float(exact[i])) <= t[0, i] * K * 2.0 ** -51


def test_tq2_gemm_i8_exact_bruteforce(orc):
    """int8 activations against TQ2_0 blocks: the oracle's fp64 value against
    the exact rational s_tok * sum_b s_b * sum_{k in b} w q, with the weights
    decoded by the independent pure-Python unpacker."""
    N, K, M = 3, 512, 2
    w = synth.ternary(85, N, K)
    sc = synth.uniform_f16_bits(86, N * K // 256, 0.005, 0.05)
    q, s = orc.quantize_f32(synth.normal_f32(87, M, K))
    b = orc.tq2_encode(w, sc)
    y, t = orc.tq2_gemm_i8(b, N, K, q, s)
    wb, scb = brute.tq2_unpack(b.tolist(), N, K)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for bi in range(K // 256):
                d = sum(wb[n][k] * int(q[m, k]) for k in range(bi * 256, bi * 256 + 256))
                tot += brute.f16(scb[n * (K // 256) + bi]) * d
            exact = Fraction(float(s[m])) * tot
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(t[m, n]) * 2 ** -48


@pytest.mark.parametrize("N,K,M", [(29, 512, 1), (8, 768, 5), (4, 2560, 17)])
def test_tq2_gemm_i8_vs_numpy_and_gemv(orc, N, K, M):
    """The same product three ways: numpy over the decoded weights, and the
    fp32-activation oracle on q (exact integers) times s_tok."""
    w = synth.ternary(95 + N, N, K)
    sc = synth.uniform_f16_bits(96 + N, N * K // 256, 0.005, 0.05)
    q, s = orc.quantize_f32(synth.normal_f32(97 + N, M, K))
    b = orc.tq2_encode(w, sc)
    y, t = orc.tq2_gemm_i8(b, N, K, q, s)
    sb = sc.view(np.float16).astype(np.float64).reshape(N, K // 256)
    q64 = q.astype(np.float64).reshape(M, K // 256, 256)
    w64 = w.astype(np.float64).reshape(N, K // 256, 256)
    ref = s.astype(np.float64)[:, None] * np.einsum("mbk,nbk,nb->mn", q64, w64, sb)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    tref = s.astype(np.float64)[:, None] * np.einsum("mbk,nb->mn", np.abs(q64), np.abs(sb))
    np.testing.assert_allclose(t, tref, rtol=1e-12)
    yg, _ = orc.tq2_gemv_f32(b, N, K, q.astype(np.float32))
    np.testing.assert_allclose(y, s.astype(np.float64)[:, None] * yg, rtol=1e-12, atol=1e-13)


def test_tq2_invalid_code_and_roundtrip(orc):
    w = synth.ternary(91, 4, 256)
    sc = synth.uniform_f16_bits(92, 4, 0.005, 0.05)
    b = orc.tq2_encode(w, sc)
    wd, scd, bad = orc.tq2_decode(b, 4, 256)
    assert np.array_equal(wd, w) and np.array_equal(scd, sc) and bad == 0
    b2 = b.copy()
    b2[3] = (b2[3] & 0xFC) | 0b10
    wd2, _, bad2 = orc.tq2_decode(b2, 4, 256)
    assert bad2 == 1 and wd2[0, 12] == -2
    with pytest.raises(ValueError):
        orc.tq2_encode(np.zeros((1, 128), np.int8), np.zeros(1, np.uint16))


# ------------------------------------------------------------------ W1
def test_w1_stored_bit(orc):
    rows = [(int(a), int(b)) for a, b in read_golden("w1_stored_bit.txt")]
    w = np.zeros((1, 32), np.int8)
    for i, (v, _) in enumerate(rows):
        w[0, i] = v
    bits = orc.w1_encode(w)
    for i, (_, b) in enumerate(rows):
        assert (int(bits[0, 0]) >> i) & 1 == b


def test_w1_bit_order_pages(orc):
    """Element k of a row sits at bit k & 31 of word k >> 5 (the WHT
    sign-table page, tests/golden/w1_bit_order.txt), and the four elements
    4t .. 4t+3 form nibble t & 7 of word t >> 3: a lone +1 among -1 encodes to
    exactly that one bit, a +1 nibble to exactly that nibble, and decoding the
    single-bit word gives the lone +1 back at k."""
    K = 128
    rows = [tuple(int(v) for v in r) for r in read_golden("w1_bit_order.txt")]
    assert len(rows) >= 10
    for e, word, bit in rows:
        assert (word, bit) == (e >> 5, e & 31)
        w = -np.ones((1, K), np.int8)
        w[0, e] = 1
        packed = orc.w1_encode(w)
        want = np.zeros((1, K // 32), np.uint32)
        want[0, word] = np.uint32(1) << np.uint32(bit)
        assert np.array_equal(packed, want), e
        back = orc.w1_decode(want, K)
        assert back[0, e] == 1 and (np.delete(back[0], e) == -1).all()
    for t in range(K // 4):
        w = -np.ones((1, K), np.int8)
        w[0, 4 * t:4 * t + 4] = 1
        packed = orc.w1_encode(w)
        want = np.zeros((1, K // 32), np.uint32)
        want[0, t >> 3] = np.uint32(0xF) << np.uint32(4 * (t & 7))
        assert np.array_equal(packed, want), t


def test_w1_worked_example(orc):
    bits = np.array([[0x0000FFFF]], np.uint32)
    w = orc.w1_decode(bits, 32)
    assert np.array_equal(w[0], np.array([1] * 16 + [-1] * 16, np.int8))
    a = np.arange(32, dtype=np.int8)[None, :]
    y, S = orc.w1a8_gemm(bits, np.array([[0x3C00]], np.uint16), 32, 32, a, np.ones(1, np.float32))
    # sum(0..15) - sum(16..31) = 120 - 376; identity: 2*120 - 496
    assert S[0, 0] == -256.0 and y[0, 0] == -256.0


def test_w1_roundtrip_and_zeros(orc):
    g = synth.rng(101)
    w = np.where(g.standard_normal((7, 160)) >= 0, 1, -1).astype(np.int8)
    assert np.array_equal(orc.w1_decode(orc.w1_encode(w), 160), w)
    t = synth.ternary(102, 3, 64)
    back = orc.w1_decode(orc.w1_encode(t), 64)
    assert np.array_equal(back, np.where(t > 0, 1, -1))
    assert not np.array_equal(back, t)


def test_w1_unit_scales_exact(orc):
    N, K, G, M = 9, 256, 64, 4
    g = synth.rng(111)
    w = np.where(g.standard_normal((N, K)) >= 0, 1, -1).astype(np.int8)
    q = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    bits = orc.w1_encode(w)
    ones = np.full((N, K // G), 0x3C00, np.uint16)
    y, S = orc.w1a8_gemm(bits, ones, K, G, q, np.ones(M, np.float32))
    ref = (q.astype(np.int64) @ w.astype(np.int64).T)
    assert np.array_equal(S, ref.astype(np.float64)) and np.array_equal(y, ref.astype(np.float32))


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_w1a8_exact_vs_bruteforce(orc, G):
    N, K, M = 3, 512, 2
    W = synth.dense_chunk(121, K, 0, rows=N)
    bits, sc = orc.w1_from_dense(W, G)
    q = synth.rng(122).integers(-127, 128, size=(M, K)).astype(np.int8)
    s_tok = synth.uniform_f32(123, M, 0.001, 0.05)
    bias = synth.uniform_f32(124, N, -1, 1)
    y, S = orc.w1a8_gemm(bits, sc, K, G, q, s_tok, bias=bias)
    for m in range(M):
        exact = brute.w1a8(bits.tolist(), sc.tolist(), K, G, q[m].tolist(), float(s_tok[m]))
        for n in range(N):
            assert S[m, n] == float(exact[n])        # the fp64 sum is exact here
            v = np.float32(np.float64(s_tok[m]) * float(exact[n])) + bias[n]
            assert y[m, n] == np.float32(v)


def test_w1_from_dense(orc):
    N, K, G = 6, 384, 128
    W = synth.dense_chunk(131, K, 0, rows=N)
    W[0, 5] = 0.0
    bits, sc = orc.w1_from_dense(W, G)
    w = orc.w1_decode(bits, K)
    assert np.array_equal(w, np.where(W > 0, 1, -1))
    ref = np.abs(W.astype(np.float64)).reshape(N, K // G, G).mean(-1).astype(np.float16).view(np.uint16)
    assert np.array_equal(sc, ref)
    # constant-magnitude rows: the scale is that magnitude in fp16
    Wc = np.full((1, 128), -0.015625, np.float32)
    _, scc = orc.w1_from_dense(Wc, 128)
    assert scc[0, 0] == np.float16(0.015625).view(np.uint16)


def test_w1_footprint_table():
    """Size formula bits/8 + 2 bytes per G weights against the card's table."""
    for layer, N, K, bf16_mb, tern_mb, bin_mb, ratio in read_golden("binary_gemm_footprint.txt"):
        N, K = int(N), int(K)
        mib = 2.0 ** 20
        bf16 = 2 * N * K
        scales = 2 * N * K // 128
        tern = N * K // 4 + scales
        binary = N * K // 8 + scales
        assert f"{bf16 / mib:.1f}" == bf16_mb, layer
        assert f"{tern / mib:.1f}" == tern_mb, layer
        assert f"{binary / mib:.1f}" == bin_mb, layer
        assert f"{tern / binary:.2f}" == ratio, layer


# ------------------------------------------------------------------ activations
def _rne_brute(v):
    """Nearest integer to the fp32 value v, ties to even, by search."""
    fv = Fraction(float(v))
    lo = int(np.floor(float(v)))
    best = None
    for c in (lo - 1, lo, lo + 1, lo + 2):
        d = abs(fv - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_quantize_invariants(orc):
    M, K = 6, 1000
    x = synth.normal_f32(141, M, K)
    x[2] *= 1e-30
    x[3] = 0.0
    x[4, 17] = -1e4
    q, s = orc.quantize_f32(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert s[3] == 0.0 and np.all(q[3] == 0)
    for m in (0, 1, 2, 4, 5):
        a = np.abs(x[m]).max()
        assert s[m] == np.float32(a) / np.float32(127.0)
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(q[m, j])) == 127
        err = np.abs(x[m].astype(np.float64) - q[m].astype(np.float64) * np.float64(s[m]))
        assert err.max() <= 0.5 * float(s[m]) * (1 + 1e-5)
        assert err.max() < 0.01 * a                     # card: < 1% of the row max
        inv = np.float32(127.0) / np.float32(a)
        prod = (x[m] * inv).astype(np.float32)
        for k in range(0, K, 37):
            assert q[m, k] == max(-127, min(127, _rne_brute(prod[k])))


def test_quantize_ties_to_even(orc):
    x = np.array([[127.0, 2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -126.5]], np.float32)
    q, s = orc.quantize_f32(x)
    assert q[0].tolist() == [127, 2, -4, 0, 2, 0, 126, -126]
    assert s[0] == 1.0


def test_quantize_bf16_matches_f32(orc):
    xb = synth.normal_bf16_bits(151, 4, 512)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    q1, s1 = orc.quantize_bf16(xb)
    q2, s2 = orc.quantize_f32(xf)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


# ------------------------------------------------------------------ fused epilogues
def test_relu2_mul_closed_forms(orc):
    """[BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"]: max(0, gate)^2 * up, values
    worked by hand: negative and zero gates give 0 whatever up is (a dropped
    ReLU would give 63 and -7 for the first two), 0.5^2 * 4 = 1, 2^2 * 3 = 12,
    3^2 * -1 = -9 (a missing square would give 1.5*... and -3)."""
    g = [-3.0, -0.0, 0.0, 0.5, 2.0, 3.0, -1e30]
    u = [7.0, -7.0, 7.0, 4.0, 3.0, -1.0, 5.0]
    assert orc.relu2_mul(g, u).tolist() == [0.0, 0.0, 0.0, 1.0, 12.0, -9.0, 0.0]


def test_relu2_mul_scaling_and_products(orc):
    """Homogeneity (degree 2 in a positive gate scale, 1 in the up scale) and
    the product of the oracle's own exact gemv results for a one-hot gate row:
    gate = s_g x_k, up = s_u x_j, so out = s_g^2 x_k^2 s_u x_j when x_k > 0."""
    rng = np.random.default_rng(5)
    g, u = rng.normal(size=64), rng.normal(size=64)
    base = orc.relu2_mul(g, u)
    assert np.array_equal(orc.relu2_mul(4.0 * g, 0.5 * u), 8.0 * base)   # powers of two: exact
    K = 128
    x = np.zeros((1, K), np.float32)
    x[0, 5], x[0, 9] = 3.0, -2.0
    wg = np.zeros((1, K), np.int8); wg[0, 5] = 1
    wu = np.zeros((1, K), np.int8); wu[0, 9] = -1
    pg = orc.i2s_encode(wg, 0.5)
    pu = orc.i2s_encode(wu, 0.25)
    gate, _ = orc.i2s_gemv_f32(pg, 1, K, x)
    up, _ = orc.i2s_gemv_f32(pu, 1, K, x)
    assert gate[0, 0] == 1.5 and up[0, 0] == 0.5
    assert orc.relu2_mul(gate, up)[0, 0] == 1.5 * 1.5 * 0.5


def test_rmsnorm_closed_forms(orc):
    """[BL "Fused RMSNorm + BitLinear + Residual Add M=1 Kernel"]: with unit
    weights and eps = 0 the output has mean square 1 exactly in exact
    arithmetic; (3, 4) has mean square 12.5, so xn = (3, 4) / sqrt(12.5);
    a positive rescaling of x changes nothing when eps = 0; eps enters under
    the root (x = (1, 1), eps = 3 gives 1/2); the weights scale elementwise;
    a zero row gives 0 (the 0/0 reading)."""
    xn = orc.rmsnorm([[3.0, 4.0]], [1.0, 1.0], 0.0)[0]
    assert abs(xn[0] - 3.0 / 12.5 ** 0.5) < 1e-15 and abs(xn[1] - 4.0 / 12.5 ** 0.5) < 1e-15
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3, 256))
    one = orc.rmsnorm(x, np.ones(256), 0.0)
    assert np.allclose(np.mean(one * one, axis=1), 1.0, rtol=1e-14, atol=0)
    assert np.allclose(orc.rmsnorm(7.5 * x, np.ones(256), 0.0), one, rtol=1e-14, atol=0)
    assert orc.rmsnorm([[1.0, 1.0]], [1.0, 1.0], 3.0).tolist() == [[0.5, 0.5]]
    assert orc.rmsnorm([[1.0, 1.0]], [2.0, -4.0], 3.0).tolist() == [[1.0, -2.0]]
    assert orc.rmsnorm([[0.0, 0.0]], [1.0, 1.0], 0.0).tolist() == [[0.0, 0.0]]
