"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, its host-side packers agree byte for byte with the oracle's encoders,
and every device entry point rejects bad arguments on the host, before any
launch (so these run without a GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(ll_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"
    assert L.ll_abi_version() == 5
    assert L.ll_strerror(-5) == "workspace missing or too small"


@pytest.mark.parametrize("N,K", [(1, 128), (7, 384), (256, 512), (33, 2560)])
def test_pack_i2s_matches_oracle(orc, N, K):
    w = synth.ternary(1000 + N, N, K)
    p = L.ll_pack_i2s(w, 0.0625)
    assert np.array_equal(p, orc.i2s_encode(w, 0.0625))
    w2, s = L.ll_unpack_i2s(p, N, K)
    assert np.array_equal(w2, w) and s == 0.0625


@pytest.mark.parametrize("N,K", [(1, 256), (5, 768), (64, 2560)])
def test_pack_tq2_matches_oracle(orc, N, K):
    w = synth.ternary(2000 + N, N, K)
    sc = synth.uniform_f16_bits(2001 + N, N * K // 256, 0.005, 0.05)
    b = L.ll_pack_tq2(w, sc)
    assert np.array_equal(b, orc.tq2_encode(w, sc))
    w2, sc2 = L.ll_unpack_tq2(b, N, K)
    assert np.array_equal(w2, w) and np.array_equal(sc2, sc)
    codes, sc3 = L.ll_tq2_split(b, N, K)
    blocks = b.reshape(-1, 66)
    assert np.array_equal(codes.reshape(-1, 64), blocks[:, :64])
    assert np.array_equal(sc3, sc)


@pytest.mark.parametrize("N,K", [(1, 32), (9, 160), (40, 5120)])
def test_pack_w1_matches_oracle(orc, N, K):
    w = synth.ternary(3000 + N, N, K)
    bits = L.ll_pack_w1(w)
    assert np.array_equal(bits, orc.w1_encode(w))
    assert np.array_equal(L.ll_unpack_w1(bits, K), orc.w1_decode(bits, K))


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_w1_from_dense_matches_oracle(orc, G):
    W = synth.dense_chunk(4000 + G, 512, 0, rows=11)
    W[3, 7] = 0.0
    W[4] = 0.0
    b1, s1 = L.ll_w1_from_dense(W, G)
    b2, s2 = orc.w1_from_dense(W, G)
    assert np.array_equal(b1, b2) and np.array_equal(s1, s2)


def test_packed_sizes():
    # i2_s 256x512: 32,768 code bytes + 4-byte scale
    assert L.ll_packed_size(L.LL_FMT_I2S, 256, 512) == (32772, 0)
    assert L.ll_packed_size(L.LL_FMT_I2S, 2560, 2560) == (1638404, 0)
    assert L.ll_packed_size(L.LL_FMT_I2S, 6912, 2560) == (4423684, 0)
    assert L.ll_packed_size(L.LL_FMT_TQ2_0, 6912, 2560) == (66 * 6912 * 10, 2 * 6912 * 10)
    assert L.ll_packed_size(L.LL_FMT_W1, 248320, 5120, 128) == (158924800, 19865600)
    assert L.ll_packed_size(L.LL_FMT_I2S, 4, 100) == (0, 0)
    assert L.ll_packed_size(L.LL_FMT_W1, 4, 96, 64) == (0, 0)


def test_packers_reject_bad_input():
    with pytest.raises(L.LowbitError) as e:
        L.ll_pack_i2s(np.zeros((2, 100), np.int8), 1.0)
    assert e.value.status == -2
    with pytest.raises(L.LowbitError) as e:
        L.ll_pack_i2s(np.full((1, 128), 3, np.int8), 1.0)
    assert e.value.status == -4
    with pytest.raises(L.LowbitError) as e:
        L.ll_pack_tq2(np.zeros((1, 128), np.int8), np.zeros(1, np.uint16))
    assert e.value.status == -2
    with pytest.raises(L.LowbitError) as e:
        L.ll_w1_from_dense(np.zeros((1, 96), np.float32), 64)
    assert e.value.status == -2


def test_validate_finds_first_bad_code():
    w = synth.ternary(5, 3, 256)
    p = L.ll_pack_i2s(w, 1.0)
    assert L.ll_validate(L.LL_FMT_I2S, p, 3, 256) == (0, -1)
    p[64 + 40] |= 0x0C           # row 1, group 0... byte 40 of row 1 -> group 1, r%32 = 8, shift 2
    rc, bad = L.ll_validate(L.LL_FMT_I2S, p, 3, 256)
    assert rc == -4 and bad == 256 + 128 + 64 + 8
    codes = np.zeros(256 // 4, np.uint8)
    codes[10] = 0b00100000       # element 4*10 + 2
    assert L.ll_validate(L.LL_FMT_TQ2_0, codes, 1, 256) == (-4, 42)


# ------------------------------------------------------------- device-entry validation (no GPU needed)
CB = 4096                                          # LL_WORKSPACE_COUNTER_BYTES
FAKE = 0x10000            # aligned, never dereferenced: validation fails first


def _w(fmt=L.LL_FMT_I2S, N=64, K=256, group=128, codes=FAKE, scales=FAKE):
    return L.ll_weights(fmt, group, N, K, C.c_void_p(codes), C.c_void_p(scales))


def _gemv(w, act=L.LL_ACT_F32, x=FAKE, xs=FAKE, M=1, bias=None, y=FAKE, ws=FAKE, wsb=1 << 30):
    lib = L.lib()
    return lib.ll_bitlinear_gemv(C.byref(w), act, C.c_void_p(x), C.c_void_p(xs), M, C.c_void_p(bias) if bias else None,
                                 C.c_void_p(y), C.c_void_p(ws) if ws else None, wsb, None)


def test_gemv_argument_errors():
    assert _gemv(_w(), M=0) == -2
    assert _gemv(_w(), M=17) == -2
    assert _gemv(_w(K=200)) == -2
    assert _gemv(_w(fmt=7)) == -1
    assert _gemv(_w(codes=0)) == -1
    assert _gemv(_w(codes=FAKE + 4)) == -3
    assert _gemv(_w(), x=FAKE + 8) == -3
    assert _gemv(_w(), y=0) == -1
    assert _gemv(_w(), M=2, ws=0) == -5          # fp32 activations, M > 1: operand workspace needed
    assert _gemv(_w(), M=6, wsb=16) == -5
    assert _gemv(_w(fmt=L.LL_FMT_TQ2_0, scales=0)) == -1
    assert _gemv(_w(fmt=L.LL_FMT_W1, K=256, group=96)) == -2
    assert _gemv(_w(), act=9) == -1
    assert _gemv(_w(), act=L.LL_ACT_I8, xs=0) == -1
    assert _gemv(_w(), M=0) == -2 and b"M must be" in L.lib().ll_last_error()


def test_gemm_and_quantize_argument_errors():
    lib = L.lib()
    w = _w()
    assert lib.ll_bitlinear_gemm(C.byref(w), C.c_void_p(FAKE), C.c_void_p(FAKE), 0, None, C.c_void_p(FAKE), None,
                                 None, 0, None) == -2
    assert lib.ll_bitlinear_gemm(C.byref(w), C.c_void_p(FAKE + 1), C.c_void_p(FAKE), 32, None, C.c_void_p(FAKE),
                                 None, None, 0, None) == -3
    assert lib.ll_quantize_act(C.c_void_p(FAKE), 5, 4, 4, C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -1
    assert lib.ll_quantize_act(C.c_void_p(FAKE), L.LL_DT_F32, 0, 4, C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -1
    assert lib.ll_quantize_act(None, L.LL_DT_F32, 2, 4, C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -1
    assert lib.ll_quantize_act(C.c_void_p(FAKE), L.LL_DT_F32, 2, 4, C.c_void_p(FAKE), C.c_void_p(FAKE),
                               C.c_void_p(FAKE + 2), None) == -3


def test_binary_linear_arguments_and_workspace():
    """ll_binary_linear: errors found before any launch, and the workspace
    layout (split-K counters | the product's data | int8 x | token scales |
    token sums, each on a 256-byte boundary); TQ2_0 products refuse acc_out."""
    lib = L.lib()
    w = _w(N=64, K=256)
    M = 3
    n = lib.ll_binary_linear_workspace_size(C.byref(w), M)
    # counters 4096, no split data for one 128-row tile, x 768 -> 768, scales 12 -> 256, sums 12
    assert lib.ll_gemm_workspace_size(C.byref(w), M) == 0
    assert n == CB + 768 + 256 + 12
    wt = _w(fmt=L.LL_FMT_TQ2_0, N=64, K=256)
    assert lib.ll_binary_linear_workspace_size(C.byref(wt), M) == n
    w1 = _w(fmt=L.LL_FMT_W1, N=64, K=256, group=128)
    assert lib.ll_binary_linear_workspace_size(C.byref(w1), M) > CB + 768 + 256 + 12
    assert lib.ll_binary_linear_workspace_size(C.byref(w), 0) == C.c_size_t(-1).value

    def call(w, x=FAKE, M=M, y=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.ll_binary_linear(C.byref(w), C.c_void_p(x) if x else None, M, None, C.c_void_p(y) if y else None,
                                    C.c_void_p(ws) if ws else None, wsb, None)
    assert call(w, M=0) == -2
    assert call(w, x=0) == -1
    assert call(w, x=FAKE + 1) == -3
    assert call(w, ws=0) == -5
    assert call(w, wsb=n - 1) == -5
    assert call(w, ws=FAKE + 8) == -3
    assert call(_w(K=200)) == -2                       # i2_s needs K % 128 == 0
    assert call(_w(fmt=L.LL_FMT_TQ2_0, scales=0)) == -1
    assert lib.ll_bitlinear_gemm(C.byref(wt), C.c_void_p(FAKE), C.c_void_p(FAKE), 32, None, C.c_void_p(FAKE),
                                 C.c_void_p(FAKE), C.c_void_p(FAKE), 1 << 30, None) == -1


def test_workspace_sizes():
    w = _w(N=6912, K=2560)
    # fp32 activations: int8 planes (M <= 3) = 5M*K bytes + exponents + row sums
    assert L.lib().ll_gemv_workspace_size(C.byref(w), L.LL_ACT_F32, 2) == CB + (10 * 2560 + 8 + 10 * 4 + 15) // 16 * 16
    # M = 1 with K <= 8192 builds the planes inside the product kernel
    assert L.lib().ll_gemv_workspace_size(C.byref(w), L.LL_ACT_F32, 1) == 0
    w2 = _w(N=64, K=8320)
    assert L.lib().ll_gemv_workspace_size(C.byref(w2), L.LL_ACT_F32, 1) == CB + (5 * 8320 + 4 + 5 * 4 + 15) // 16 * 16
    assert L.lib().ll_gemv_workspace_size(C.byref(w), L.LL_ACT_F32, 8) > 0
    assert L.lib().ll_gemv_workspace_size(C.byref(w), L.LL_ACT_I8, 1) == 0
    assert L.lib().ll_gemv_workspace_size(C.byref(w), L.LL_ACT_F32, 17) == 2 ** 64 - 1


def _item(N, K, x, y):
    return L.ll_gemv_item(_w(N=N, K=K), C.c_void_p(x), None, C.c_void_p(y))


def test_plan_bytes_hold_every_activation_layout():
    """Host-only: a plan prepares every distinct activation into plan memory
    (also where a single call of that shape needs no workspace), so its size
    covers each one's operands (5K int8 plane bytes per token)."""
    lib = L.lib()
    two = (L.ll_gemv_item * 2)(_item(2560, 2560, FAKE, FAKE), _item(2560, 6912, FAKE + 0x10000, FAKE))
    split = (L.ll_gemv_item * 2)(_item(2560, 2560, FAKE, FAKE), _item(100, 8448, FAKE + 0x10000, FAKE))
    assert lib.ll_gemv_plan_bytes(two, 2, L.LL_ACT_F32, 1) >= 5 * (2560 + 6912)
    assert lib.ll_gemv_plan_bytes(split, 2, L.LL_ACT_F32, 1) >= 5 * (2560 + 8448)
    fused = two
    # two products sharing x (same pointer and K) share one layout
    shared = (L.ll_gemv_item * 3)(_item(64, 2560, FAKE, FAKE), _item(64, 2560, FAKE, FAKE), _item(64, 8448, FAKE * 3, FAKE))
    b_shared = lib.ll_gemv_plan_bytes(shared, 3, L.LL_ACT_F32, 1)
    assert 5 * (2560 + 8448) <= b_shared < 5 * (2 * 2560 + 8448)
    assert lib.ll_gemv_plan_bytes(fused, 2, L.LL_ACT_I8, 1) == 2 ** 64 - 1


def _pair(N, K, x, y, N2=None, K2=None, bias=None, epi=1):
    return L.ll_gemv_item_ex(_w(N=N, K=K), _w(N=N2 or N, K=K2 or K), C.c_void_p(x),
                             None if bias is None else C.c_void_p(bias), C.c_void_p(y), epi)


def test_plan_ex_gated_pair_validation():
    """Host-only: a gated pair (LL_EPI_RELU2_MUL) shares its activation layout
    with a plain item of the same x and K, and is rejected with M != 1, a
    bias, gate and up of different N or K, or an unknown epilogue code."""
    lib = L.lib()
    plain = L.ll_gemv_item_ex(_w(N=2560, K=2560), L.ll_weights(), C.c_void_p(FAKE), None, C.c_void_p(FAKE), 0)
    ok = (L.ll_gemv_item_ex * 2)(plain, _pair(6912, 2560, FAKE, FAKE))
    b_ok = lib.ll_gemv_plan_bytes_ex(ok, 2, L.LL_ACT_F32, 1)
    assert b_ok != 2 ** 64 - 1 and b_ok >= 5 * 2560
    one = (L.ll_gemv_item * 1)(_item(2560, 2560, FAKE, FAKE))
    assert b_ok < lib.ll_gemv_plan_bytes(one, 1, L.LL_ACT_F32, 1) + 5 * 2560   # one layout for the shared x
    assert lib.ll_gemv_plan_bytes_ex(ok, 2, L.LL_ACT_F32, 2) == 2 ** 64 - 1     # M != 1
    plan = L.ll_gemv_plan()
    cases = [(_pair(64, 2560, FAKE, FAKE, K2=5120), -2),
             (_pair(64, 2560, FAKE, FAKE, N2=65), -2),
             (_pair(64, 2560, FAKE, FAKE, bias=FAKE), -1),
             (_pair(64, 2560, FAKE, FAKE, epi=7), -1)]
    for item, want in cases:
        arr = (L.ll_gemv_item_ex * 1)(item)
        assert lib.ll_gemv_plan_bytes_ex(arr, 1, L.LL_ACT_F32, 1) == 2 ** 64 - 1
        assert lib.ll_gemv_plan_init_ex(arr, 1, L.LL_ACT_F32, 1, None, 0, C.byref(plan)) == want


def _item_i8(N, K, xq, y, group=128, fmt=None, xs=None, bias=None):
    return L.ll_gemv_item_i8(_w(fmt=L.LL_FMT_W1 if fmt is None else fmt, N=N, K=K, group=group), C.c_void_p(xq),
                             C.c_void_p(FAKE if xs is None else xs), None if bias is None else C.c_void_p(bias),
                             C.c_void_p(y))


def test_i2s_rows_longer_than_2_20_are_rejected():
    """i2_s products keep whole-row sums in int32, so every device entry point
    refuses K > 2^20 on the host (LL_ERANGE) and accepts K = 2^20 as far as
    validation goes (the byte-size check of a plan)."""
    lib = L.lib()
    big = _w(N=64, K=(1 << 20) + 128)
    assert _gemv(big) == -7
    assert _gemv(big, act=L.LL_ACT_I8) == -7
    assert lib.ll_bitlinear_gemm(C.byref(big), C.c_void_p(FAKE), C.c_void_p(FAKE), 32, None, C.c_void_p(FAKE), None,
                                 C.c_void_p(FAKE), 1 << 30, None) == -7
    plan = L.ll_gemv_plan()
    arr = (L.ll_gemv_item * 1)(_item(64, (1 << 20) + 128, FAKE, FAKE))
    assert lib.ll_gemv_plan_bytes(arr, 1, L.LL_ACT_F32, 1) == 2 ** 64 - 1
    assert lib.ll_gemv_plan_init(arr, 1, L.LL_ACT_F32, 1, None, 0, C.byref(plan)) == -7
    ok = (L.ll_gemv_item * 1)(_item(64, 1 << 20, FAKE, FAKE))
    assert lib.ll_gemv_plan_bytes(ok, 1, L.LL_ACT_F32, 1) != 2 ** 64 - 1


def test_plan_i8_layout_and_validation():
    """Host-only: a W1A8 plan holds one prepared operand per distinct (xq, K)
    (A digit rows of K / 128 chunks x 2M rows x 128 B, then M x K / 128
    int32 group sums) and rejects other formats, group sizes, M outside
    [1, 8], operands too large for the streaming product, NULL and
    misaligned pointers, before anything is launched."""
    lib = L.lib()
    one = (L.ll_gemv_item_i8 * 1)(_item_i8(7168, 5120, FAKE, FAKE))
    b1 = lib.ll_gemv_plan_bytes_i8(one, 1, 1)
    ops = 40 * 2 * 128 + 40 * 4
    assert ops <= b1 < ops + 4096
    shared = (L.ll_gemv_item_i8 * 3)(_item_i8(7168, 5120, FAKE, FAKE), _item_i8(17408, 5120, FAKE, FAKE),
                                     _item_i8(5120, 17408, FAKE * 3, FAKE))
    b3 = lib.ll_gemv_plan_bytes_i8(shared, 3, 1)
    ops3 = ops + 136 * 2 * 128 + 136 * 4
    assert ops3 <= b3 < ops3 + 8192
    assert lib.ll_gemv_plan_bytes_i8(one, 1, 8) > lib.ll_gemv_plan_bytes_i8(one, 1, 1)
    plan = L.ll_gemv_plan()
    cases = [(_item_i8(64, 5120, FAKE, FAKE, fmt=L.LL_FMT_I2S), 1, -1),      # another format
             (_item_i8(64, 5120, FAKE, FAKE, group=64), 1, -2),              # group 64
             (_item_i8(64, 5120, FAKE, FAKE), 9, -2),                        # M = 9
             (_item_i8(64, 5120, FAKE, FAKE), 0, -2),                        # M = 0
             (_item_i8(64, 6400, FAKE, FAKE), 8, -7),                        # operand of 8 x 6400 too large
             (_item_i8(64, 50304, FAKE, FAKE), 1, -7),                       # 1 x 50304 too large
             (_item_i8(64, 5120, FAKE + 8, FAKE), 1, -3),                    # xq not 16-byte aligned
             (_item_i8(64, 5120, FAKE, FAKE + 2), 1, -3),                    # y not 4-byte aligned
             (_item_i8(64, 5120, 0, FAKE), 1, -1)]                           # NULL xq
    for item, M, want in cases:
        arr = (L.ll_gemv_item_i8 * 1)(item)
        assert lib.ll_gemv_plan_bytes_i8(arr, 1, M) == 2 ** 64 - 1, (M, want)
        assert lib.ll_gemv_plan_init_i8(arr, 1, M, None, 0, C.byref(plan)) == want, (M, want)
    assert lib.ll_gemv_plan_bytes_i8((L.ll_gemv_item_i8 * 1)(_item_i8(64, 6272, FAKE, FAKE)), 1, 8) != 2 ** 64 - 1
    assert lib.ll_gemv_plan_bytes_i8((L.ll_gemv_item_i8 * 1)(_item_i8(64, 50176, FAKE, FAKE)), 1, 1) != 2 ** 64 - 1
    assert lib.ll_gemv_plan_init_i8(one, 1, 1, None, 0, C.byref(plan)) == -5     # no memory


def test_w1_device_argument_errors_and_workspace():
    lib = L.lib()
    w = _w(fmt=L.LL_FMT_W1, N=64, K=5120, group=128)
    # A rows: 40 chunks x (2 digits x 8 tokens) x 128 B, then int32 group sums [8][40]; one row block
    # of 128 splits K five ways (one per 1024-k window): fp64 partial sums [5][128][tokens] at the
    # next 256-byte boundary; all of it after the 4096-byte counter region (one counter in use)
    assert lib.ll_gemv_workspace_size(C.byref(w), L.LL_ACT_I8, 8) == CB + 40 * 16 * 128 + 8 * 40 * 4 + 5 * 128 * 8 * 8
    base1 = 40 * 2 * 128 + 40 * 4
    assert lib.ll_gemv_workspace_size(C.byref(w), L.LL_ACT_I8, 1) == CB + (base1 + 255) // 256 * 256 + 5 * 128 * 8
    # a wide matrix (1940 row blocks) is not split
    wide = _w(fmt=L.LL_FMT_W1, N=248320, K=5120, group=128)
    assert lib.ll_gemv_workspace_size(C.byref(wide), L.LL_ACT_I8, 1) == CB + base1
    # G = 32: four group slots per 128-k chunk; passes of 2 tokens (a 4-token pass has 32 A rows,
    # more than the streamed product takes, and two streamed passes beat one windowed pass)
    w32 = _w(fmt=L.LL_FMT_W1, N=64, K=512, group=32)
    assert lib.ll_gemm_workspace_size(C.byref(w32), 100) == CB + 4 * 16 * 128 + 2 * 16 * 4
    assert _gemv(w, act=L.LL_ACT_I8, M=8, ws=0) == -5
    assert _gemv(w, act=L.LL_ACT_I8, M=8, wsb=16) == -5
    assert _gemv(_w(fmt=L.LL_FMT_W1, K=160, group=32), act=L.LL_ACT_I8) == -2      # K % 128 on the device
    assert _gemv(_w(fmt=L.LL_FMT_W1, K=384, group=96), act=L.LL_ACT_I8) == -2      # group 96
    assert _gemv(_w(fmt=L.LL_FMT_W1, K=512, group=128, scales=0), act=L.LL_ACT_I8) == -1
    assert lib.ll_bitlinear_gemm(C.byref(w), C.c_void_p(FAKE), C.c_void_p(FAKE), 32, None, C.c_void_p(FAKE),
                                 C.c_void_p(FAKE), C.c_void_p(FAKE), 1 << 30, None) == -1   # acc_out with W1
