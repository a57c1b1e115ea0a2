"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer-activation paths must be bit-exact; fp32
activation paths must satisfy |y_gpu - y_ref| <= 1e-5 * T + 1e-6.

Every output is compared: small shapes (they still span several tiles and
a ragged tail) and the full configuration sizes, the latter in the launch
configuration the benchmark times, with the oracle's rows split over every
host core (oracle.cores())."""
import numpy as np
import pytest

import oracle
from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth
from gpu_util import TH, announce, f32_tol_ok, make_i2s, make_tq2, relu2_mul_tol_ok, torch

pytestmark = pytest.mark.gpu


def _x(seed, M, K):
    return synth.normal_f32(seed, M, K)


# ------------------------------------------------------------------ quantize
@pytest.mark.parametrize("M,K,dtype", [(1, 512, "f32"), (7, 2560, "f32"), (512, 2560, "bf16"), (512, 6912, "bf16"),
                                       (3, 1000, "f32"), (5, 1001, "bf16"), (16, 5120, "f32")])
def test_quantize_bitexact(M, K, dtype):
    t = torch()
    announce("quantize", M, K, dtype)
    if dtype == "bf16":
        xb = synth.normal_bf16_bits(11 + M, M, K)
        xb[0, :] = 0                                   # zero token
        x = t.from_numpy(xb.view(np.int16)).cuda().view(t.bfloat16)
        q_ref, s_ref = oracle.quantize_bf16(xb)
    else:
        xf = _x(12 + M, M, K)
        xf[-1, :] = 0.0
        if K >= 8:
            xf[0, :4] = [127.0, 2.5, -3.5, 0.5]        # exact ties when absmax is 127
            xf[0, 4:] = np.clip(xf[0, 4:], -100, 100)
        x = t.from_numpy(xf).cuda()
        q_ref, s_ref = oracle.quantize_f32(xf)
    xq, xs, xsum = L.quantize(x, with_sum=True)
    t.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(xsum.cpu().numpy().astype(np.int64), q_ref.astype(np.int64).sum(axis=1))
    xq2, xs2 = L.quantize(x)                           # without the sums: the same codes
    t.cuda.synchronize()
    assert np.array_equal(xq2.cpu().numpy(), q_ref)


# ------------------------------------------------------------------ i2_s, fp32 activations
# A single call with M = 1 up to K = 8192 runs the fused kernel (planes built
# per workgroup); K = 8320 and M = 2, 3 the preparation + product pair;
# M > 3 the same kernels in passes of up to three tokens.
I2S_F32_SMALL = [(256, 512, 1), (37, 384, 1), (16, 128, 1), (1, 128, 1), (100, 640, 2), (77, 512, 5),
                 (64, 256, 6), (50, 384, 11), (33, 512, 16), (129, 1024, 3), (40, 8192, 1), (70, 8320, 1),
                 (65, 1152, 2), (3, 3200, 1)]


@pytest.mark.parametrize("N,K,M", I2S_F32_SMALL)
def test_i2s_gemv_f32_small(N, K, M):
    t = torch()
    w, scale, packed = make_i2s(100 + N + K + M, N, K, scale=0.0625 if (N, K) == (256, 512) else None)
    x = _x(200 + N + M, M, K)
    bias = synth.uniform_f32(300 + N, N, -1, 1) if M == 2 else None
    announce("i2s gemv f32", N, K, M)
    W = L.upload_i2s(packed, N, K)
    y = L.gemv(W, t.from_numpy(x).cuda(), bias=None if bias is None else t.from_numpy(bias).cuda())
    y = y.cpu().numpy()
    y_ref, tsum = oracle.i2s_gemv_f32(packed, N, K, x)
    if bias is not None:
        y_ref = y_ref + bias.astype(np.float64)[None, :]
    ok, worst = f32_tol_ok(y, y_ref, tsum)
    assert ok, "worst error / bound = %.3f" % worst


I2S_DECODE = [(2560, 2560, 201), (6912, 2560, 205), (2560, 6912, 207)]


@pytest.mark.parametrize("N,K,seed", I2S_DECODE)
def test_i2s_gemv_f32_decode_full(N, K, seed):
    t = torch()
    w, scale, packed = make_i2s(seed, N, K)
    x = _x(seed + 50, 1, K)
    announce("i2s gemv f32 full", N, K)
    W = L.upload_i2s(packed, N, K)
    y = L.gemv(W, t.from_numpy(x).cuda()).cpu().numpy()
    y_ref, tsum = oracle.i2s_gemv_f32(packed, N, K, x, threads=TH)
    ok, worst = f32_tol_ok(y, y_ref, tsum)
    assert ok, "worst error / bound = %.3f" % worst


def test_i2s_gemv_f32_closed_forms():
    """One-hot rows locate every k end to end; all-zero rows give exactly 0."""
    t = torch()
    K = 512
    N = 128
    w = np.zeros((N, K), np.int8)
    ks = np.arange(N) * 4 + 1
    w[np.arange(N), ks] = np.where(np.arange(N) % 2 == 0, 1, -1)
    w[-1] = 0
    packed = L.ll_pack_i2s(w, 1.0)
    x = _x(77, 1, K)
    announce("i2s gemv onehot")
    y = L.gemv(L.upload_i2s(packed, N, K), t.from_numpy(x).cuda()).cpu().numpy()[0]
    expect = np.where(np.arange(N) % 2 == 0, 1.0, -1.0) * x[0, ks]
    expect[-1] = 0.0
    assert np.array_equal(y, expect.astype(np.float32))


def test_i2s_gemv_f32_deterministic():
    t = torch()
    N, K = 1000, 2560
    _, _, packed = make_i2s(5, N, K)
    x = t.from_numpy(_x(6, 1, K)).cuda()
    W = L.upload_i2s(packed, N, K)
    announce("i2s gemv determinism")
    a = L.gemv(W, x).cpu().numpy()
    b = L.gemv(W, x).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ TQ2_0, fp32 activations
@pytest.mark.parametrize("N,K,M", [(17, 256, 1), (100, 512, 8), (40, 768, 16), (6, 1024, 3), (256, 2560, 1),
                                   (9, 8192, 1), (5, 8448, 1), (70, 1280, 2)])
def test_tq2_gemv_f32_small(N, K, M):
    t = torch()
    w, sc, blocks = make_tq2(400 + N + M, N, K)
    x = _x(500 + N + M, M, K)
    announce("tq2 gemv f32", N, K, M)
    W = L.upload_tq2(blocks, N, K)
    y = L.gemv(W, t.from_numpy(x).cuda()).cpu().numpy()
    y_ref, tsum = oracle.tq2_gemv_f32(blocks, N, K, x)
    ok, worst = f32_tol_ok(y, y_ref, tsum)
    assert ok, "worst error / bound = %.3f" % worst


@pytest.mark.parametrize("M", [1, 8, 16])
def test_tq2_gemv_f32_full(M):
    t = torch()
    N, K = 6912, 2560
    w, sc, blocks = make_tq2(301, N, K)
    x = _x(302 + M, M, K)
    announce("tq2 gemv f32 full", M)
    W = L.upload_tq2(blocks, N, K)
    y = L.gemv(W, t.from_numpy(x).cuda()).cpu().numpy()
    y_ref, tsum = oracle.tq2_gemv_f32(blocks, N, K, x, threads=TH)
    ok, worst = f32_tol_ok(y, y_ref, tsum)
    assert ok, "worst error / bound = %.3f" % worst


# ------------------------------------------------------------------ i2_s, int8 activations (GEMM)
def _i2s_i8_case(N, K, M, seed, rows=None, bias=False):
    t = torch()
    w, scale, packed = make_i2s(seed, N, K)
    xb = synth.normal_bf16_bits(seed + 3, M, K)
    q, s = oracle.quantize_bf16(xb)
    W = L.upload_i2s(packed, N, K)
    b = synth.uniform_f32(seed + 4, N, -1, 1) if bias else None
    y, acc = L.gemm(W, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(),
                    bias=None if b is None else t.from_numpy(b).cuda(), want_acc=True)
    y = y.cpu().numpy()
    acc = acc.cpu().numpy()
    y_ref, acc_ref = oracle.i2s_gemm_i8(packed, N, K, q, s, rows, threads=TH)
    if rows is not None:
        y, acc = y[:, rows], acc[:, rows]
    if b is not None:
        bb = b if rows is None else b[rows]
        y_ref = (y_ref + bb[None, :]).astype(np.float32)
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


# Tile paths (narrow 64 x 128 tiles unless noted): K split (5, 2560, 300) two ways, (150, 2688, 33) two
# uneven ways, (64, 4096, 40) three uneven ways, (100, 5120, 70) four ways; two halves along K
# (128, 256, 128), (200, 512, 17), (300, 2048, 200); four waves, odd group counts (77, 384, 65),
# (130, 640, 129), (257, 1664, 130); wide 128 x 128 tiles with ragged rows and columns (1300, 384, 1500)
@pytest.mark.parametrize("N,K,M", [(77, 384, 65), (128, 256, 128), (200, 512, 17), (33, 128, 1), (130, 640, 129),
                                   (5, 2560, 300), (300, 2048, 200), (64, 4096, 40), (257, 1664, 130),
                                   (100, 5120, 70), (150, 2688, 33), (1300, 384, 1500)])
def test_i2s_gemm_i8_small(N, K, M):
    announce("i2s gemm i8", N, K, M)
    _i2s_i8_case(N, K, M, 600 + N + M, bias=(M == 65))


@pytest.mark.parametrize("N,K", [(6912, 2560), (2560, 6912)])
def test_i2s_gemm_i8_prefill_full(N, K):
    announce("i2s gemm i8 full", N, K)
    _i2s_i8_case(N, K, 512, 401 if N == 6912 else 402)


# ------------------------------------------------------------------ TQ2_0, int8 activations (GEMM)
def _tq2_i8_case(N, K, M, seed, rows=None, bias=False, repeat=1):
    """fp32 bound against the oracle's fp64 value: the kernel scales each
    256-k block's exact int32 sum into fp32 (the same bound as the
    fp32-activation paths, with T = s_tok * sum_b |s_b| sum_{k in b} |q|)."""
    t = torch()
    w, sc, blocks = make_tq2(seed, N, K)
    q, s = oracle.quantize_bf16(synth.normal_bf16_bits(seed + 3, M, K))
    W = L.upload_tq2(blocks, N, K)
    b = synth.uniform_f32(seed + 4, N, -1, 1) if bias else None
    outs = []
    for _ in range(repeat):
        y, _ = L.gemm(W, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), bias=None if b is None else t.from_numpy(b).cuda())
        outs.append(y.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), "repeated calls differ"
    y = outs[0] if rows is None else outs[0][:, rows]
    y_ref, tsum = oracle.tq2_gemm_i8(blocks, N, K, q, s, rows, threads=TH)
    if b is not None:
        y_ref = y_ref + (b if rows is None else b[rows])[None, :].astype(np.float64)
    ok, worst = f32_tol_ok(y, y_ref, tsum)
    assert ok, "N=%d K=%d M=%d: worst error / bound %.3f" % (N, K, M, worst)


# split K (whole 256-k blocks): (5, 2560, 300) two ways (5 + 5 blocks), (150, 2816, 33) two uneven ways
# (5 + 6), (64, 4096, 40) three uneven ways (5 + 5 + 6), (64, 5376, 40) four uneven ways (5 + 5 + 5 + 6);
# the others unsplit.  Narrow tiles run as two halves of whole blocks along K: (77, 512, 65) one block
# each, (200, 768, 17) one and two; (128, 256, 128) has a single block, so it keeps the wide tiles
@pytest.mark.parametrize("N,K,M", [(77, 512, 65), (128, 256, 128), (200, 768, 17), (33, 256, 1), (130, 1280, 129),
                                   (5, 2560, 300), (300, 2048, 200), (64, 4096, 40), (257, 1792, 130),
                                   (150, 2816, 33), (64, 5376, 40)])
def test_tq2_gemm_i8_small(N, K, M):
    announce("tq2 gemm i8", N, K, M)
    _tq2_i8_case(N, K, M, 620 + N + M, bias=(M == 65), repeat=2 if K >= 1792 else 1)


@pytest.mark.parametrize("N,K", [(6912, 2560), (2560, 6912)])
def test_tq2_gemm_i8_prefill_full(N, K):
    announce("tq2 gemm i8 full", N, K)
    _tq2_i8_case(N, K, 512, 411 if N == 6912 else 412)


def test_i2s_gemm_i8_workspace_reuse():
    """Two calls sharing one (zero-filled once) workspace: the split-K tile
    counters are left zero by the first call, so the second is exact too."""
    t = torch()
    N, K, M = 2560, 6912, 256
    w, scale, packed = make_i2s(650, N, K)
    W = L.upload_i2s(packed, N, K)
    ws = t.zeros((max(L.ll_gemm_workspace_size(W, M), 16),), dtype=t.uint8, device="cuda")
    assert L.ll_gemm_workspace_size(W, M) > 0
    for rnd in range(2):
        q, s = oracle.quantize_bf16(synth.normal_bf16_bits(652 + rnd, M, K))
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        announce("gemm workspace reuse", rnd)
        L.ll_bitlinear_gemm(W, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), M, None, y, None, ws)
        y_ref, _ = oracle.i2s_gemm_i8(packed, N, K, q, s, threads=TH)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), rnd


# ------------------------------------------------------------------ int8 activations at decode sizes (M <= 16)
def _gemv_i8_case(fmt, N, K, M, seed, bias=False):
    """ll_bitlinear_gemv with int8 activations, every output: i2_s bit for
    bit against the oracle (y = ((float)acc * s_tok) * s_w, then + bias),
    TQ2_0 inside the fp32 bound; every output written (y starts as NaN)."""
    t = torch()
    if fmt == "i2s":
        w, scale, packed = make_i2s(seed, N, K)
        W = L.upload_i2s(packed, N, K)
    else:
        w, sc, blocks = make_tq2(seed, N, K)
        W = L.upload_tq2(blocks, N, K)
    q, s = oracle.quantize_bf16(synth.normal_bf16_bits(seed + 3, M, K))
    b = synth.uniform_f32(seed + 4, N, -1, 1) if bias else None
    assert L.ll_gemv_workspace_size(W, L.LL_ACT_I8, M) == 0
    y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    L.ll_bitlinear_gemv(W, L.LL_ACT_I8, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), M,
                        None if b is None else t.from_numpy(b).cuda(), y, None)
    y = y.cpu().numpy()
    bb = b
    if fmt == "i2s":
        y_ref, _ = oracle.i2s_gemm_i8(packed, N, K, q, s, None, threads=TH)
        if bb is not None:
            y_ref = (y_ref + bb[None, :]).astype(np.float32)
        bad = np.argwhere(y.view(np.uint32) != y_ref.view(np.uint32))
        assert bad.size == 0, "N=%d K=%d M=%d: %d outputs differ, first %s" % (N, K, M, len(bad), bad[:4].tolist())
    else:
        y_ref, tsum = oracle.tq2_gemm_i8(blocks, N, K, q, s, None, threads=TH)
        if bb is not None:
            y_ref = y_ref + bb[None, :].astype(np.float64)
        ok, worst = f32_tol_ok(y, y_ref, tsum)
        assert ok, "N=%d K=%d M=%d: worst error / bound %.3f" % (N, K, M, worst)


# ragged N (33, 37, 77, 130, 300), ragged last window (K = 384, 1152, 1280, 8448), every row capacity
# (M = 1, 2, 3..4, 5..8, 9..16), bias
@pytest.mark.parametrize("N,K,M,bias", [(300, 1024, 4, False), (33, 128, 1, True), (37, 384, 2, False),
                                        (130, 1152, 3, True), (300, 2560, 7, False), (64, 8448, 16, True),
                                        (100, 4096, 13, False), (77, 768, 16, False), (16, 256, 9, True)])
def test_i2s_gemv_i8_small(N, K, M, bias):
    announce("i2s gemv i8", N, K, M)
    _gemv_i8_case("i2s", N, K, M, 700 + N + M, bias)


@pytest.mark.parametrize("N,K,M,bias", [(300, 1024, 5, False), (33, 256, 1, True), (37, 512, 2, False),
                                        (130, 1280, 3, True), (300, 2560, 7, False), (64, 8448, 16, True),
                                        (100, 4096, 11, False), (77, 768, 16, False), (16, 256, 9, True)])
def test_tq2_gemv_i8_small(N, K, M, bias):
    announce("tq2 gemv i8", N, K, M)
    _gemv_i8_case("tq2", N, K, M, 720 + N + M, bias)


# the decode shapes at full size, every output
@pytest.mark.parametrize("fmt", ["i2s", "tq2"])
@pytest.mark.parametrize("N,K,M", [(2560, 2560, 1), (6912, 2560, 8), (2560, 6912, 16)])
def test_gemv_i8_decode_shapes(fmt, N, K, M):
    announce("gemv i8 decode", fmt, N, K, M)
    _gemv_i8_case(fmt, N, K, M, 740 + N + M, bias=(M == 8))


# ------------------------------------------------------------------ prepared batch
@pytest.mark.parametrize("fmt,M,big", [("i2s", 1, False), ("i2s", 1, True), ("i2s", 2, False), ("i2s", 4, False),
                                      ("i2s", 5, False), ("i2s", 16, True), ("tq2", 1, False), ("tq2", 1, True),
                                      ("tq2", 3, False), ("tq2", 8, False), ("tq2", 16, False)])
def test_gemv_plan_matches_oracle(fmt, M, big):
    """A prepared batch of products with mixed N and K (some sharing x) against
    the oracle, every row, run twice (second run with new x contents).  With
    big, one product has K = 8448 (33 plane blocks, a ragged last window)."""
    t = torch()
    shapes = [(2560, 2560, 0), (6912, 2560, 0), (2560, 6912, 1), (37, 384 if fmt == "i2s" else 512, 2),
              (16, 256, 3)] + ([(100, 8448, 4)] if big else [])
    xs_np = {}
    items, refs = [], []
    for i, (N, K, slot) in enumerate(shapes):
        if fmt == "i2s":
            w, scale, packed = make_i2s(700 + i, N, K)
            W = L.upload_i2s(packed, N, K)
        else:
            w, sc, packed = make_tq2(700 + i, N, K)
            W = L.upload_tq2(packed, N, K)
        if slot not in xs_np:
            xs_np[slot] = (_x(800 + slot, M, K), None)
        x = xs_np[slot][0]
        if xs_np[slot][1] is None:
            xs_np[slot] = (x, t.from_numpy(x).cuda())
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        items.append((W, xs_np[slot][1], None, y))
        refs.append((packed, N, K, slot))
    announce("gemv plan", fmt, M)
    plan = L.GemvPlan(items, M)
    for rnd in range(2):
        if rnd == 1:
            for slot, (x, xd) in xs_np.items():
                x2 = _x(900 + slot, M, x.shape[1])
                xd.copy_(t.from_numpy(x2))
                xs_np[slot] = (x2, xd)
        plan.run()
        t.cuda.synchronize()
        for (W, xd, _, y), (packed, N, K, slot) in zip(items, refs):
            fn = oracle.i2s_gemv_f32 if fmt == "i2s" else oracle.tq2_gemv_f32
            y_ref, tsum = fn(packed, N, K, xs_np[slot][0], threads=TH)
            ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
            assert ok, "N=%d K=%d round %d: worst error / bound %.3f" % (N, K, rnd, worst)


@pytest.mark.parametrize("fmt", ["i2s", "tq2"])
def test_gemv_plan_relu2_mul_and_residual(fmt):
    """Fused epilogues of a one-token prepared batch against the oracle: gated
    pairs y = relu(gate)^2 * up [BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"] (the
    FFN shape 6912 x 2560 and a ragged 100-row pair with another x), mixed
    with a plain product whose bias is the residual stream [BL "Fused
    BitLinear + Residual Add Kernel"]; run twice with new x contents."""
    t = torch()
    K, Kr = 2560, 384 if fmt == "i2s" else 512
    mk = (lambda s, N, K: make_i2s(s, N, K)) if fmt == "i2s" else (lambda s, N, K: make_tq2(s, N, K))
    up = (lambda p, N, K: L.upload_i2s(p, N, K)) if fmt == "i2s" else (lambda p, N, K: L.upload_tq2(p, N, K))
    fn = oracle.i2s_gemv_f32 if fmt == "i2s" else oracle.tq2_gemv_f32
    xs = {0: _x(830, 1, K), 1: _x(831, 1, Kr)}
    xd = {k: t.from_numpy(v).cuda() for k, v in xs.items()}
    pairs, items = [], []
    for i, (N, KK, slot) in enumerate([(6912, K, 0), (100, Kr, 1)]):
        pg, pu = mk(840 + 2 * i, N, KK)[2], mk(841 + 2 * i, N, KK)[2]
        y = t.empty((1, N), dtype=t.float32, device="cuda")
        items.append(L.Relu2Mul(up(pg, N, KK), up(pu, N, KK), xd[slot], y))
        pairs.append((pg, pu, N, KK, slot, y))
    pp = mk(850, 2560, K)[2]
    res = synth.normal_f32(851, 1, 2560)[0]
    yp = t.empty((1, 2560), dtype=t.float32, device="cuda")
    items.append((up(pp, 2560, K), xd[0], t.from_numpy(res).cuda(), yp))
    announce("gemv plan relu2 mul", fmt)
    plan = L.GemvPlan(items, 1)
    for rnd in range(2):
        if rnd == 1:
            for slot in xs:
                xs[slot] = _x(860 + slot, 1, xs[slot].shape[1])
                xd[slot].copy_(t.from_numpy(xs[slot]))
        plan.run()
        t.cuda.synchronize()
        for pg, pu, N, KK, slot, y in pairs:
            g_ref, tg = fn(pg, N, KK, xs[slot], threads=TH)
            u_ref, tu = fn(pu, N, KK, xs[slot], threads=TH)
            ok, worst = relu2_mul_tol_ok(y.cpu().numpy(), g_ref, tg, u_ref, tu)
            assert ok, "pair N=%d K=%d round %d: worst error / bound %.3f" % (N, KK, rnd, worst)
            assert (g_ref > 0).any() and (g_ref < 0).any()
        y_ref, tsum = fn(pp, 2560, K, xs[0], threads=TH)
        want = y_ref + res.astype(np.float64)[None, :]
        got = yp.cpu().numpy().astype(np.float64)
        bound = 1e-5 * tsum + 1e-6 + 2.0 ** -23 * np.abs(want)
        assert (np.abs(got - want) <= bound).all(), "residual round %d" % rnd


@pytest.mark.parametrize("fmt", ["i2s", "tq2"])
def test_gemv_plan_rmsnorm_prologue(fmt):
    """RMSNorm prologue of a one-token prepared batch [BL "Fused RMSNorm +
    BitLinear + Residual Add M=1 Kernel"] against the oracle (xn from
    oracle.rmsnorm in fp64): two normed products sharing x and the norm (one
    prepared operand), a plain product of the same x (its own), a normed
    gated pair, and a zero row with eps = 0 whose output is the residual bit
    for bit.  Outputs carry the residual add where the page's kernel has it."""
    t = torch()
    K, N = 2560, 2560
    mk = (lambda s, N, K: make_i2s(s, N, K)[2]) if fmt == "i2s" else (lambda s, N, K: make_tq2(s, N, K)[2])
    up = (lambda p, N, K: L.upload_i2s(p, N, K)) if fmt == "i2s" else (lambda p, N, K: L.upload_tq2(p, N, K))
    fn = oracle.i2s_gemv_f32 if fmt == "i2s" else oracle.tq2_gemv_f32
    eps = 1e-5
    x0 = _x(870, 1, K)
    x2 = _x(871, 1, K)
    x3 = np.zeros((1, K), np.float32)
    g0 = synth.uniform_f32(872, K, 0.5, 1.5)
    g2 = synth.uniform_f32(873, K, 0.5, 1.5)
    d = {k: t.from_numpy(v).cuda() for k, v in dict(x0=x0, x2=x2, x3=x3, g0=g0, g2=g2).items()}
    res = synth.normal_f32(874, 1, N)[0]
    resd = t.from_numpy(res).cuda()
    P = {name: mk(880 + i, N if name not in ("gate", "up") else 6912, K)
         for i, name in enumerate(["q", "k", "v", "o", "gate", "up"])}
    Wd = {name: up(p, N if name not in ("gate", "up") else 6912, K) for name, p in P.items()}
    Y = {name: t.empty((1, N if name != "ffn" else 6912), dtype=t.float32, device="cuda")
         for name in ["q", "k", "v", "o", "ffn"]}
    items = [L.Normed(Wd["q"], d["x0"], d["g0"], eps, resd, Y["q"]),
             L.Normed(Wd["k"], d["x0"], d["g0"], eps, None, Y["k"]),
             (Wd["v"], d["x0"], None, Y["v"]),
             L.Relu2Mul(Wd["gate"], Wd["up"], d["x2"], Y["ffn"], norm=(d["g2"], eps)),
             L.Normed(Wd["o"], d["x3"], d["g0"], 0.0, resd, Y["o"])]
    announce("gemv plan rmsnorm", fmt)
    plan = L.GemvPlan(items, 1)
    assert plan.plan.nprep == 4                      # (x0, g0), x0 plain, (x2, g2), (x3, g0, eps 0)
    plan.run()
    t.cuda.synchronize()
    xn0 = oracle.rmsnorm(x0, g0, eps).astype(np.float32)
    xn2 = oracle.rmsnorm(x2, g2, eps).astype(np.float32)
    for name, xin, add in [("q", xn0, res), ("k", xn0, None), ("v", x0, None)]:
        y_ref, tsum = fn(P[name], N, K, xin, threads=TH)
        want = y_ref + (0.0 if add is None else add.astype(np.float64)[None, :])
        got = Y[name].cpu().numpy().astype(np.float64)
        bound = 1e-5 * tsum + 1e-6 + 2.0 ** -23 * np.abs(want)
        assert (np.abs(got - want) <= bound).all(), name
    g_ref, tg = fn(P["gate"], 6912, K, xn2, threads=TH)
    u_ref, tu = fn(P["up"], 6912, K, xn2, threads=TH)
    ok, worst = relu2_mul_tol_ok(Y["ffn"].cpu().numpy(), g_ref, tg, u_ref, tu)
    assert ok, "normed gated pair: worst error / bound %.3f" % worst
    assert np.array_equal(Y["o"].cpu().numpy()[0].view(np.uint32), res.view(np.uint32))


@pytest.mark.parametrize("fmt", ["i2s", "tq2"])
def test_gemv_plan_one_token_edges(fmt):
    """One-token prepared batch (the fp4 digit-plane engine) on the cases its
    activation split has to survive: an all-zero token (y = bias exactly),
    every element at +-max|x| (largest digit words), magnitudes near 1e30 and
    1e-30 (exponent scaling in two steps), one large element among tiny ones
    (sum|x| close to max|x|, so the bound is tight), the shortest rows (one
    group / one block), row counts that end inside a column block, and
    biases."""
    t = torch()
    base = 256 if fmt == "tq2" else 128
    rng = synth.rng(4300)
    cases = []
    for i, (N, K) in enumerate([(90, 1024), (33, 2 * base), (1, base), (257, 2560), (70, 3 * base),
                                (17, 1536), (300, 768)]):
        x = synth.normal_f32(4310 + i, 1, K)
        if i == 0:
            x[:] = 0.0
        elif i == 1:
            x[:] = np.where(rng.random(K) < 0.5, -1.0, 1.0).astype(np.float32) * np.float32(3.0)
        elif i == 3:
            x *= np.float32(1e30)
        elif i == 4:
            x *= np.float32(1e-30)
        elif i == 5:
            x *= np.float32(1e-6)
            x[0, 7] = np.float32(-40.0)
        bias = synth.uniform_f32(4320 + i, N, -1, 1) if i % 2 == 0 else None
        cases.append((N, K, x, bias))
    items, refs = [], []
    for i, (N, K, x, bias) in enumerate(cases):
        if fmt == "i2s":
            _, _, packed = make_i2s(4330 + i, N, K)
            W = L.upload_i2s(packed, N, K)
        else:
            _, _, packed = make_tq2(4330 + i, N, K)
            W = L.upload_tq2(packed, N, K)
        y = t.empty((1, N), dtype=t.float32, device="cuda")
        b = None if bias is None else t.from_numpy(bias).cuda()
        items.append((W, t.from_numpy(x).cuda(), b, y))
        refs.append((packed, N, K, x, bias))
    announce("plan one-token edges", fmt)
    plan = L.GemvPlan(items, 1)
    plan.run()
    t.cuda.synchronize()
    fn = oracle.i2s_gemv_f32 if fmt == "i2s" else oracle.tq2_gemv_f32
    for i, ((_, _, _, y), (packed, N, K, x, bias)) in enumerate(zip(items, refs)):
        got = y.cpu().numpy()
        if i == 0:
            assert np.array_equal(got[0], bias)
            continue
        y_ref, tsum = fn(packed, N, K, x)
        if bias is not None:
            y_ref = y_ref + bias.astype(np.float64)[None, :]
        ok, worst = f32_tol_ok(got, y_ref, tsum)
        assert ok, "case %d (N=%d K=%d): worst error / bound %.3f" % (i, N, K, worst)


@pytest.mark.parametrize("fmt,M", [("i2s", 1), ("tq2", 1), ("i2s", 3)])
def test_gemv_plan_graph_replay(fmt, M):
    """A prepared batch captured in a HIP graph (its two launches): several
    replays, with eager work (new activations, an eager run of the same plan)
    between them, each equal bit for bit to the eager result on the same
    inputs."""
    t = torch()
    shapes = [(2560, 2560, 0), (6912, 2560, 0), (2560, 6912, 1)]
    items, xs_d = [], {}
    for i, (N, K, slot) in enumerate(shapes):
        if fmt == "i2s":
            _, _, packed = make_i2s(7700 + i, N, K)
            W = L.upload_i2s(packed, N, K)
        else:
            _, _, packed = make_tq2(7700 + i, N, K)
            W = L.upload_tq2(packed, N, K)
        if slot not in xs_d:
            xs_d[slot] = t.from_numpy(_x(7800 + slot, M, K)).cuda()
        items.append((W, xs_d[slot], None, t.empty((M, N), dtype=t.float32, device="cuda")))
    plan = L.GemvPlan(items, M)
    announce("plan graph replay", fmt, M)
    plan.run()
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        plan.prepare(None)
        plan.product(None)
    for rnd in range(3):
        for slot, xd in xs_d.items():
            xd.copy_(t.from_numpy(_x(7900 + 10 * rnd + slot, M, xd.shape[1])))
        plan.run()                                     # eager result on these inputs
        t.cuda.synchronize()
        eager = [y.clone() for (_, _, _, y) in items]
        for (_, _, _, y) in items:
            y.zero_()
        g.replay()
        t.cuda.synchronize()
        for (_, _, _, y), ye in zip(items, eager):
            assert t.equal(y.view(t.int32), ye.view(t.int32)), rnd


@pytest.mark.parametrize("fmt,M", [("i2s", 1), ("i2s", 2), ("tq2", 1), ("tq2", 3), ("i2s", 6)])
def test_gemv_f32_zero_token(fmt, M):
    """An all-zero token gives exactly the bias (no exponent, no planes); the
    other tokens still match the oracle."""
    t = torch()
    N, K = 90, 1024
    if fmt == "i2s":
        _, _, packed = make_i2s(41 + M, N, K)
        W = L.upload_i2s(packed, N, K)
        fn = oracle.i2s_gemv_f32
    else:
        _, _, packed = make_tq2(42 + M, N, K)
        W = L.upload_tq2(packed, N, K)
        fn = oracle.tq2_gemv_f32
    x = _x(43 + M, M, K)
    x[0, :] = 0.0
    bias = synth.uniform_f32(44, N, -1, 1)
    announce("zero token", fmt, M)
    y = L.gemv(W, t.from_numpy(x).cuda(), bias=t.from_numpy(bias).cuda()).cpu().numpy()
    assert np.array_equal(y[0], bias)
    y_ref, tsum = fn(packed, N, K, x)
    ok, worst = f32_tol_ok(y, y_ref + bias.astype(np.float64)[None, :], tsum)
    assert ok, "worst error / bound = %.3f" % worst


# ------------------------------------------------------------------ the benchmarked configurations
def _bench():
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    return bench


def test_decode_step_as_benched():
    """The headline workload exactly as bench.py builds and launches it: the
    30-layer i2_s decode step (210 products, 594.7 MB, one prepared batch),
    every output of every product against the oracle."""
    t = torch()
    bench = _bench()
    packed, items, wbytes = bench.build_decode_step(L, synth, t, "cuda")
    assert wbytes == 594740040 and len(items) == 210
    plan = L.GemvPlan(items, 1)
    announce("decode step as benched", plan.plan.tiles)
    plan.run()
    t.cuda.synchronize()
    for layer in range(bench.LAYERS):
        for r, (name, N, K, _) in enumerate(bench.ROLES):
            W, x, _, y = items[7 * layer + r]
            y_ref, tsum = oracle.i2s_gemv_f32(packed[name][0], N, K, x.cpu().numpy(), threads=TH)
            ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
            assert ok, "layer %d %s: worst error / bound %.3f" % (layer, name, worst)


def test_fused_decode_step_as_benched():
    """The fused decode step of bench.py's extras (RMSNorm prologues, gated
    ReLU² pairs, residual adds on O and down), every output of every layer
    against the oracle's rmsnorm, products and relu2_mul."""
    t = torch()
    bench = _bench()
    packed, items, wbytes = bench.build_decode_step(L, synth, t, "cuda")
    fused, extra = bench.fused_decode_items(L, synth, t, "cuda", items)
    plan = L.GemvPlan(fused, 1)
    announce("fused decode step as benched", plan.plan.tiles)
    plan.run()
    t.cuda.synchronize()
    eps = 1e-5
    for layer in range(bench.LAYERS):
        by = {name: items[7 * layer + r] for r, (name, _, _, _) in enumerate(bench.ROLES)}
        norms, res = [n.cpu().numpy() for n in extra[layer][0]], [v.cpu().numpy() for v in extra[layer][1]]
        xs = {name: by[name][1].cpu().numpy() for name in by}
        for name, nidx, radd in [("q", 0, None), ("k", 0, None), ("v", 0, None), ("o", 1, 0), ("down", 3, 1)]:
            _, N, K, _ = [rr for rr in bench.ROLES if rr[0] == name][0]
            xn = oracle.rmsnorm(xs[name], norms[nidx], eps).astype(np.float32)
            y_ref, tsum = oracle.i2s_gemv_f32(packed[name][0], N, K, xn, threads=TH)
            want = y_ref + (0.0 if radd is None else res[radd].astype(np.float64)[None, :])
            got = by[name][3].cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= 1e-5 * tsum + 1e-6 + 2.0 ** -23 * np.abs(want)).all(), (layer, name)
        N, K = bench.FFN, bench.HIDDEN
        xn = oracle.rmsnorm(xs["up"], norms[2], eps).astype(np.float32)
        g_ref, tg = oracle.i2s_gemv_f32(packed["gate"][0], N, K, xn, threads=TH)
        u_ref, tu = oracle.i2s_gemv_f32(packed["up"][0], N, K, xn, threads=TH)
        ok, worst = relu2_mul_tol_ok(by["up"][3].cpu().numpy(), g_ref, tg, u_ref, tu)
        assert ok, "layer %d gated pair: worst error / bound %.3f" % (layer, worst)


# ------------------------------------------------------------------ one workspace, many shapes and entry points
def test_workspace_shared_across_shapes_and_entry_points():
    """One zero-filled workspace serves, in turn: a W1 product of a narrow
    matrix at M = 8 and M = 1 (split K, counters), an fp32 single call whose
    int8 planes fill the data region, an i2_s GEMM split three ways at M = 512
    and again at M = 640 (other tile counts), and the W1 product again.  The
    split counters sit at the start of every workspace, which no call writes
    with data, so each call is exact whatever ran before it."""
    import gpu_util
    t = torch()
    K, G = 5120, 128
    bits, scales = gpu_util.make_w1(501, 7168, K, G)
    W1 = L.upload_w1(bits, scales, K, G)
    _, _, p_i2s = make_i2s(402, 2560, 6912)
    Wi = L.upload_i2s(p_i2s, 2560, 6912)
    _, _, p_f = make_i2s(403, 3000, 2560)
    Wf = L.upload_i2s(p_f, 3000, 2560)
    need = max(L.ll_gemv_workspace_size(W1, L.LL_ACT_I8, 8), L.ll_gemv_workspace_size(Wf, L.LL_ACT_F32, 5),
               L.ll_gemm_workspace_size(Wi, 512), L.ll_gemm_workspace_size(Wi, 640))
    ws = t.zeros((need,), dtype=t.uint8, device="cuda")

    def w1(M, seed):
        q, s = oracle.quantize_f32(_x(seed, M, K))
        y = t.empty((M, 7168), dtype=t.float32, device="cuda")
        announce("shared workspace w1", M)
        L.ll_bitlinear_gemv(W1, L.LL_ACT_I8, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), M, None, y, ws)
        y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s, threads=TH)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), ("w1", M)

    def f32(M, seed):
        x = _x(seed, M, 2560)
        y = t.empty((M, 3000), dtype=t.float32, device="cuda")
        announce("shared workspace f32", M)
        L.ll_bitlinear_gemv(Wf, L.LL_ACT_F32, t.from_numpy(x).cuda(), None, M, None, y, ws)
        y_ref, tsum = oracle.i2s_gemv_f32(p_f, 3000, 2560, x, threads=TH)
        ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
        assert ok, ("f32", M, worst)

    def gemm(M, seed):
        q, s = oracle.quantize_bf16(synth.normal_bf16_bits(seed, M, 6912))
        y = t.empty((M, 2560), dtype=t.float32, device="cuda")
        announce("shared workspace gemm", M)
        L.ll_bitlinear_gemm(Wi, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), M, None, y, None, ws)
        y_ref, _ = oracle.i2s_gemm_i8(p_i2s, 2560, 6912, q, s, threads=TH)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), ("gemm", M)

    w1(8, 9100)
    w1(1, 9101)
    f32(5, 9102)
    w1(1, 9103)
    gemm(512, 9104)
    gemm(640, 9105)
    w1(8, 9106)
    assert not ws[:4096].any().item()          # counters left zero


# ------------------------------------------------------------------ TQ2_0 prepared batch at the full shape
@pytest.mark.parametrize("M", [1, 8, 16])
def test_tq2_plan_full(M):
    """TQ2_0 6912 x 2560 as a prepared batch (the fp4 engine, all M tokens in
    one pass over the weights), every output."""
    t = torch()
    N, K = 6912, 2560
    _, _, blocks = make_tq2(301, N, K)
    x = _x(304 + M, M, K)
    W = L.upload_tq2(blocks, N, K)
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    plan = L.GemvPlan([(W, t.from_numpy(x).cuda(), None, y)], M)
    announce("tq2 plan full", M)
    plan.run()
    t.cuda.synchronize()
    y_ref, tsum = oracle.tq2_gemv_f32(blocks, N, K, x, threads=TH)
    ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
    assert ok, "worst error / bound %.3f" % worst


# ------------------------------------------------------------------ the fp4 engine's K limit
def test_plan_k_limit_of_the_fp4_engine():
    """Rows of K = 2^17 still run on the fp4 digit engine; a batch holding a
    row of K = 2^17 + 128 runs on the int8-plane engine instead (its rounding
    error stays inside the bound for any K).  One large element among small
    ones keeps sum|x| close to max|x|, where the bound is tightest."""
    t = torch()
    for K in (1 << 17, (1 << 17) + 128):
        N = 40
        _, _, packed = make_i2s(9200 + K % 7, N, K)
        x = _x(9201, 1, K) * np.float32(1e-3)
        x[0, 5] = np.float32(9.0)
        W = L.upload_i2s(packed, N, K)
        y = t.empty((1, N), dtype=t.float32, device="cuda")
        plan = L.GemvPlan([(W, t.from_numpy(x).cuda(), None, y)], 1)
        announce("plan K limit", K)
        plan.run()
        t.cuda.synchronize()
        y_ref, tsum = oracle.i2s_gemv_f32(packed, N, K, x, threads=TH)
        ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
        assert ok, "K=%d: worst error / bound %.3f" % (K, worst)


def test_tq2_plan_longest_rows_several_tokens():
    """TQ2_0 rows of K = 2^17 (the fp4 engine's limit) for three tokens: one
    large element among small ones keeps sum|x| close to max|x|, and 512
    block-scaled sums per row are accumulated; the result stays inside the
    bound (the block sums are folded exactly and added in fp64)."""
    t = torch()
    N, K, M = 40, 1 << 17, 3
    _, _, blocks = make_tq2(9300, N, K)
    x = _x(9301, M, K) * np.float32(1e-3)
    x[:, 7] = np.float32(9.0)
    W = L.upload_tq2(blocks, N, K)
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    plan = L.GemvPlan([(W, t.from_numpy(x).cuda(), None, y)], M)
    announce("tq2 plan longest rows", N, K, M)
    plan.run()
    t.cuda.synchronize()
    y_ref, tsum = oracle.tq2_gemv_f32(blocks, N, K, x, threads=TH)
    ok, worst = f32_tol_ok(y.cpu().numpy(), y_ref, tsum)
    assert ok, "worst error / bound %.3f" % worst


# ------------------------------------------------------------------ single calls: extreme activations
@pytest.mark.parametrize("fmt,M", [("i2s", 1), ("i2s", 2), ("i2s", 5), ("tq2", 1), ("tq2", 3)])
def test_gemv_f32_single_call_extreme_x(fmt, M):
    """The single-call fp32 engine (int8 planes; fused at M = 1) on
    activations at the ends of the fp32 range: every token subnormal
    (|x| < 2^-126), subnormals beside one normal element, elements near the
    largest finite fp32 (K and the scale keep y finite), and +-max|x|
    everywhere.  Every token of a call gets the same case."""
    t = torch()
    N, K = 70, 256 if fmt == "tq2" else 128
    rng = synth.rng(9300 + M)
    sign = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    cases = {
        "subnormal": (synth.normal_f32(9301, M, K) * np.float32(1e-41)).astype(np.float32),
        "subnormal_and_one_normal": None,
        "near_max": sign * np.float32(3.0e38) * rng.random((M, K)).astype(np.float32),
        "max_everywhere": sign * np.float32(2.5e37),
    }
    mixed = (synth.normal_f32(9302, M, K) * np.float32(1e-40)).astype(np.float32)
    mixed[:, 3] = np.float32(1.5e-30)
    cases["subnormal_and_one_normal"] = mixed
    if fmt == "i2s":
        _, _, packed = make_i2s(9310, N, K, scale=1e-3)
        W = L.upload_i2s(packed, N, K)
        fn = oracle.i2s_gemv_f32
    else:
        w = synth.ternary(9311, N, K)
        sc = np.full(N * K // 256, 0x1400, np.uint16)            # fp16 2^-10
        packed = L.ll_pack_tq2(w, sc)
        W = L.upload_tq2(packed, N, K)
        fn = oracle.tq2_gemv_f32
    for name, x in cases.items():
        assert np.isfinite(x).all()
        announce("single call extreme x", fmt, M, name)
        y = L.gemv(W, t.from_numpy(np.ascontiguousarray(x)).cuda()).cpu().numpy()
        y_ref, tsum = fn(packed, N, K, x)
        assert np.isfinite(y_ref).all() and (np.abs(y_ref) < 3.4e38).all()
        ok, worst = f32_tol_ok(y, y_ref, tsum)
        assert ok, "%s: worst error / bound %.3f" % (name, worst)
