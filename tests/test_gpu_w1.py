"""GPU parity of the W1A8 path (binary sign-bit weights, fp16 group scales,
int8 per-token activations) against the CPU oracle: bit-exact, every element
of the small shapes and of the full workload shapes (hidden 5120, G = 128,
N = 7168 / 17408 / 248320, M = 1 and 8), the oracle's rows split over every
host core for the latter."""
import numpy as np
import pytest

import oracle
from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth
from gpu_util import TH, announce, make_w1, torch

pytestmark = pytest.mark.gpu


def _acts(seed, M, K):
    """int8 activations and per-token scales from the oracle's quantizer."""
    return oracle.quantize_f32(synth.normal_f32(seed, M, K))


def _run(bits, scales, K, G, q, s, bias=None, rows=None, use_gemm=False):
    t = torch()
    W = L.upload_w1(bits, scales, K, G)
    xq = t.from_numpy(q).cuda()
    xs = t.from_numpy(s).cuda()
    b = None if bias is None else t.from_numpy(bias).cuda()
    if use_gemm:
        y, _ = L.gemm(W, xq, xs, bias=b)
    else:
        y = L.gemv(W, xq, xs, bias=b)
    y = y.cpu().numpy()
    y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s, bias=bias, rows=rows, threads=TH)
    if rows is not None:
        y = y[:, rows]
    return y, y_ref


# (N, K, G, M): ragged row counts (the workgroup covers 128 rows), every group
# size, token counts that need one or two A row blocks and several passes, and
# every number of units packed into one accumulator (8, 4, 2) with the last
# packed set of the matrix cut short by the end of K
W1_SMALL = [(37, 128, 128, 1), (64, 256, 32, 3), (100, 512, 64, 8), (130, 1024, 128, 16), (7, 384, 128, 2),
            (33, 2048, 256, 5), (250, 1152, 32, 4), (16, 5120, 128, 8), (129, 640, 64, 1), (40, 256, 256, 1),
            (300, 1280, 64, 9), (90, 2304, 32, 11), (50, 1152, 128, 4), (77, 1536, 128, 3), (45, 640, 32, 1),
            (61, 896, 64, 2), (23, 768, 256, 2), (140, 2944, 128, 1)]


@pytest.mark.parametrize("N,K,G,M", W1_SMALL)
def test_w1a8_small_bitexact(N, K, G, M):
    bits, scales = make_w1(5000 + N + G, N, K, G)
    q, s = _acts(5100 + M + K, M, K)
    bias = synth.uniform_f32(5200 + N, N, -1, 1) if M == 3 else None
    announce("w1a8 small", N, K, G, M)
    y, y_ref = _run(bits, scales, K, G, q, s, bias=bias)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), \
        "mismatches: %d" % int((y.view(np.uint32) != y_ref.view(np.uint32)).sum())


@pytest.mark.parametrize("N,K,G,M", [(70, 1024, 64, 40), (20, 512, 32, 9), (129, 2560, 256, 33)])
def test_w1a8_gemm_passes_bitexact(N, K, G, M):
    """ll_bitlinear_gemm with W1 and a group size other than 128: M above one
    pass of tokens, exact fp64 group scaling."""
    bits, scales = make_w1(5300 + N, N, K, G)
    q, s = _acts(5400 + M, M, K)
    announce("w1a8 gemm", N, K, G, M)
    y, y_ref = _run(bits, scales, K, G, q, s, use_gemm=True)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


def _w1_bound(scales, K, G, q, s, rows=None):
    """T = s_tok * sum_g |s_g| * sum_{k in g} |q_k| for the fp32 bound of the
    matrix-core path (group scaling in fp32)."""
    sg = np.abs(scales.view(np.float16).astype(np.float64))
    if rows is not None:
        sg = sg[rows]
    qa = np.abs(q.astype(np.float64)).reshape(q.shape[0], K // G, G).sum(axis=2)
    return s.astype(np.float64)[:, None] * (qa @ sg.T)


# G = 128 above 16 tokens: the int8 matrix cores.  Ragged tiles, five groups
# (K = 640), a bias, and split K: (5, 2560, 300) two ways, (64, 4096, 40)
# three uneven ways (10 + 11 + 11 groups), (64, 5376, 40) four uneven ways;
# (300, 2048, 200) and (257, 1664, 130) unsplit.
@pytest.mark.parametrize("N,K,M", [(70, 1024, 40), (200, 640, 17), (130, 1280, 129), (5, 2560, 300), (64, 4096, 40),
                                   (300, 2048, 200), (257, 1664, 130), (64, 5376, 40)])
def test_w1a8_gemm_mfma_within_bound(N, K, M):
    G = 128
    bits, scales = make_w1(5600 + N, N, K, G)
    q, s = _acts(5700 + M, M, K)
    bias = synth.uniform_f32(5800 + N, N, -1, 1) if M == 129 else None
    announce("w1a8 gemm mfma", N, K, M)
    t = torch()
    W = L.upload_w1(bits, scales, K, G)
    outs = []
    for _ in range(2 if K >= 1664 else 1):
        y, _ = L.gemm(W, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), bias=None if bias is None else t.from_numpy(bias).cuda())
        outs.append(y.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), "repeated calls differ"
    y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s, bias=bias)
    bound = 1e-5 * _w1_bound(scales, K, G, q, s) + 1e-6
    err = np.abs(outs[0].astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= bound).all(), "worst error / bound %.3f" % float((err / bound).max())


def test_w1a8_gemm_mfma_gate_full():
    """The gate shape (17408 x 5120, G = 128) at M = 512 on the matrix cores,
    every output."""
    N, K, G, M = 17408, 5120, 128, 512
    bits, scales = make_w1(5900, N, K, G)
    q, s = _acts(5901, M, K)
    announce("w1a8 gemm mfma gate")
    t = torch()
    W = L.upload_w1(bits, scales, K, G)
    y, _ = L.gemm(W, t.from_numpy(q).cuda(), t.from_numpy(s).cuda())
    y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s, threads=TH)
    bound = 1e-5 * _w1_bound(scales, K, G, q, s) + 1e-6
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= bound).all(), "worst error / bound %.3f" % float((err / bound).max())


@pytest.mark.parametrize("N,M", [(7168, 1), (7168, 8), (17408, 1), (17408, 8), (248320, 1), (248320, 8)])
def test_w1a8_full_shapes(N, M):
    K, G = 5120, 128
    bits, scales = make_w1(501 if N == 7168 else 502 if N == 17408 else 503, N, K, G)
    q, s = _acts(510 + M, M, K)
    announce("w1a8 full", N, M)
    y, y_ref = _run(bits, scales, K, G, q, s)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


def test_w1a8_end_to_end_from_fp32():
    """fp32 x -> ll_quantize_act on the GPU -> W1 product, against the oracle's
    quantizer and product."""
    t = torch()
    N, K, G, M = 200, 1024, 128, 8
    bits, scales = make_w1(5500, N, K, G)
    x = synth.normal_f32(5501, M, K)
    announce("w1a8 end to end")
    xq, xs = L.quantize(t.from_numpy(x).cuda())
    W = L.upload_w1(bits, scales, K, G)
    y = L.gemv(W, xq, xs).cpu().numpy()
    q, s = oracle.quantize_f32(x)
    y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("G", [32, 128])
def test_w1a8_extreme_and_zero_tokens(G):
    """Tokens at +-127 everywhere (largest digits of the activation split), a
    token of all zeros with scale 0 (y = bias exactly), alternating signs."""
    N, K, M = 150, 768, 4
    bits, scales = make_w1(5600 + G, N, K, G)
    q = np.empty((M, K), np.int8)
    q[0] = 127
    q[1] = -127
    q[2] = 0
    q[3] = np.where(np.arange(K) % 2 == 0, 127, -128 + 1).astype(np.int8)
    s = np.array([0.5, 0.25, 0.0, 1.0], np.float32)
    bias = synth.uniform_f32(5601, N, -1, 1)
    announce("w1a8 extremes", G)
    y, y_ref = _run(bits, scales, K, G, q, s, bias=bias)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
    assert np.array_equal(y[2], bias)


def test_w1a8_unit_scales_integer_result():
    """Unit group scales and unit token scale: y is the exact integer dot."""
    N, K, G, M = 64, 512, 128, 2
    rng = synth.rng(5700)
    bits = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = np.full((N, K // G), 0x3C00, np.uint16)          # fp16 1.0
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    s = np.ones(M, np.float32)
    announce("w1a8 unit scales")
    y, y_ref = _run(bits, scales, K, G, q, s)
    w = L.ll_unpack_w1(bits, K).astype(np.int64)
    exact = (q.astype(np.int64) @ w.T).astype(np.float32)
    assert np.array_equal(y, exact) and np.array_equal(y_ref, exact)


@pytest.mark.parametrize("M,K", [(1, 5120), (8, 5120), (8, 8192)])
def test_w1a8_split_workspace_reuse(M, K):
    """A narrow matrix splits K: K = 5120 streams, its windows split over the
    waves of a workgroup; K = 8192 at M = 8 (an A operand too large for the
    streaming product) splits K over workgroups, with partial sums and
    per-row-block counters in the workspace.  Three calls in a row on one
    zero-filled workspace, with new activations each time, stay bit-exact
    (the counters are left zero by every call)."""
    t = torch()
    N, G = 300, 128
    bits, scales = make_w1(5800 + M, N, K, G)
    W = L.upload_w1(bits, scales, K, G)
    nws = L.ll_gemv_workspace_size(W, L.LL_ACT_I8, M)
    ws = t.zeros((nws,), dtype=t.uint8, device="cuda")
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    for rnd in range(3):
        q, s = _acts(5810 + 10 * M + rnd, M, K)
        announce("w1a8 split reuse", M, rnd)
        L.ll_bitlinear_gemv(W, L.LL_ACT_I8, t.from_numpy(q).cuda(), t.from_numpy(s).cuda(), M, None, y, ws)
        y_ref, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), rnd


def _plan_case(shapes, M, seed, bias_at=()):
    """Runs a W1A8 prepared batch twice (the second time with new activation
    contents and scales in the same buffers) and compares every output with
    the oracle bit for bit.  shapes: (N, K, activation slot)."""
    t = torch()
    acts, items, refs = {}, [], []
    for i, (N, K, slot) in enumerate(shapes):
        bits, scales = make_w1(seed + i, N, K, 128)
        W = L.upload_w1(bits, scales, K, 128)
        if slot not in acts:
            q, s = _acts(seed + 100 + slot, M, K)
            acts[slot] = [q, s, t.from_numpy(q).cuda(), t.from_numpy(s).cuda()]
        b = synth.uniform_f32(seed + 200 + i, N, -1, 1) if i in bias_at else None
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        a = acts[slot]
        items.append((W, a[2], a[3], None if b is None else t.from_numpy(b).cuda(), y))
        refs.append((bits, scales, K, slot, b))
    plan = L.GemvPlanI8(items, M)
    for rnd in range(2):
        if rnd == 1:
            for slot, a in acts.items():
                q, s = _acts(seed + 300 + slot, M, a[0].shape[1])
                a[2].copy_(t.from_numpy(q))
                a[3].copy_(t.from_numpy(s))
                a[0], a[1] = q, s
        announce("w1a8 plan", M, len(shapes), rnd)
        plan.run()
        t.cuda.synchronize()
        for (W, _, _, _, y), (bits, scales, K, slot, b) in zip(items, refs):
            y_ref, _ = oracle.w1a8_gemm(bits, scales, K, 128, acts[slot][0], acts[slot][1], bias=b, threads=TH)
            got = y.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), y_ref.view(np.uint32)), \
                "N=%d K=%d round %d: %d mismatches" % (W.N, K, rnd, int((got.view(np.uint32) != y_ref.view(np.uint32)).sum()))


# every token count (packed units 8 / 4 / 2 / 1); with scv every K is a multiple of 1024 (row-vector scale
# loads), else one K = 1152 ends in a cut window; ragged N (37, 130, 300, 1000) and a 16-row matrix
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("scv", [True, False])
def test_w1a8_plan_matches_oracle(M, scv):
    shapes = [(300, 5120, 0), (37, 5120, 0), (1000, 2048, 1), (16, 1024, 2)]
    shapes += [] if scv else [(130, 1152, 3), (20, 128, 4)]
    shapes += [(50, 17408, 5)] if M <= 2 else []
    _plan_case(shapes, M, 6000 + 10 * M + int(scv), bias_at=(1, 3))


def test_w1a8_plan_decode_layer():
    """One decoder layer of the hidden-5120 shapes as one batch at M = 1: QKV
    7168, O 5120, gate and up 17408 (one activation), down 5120 x 17408."""
    shapes = [(7168, 5120, 0), (5120, 5120, 1), (17408, 5120, 2), (17408, 5120, 2), (5120, 17408, 3)]
    _plan_case(shapes, 1, 6500)


@pytest.mark.parametrize("M", [1, 2])
def test_w1a8_plan_decode_layers_streamed(M):
    """Four decoder layers in one batch: more workgroups than the device holds
    at once, so most products get fewer workgroups than blocks and each wave
    streams several blocks back to back.  The layers share weights and
    activations (separate device copies), so every layer's outputs equal the
    oracle's of the first; every output is compared bit for bit."""
    t = torch()
    shapes = [(7168, 5120, 0), (5120, 5120, 1), (17408, 5120, 2), (17408, 5120, 2), (5120, 17408, 3)]
    acts, host, items = {}, [], []
    for i, (N, K, slot) in enumerate(shapes):
        bits, scales = make_w1(6600 + i, N, K, 128)
        if slot not in acts:
            q, s = _acts(6700 + slot, M, K)
            acts[slot] = (q, s, t.from_numpy(q).cuda(), t.from_numpy(s).cuda())
        host.append((bits, scales, K, slot))
    outs = []
    for layer in range(4):
        for i, (N, K, slot) in enumerate(shapes):
            bits, scales, _, _ = host[i]
            y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
            items.append((L.upload_w1(bits, scales, K, 128), acts[slot][2], acts[slot][3], None, y))
            outs.append((i, y))
    plan = L.GemvPlanI8(items, M)
    assert plan.plan.tiles < sum((N + 255) // 256 for N, _, _ in shapes) * 4    # fewer workgroups than blocks / 8
    announce("w1a8 plan 4 layers", M)
    plan.run()
    t.cuda.synchronize()
    refs = [oracle.w1a8_gemm(b, sc, K, 128, acts[slot][0], acts[slot][1], threads=TH)[0] for b, sc, K, slot in host]
    for i, y in outs:
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), refs[i].view(np.uint32)), \
            "product %d: %d mismatches" % (i, int((got.view(np.uint32) != refs[i].view(np.uint32)).sum()))
