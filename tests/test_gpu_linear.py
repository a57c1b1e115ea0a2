"""GPU parity of the one-shot bf16 layer, ll_binary_linear (bf16 x -> per-token
int8 quantization -> the format's int8 product -> bias in fp32 -> bf16 y,
rounded to nearest with ties to even), against the oracle's quantize_bf16,
its int8 product and f32_to_bf16.  i2_s and W1 products are bit-exact in
fp32, so their bf16 outputs must match bit for bit; TQ2_0 (fp32 block
scaling) must lie within its fp32 bound plus half a bf16 ulp."""
import numpy as np
import pytest

import oracle
from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth
from gpu_util import TH, announce, make_i2s, make_tq2, make_w1, torch

pytestmark = pytest.mark.gpu


def _bf16_dev(xb):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(t.bfloat16)


def _bits(y):
    t = torch()
    return y.view(t.int16).cpu().numpy().view(np.uint16)


def _bias(seed, N, on):
    if not on:
        return None, None
    b = synth.uniform_f32(seed, N, -1, 1)
    return b, torch().from_numpy(b).cuda()


# ragged rows and tokens, one token, a bias, split K (300 x 2048 at M = 200: four ways)
@pytest.mark.parametrize("N,K,M,with_bias", [(200, 512, 17, False), (77, 384, 1, True), (130, 1280, 129, True),
                                             (300, 2048, 200, False)])
def test_binary_linear_i2s_bitexact(N, K, M, with_bias):
    w, scale, packed = make_i2s(7000 + N, N, K)
    xb = synth.normal_bf16_bits(7100 + M, M, K)
    b, bd = _bias(7200 + N, N, with_bias)
    W = L.upload_i2s(packed, N, K)
    announce("binary_linear i2s", N, K, M)
    y = _bits(L.binary_linear(W, _bf16_dev(xb), bias=bd))
    q, s = oracle.quantize_bf16(xb)
    y32, _ = oracle.i2s_gemm_i8(packed, N, K, q, s)
    if b is not None:
        y32 = (y32 + b[None, :]).astype(np.float32)
    assert np.array_equal(y, oracle.f32_to_bf16(y32))


def test_binary_linear_i2s_prefill_full():
    N, K, M = 6912, 2560, 512
    w, scale, packed = make_i2s(7300, N, K)
    xb = synth.normal_bf16_bits(7301, M, K)
    W = L.upload_i2s(packed, N, K)
    announce("binary_linear i2s full")
    y = _bits(L.binary_linear(W, _bf16_dev(xb)))
    q, s = oracle.quantize_bf16(xb)
    y32, _ = oracle.i2s_gemm_i8(packed, N, K, q, s, threads=TH)
    assert np.array_equal(y, oracle.f32_to_bf16(y32))


# W1 with the binary-gemm card's shapes scaled down: one pass, several passes of 16 tokens, G = 32 / 128
@pytest.mark.parametrize("N,K,G,M,with_bias", [(100, 512, 128, 8, True), (70, 1024, 32, 40, False),
                                               (129, 2560, 128, 3, False)])
def test_binary_linear_w1_bitexact(N, K, G, M, with_bias):
    bits, scales = make_w1(7400 + N, N, K, G)
    xb = synth.normal_bf16_bits(7500 + M, M, K)
    b, bd = _bias(7600 + N, N, with_bias)
    W = L.upload_w1(bits, scales, K, G)
    announce("binary_linear w1", N, K, G, M)
    y = _bits(L.binary_linear(W, _bf16_dev(xb), bias=bd))
    q, s = oracle.quantize_bf16(xb)
    y32, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s, bias=b)
    assert np.array_equal(y, oracle.f32_to_bf16(y32))


# W1 with G = 128 above 16 tokens: the int8 matrix cores with fp32 group
# scaling and the bf16 rounding in their epilogue; (300, 2048, 200) splits K
# four ways, (130, 1280, 129) has ragged tiles and a bias
@pytest.mark.parametrize("N,K,M,with_bias", [(300, 2048, 200, False), (130, 1280, 129, True)])
def test_binary_linear_w1_mfma_within_bound(N, K, M, with_bias):
    G = 128
    bits, scales = make_w1(7450 + N, N, K, G)
    xb = synth.normal_bf16_bits(7550 + M, M, K)
    b, bd = _bias(7650 + N, N, with_bias)
    W = L.upload_w1(bits, scales, K, G)
    announce("binary_linear w1 mfma", N, K, M)
    y = _bits(L.binary_linear(W, _bf16_dev(xb), bias=bd))
    yv = np.array([oracle.bf16_to_f32(int(v)) for v in y.reshape(-1)], np.float64).reshape(y.shape)
    q, s = oracle.quantize_bf16(xb)
    y_ref, S = oracle.w1a8_gemm(bits, scales, K, G, q, s, bias=b, threads=TH)
    # fp32 bound of the matrix-core path (T = s_tok sum_g |s_g| sum_{k in g} |q|), then half a bf16 ulp
    sg = np.abs(scales.view(np.float16).astype(np.float64))
    qa = np.abs(q.astype(np.float64)).reshape(M, K // G, G).sum(axis=2)
    tsum = s.astype(np.float64)[:, None] * (qa @ sg.T)
    exact = s.astype(np.float64)[:, None] * S + (0.0 if b is None else b.astype(np.float64)[None, :])
    bound = 1e-5 * tsum + 1e-6 + np.abs(exact) * 2.0 ** -8 + 2.0 ** -24 * np.abs(exact)
    assert (np.abs(yv - exact) <= bound).all(), "worst %.3f" % float((np.abs(yv - exact) / bound).max())
    assert y_ref.shape == y.shape


@pytest.mark.parametrize("N,K,M", [(150, 768, 33), (64, 2048, 5)])
def test_binary_linear_tq2_within_bound(N, K, M):
    w, sc, blocks = make_tq2(7700 + N, N, K)
    xb = synth.normal_bf16_bits(7800 + M, M, K)
    W = L.upload_tq2(blocks, N, K)
    announce("binary_linear tq2", N, K, M)
    y = _bits(L.binary_linear(W, _bf16_dev(xb)))
    yv = np.array([oracle.bf16_to_f32(int(v)) for v in y.reshape(-1)], np.float64).reshape(y.shape)
    q, s = oracle.quantize_bf16(xb)
    y_ref, tsum = oracle.tq2_gemm_i8(blocks, N, K, q, s)
    bound = 1e-5 * tsum + 1e-6 + np.abs(y_ref) * 2.0 ** -8      # fp32 bound, then half a bf16 ulp
    assert (np.abs(yv - y_ref) <= bound).all()


def test_binary_linear_workspace_reuse():
    """Two calls sharing one workspace (zero-filled once; split K leaves its
    counters zero), the second with other activations: both exact."""
    t = torch()
    N, K, M = 2560, 6912, 256
    w, scale, packed = make_i2s(7900, N, K)
    W = L.upload_i2s(packed, N, K)
    ws = t.zeros((L.ll_binary_linear_workspace_size(W, M),), dtype=t.uint8, device="cuda")
    for rnd in range(2):
        xb = synth.normal_bf16_bits(7902 + rnd, M, K)
        announce("binary_linear workspace reuse", rnd)
        y = _bits(L.binary_linear(W, _bf16_dev(xb), workspace=ws))
        q, s = oracle.quantize_bf16(xb)
        y32, _ = oracle.i2s_gemm_i8(packed, N, K, q, s, threads=TH)
        assert np.array_equal(y, oracle.f32_to_bf16(y32)), rnd
