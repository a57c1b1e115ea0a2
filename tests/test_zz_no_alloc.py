"""The allocation-free product ll_bitlinear_gemm_noalloc (static device
scratch) against ll_bitlinear_gemm with its own zero-filled workspace, bit
for bit (the fp32 paths run the same kernels in the same order, so their
bits agree too), through the C ABI, on calls in a row that leave the
scratch holding the previous call's contents:
  1. i2_s 2560 x 6912 at M = 256: 128 x 64 tiles split K three ways
     (partial tiles and counters in the scratch), acc_out too;
  2. i2_s 300 x 2048 at M = 200, smaller: four splits, other tile counts;
  3. W1 with G = 64 at M = 40: passes of 16 tokens whose prepared operands
     live in the scratch;
  4. TQ2_0 257 x 1792 at M = 130: three uneven splits of whole blocks.
Also: a product whose scratch need exceeds the array is refused before any
launch, with LL_EWORKSPACE."""
import ctypes as C

import numpy as np
import pytest

import oracle
from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth
from gpu_util import announce, make_i2s, make_tq2, make_w1, torch

pytestmark = pytest.mark.gpu


def _pair(W, q, s, M, N, want_acc):
    t = torch()
    xq, xs = t.from_numpy(q).cuda(), t.from_numpy(s).cuda()
    y_ref = t.empty((M, N), dtype=t.float32, device="cuda")
    y_new = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    a_ref = t.empty((M, N), dtype=t.int32, device="cuda") if want_acc else None
    a_new = t.full((M, N), -7, dtype=t.int32, device="cuda") if want_acc else None
    nws = L.ll_gemm_workspace_size(W, M)
    ws = t.zeros((max(nws, 16),), dtype=t.uint8, device="cuda")
    L.ll_bitlinear_gemm(W, xq, xs, M, None, y_ref, a_ref, ws)
    L.ll_bitlinear_gemm_noalloc(W, xq, xs, M, None, y_new, a_new)
    t.cuda.synchronize()
    assert nws <= L.ll_gemm_noalloc_scratch_bytes()
    assert np.array_equal(y_new.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))
    if want_acc:
        assert np.array_equal(a_new.cpu().numpy(), a_ref.cpu().numpy())
    return y_new.cpu().numpy()


def test_noalloc_matches_workspace_product():
    # 1: large split-K i2_s product
    N, K, M = 2560, 6912, 256
    _, _, packed = make_i2s(402, N, K)
    W = L.upload_i2s(packed, N, K)
    q, s = oracle.quantize_bf16(synth.normal_bf16_bits(9500, M, K))
    announce("noalloc i2s", N, K, M)
    assert L.ll_gemm_workspace_size(W, M) > 4096          # the scratch holds partial tiles
    y = _pair(W, q, s, M, N, True)
    rows = synth.sample_rows(9501, N, 16)
    y_or, _ = oracle.i2s_gemm_i8(packed, N, K, q, s, rows, threads=oracle.cores())
    assert np.array_equal(y[:, rows].view(np.uint32), y_or.view(np.uint32))
    # 2: smaller i2_s product on the same scratch
    N, K, M = 300, 2048, 200
    _, _, packed = make_i2s(9502, N, K)
    W = L.upload_i2s(packed, N, K)
    q, s = oracle.quantize_bf16(synth.normal_bf16_bits(9503, M, K))
    announce("noalloc i2s small", N, K, M)
    y = _pair(W, q, s, M, N, True)
    y_or, _ = oracle.i2s_gemm_i8(packed, N, K, q, s)
    assert np.array_equal(y.view(np.uint32), y_or.view(np.uint32))
    # 3: W1 passes (G = 64) with prepared operands in the scratch
    N, K, G, M = 70, 1024, 64, 40
    bits, scales = make_w1(9504, N, K, G)
    W = L.upload_w1(bits, scales, K, G)
    q, s = oracle.quantize_f32(synth.normal_f32(9505, M, K))
    announce("noalloc w1", N, K, G, M)
    y = _pair(W, q, s, M, N, False)
    y_or, _ = oracle.w1a8_gemm(bits, scales, K, G, q, s)
    assert np.array_equal(y.view(np.uint32), y_or.view(np.uint32))
    # 4: TQ2_0, three uneven splits
    N, K, M = 257, 1792, 130
    _, _, blocks = make_tq2(9506, N, K)
    W = L.upload_tq2(blocks, N, K)
    q, s = oracle.quantize_bf16(synth.normal_bf16_bits(9507, M, K))
    announce("noalloc tq2", N, K, M)
    _pair(W, q, s, M, N, False)


def test_noalloc_refuses_beyond_the_scratch():
    """W1 passes of 4 tokens with G = 32 at K = 2^20 need 32 MiB of prepared
    operands plus group sums: more than the scratch, refused with
    LL_EWORKSPACE (nothing launched, no device pointer touched)."""
    w = L.ll_weights(L.LL_FMT_W1, 32, 64, 1 << 20, C.c_void_p(0x10000), C.c_void_p(0x10000))
    assert L.lib().ll_gemm_workspace_size(C.byref(w), 16) > L.ll_gemm_noalloc_scratch_bytes()
    rc = L.lib().ll_bitlinear_gemm_noalloc(C.byref(w), C.c_void_p(0x10000), C.c_void_p(0x10000), 16, None,
                                          C.c_void_p(0x10000), None, None)
    assert rc == -5
    assert b"static scratch" in L.lib().ll_last_error()
