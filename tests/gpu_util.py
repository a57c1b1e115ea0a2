"""Helpers for the GPU parity tests: seeded inputs (binary_bit_weight_amd.synth),
library calls through the C ABI (binary_bit_weight_amd.lowbit) and the CPU
oracle on the same inputs."""
import sys

import numpy as np

import oracle
from binary_bit_weight_amd import lowbit as L
from binary_bit_weight_amd import synth


TH = oracle.cores()        # host threads of the oracle on full-size comparisons


def torch():
    import torch as t
    return t


def announce(*parts):
    """Names the case about to touch the GPU (flushed before the launch)."""
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def f32_tol_ok(y_gpu, y_ref, tsum):
    """The fp32 bound |y_gpu - y_ref| <= 1e-5 * T + 1e-6 (T = scale * sum|x|
    for i2_s, sum_b |s_b| * sum_{k in b} |x| for TQ2_0)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = 1e-5 * tsum + 1e-6
    bad = err > bound
    return (not bad.any()), float((err / bound).max())


def relu2_mul_tol_ok(out_gpu, g_ref, tg, u_ref, tu):
    """Bound for out = (r * r) * u computed in fp32 from gate and up products
    that each meet the fp32 bound (eg = 1e-5 tg + 1e-6, eu likewise): with
    r = max(0, g) (1-Lipschitz), the product rule gives
    |out - r^2 u| <= (2 r + eg) eg (|u| + eu) + r^2 eu, plus the two fp32
    multiplies, each within 2^-24 relative: 2^-22 (r + eg)^2 (|u| + eu)."""
    eg = 1e-5 * tg + 1e-6
    eu = 1e-5 * tu + 1e-6
    r = np.maximum(g_ref, 0.0)
    ref = r * r * u_ref
    bound = (2 * r + eg) * eg * (np.abs(u_ref) + eu) + r * r * eu + 2.0 ** -22 * (r + eg) ** 2 * (np.abs(u_ref) + eu)
    err = np.abs(out_gpu.astype(np.float64) - ref)
    return (not (err > bound).any()), float((err / bound).max())


def make_i2s(seed, N, K, scale=None, p0=0.4):
    w = synth.ternary(seed, N, K, p0)
    if scale is None:
        scale = float(synth.uniform_f32(seed + 1, 1, 0.01, 0.1)[0])
    packed = L.ll_pack_i2s(w, scale)
    return w, np.float32(scale), packed


def make_tq2(seed, N, K):
    w = synth.ternary(seed, N, K)
    sc = synth.uniform_f16_bits(seed + 1, N * K // 256, 0.005, 0.05)
    blocks = L.ll_pack_tq2(w, sc)
    return w, sc, blocks


_W1_CACHE = {}


def make_w1(seed, N, K, G):
    """Binary weights of the W1A8 recipe: dense N(0, 0.02) rows (generated in
    4096-row chunks) -> ll_w1_from_dense (sign bits, fp16 group mean-abs
    scales).  Returns (bits uint32 [N, K/32], scales uint16 [N, K/G]); cached
    per process for the large shapes."""
    key = (seed, N, K, G)
    if key in _W1_CACHE:
        return _W1_CACHE[key]
    bits = np.empty((N, K // 32), np.uint32)
    scales = np.empty((N, K // G), np.uint16)
    for c in range((N + synth.CHUNK_ROWS - 1) // synth.CHUNK_ROWS):
        r0 = c * synth.CHUNK_ROWS
        rows = min(synth.CHUNK_ROWS, N - r0)
        b, s = L.ll_w1_from_dense(synth.dense_chunk(seed, K, c, rows), G)
        bits[r0:r0 + rows], scales[r0:r0 + rows] = b, s
    if N * K >= 1 << 26:
        _W1_CACHE[key] = (bits, scales)
    return bits, scales
