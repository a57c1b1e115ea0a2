"""CPU oracle for the packed low-bit BitLinear product -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct reference implementations (``oracle.c``,
accumulating in int64 / fp64), wrapped for numpy.  Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library never imports it, and it imports
nothing from the product library.

Functions whose result is not pinned to an external fact are listed in the
module docstring of ``tests/test_oracle_pins.py`` as "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no contraction, no fast-math).

    ORACLE_LIB_OVERRIDE names an already built library to load instead; the
    mutant test uses it to load oracles with planted mistakes."""
    override = os.environ.get("ORACLE_LIB_OVERRIDE")
    if override:
        return override
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        P = C.c_void_p
        I64 = C.c_int64
        sig = {
            "orc_f16_to_f64": (C.c_double, [C.c_uint16]),
            "orc_f64_to_f16": (C.c_uint16, [C.c_double]),
            "orc_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_f32_to_bf16": (C.c_uint16, [C.c_float]),
            "orc_i2s_encode": (C.c_int, [P, I64, I64, C.c_float, P]),
            "orc_i2s_decode": (I64, [P, I64, I64, P, P]),
            "orc_i2s_gemv_f32": (None, [P, I64, I64, P, I64, P, I64, P, P]),
            "orc_i2s_gemm_i8": (None, [P, I64, I64, P, P, I64, P, I64, P, P]),
            "orc_tq2_encode": (C.c_int, [P, P, I64, I64, P]),
            "orc_tq2_decode": (I64, [P, I64, I64, P, P]),
            "orc_tq2_gemv_f32": (None, [P, I64, I64, P, I64, P, I64, P, P]),
            "orc_tq2_gemm_i8": (None, [P, I64, I64, P, P, I64, P, I64, P, P]),
            "orc_w1_encode": (C.c_int, [P, I64, I64, P]),
            "orc_w1_decode": (None, [P, I64, I64, P]),
            "orc_w1_from_dense": (C.c_int, [P, I64, I64, C.c_int32, P, P]),
            "orc_w1a8_gemm": (I64, [P, P, I64, I64, C.c_int32, P, P, I64, P, P, I64, P, P]),
            "orc_quantize_f32": (None, [P, I64, I64, P, P]),
            "orc_quantize_bf16": (None, [P, I64, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(_lib, name)
            f.restype = res
            f.argtypes = args
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def cores() -> int:
    """Host threads of the all-core runs: the CPUs this process may use, at
    most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _by_rows(call, rows, N, threads):
    """All-core form of a product: call(sub) evaluates the output rows `sub`
    (int64 indices; None = all N rows) and returns arrays of shape
    [M, len(sub)].  With threads > 1 the rows are cut into that many
    contiguous slices, each evaluated by the same C function on its own
    thread (ctypes releases the GIL for the call), and the results are
    joined along the row axis.  Only the partition differs from a single
    call: every output comes from the same scalar loop."""
    if threads is None or threads <= 1:
        return call(None if rows is None else _c(rows, np.int64))
    r = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    parts = [p for p in np.array_split(r, min(threads, max(1, r.size))) if p.size]
    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(call, parts))
    return tuple(np.concatenate([part[i] for part in res], axis=1) for i in range(len(res[0])))


def _rows(rows, N):
    if rows is None:
        return None, N
    r = _c(rows, np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < N))
    return r, r.size


# ---------------------------------------------------------------- scalars
def f16_to_f64(h: int) -> float:
    return lib().orc_f16_to_f64(int(h))


def f64_to_f16(v: float) -> int:
    return lib().orc_f64_to_f16(float(v))


def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(int(b))


def f32_to_bf16(y):
    """bf16 bits (round to nearest, ties to even) of every fp32 value of y."""
    y = np.asarray(y, np.float32)
    f = lib().orc_f32_to_bf16
    return np.array([f(float(v)) for v in y.reshape(-1)], np.uint16).reshape(y.shape)


# ---------------------------------------------------------------- i2_s
def i2s_encode(w: np.ndarray, scale: float) -> np.ndarray:
    w = _c(w, np.int8)
    N, K = w.shape
    out = np.zeros(N * K // 4 + 4, np.uint8)
    rc = lib().orc_i2s_encode(_p(w), N, K, float(scale), _p(out))
    if rc:
        raise ValueError("orc_i2s_encode: %d" % rc)
    return out


def i2s_decode(packed: np.ndarray, N: int, K: int):
    packed = _c(packed, np.uint8)
    assert packed.size == N * K // 4 + 4
    w = np.empty((N, K), np.int8)
    s = np.zeros(1, np.float32)
    bad = lib().orc_i2s_decode(_p(packed), N, K, _p(w), _p(s))
    return w, float(s[0]), int(bad)


def i2s_gemv_f32(packed, N, K, x, rows=None, threads=None):
    """y[m, i] = scale * sum_k w[rows[i], k] * x[m, k] in fp64; also T.
    threads: rows split over that many host threads (_by_rows)."""
    packed = _c(packed, np.uint8)
    x = _c(np.atleast_2d(x), np.float32)
    M = x.shape[0]
    assert x.shape[1] == K

    def one(sub):
        r, nr = _rows(sub, N)
        y = np.empty((M, nr), np.float64)
        t = np.empty((M, nr), np.float64)
        lib().orc_i2s_gemv_f32(_p(packed), N, K, _p(x), M, _p(r), nr, _p(y), _p(t))
        return y, t
    return _by_rows(one, rows, N, threads)


def i2s_gemm_i8(packed, N, K, q, s_tok, rows=None, threads=None):
    packed = _c(packed, np.uint8)
    q = _c(np.atleast_2d(q), np.int8)
    s_tok = _c(s_tok, np.float32)
    M = q.shape[0]

    def one(sub):
        r, nr = _rows(sub, N)
        y = np.empty((M, nr), np.float32)
        acc = np.empty((M, nr), np.int64)
        lib().orc_i2s_gemm_i8(_p(packed), N, K, _p(q), _p(s_tok), M, _p(r), nr, _p(y), _p(acc))
        return y, acc
    return _by_rows(one, rows, N, threads)


# ---------------------------------------------------------------- TQ2_0
def tq2_encode(w, scales_f16_bits):
    w = _c(w, np.int8)
    N, K = w.shape
    sc = _c(scales_f16_bits, np.uint16)
    if K % 256 or sc.size != N * K // 256:
        raise ValueError("TQ2_0 needs K % 256 == 0 and one scale per block")
    out = np.zeros(66 * N * K // 256, np.uint8)
    rc = lib().orc_tq2_encode(_p(w), _p(sc), N, K, _p(out))
    if rc:
        raise ValueError("orc_tq2_encode: %d" % rc)
    return out


def tq2_decode(blocks, N, K):
    blocks = _c(blocks, np.uint8)
    assert blocks.size == 66 * N * K // 256
    w = np.empty((N, K), np.int8)
    sc = np.empty(N * K // 256, np.uint16)
    bad = lib().orc_tq2_decode(_p(blocks), N, K, _p(w), _p(sc))
    return w, sc, int(bad)


def tq2_gemv_f32(blocks, N, K, x, rows=None, threads=None):
    blocks = _c(blocks, np.uint8)
    x = _c(np.atleast_2d(x), np.float32)
    M = x.shape[0]

    def one(sub):
        r, nr = _rows(sub, N)
        y = np.empty((M, nr), np.float64)
        t = np.empty((M, nr), np.float64)
        lib().orc_tq2_gemv_f32(_p(blocks), N, K, _p(x), M, _p(r), nr, _p(y), _p(t))
        return y, t
    return _by_rows(one, rows, N, threads)


def tq2_gemm_i8(blocks, N, K, q, s_tok, rows=None, threads=None):
    """int8 activations q [M, K] with scales s_tok [M] against TQ2_0 blocks:
    y = s_tok * sum_b s_b * sum_{k in b} w q in fp64 (exact integer block
    sums), and T = s_tok * sum_b |s_b| * sum_{k in b} |q|, both [M, len(rows)]."""
    blocks = _c(blocks, np.uint8)
    q = _c(np.atleast_2d(q), np.int8)
    s_tok = _c(s_tok, np.float32)
    M = q.shape[0]
    assert q.shape[1] == K and s_tok.size == M

    def one(sub):
        r, nr = _rows(sub, N)
        y = np.empty((M, nr), np.float64)
        t = np.empty((M, nr), np.float64)
        lib().orc_tq2_gemm_i8(_p(blocks), N, K, _p(q), _p(s_tok), M, _p(r), nr, _p(y), _p(t))
        return y, t
    return _by_rows(one, rows, N, threads)


# ---------------------------------------------------------------- W1
def w1_encode(w):
    w = _c(w, np.int8)
    N, K = w.shape
    out = np.zeros((N, K // 32), np.uint32)
    rc = lib().orc_w1_encode(_p(w), N, K, _p(out))
    if rc:
        raise ValueError("orc_w1_encode: %d" % rc)
    return out


def w1_decode(bits, K):
    bits = _c(bits, np.uint32)
    N = bits.shape[0]
    w = np.empty((N, K), np.int8)
    lib().orc_w1_decode(_p(bits), N, K, _p(w))
    return w


def w1_from_dense(W, G):
    W = _c(W, np.float32)
    N, K = W.shape
    bits = np.zeros((N, K // 32), np.uint32)
    sc = np.zeros((N, K // G), np.uint16)
    rc = lib().orc_w1_from_dense(_p(W), N, K, int(G), _p(bits), _p(sc))
    if rc:
        raise ValueError("orc_w1_from_dense: %d" % rc)
    return bits, sc


def w1a8_gemm(bits, scales, K, G, q, s_tok, bias=None, rows=None, threads=None):
    bits = _c(bits, np.uint32)
    scales = _c(scales, np.uint16)
    N = bits.shape[0]
    q = _c(np.atleast_2d(q), np.int8)
    s_tok = _c(s_tok, np.float32)
    M = q.shape[0]
    b = None if bias is None else _c(bias, np.float32)

    def one(sub):
        r, nr = _rows(sub, N)
        y = np.empty((M, nr), np.float32)
        S = np.empty((M, nr), np.float64)
        mism = lib().orc_w1a8_gemm(_p(bits), _p(scales), N, K, int(G), _p(q), _p(s_tok), M, _p(b),
                                   _p(r), nr, _p(y), _p(S))
        if mism:
            raise AssertionError("W1 identity disagreed %d times" % mism)
        return y, S
    return _by_rows(one, rows, N, threads)


# ---------------------------------------------------------------- activations
def quantize_f32(x):
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    lib().orc_quantize_f32(_p(x), M, K, _p(q), _p(s))
    return q, s


def quantize_bf16(xb):
    xb = _c(np.atleast_2d(xb), np.uint16)
    M, K = xb.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    lib().orc_quantize_bf16(_p(xb), M, K, _p(q), _p(s))
    return q, s


# ---------------------------------------------------------------- fused epilogues
def relu2_mul(gate, up):
    """[BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"] out = (r * r) * up with
    r = max(0, gate), elementwise in fp64; gate and up are the two products
    of one activation (the exact values of the oracle's gemv functions)."""
    g = np.asarray(gate, np.float64)
    u = np.asarray(up, np.float64)
    r = np.where(g > 0.0, g, 0.0)
    return (r * r) * u


def rmsnorm(x, w, eps):
    """[BL "Fused RMSNorm + BitLinear + Residual Add M=1 Kernel"] the
    normalised activation x * rinv * w with rinv = 1 / sqrt(mean(x^2) + eps),
    in fp64 (a zero row with eps = 0 gives 0: the reading for 0 / 0)."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    w = np.asarray(w, np.float64)
    den = np.mean(x * x, axis=1, keepdims=True) + float(eps)
    rinv = np.where(den > 0.0, 1.0 / np.sqrt(np.where(den > 0.0, den, 1.0)), 0.0)
    return x * rinv * w[None, :]
