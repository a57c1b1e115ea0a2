"""Python binding of the C ABI in include/lowbit.h (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: host functions take and return numpy arrays, device
functions take torch tensors that already live on the GPU (torch provides the
memory and the stream) and enqueue the library's HIP kernels.  A nonzero
status raises :class:`LowbitError` with the library's own message.

The library must be built (``python -m binary_bit_weight_amd.build``); there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblowbit.so")

LL_FMT_I2S, LL_FMT_TQ2_0, LL_FMT_W1 = 1, 2, 3
LL_ACT_F32, LL_ACT_I8 = 1, 2
LL_DT_F32, LL_DT_BF16 = 1, 2

STATUS_NAMES = {0: "LL_OK", -1: "LL_EINVAL", -2: "LL_ESHAPE", -3: "LL_EALIGN", -4: "LL_ECODE",
                -5: "LL_EWORKSPACE", -6: "LL_EHIP", -7: "LL_ERANGE"}

# Every entry point lowbit.h declares, with (restype, argtypes).
_P, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
SIGNATURES = {
    "ll_abi_version": (C.c_int, []),
    "ll_strerror": (C.c_char_p, [C.c_int]),
    "ll_last_error": (C.c_char_p, []),
    "ll_packed_size": (_SZ, [_I32, _I64, _I64, _I32, _P]),
    "ll_pack_i2s": (C.c_int, [_P, _I64, _I64, C.c_float, _P]),
    "ll_unpack_i2s": (C.c_int, [_P, _I64, _I64, _P, _P]),
    "ll_pack_tq2": (C.c_int, [_P, _P, _I64, _I64, _P]),
    "ll_unpack_tq2": (C.c_int, [_P, _I64, _I64, _P, _P]),
    "ll_tq2_split": (C.c_int, [_P, _I64, _I64, _P, _P]),
    "ll_pack_w1": (C.c_int, [_P, _I64, _I64, _P]),
    "ll_unpack_w1": (C.c_int, [_P, _I64, _I64, _P]),
    "ll_w1_from_dense": (C.c_int, [_P, _I64, _I64, _I32, _P, _P]),
    "ll_validate": (C.c_int, [_I32, _P, _I64, _I64, _P]),
    "ll_quantize_act": (C.c_int, [_P, _I32, _I64, _I64, _P, _P, _P, _P]),
    "ll_gemv_workspace_size": (_SZ, [_P, _I32, _I64]),
    "ll_bitlinear_gemv": (C.c_int, [_P, _I32, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "ll_gemm_workspace_size": (_SZ, [_P, _I64]),
    "ll_bitlinear_gemm": (C.c_int, [_P, _P, _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "ll_probe_stream_read": (C.c_int, [_P, _SZ, _P, _I32, _P]),
    "ll_gemm_noalloc_scratch_bytes": (_SZ, []),
    "ll_bitlinear_gemm_noalloc": (C.c_int, [_P, _P, _P, _I64, _P, _P, _P, _P]),
    "ll_binary_linear_workspace_size": (_SZ, [_P, _I64]),
    "ll_binary_linear": (C.c_int, [_P, _P, _I64, _P, _P, _P, _SZ, _P]),
}


class LowbitError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, msg))
        self.status = status


class ll_weights(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("group", C.c_int32), ("N", C.c_int64), ("K", C.c_int64),
                ("codes", C.c_void_p), ("scales", C.c_void_p)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("liblowbit.so is not built; run `python -m binary_bit_weight_amd.build`")
        # torch ships its own HIP runtime under the same soname.  Loading it
        # first lets the library bind to that copy; loaded the other way round
        # the process would hold two HIP/HSA runtimes, and the second one finds
        # no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise LowbitError(rc, lib().ll_last_error().decode())


def _np(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


def _dev(t):
    """Device pointer of a torch tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ info
def ll_abi_version() -> int:
    return lib().ll_abi_version()


def ll_strerror(status: int) -> str:
    return lib().ll_strerror(status).decode()


# ------------------------------------------------------------------ host formats
def ll_packed_size(fmt, N, K, group=0):
    sb = C.c_size_t(0)
    n = lib().ll_packed_size(fmt, N, K, group, C.byref(sb))
    return int(n), int(sb.value)


def ll_pack_i2s(w, scale):
    w, pw = _np(w, np.int8)
    N, K = w.shape
    out = np.zeros(N * K // 4 + 4, np.uint8)
    _check(lib().ll_pack_i2s(pw, N, K, float(scale), out.ctypes.data_as(C.c_void_p)))
    return out


def ll_unpack_i2s(packed, N, K):
    packed, pp = _np(packed, np.uint8)
    w = np.empty((N, K), np.int8)
    s = np.zeros(1, np.float32)
    _check(lib().ll_unpack_i2s(pp, N, K, w.ctypes.data_as(C.c_void_p), s.ctypes.data_as(C.c_void_p)))
    return w, float(s[0])


def ll_pack_tq2(w, scales):
    w, pw = _np(w, np.int8)
    sc, ps = _np(scales, np.uint16)
    N, K = w.shape
    out = np.zeros(66 * N * K // 256, np.uint8)
    _check(lib().ll_pack_tq2(pw, ps, N, K, out.ctypes.data_as(C.c_void_p)))
    return out


def ll_unpack_tq2(blocks, N, K):
    blocks, pb = _np(blocks, np.uint8)
    w = np.empty((N, K), np.int8)
    sc = np.empty(N * K // 256, np.uint16)
    _check(lib().ll_unpack_tq2(pb, N, K, w.ctypes.data_as(C.c_void_p), sc.ctypes.data_as(C.c_void_p)))
    return w, sc


def ll_tq2_split(blocks, N, K):
    blocks, pb = _np(blocks, np.uint8)
    codes = np.empty(N * K // 4, np.uint8)
    sc = np.empty(N * K // 256, np.uint16)
    _check(lib().ll_tq2_split(pb, N, K, codes.ctypes.data_as(C.c_void_p), sc.ctypes.data_as(C.c_void_p)))
    return codes, sc


def ll_pack_w1(w):
    w, pw = _np(w, np.int8)
    N, K = w.shape
    out = np.zeros((N, K // 32), np.uint32)
    _check(lib().ll_pack_w1(pw, N, K, out.ctypes.data_as(C.c_void_p)))
    return out


def ll_unpack_w1(bits, K):
    bits, pb = _np(bits, np.uint32)
    N = bits.shape[0]
    w = np.empty((N, K), np.int8)
    _check(lib().ll_unpack_w1(pb, N, K, w.ctypes.data_as(C.c_void_p)))
    return w


def ll_w1_from_dense(W, group):
    W, pW = _np(W, np.float32)
    N, K = W.shape
    bits = np.zeros((N, K // 32), np.uint32)
    sc = np.zeros((N, K // group), np.uint16)
    _check(lib().ll_w1_from_dense(pW, N, K, int(group), bits.ctypes.data_as(C.c_void_p),
                                  sc.ctypes.data_as(C.c_void_p)))
    return bits, sc


def ll_validate(fmt, codes, N, K):
    """(status, first bad element index or -1); does not raise on LL_ECODE."""
    codes, pc = _np(codes, np.uint8)
    bad = C.c_int64(-1)
    rc = lib().ll_validate(fmt, pc, N, K, C.byref(bad))
    if rc not in (0, -4):
        _check(rc)
    return rc, int(bad.value)


# ------------------------------------------------------------------ device
class Weights:
    """A packed weight matrix in device memory plus its ll_weights descriptor.

    codes / scales are torch GPU tensors holding exactly the layouts lowbit.h
    documents for ll_weights (the object keeps them alive)."""

    def __init__(self, fmt, N, K, codes, scales=None, group=0):
        self.fmt, self.N, self.K, self.group = fmt, N, K, group
        self.codes, self.scales = codes, scales
        self.desc = ll_weights(fmt, group, N, K, _dev(codes), _dev(scales))

    @property
    def ref(self):
        return C.byref(self.desc)


def ll_quantize_act(x, xq, xs, stream=None, xsum=None):
    import torch
    M, K = x.shape
    dt = LL_DT_BF16 if x.dtype == torch.bfloat16 else LL_DT_F32
    _check(lib().ll_quantize_act(_dev(x), dt, M, K, _dev(xq), _dev(xs), _dev(xsum), _stream(stream)))


def ll_gemv_workspace_size(w: Weights, act, M):
    return int(lib().ll_gemv_workspace_size(w.ref, act, M))


def ll_bitlinear_gemv(w: Weights, act, x, xs, M, bias, y, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ll_bitlinear_gemv(w.ref, act, _dev(x), _dev(xs), M, _dev(bias), _dev(y), _dev(workspace),
                                   ws_bytes, _stream(stream)))


def ll_gemm_workspace_size(w: Weights, M):
    return int(lib().ll_gemm_workspace_size(w.ref, M))


def ll_bitlinear_gemm(w: Weights, xq, xs, M, bias, y, acc_out=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ll_bitlinear_gemm(w.ref, _dev(xq), _dev(xs), M, _dev(bias), _dev(y), _dev(acc_out),
                                   _dev(workspace), ws_bytes, _stream(stream)))


def ll_probe_stream_read(buf, sink, blocks, stream=None):
    """Streams every byte of the device tensor buf once (diagnostic)."""
    _check(lib().ll_probe_stream_read(_dev(buf), buf.numel() * buf.element_size(), _dev(sink), blocks,
                                      _stream(stream)))


def ll_gemm_noalloc_scratch_bytes() -> int:
    return int(lib().ll_gemm_noalloc_scratch_bytes())


def ll_bitlinear_gemm_noalloc(w: Weights, xq, xs, M, bias, y, acc_out=None, stream=None):
    _check(lib().ll_bitlinear_gemm_noalloc(w.ref, _dev(xq), _dev(xs), M, _dev(bias), _dev(y), _dev(acc_out),
                                           _stream(stream)))


def ll_binary_linear_workspace_size(w: Weights, M) -> int:
    n = lib().ll_binary_linear_workspace_size(w.ref, M)
    if n == C.c_size_t(-1).value:
        raise RuntimeError("ll_binary_linear_workspace_size: unsupported weights or M")
    return int(n)


def ll_binary_linear(w: Weights, x, M, bias, y, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ll_binary_linear(w.ref, _dev(x), M, _dev(bias), _dev(y), _dev(workspace), ws_bytes,
                                  _stream(stream)))


# ------------------------------------------------------------------ conveniences
# Allocation and upload helpers around the entry points above (torch provides
# the memory); each call still ends in exactly one library entry point.
def _to_gpu(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_i2s(packed, N, K, device="cuda") -> Weights:
    """Device copy of an ll_pack_i2s buffer (codes + tail scale)."""
    return Weights(LL_FMT_I2S, N, K, _to_gpu(np.asarray(packed, np.uint8), device))


def upload_tq2(blocks, N, K, device="cuda") -> Weights:
    """Splits 66-byte TQ2_0 blocks on the host (ll_tq2_split) and uploads both arrays."""
    codes, sc = ll_tq2_split(blocks, N, K)
    return Weights(LL_FMT_TQ2_0, N, K, _to_gpu(codes, device), _to_gpu(sc.view(np.int16), device))


def upload_w1(bits, scales, K, group, device="cuda") -> Weights:
    bits = np.asarray(bits, np.uint32)
    return Weights(LL_FMT_W1, bits.shape[0], K, _to_gpu(bits.view(np.int32), device),
                   _to_gpu(np.asarray(scales, np.uint16).view(np.int16), device), group)


def quantize(x, stream=None, with_sum=False):
    """(xq int8 [M,K], xs fp32 [M]) = ll_quantize_act(x); with_sum also
    returns xsum int32 [M] = sum_k xq[m,k]."""
    import torch
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    xsum = torch.empty((M,), dtype=torch.int32, device=x.device) if with_sum else None
    ll_quantize_act(x, xq, xs, stream, xsum)
    return (xq, xs, xsum) if with_sum else (xq, xs)


def gemv(w: Weights, x, xs=None, bias=None, stream=None):
    """y [M,N] fp32 = ll_bitlinear_gemv; x fp32 [M,K], or int8 [M,K] with xs."""
    import torch
    M = x.shape[0]
    act = LL_ACT_I8 if x.dtype == torch.int8 else LL_ACT_F32
    y = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    nws = ll_gemv_workspace_size(w, act, M)
    # zero-filled: split-K counters (W1) must start at zero (each call leaves them zero)
    ws = torch.zeros((max(nws, 16),), dtype=torch.uint8, device=x.device) if nws else None
    ll_bitlinear_gemv(w, act, x, xs, M, bias, y, ws, stream)
    return y


def binary_linear(w: Weights, x, bias=None, stream=None, workspace=None):
    """y bf16 [M,N] = ll_binary_linear(x bf16 [M,K]); a zero-filled workspace
    is allocated unless one is given."""
    import torch
    M = x.shape[0]
    y = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.zeros((ll_binary_linear_workspace_size(w, M),), dtype=torch.uint8, device=x.device)
    ll_binary_linear(w, x, M, bias, y, workspace, stream)
    return y


def gemm(w: Weights, xq, xs, bias=None, want_acc=False, stream=None):
    """(y [M,N] fp32, acc int32 [M,N] or None) = ll_bitlinear_gemm."""
    import torch
    M = xq.shape[0]
    y = torch.empty((M, w.N), dtype=torch.float32, device=xq.device)
    acc = torch.empty((M, w.N), dtype=torch.int32, device=xq.device) if want_acc else None
    nws = ll_gemm_workspace_size(w, M)
    # zero-filled: the split-K tile counters must start at zero (each call leaves them zero)
    ws = torch.zeros((max(nws, 16),), dtype=torch.uint8, device=xq.device) if nws else None
    ll_bitlinear_gemm(w, xq, xs, M, bias, y, acc, ws, stream)
    return y, acc


# ------------------------------------------------------------------ prepared batches
class ll_gemv_item(C.Structure):
    _fields_ = [("w", ll_weights), ("x", C.c_void_p), ("bias", C.c_void_p), ("y", C.c_void_p)]


LL_EPI_NONE, LL_EPI_RELU2_MUL = 0, 1


class ll_gemv_item_ex(C.Structure):
    _fields_ = [("w", ll_weights), ("w2", ll_weights), ("x", C.c_void_p), ("bias", C.c_void_p), ("y", C.c_void_p),
                ("epilogue", C.c_int32), ("norm_eps", C.c_float), ("norm_w", C.c_void_p)]


class ll_gemv_plan(C.Structure):
    _fields_ = [("mem", C.c_void_p), ("bytes", C.c_size_t), ("count", C.c_int32), ("nprep", C.c_int32),
                ("act", C.c_int32), ("fmt", C.c_int32), ("M", C.c_int64), ("tiles", C.c_int64),
                ("prep_entries", C.c_int64), ("kmax", C.c_int64), ("prob_table", C.c_void_p),
                ("prep_table", C.c_void_p), ("map_table", C.c_void_p), ("epilogues", C.c_int32),
                ("flags", C.c_int32)]


class ll_gemv_item_i8(C.Structure):
    _fields_ = [("w", ll_weights), ("xq", C.c_void_p), ("xs", C.c_void_p), ("bias", C.c_void_p), ("y", C.c_void_p)]


SIGNATURES.update({
    "ll_gemv_plan_bytes": (_SZ, [_P, _I32, _I32, _I64]),
    "ll_gemv_plan_init": (C.c_int, [_P, _I32, _I32, _I64, _P, _SZ, _P]),
    "ll_gemv_plan_bytes_ex": (_SZ, [_P, _I32, _I32, _I64]),
    "ll_gemv_plan_init_ex": (C.c_int, [_P, _I32, _I32, _I64, _P, _SZ, _P]),
    "ll_gemv_plan_bytes_i8": (_SZ, [_P, _I32, _I64]),
    "ll_gemv_plan_init_i8": (C.c_int, [_P, _I32, _I64, _P, _SZ, _P]),
    "ll_gemv_plan_run": (C.c_int, [_P, _P]),
    "ll_gemv_plan_prepare": (C.c_int, [_P, _P]),
    "ll_gemv_plan_product": (C.c_int, [_P, _P]),
})


class Relu2Mul:
    """A gated pair for GemvPlan (M = 1): y = relu(W_gate x)^2 * (W_up x)
    [BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"], both products from one x
    (optionally RMS-normalised: norm = (weights [K], eps))."""

    def __init__(self, w_gate, w_up, x, y, norm=None):
        self.w_gate, self.w_up, self.x, self.y, self.norm = w_gate, w_up, x, y, norm


class Normed:
    """A product of an RMS-normalised activation for GemvPlan (M = 1) [BL
    "Fused RMSNorm + BitLinear + Residual Add M=1 Kernel"]: y = W xn (+ bias,
    the residual) with xn = x / sqrt(mean(x^2) + eps) * norm_w."""

    def __init__(self, w, x, norm_w, eps, bias, y):
        self.w, self.x, self.norm_w, self.eps, self.bias, self.y = w, x, norm_w, eps, bias, y


class GemvPlan:
    """A prepared batch of fp32-activation decode products (ll_gemv_plan_*).

    items: list of (Weights, x, bias_or_None, y) with GPU tensors, or
    Relu2Mul gated pairs (ll_gemv_plan_init_ex); the plan keeps them alive.
    With M = 1 the bias is the residual add.  run() = prepare() + product()."""

    def __init__(self, items, M):
        import torch
        self.items = list(items)
        arr = (ll_gemv_item_ex * len(self.items))()
        for i, it in enumerate(self.items):
            if isinstance(it, Relu2Mul):
                nw, eps = it.norm if it.norm is not None else (None, 0.0)
                arr[i] = ll_gemv_item_ex(it.w_gate.desc, it.w_up.desc, _dev(it.x), None, _dev(it.y), LL_EPI_RELU2_MUL,
                                         float(eps), _dev(nw))
            elif isinstance(it, Normed):
                arr[i] = ll_gemv_item_ex(it.w.desc, ll_weights(), _dev(it.x), _dev(it.bias), _dev(it.y), LL_EPI_NONE,
                                         float(it.eps), _dev(it.norm_w))
            else:
                w, x, b, y = it
                arr[i] = ll_gemv_item_ex(w.desc, ll_weights(), _dev(x), _dev(b), _dev(y), LL_EPI_NONE, 0.0, None)
        self._arr = arr
        self.plan = ll_gemv_plan()
        n = lib().ll_gemv_plan_bytes_ex(arr, len(self.items), LL_ACT_F32, M)
        if n == 2 ** 64 - 1:   # invalid items: let init report which one
            _check(lib().ll_gemv_plan_init_ex(arr, len(self.items), LL_ACT_F32, M, None, 0, C.byref(self.plan)))
        dev = self.items[0].x.device if isinstance(self.items[0], (Relu2Mul, Normed)) else self.items[0][1].device
        self.mem = torch.empty((max(int(n), 16),), dtype=torch.uint8, device=dev)
        _check(lib().ll_gemv_plan_init_ex(arr, len(self.items), LL_ACT_F32, M, _dev(self.mem), int(n),
                                          C.byref(self.plan)))

    def prepare(self, stream=None):
        _check(lib().ll_gemv_plan_prepare(C.byref(self.plan), _stream(stream)))

    def product(self, stream=None):
        _check(lib().ll_gemv_plan_product(C.byref(self.plan), _stream(stream)))

    def run(self, stream=None):
        _check(lib().ll_gemv_plan_run(C.byref(self.plan), _stream(stream)))


class GemvPlanI8:
    """A prepared batch of W1A8 decode products (ll_gemv_plan_init_i8): items
    (Weights with group 128, xq int8 [M,K], xs fp32 [M], bias_or_None, y fp32
    [M,N]) as GPU tensors; the plan keeps them alive.  run() = prepare() +
    product()."""

    def __init__(self, items, M):
        import torch
        self.items = list(items)
        arr = (ll_gemv_item_i8 * len(self.items))()
        for i, (w, xq, xs, b, y) in enumerate(self.items):
            arr[i] = ll_gemv_item_i8(w.desc, _dev(xq), _dev(xs), _dev(b), _dev(y))
        self._arr = arr
        self.plan = ll_gemv_plan()
        n = lib().ll_gemv_plan_bytes_i8(arr, len(self.items), M)
        if n == 2 ** 64 - 1:   # invalid items: let init report which one
            _check(lib().ll_gemv_plan_init_i8(arr, len(self.items), M, None, 0, C.byref(self.plan)))
        self.mem = torch.empty((max(int(n), 16),), dtype=torch.uint8, device=self.items[0][1].device)
        _check(lib().ll_gemv_plan_init_i8(arr, len(self.items), M, _dev(self.mem), int(n), C.byref(self.plan)))

    def prepare(self, stream=None):
        _check(lib().ll_gemv_plan_prepare(C.byref(self.plan), _stream(stream)))

    def product(self, stream=None):
        _check(lib().ll_gemv_plan_product(C.byref(self.plan), _stream(stream)))

    def run(self, stream=None):
        _check(lib().ll_gemv_plan_run(C.byref(self.plan), _stream(stream)))
