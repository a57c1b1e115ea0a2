// Device entry points of lowbit.h: host-side argument validation, then the
// kernel launchers.  Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <tuple>
#include <vector>

#include "internal.h"
#include "launch.h"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ll_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return LL_OK;
    return ll::failf(LL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape and pointer checks common to every product entry point.
// The W1 device kernels work on 128-k chunks: K % 128 == 0, G in {32, 64, 128, 256}.
ll_status check_w1_device(const ll_weights* w, const char* fn) {
    if (w->K % 128) return ll::failf(LL_ESHAPE, "%s: the W1 device path needs K %% 128 == 0", fn);
    if (w->group != 32 && w->group != 64 && w->group != 128 && w->group != 256)
        return ll::failf(LL_ESHAPE, "%s: the W1 device path needs group 32, 64, 128 or 256", fn);
    return LL_OK;
}

ll_status check_weights(const ll_weights* w, const char* fn) {
    if (!w) return ll::failf(LL_EINVAL, "%s: weights descriptor is NULL", fn);
    if (w->N <= 0 || w->K <= 0) return ll::failf(LL_EINVAL, "%s: N and K must be positive", fn);
    if (w->N > (int64_t(1) << 31) - 1 || w->K > (int64_t(1) << 24))
        return ll::failf(LL_ERANGE, "%s: N must be < 2^31 and K <= 2^24", fn);
    if (!w->codes) return ll::failf(LL_EINVAL, "%s: codes pointer is NULL", fn);
    if (!aligned(w->codes, 16)) return ll::failf(LL_EALIGN, "%s: codes must be 16-byte aligned", fn);
    switch (w->fmt) {
    case LL_FMT_I2S:
        if (w->K % 128) return ll::failf(LL_ESHAPE, "%s: i2_s needs K %% 128 == 0", fn);
        // the products sum a code field's terms (up to 2 * 16 * 127 each) over
        // up to K / 2 elements in one int32 accumulator
        if (w->K > (int64_t(1) << 20)) return ll::failf(LL_ERANGE, "%s: i2_s needs K <= 2^20 (exact int32 sums)", fn);
        return LL_OK;
    case LL_FMT_TQ2_0:
        if (w->K % 256) return ll::failf(LL_ESHAPE, "%s: TQ2_0 needs K %% 256 == 0", fn);
        if (!w->scales) return ll::failf(LL_EINVAL, "%s: TQ2_0 scales pointer is NULL", fn);
        if (!aligned(w->scales, 2)) return ll::failf(LL_EALIGN, "%s: scales must be 2-byte aligned", fn);
        return LL_OK;
    case LL_FMT_W1:
        if (w->group <= 0 || w->group % 32 || w->K % w->group)
            return ll::failf(LL_ESHAPE, "%s: W1 needs group a positive multiple of 32 dividing K", fn);
        if (!w->scales) return ll::failf(LL_EINVAL, "%s: W1 scales pointer is NULL", fn);
        if (!aligned(w->scales, 2)) return ll::failf(LL_EALIGN, "%s: scales must be 2-byte aligned", fn);
        return LL_OK;
    default:
        return ll::failf(LL_EINVAL, "%s: unknown format %d", fn, int(w->fmt));
    }
}

static_assert(llk::kCounterBytes == LL_WORKSPACE_COUNTER_BYTES, "counter region size of lowbit.h");

// A device workspace: split-K counters in its first llk::kCounterBytes, then
// the data region a product's launcher lays out.
struct Workspace {
    int32_t* counters;
    void* data;
};
Workspace split_ws(void* ws) {
    char* b = static_cast<char*>(ws);
    return {reinterpret_cast<int32_t*>(b), b ? b + llk::kCounterBytes : nullptr};
}
// Bytes of a workspace whose data region needs `data` bytes (0: no workspace).
size_t with_counters(size_t data) { return data ? llk::kCounterBytes + data : 0; }

ll_status check_workspace(void* ws, size_t bytes, size_t need, const char* fn) {
    if (need == 0) return LL_OK;
    if (!ws || bytes < need) return ll::failf(LL_EWORKSPACE, "%s: workspace of %zu bytes required", fn, need);
    if (!aligned(ws, 16)) return ll::failf(LL_EALIGN, "%s: workspace must be 16-byte aligned", fn);
    return LL_OK;
}

}  // namespace

namespace llk {

hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::vector<std::tuple<const void*, int, size_t>> done;   // (kernel, device, bytes allowed)
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& d : done)
        if (std::get<0>(d) == kernel && std::get<1>(d) == dev && std::get<2>(d) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e == hipSuccess) done.emplace_back(kernel, dev, bytes);
    return e;
}

}  // namespace llk

extern "C" {

ll_status ll_quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* xq, float* xs, int32_t* xsum,
                          void* stream) {
    if (!x || !xq || !xs) return ll::fail(LL_EINVAL, "ll_quantize_act: NULL pointer");
    if (x_dtype != LL_DT_F32 && x_dtype != LL_DT_BF16) return ll::fail(LL_EINVAL, "ll_quantize_act: unknown dtype");
    if (M <= 0 || K <= 0) return ll::fail(LL_EINVAL, "ll_quantize_act: M and K must be positive");
    if (M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 20)) return ll::fail(LL_ERANGE, "ll_quantize_act: M < 2^31, K <= 2^20");
    if (!aligned(x, x_dtype == LL_DT_F32 ? 4 : 2) || !aligned(xs, 4) || (xsum && !aligned(xsum, 4)))
        return ll::fail(LL_EALIGN, "ll_quantize_act: x / xs / xsum not aligned to their element size");
    return hip_status(llk::launch_quantize(x, x_dtype == LL_DT_BF16, M, K, xq, xs, xsum, static_cast<hipStream_t>(stream)),
                      "ll_quantize_act");
}

size_t ll_gemv_workspace_size(const ll_weights* w, int32_t act, int64_t M) {
    if (!w || M < 1 || M > 16 || w->K <= 0) return size_t(-1);
    if (act == LL_ACT_F32) return with_counters(llk::planes_workspace(M, w->K));
    if (act == LL_ACT_I8)
        return w->fmt == LL_FMT_W1 && w->group > 0 ? with_counters(llk::w1_workspace(M, w->N, w->K, w->group)) : 0;
    return size_t(-1);
}

ll_status ll_bitlinear_gemv(const ll_weights* w, int32_t act, const void* x, const float* xs, int64_t M,
                            const float* bias, float* y, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ll_bitlinear_gemv";
    ll_status st = check_weights(w, fn);
    if (st) return st;
    if (M < 1 || M > 16) return ll::fail(LL_ESHAPE, "ll_bitlinear_gemv: M must be in [1, 16] (use ll_bitlinear_gemm above)");
    if (!x || !y) return ll::fail(LL_EINVAL, "ll_bitlinear_gemv: x or y is NULL");
    if (!aligned(x, 16)) return ll::fail(LL_EALIGN, "ll_bitlinear_gemv: x must be 16-byte aligned");
    if (!aligned(y, 4) || (bias && !aligned(bias, 4))) return ll::fail(LL_EALIGN, "ll_bitlinear_gemv: y / bias must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (act == LL_ACT_F32) {
        if (w->fmt != LL_FMT_I2S && w->fmt != LL_FMT_TQ2_0)
            return ll::fail(LL_EINVAL, "ll_bitlinear_gemv: fp32 activations need format i2_s or TQ2_0");
        const size_t need = with_counters(llk::planes_workspace(M, w->K));
        st = check_workspace(workspace, workspace_bytes, need, fn);
        if (st) return st;
        return hip_status(llk::launch_gemv_planes(w->fmt, w->codes, w->scales, w->N, w->K, static_cast<const float*>(x),
                                                  M, bias, y, need ? split_ws(workspace).data : nullptr, s),
                          fn);
    }
    if (act == LL_ACT_I8) {
        if (!xs) return ll::fail(LL_EINVAL, "ll_bitlinear_gemv: int8 activations need their scales xs");
        if (!aligned(xs, 4)) return ll::fail(LL_EALIGN, "ll_bitlinear_gemv: xs must be 4-byte aligned");
        if (w->fmt == LL_FMT_I2S || w->fmt == LL_FMT_TQ2_0)
            return hip_status(llk::launch_gemv_i8_planes(w->fmt, w->codes, w->scales, w->N, w->K,
                                                         static_cast<const int8_t*>(x), xs, M, bias, y, s),
                              fn);
        if (w->fmt == LL_FMT_W1) {
            st = check_w1_device(w, fn);
            if (st) return st;
            const size_t need = with_counters(llk::w1_workspace(M, w->N, w->K, w->group));
            st = check_workspace(workspace, workspace_bytes, need, fn);
            if (st) return st;
            const Workspace ws = split_ws(workspace);
            return hip_status(llk::launch_w1_gemv(static_cast<const uint32_t*>(w->codes),
                                                  static_cast<const uint16_t*>(w->scales), w->N, w->K, w->group,
                                                  static_cast<const int8_t*>(x), xs, M, bias, y, ws.counters, ws.data,
                                                  s),
                              fn);
        }
        return ll::fail(LL_EINVAL, "ll_bitlinear_gemv: int8 activations with this format are not supported");
    }
    return ll::fail(LL_EINVAL, "ll_bitlinear_gemv: unknown activation type");
}

// W1 with group size 128 above 16 tokens runs on the int8 matrix cores
// (fp32 group scaling); other W1 products run as passes of up to 16 tokens
// with exact fp64 group scaling.
static bool w1_mfma(const ll_weights* w, int64_t M) { return w->fmt == LL_FMT_W1 && w->group == 128 && M > 16; }

// The product of ll_bitlinear_gemm on validated arguments; ws: a workspace
// of ll_gemm_workspace_size bytes, or NULL when that is 0.
// xsum (i2_s): per-token sums of xq from the quantization, or NULL; y16:
// bf16 output written instead of y, or NULL.
static hipError_t run_gemm(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M, const float* bias,
                           float* y, int32_t* acc_out, void* ws, hipStream_t s, const int32_t* xsum = nullptr,
                           uint16_t* y16 = nullptr) {
    const Workspace W = split_ws(ws);
    if (w1_mfma(w, M))
        return llk::launch_gemm_i8_w1(static_cast<const uint32_t*>(w->codes), static_cast<const uint16_t*>(w->scales),
                                      w->N, w->K, xq, xs, M, bias, y, W.counters, W.data, s, y16);
    if (w->fmt == LL_FMT_W1)
        return llk::launch_w1_gemv(static_cast<const uint32_t*>(w->codes), static_cast<const uint16_t*>(w->scales), w->N,
                                   w->K, w->group, xq, xs, M, bias, y, W.counters, W.data, s, y16);
    if (w->fmt == LL_FMT_TQ2_0)
        return llk::launch_gemm_i8_tq2(static_cast<const uint8_t*>(w->codes), static_cast<const uint16_t*>(w->scales),
                                       w->N, w->K, xq, xs, M, bias, y, W.counters, W.data, s, y16);
    return llk::launch_gemm_i8_i2s(static_cast<const uint8_t*>(w->codes), w->N, w->K, xq, xs, M, bias, y, acc_out,
                                   W.counters, W.data, s, xsum, y16);
}

// Data-region bytes of the product ll_bitlinear_gemm runs (0: no workspace).
static size_t gemm_data_bytes(const ll_weights* w, int64_t M) {
    if (w1_mfma(w, M)) return llk::gemm_i8_workspace(M, w->N, w->K, LL_FMT_W1);
    if (w->fmt == LL_FMT_W1) return llk::w1_workspace(M, w->N, w->K, w->group);
    return llk::gemm_i8_workspace(M, w->N, w->K, w->fmt);
}

size_t ll_gemm_workspace_size(const ll_weights* w, int64_t M) {
    if (!w || M < 1 || w->K <= 0 || w->N <= 0) return size_t(-1);
    if (w->fmt == LL_FMT_W1 && w->group <= 0) return size_t(-1);
    if (w->fmt != LL_FMT_I2S && w->fmt != LL_FMT_TQ2_0 && w->fmt != LL_FMT_W1) return size_t(-1);
    return with_counters(gemm_data_bytes(w, M));
}

// Argument checks of ll_bitlinear_gemm and its allocation-free variant.
static ll_status check_gemm(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M, const float* bias,
                            const float* y, const int32_t* acc_out, const char* fn) {
    ll_status st = check_weights(w, fn);
    if (st) return st;
    if (M < 1 || M > 65535 * 128) return ll::failf(LL_ESHAPE, "%s: M must be in [1, 65535*128]", fn);
    if (!xq || !xs || !y) return ll::failf(LL_EINVAL, "%s: xq, xs or y is NULL", fn);
    if (!aligned(xq, 16)) return ll::failf(LL_EALIGN, "%s: xq must be 16-byte aligned", fn);
    if (!aligned(xs, 4) || !aligned(y, 4) || (bias && !aligned(bias, 4)) || (acc_out && !aligned(acc_out, 4)))
        return ll::failf(LL_EALIGN, "%s: xs / y / bias / acc_out must be 4-byte aligned", fn);
    if (w->fmt == LL_FMT_W1) {
        st = check_w1_device(w, fn);
        if (st) return st;
        if (acc_out) return ll::failf(LL_EINVAL, "%s: acc_out is not available for W1 (per-group scales)", fn);
    }
    if (w->fmt != LL_FMT_I2S && w->fmt != LL_FMT_TQ2_0 && w->fmt != LL_FMT_W1)
        return ll::failf(LL_EINVAL, "%s: formats i2_s, TQ2_0 and W1 only", fn);
    if (w->fmt == LL_FMT_TQ2_0 && acc_out)
        return ll::failf(LL_EINVAL, "%s: acc_out is not available for TQ2_0 (per-block scales)", fn);
    return LL_OK;
}

ll_status ll_bitlinear_gemm(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M, const float* bias,
                            float* y, int32_t* acc_out, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ll_bitlinear_gemm";
    ll_status st = check_gemm(w, xq, xs, M, bias, y, acc_out, fn);
    if (st) return st;
    const size_t need = with_counters(gemm_data_bytes(w, M));
    st = check_workspace(workspace, workspace_bytes, need, fn);
    if (st) return st;
    return hip_status(run_gemm(w, xq, xs, M, bias, y, acc_out, need ? workspace : nullptr, static_cast<hipStream_t>(stream)),
                      fn);
}

ll_status ll_probe_stream_read(const void* p, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    if (!p || !sink) return ll::fail(LL_EINVAL, "ll_probe_stream_read: NULL pointer");
    if (bytes == 0 || bytes % 16) return ll::fail(LL_ESHAPE, "ll_probe_stream_read: bytes must be a positive multiple of 16");
    if (blocks < 1 || blocks > 65535) return ll::fail(LL_EINVAL, "ll_probe_stream_read: blocks must be in [1, 65535]");
    if (!aligned(p, 16) || !aligned(sink, 4)) return ll::fail(LL_EALIGN, "ll_probe_stream_read: p 16-byte, sink 4-byte aligned");
    return hip_status(llk::launch_stream_read(p, bytes, sink, blocks, static_cast<hipStream_t>(stream)),
                      "ll_probe_stream_read");
}

size_t ll_gemm_noalloc_scratch_bytes(void) { return llk::static_scratch_bytes(); }

ll_status ll_bitlinear_gemm_noalloc(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M,
                                    const float* bias, float* y, int32_t* acc_out, void* stream) {
    const char* fn = "ll_bitlinear_gemm_noalloc";
    ll_status st = check_gemm(w, xq, xs, M, bias, y, acc_out, fn);
    if (st) return st;
    const size_t need = with_counters(gemm_data_bytes(w, M));
    if (need > llk::static_scratch_bytes())
        return ll::failf(LL_EWORKSPACE, "%s: this product needs %zu bytes of scratch, more than the %zu-byte static scratch",
                         fn, need, llk::static_scratch_bytes());
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (need) {
        st = hip_status(llk::static_scratch(&ws, s), fn);
        if (st) return st;
    }
    return hip_status(run_gemm(w, xq, xs, M, bias, y, acc_out, ws, s), fn);
}

// One-shot bf16 layer: workspace = split-K counters | the product's data
// region | int8 x [M K] | token scales [M] | token sums of q [M], each part
// on a 256-byte boundary.  Two launches: the quantization (which also sums
// each token's codes, the offset term of the i2_s product), then the product
// with the bias and the bf16 rounding in its epilogue.
static size_t round256(size_t b) { return (b + 255) / 256 * 256; }
struct LinearLayout {
    size_t q, s, qs, total;
};
static bool linear_layout(const ll_weights* w, int64_t M, LinearLayout& L) {
    if (w->fmt != LL_FMT_I2S && w->fmt != LL_FMT_TQ2_0 && w->fmt != LL_FMT_W1) return false;
    if (w->fmt == LL_FMT_W1 && w->group <= 0) return false;
    L.q = round256(llk::kCounterBytes + gemm_data_bytes(w, M));
    L.s = L.q + round256(size_t(M) * size_t(w->K));
    L.qs = L.s + round256(size_t(M) * 4);
    L.total = L.qs + size_t(M) * 4;
    return true;
}

size_t ll_binary_linear_workspace_size(const ll_weights* w, int64_t M) {
    if (!w || M < 1 || w->N <= 0 || w->K <= 0) return size_t(-1);
    LinearLayout L;
    return linear_layout(w, M, L) ? L.total : size_t(-1);
}

ll_status ll_binary_linear(const ll_weights* w, const uint16_t* x, int64_t M, const float* bias, uint16_t* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ll_binary_linear";
    ll_status st = check_weights(w, fn);
    if (st) return st;
    if (M < 1 || M > 65535 * 128) return ll::fail(LL_ESHAPE, "ll_binary_linear: M must be in [1, 65535*128]");
    if (w->K > (int64_t(1) << 20)) return ll::fail(LL_ERANGE, "ll_binary_linear: K <= 2^20");
    if (!x || !y) return ll::fail(LL_EINVAL, "ll_binary_linear: x or y is NULL");
    if (!aligned(x, 2) || !aligned(y, 2) || (bias && !aligned(bias, 4)))
        return ll::fail(LL_EALIGN, "ll_binary_linear: x / y must be 2-byte and bias 4-byte aligned");
    if (w->fmt == LL_FMT_W1) {
        st = check_w1_device(w, fn);
        if (st) return st;
    }
    LinearLayout L;
    if (!linear_layout(w, M, L)) return ll::fail(LL_EINVAL, "ll_binary_linear: unsupported format");
    st = check_workspace(workspace, workspace_bytes, L.total, fn);
    if (st) return st;
    char* base = static_cast<char*>(workspace);
    int8_t* q = reinterpret_cast<int8_t*>(base + L.q);
    float* s = reinterpret_cast<float*>(base + L.s);
    int32_t* qs = w->fmt == LL_FMT_I2S ? reinterpret_cast<int32_t*>(base + L.qs) : nullptr;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    st = hip_status(llk::launch_quantize(x, true, M, w->K, q, s, qs, hs), fn);
    if (st) return st;
    return hip_status(run_gemm(w, q, s, M, bias, nullptr, nullptr, base, hs, qs, y), fn);
}

}  // extern "C"
