// Prepared batches of decode products (ll_gemv_plan_* in lowbit.h): the
// host validates every item once and lays out device tables inside the
// plan memory; every later run costs two launches: one preparing the
// operands of every distinct activation (into the plan memory), one walking
// the table of products.  Every K <= 2^17: fp4 digit planes on the fp4 matrix
// cores, all M <= 16 tokens in one pass over the weights (gemv_fp4.hip);
// larger K: int8 planes on the int8 matrix cores, up to three tokens per
// pass (gemv_planes.hip).  An item may carry a
// fused epilogue: a gated pair (gate and up of one activation, y = relu(g)^2
// * u, one token) runs as workgroups of 64 rows of both matrices.
// Batches of W1A8 products (int8 activations, group 128) run on the W1
// streaming product (gemv_w1.hip): the preparation forms each distinct
// activation's fp8 digit operand, the product launch runs every matrix.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <queue>
#include <utility>
#include <vector>

#include "internal.h"
#include "launch.h"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
    size_t prob_off = 0, prep_off = 0, map_off = 0, frag_off = 0, total = 0;
    std::vector<int> prep_of;          // item -> distinct activation index
    std::vector<const void*> xs;       // distinct activations (with their norm)
    std::vector<int64_t> xk;           // their K
    std::vector<const float*> xnw;     // their RMSNorm weights (or NULL)
    std::vector<float> xeps;           // and epsilon
    std::vector<size_t> frag_at;       // byte offset of each activation's operands
    int64_t tiles = 0, kmax = 0;       // workgroups of the product launch
    bool f4 = false;                   // fp4 engine (one token)
};

ll_status check_weights(const ll_weights& w, int i, int32_t fmt0) {
    if (w.fmt != fmt0) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d has a different format", i);
    if (w.N <= 0 || w.K <= 0) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: N and K must be positive", i);
    if (w.N > (int64_t(1) << 31) - 1 || w.K > (int64_t(1) << 24))
        return ll::failf(LL_ERANGE, "ll_gemv_plan: item %d: N must be < 2^31 and K <= 2^24", i);
    if (!w.codes) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: NULL codes", i);
    if (!aligned(w.codes, 16)) return ll::failf(LL_EALIGN, "ll_gemv_plan: item %d: codes must be 16-byte aligned", i);
    if (w.fmt == LL_FMT_I2S) {
        if (w.K % 128) return ll::failf(LL_ESHAPE, "ll_gemv_plan: item %d: i2_s needs K %% 128 == 0", i);
        if (w.K > (int64_t(1) << 20))
            return ll::failf(LL_ERANGE, "ll_gemv_plan: item %d: i2_s needs K <= 2^20 (exact int32 sums)", i);
    } else if (w.fmt == LL_FMT_TQ2_0) {
        if (w.K % 256) return ll::failf(LL_ESHAPE, "ll_gemv_plan: item %d: TQ2_0 needs K %% 256 == 0", i);
        if (!w.scales) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: TQ2_0 scales pointer is NULL", i);
        if (!aligned(w.scales, 2)) return ll::failf(LL_EALIGN, "ll_gemv_plan: item %d: scales must be 2-byte aligned", i);
    } else {
        return ll::fail(LL_EINVAL, "ll_gemv_plan: fp32 activations need format i2_s or TQ2_0");
    }
    return LL_OK;
}

ll_status check_item(const ll_gemv_item_ex& it, int i, int32_t act, int64_t M, int32_t fmt0) {
    if (act != LL_ACT_F32) return ll::fail(LL_EINVAL, "ll_gemv_plan: only fp32 activations are supported");
    if (M < 1 || M > 16) return ll::fail(LL_ESHAPE, "ll_gemv_plan: M must be in [1, 16]");
    ll_status st = check_weights(it.w, i, fmt0);
    if (st) return st;
    if (!it.x || !it.y) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: NULL x or y", i);
    if (!aligned(it.x, 16)) return ll::failf(LL_EALIGN, "ll_gemv_plan: item %d: x must be 16-byte aligned", i);
    if (!aligned(it.y, 4) || (it.bias && !aligned(it.bias, 4)))
        return ll::failf(LL_EALIGN, "ll_gemv_plan: item %d: y / bias must be 4-byte aligned", i);
    if (it.norm_w) {
        if (M != 1) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: the RMSNorm prologue needs M == 1", i);
        if (!aligned(it.norm_w, 16))
            return ll::failf(LL_EALIGN, "ll_gemv_plan: item %d: norm_w must be 16-byte aligned", i);
        if (!(it.norm_eps >= 0.0f) || it.norm_eps > 3.4e38f)
            return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: norm_eps must be finite and >= 0", i);
    }
    if (it.epilogue == LL_EPI_NONE) return LL_OK;
    if (it.epilogue != LL_EPI_RELU2_MUL)
        return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: unknown epilogue %d", i, int(it.epilogue));
    if (M != 1) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: the gated pair needs M == 1", i);
    if (it.bias) return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: the gated pair takes no bias", i);
    st = check_weights(it.w2, i, fmt0);
    if (st) return st;
    if (it.w2.N != it.w.N || it.w2.K != it.w.K)
        return ll::failf(LL_ESHAPE, "ll_gemv_plan: item %d: gate and up matrices differ in N or K", i);
    return LL_OK;
}

bool is_pair(const ll_gemv_item_ex& it) { return it.epilogue == LL_EPI_RELU2_MUL; }

ll_status plan_layout(const ll_gemv_item_ex* items, int32_t count, int32_t act, int64_t M, Layout& L) {
    if (!items || count <= 0) return ll::fail(LL_EINVAL, "ll_gemv_plan: no items");
    for (int i = 0; i < count; ++i) {
        ll_status st = check_item(items[i], i, act, M, items[0].w.fmt);
        if (st) return st;
    }
    L.prep_of.assign(size_t(count), -1);
    for (int i = 0; i < count; ++i) L.kmax = std::max(L.kmax, items[i].w.K);
    L.f4 = llk::f4_engine(M, L.kmax);
    for (int i = 0; i < count; ++i)
        if ((is_pair(items[i]) || items[i].norm_w) && !L.f4)
            return ll::failf(LL_EINVAL, "ll_gemv_plan: item %d: gated pairs and norms need every K <= 2^17", i);
    for (int i = 0; i < count; ++i) {
        const int64_t rows = L.f4 ? llk::f4_batch_rows(is_pair(items[i]), items[0].w.fmt, M) : llk::planes_batch_rows();
        int found = -1;
        const float eps = items[i].norm_w ? items[i].norm_eps : 0.0f;
        for (size_t j = 0; j < L.xs.size(); ++j)
            if (L.xs[j] == items[i].x && L.xk[j] == items[i].w.K && L.xnw[j] == items[i].norm_w && L.xeps[j] == eps) {
                found = int(j);
                break;
            }
        if (found < 0) {
            found = int(L.xs.size());
            L.xs.push_back(items[i].x);
            L.xk.push_back(items[i].w.K);
            L.xnw.push_back(items[i].norm_w);
            L.xeps.push_back(eps);
        }
        L.prep_of[size_t(i)] = found;
        L.tiles += (items[i].w.N + rows - 1) / rows;              // (logical) workgroups
    }
    const size_t prob_sz = L.f4 ? llk::f4_prob_bytes() : llk::planes_prob_bytes();
    // fp4 engine: one preparation entry per token of each distinct activation
    const size_t prep_sz = L.f4 ? llk::f4_prep_bytes() * size_t(M) : llk::planes_prep_bytes();
    L.prob_off = 0;
    L.prep_off = round_up(size_t(count) * prob_sz, 256);
    L.map_off = round_up(L.prep_off + L.xs.size() * prep_sz, 256);
    L.frag_off = round_up(L.map_off + size_t(L.tiles) * 4, 256);
    size_t at = L.frag_off;
    for (size_t j = 0; j < L.xs.size(); ++j) {
        L.frag_at.push_back(at);
        const size_t bytes = L.f4 ? llk::f4_operand_bytes(M, L.xk[j]) : llk::planes_operand_bytes(M, L.xk[j]);
        at = round_up(at + bytes, 256);
    }
    L.total = at;
    if (L.tiles > (int64_t(1) << 31) - 1 || L.xs.size() > 65535)
        return ll::fail(LL_ERANGE, "ll_gemv_plan: batch too large");
    return LL_OK;
}

// plain items as items without a fused epilogue
std::vector<ll_gemv_item_ex> widen(const ll_gemv_item* items, int32_t count) {
    std::vector<ll_gemv_item_ex> ex(static_cast<size_t>(count));
    for (int32_t i = 0; i < count; ++i) {
        ll_gemv_item_ex e;
        std::memset(&e, 0, sizeof e);
        e.w = items[i].w;
        e.x = items[i].x;
        e.bias = items[i].bias;
        e.y = items[i].y;
        e.epilogue = LL_EPI_NONE;
        ex[size_t(i)] = e;
    }
    return ex;
}

// ---------------------------------------------------------------- W1A8 batches
struct LayoutI8 {
    size_t prob_off = 0, prep_off = 0, map_off = 0, frag_off = 0, total = 0;
    std::vector<int> prep_of;
    std::vector<const int8_t*> xq;
    std::vector<int64_t> xk, blk0;
    std::vector<size_t> frag_at;
    int64_t tiles = 0, kmax = 0, prep_blocks = 0;    // tiles: the most workgroups any assignment uses
    bool scv = true;                   // every K a multiple of 1024
};

// Workgroups per product: start from one each and give the next one to the
// product whose waves have the longest stream of windows (a wave's blocks x
// windows per block), while the total stays within the resident workgroups
// and each product has at most one block per wave.  slots <= 0 (unknown):
// one block per wave everywhere.
std::vector<int64_t> assign_w1_wgs(const ll_gemv_item_i8* items, int32_t count, int64_t slots) {
    std::vector<int64_t> wgs(size_t(count), 1);
    if (slots <= 0) {
        for (int i = 0; i < count; ++i) wgs[size_t(i)] = llk::w1_batch_wgs(items[i].w.N);
        return wgs;
    }
    auto windows = [&](int i) {
        const int64_t per_wave = (llk::w1_batch_blocks(items[i].w.N) + 8 * wgs[size_t(i)] - 1) / (8 * wgs[size_t(i)]);
        return per_wave * ((items[i].w.K + 1023) / 1024);
    };
    std::priority_queue<std::pair<int64_t, int>> heap;
    for (int i = 0; i < count; ++i) heap.push({windows(i), i});
    int64_t total = count;
    while (total < slots && !heap.empty()) {
        const int i = heap.top().second;
        heap.pop();
        if (wgs[size_t(i)] >= llk::w1_batch_wgs(items[i].w.N)) continue;    // one block per wave already
        ++wgs[size_t(i)];
        ++total;
        heap.push({windows(i), i});
    }
    return wgs;
}

ll_status check_item_i8(const ll_gemv_item_i8& it, int i, int64_t M) {
    const ll_weights& w = it.w;
    if (w.fmt != LL_FMT_W1) return ll::failf(LL_EINVAL, "ll_gemv_plan_i8: item %d: int8 activations need format W1", i);
    if (w.N <= 0 || w.K <= 0) return ll::failf(LL_EINVAL, "ll_gemv_plan_i8: item %d: N and K must be positive", i);
    if (w.N > (int64_t(1) << 31) - 1 || w.K > (int64_t(1) << 24))
        return ll::failf(LL_ERANGE, "ll_gemv_plan_i8: item %d: N must be < 2^31 and K <= 2^24", i);
    if (w.group != 128 || w.K % 128)
        return ll::failf(LL_ESHAPE, "ll_gemv_plan_i8: item %d: group 128 and K %% 128 == 0 required", i);
    if (!w.codes || !w.scales || !it.xq || !it.xs || !it.y)
        return ll::failf(LL_EINVAL, "ll_gemv_plan_i8: item %d: NULL codes, scales, xq, xs or y", i);
    if (!aligned(w.codes, 16) || !aligned(w.scales, 2))
        return ll::failf(LL_EALIGN, "ll_gemv_plan_i8: item %d: codes must be 16-byte, scales 2-byte aligned", i);
    if (!aligned(it.xq, 16) || !aligned(it.xs, 4) || !aligned(it.y, 4) || (it.bias && !aligned(it.bias, 4)))
        return ll::failf(LL_EALIGN, "ll_gemv_plan_i8: item %d: xq must be 16-byte, xs / y / bias 4-byte aligned", i);
    if (!llk::w1_batch_fits(M, w.K))
        return ll::failf(LL_ERANGE, "ll_gemv_plan_i8: item %d: the operand of %lld tokens x K = %lld is too large", i,
                         static_cast<long long>(M), static_cast<long long>(w.K));
    return LL_OK;
}

ll_status plan_layout_i8(const ll_gemv_item_i8* items, int32_t count, int64_t M, LayoutI8& L) {
    if (!items || count <= 0) return ll::fail(LL_EINVAL, "ll_gemv_plan_i8: no items");
    if (M < 1 || M > 8) return ll::fail(LL_ESHAPE, "ll_gemv_plan_i8: M must be in [1, 8]");
    for (int i = 0; i < count; ++i) {
        ll_status st = check_item_i8(items[i], i, M);
        if (st) return st;
    }
    L.prep_of.assign(size_t(count), -1);
    for (int i = 0; i < count; ++i) {
        const int64_t K = items[i].w.K;
        L.kmax = std::max(L.kmax, K);
        L.scv = L.scv && K % 1024 == 0;
        int found = -1;
        for (size_t j = 0; j < L.xq.size(); ++j)
            if (L.xq[j] == items[i].xq && L.xk[j] == K) {
                found = int(j);
                break;
            }
        if (found < 0) {
            found = int(L.xq.size());
            L.xq.push_back(items[i].xq);
            L.xk.push_back(K);
            L.blk0.push_back(L.prep_blocks);
            L.prep_blocks += llk::w1_batch_prep_blocks(M, K);
        }
        L.prep_of[size_t(i)] = found;
        L.tiles += llk::w1_batch_wgs(items[i].w.N);
    }
    L.prob_off = 0;
    L.prep_off = round_up(size_t(count) * llk::w1_batch_prob_bytes(), 256);
    L.map_off = round_up(L.prep_off + L.xq.size() * llk::w1_batch_prep_bytes(), 256);
    L.frag_off = round_up(L.map_off + size_t(L.tiles) * 4, 256);
    size_t at = L.frag_off;
    for (size_t j = 0; j < L.xq.size(); ++j) {
        L.frag_at.push_back(at);
        at = round_up(at + llk::w1_batch_operand_bytes(M, L.xk[j]), 256);
    }
    L.total = at;
    if (L.tiles > (int64_t(1) << 31) - 1 || L.prep_blocks > (int64_t(1) << 31) - 1 || L.xq.size() > 65535)
        return ll::fail(LL_ERANGE, "ll_gemv_plan_i8: batch too large");
    return LL_OK;
}

ll_status check_plan(const ll_gemv_plan* p) {
    if (!p || !p->mem || !p->prob_table || !p->prep_table || !p->map_table || p->count <= 0 || p->nprep <= 0)
        return ll::fail(LL_EINVAL, "ll_gemv_plan: plan not initialised");
    return LL_OK;
}

ll_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return LL_OK;
    return ll::failf(LL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t ll_gemv_plan_bytes_ex(const ll_gemv_item_ex* items, int32_t count, int32_t act, int64_t M) {
    Layout L;
    if (plan_layout(items, count, act, M, L)) return size_t(-1);
    return L.total;
}

ll_status ll_gemv_plan_init_ex(const ll_gemv_item_ex* items, int32_t count, int32_t act, int64_t M, void* mem,
                               size_t bytes, ll_gemv_plan* plan) {
    if (!plan) return ll::fail(LL_EINVAL, "ll_gemv_plan_init: plan is NULL");
    Layout L;
    ll_status st = plan_layout(items, count, act, M, L);
    if (st) return st;
    if (!mem || bytes < L.total) return ll::failf(LL_EWORKSPACE, "ll_gemv_plan_init: %zu device bytes required", L.total);
    if (!aligned(mem, 16)) return ll::fail(LL_EALIGN, "ll_gemv_plan_init: mem must be 16-byte aligned");
    char* base = static_cast<char*>(mem);
    std::vector<char> host(L.frag_off, 0);
    int32_t* map = reinterpret_cast<int32_t*>(host.data() + L.map_off);
    int64_t first = 0;
    for (int i = 0; i < count; ++i) {
        const ll_gemv_item_ex& it = items[i];
        const bool pair = is_pair(it);
        char* ops = base + L.frag_at[size_t(L.prep_of[size_t(i)])];
        if (L.f4)
            llk::fill_f4_prob(host.data() + L.prob_off + size_t(i) * llk::f4_prob_bytes(), it.w.codes, it.w.scales,
                              ops, it.bias, it.y, it.w.N, it.w.K, first, pair ? it.w2.codes : nullptr,
                              pair ? it.w2.scales : nullptr, M);
        else
            llk::fill_planes_prob(host.data() + L.prob_off + size_t(i) * llk::planes_prob_bytes(), it.w.codes,
                                  it.w.scales, ops, it.bias, it.y, it.w.N, it.w.K, first);
        const int64_t rows = L.f4 ? llk::f4_batch_rows(pair, items[0].w.fmt, M) : llk::planes_batch_rows();
        const int64_t wgs = (it.w.N + rows - 1) / rows;
        for (int64_t g = 0; g < wgs; ++g) map[first + g] = i;
        first += wgs;
    }
    for (size_t j = 0; j < L.xs.size(); ++j) {
        const float* x = static_cast<const float*>(L.xs[j]);
        if (L.f4)
            for (int64_t m = 0; m < M; ++m)
                llk::fill_f4_prep(host.data() + L.prep_off + (j * size_t(M) + size_t(m)) * llk::f4_prep_bytes(),
                                  x + m * L.xk[j], base + L.frag_at[j] + m * llk::f4_op_stride(L.xk[j]), L.xk[j],
                                  L.xnw[j], L.xeps[j]);
        else
            llk::fill_planes_prep(host.data() + L.prep_off + j * llk::planes_prep_bytes(), x, base + L.frag_at[j],
                                  L.xk[j]);
    }
    st = hip_status(hipMemcpy(mem, host.data(), host.size(), hipMemcpyHostToDevice), "ll_gemv_plan_init");
    if (st) return st;
    ll_gemv_plan p;
    std::memset(&p, 0, sizeof p);
    p.mem = mem;
    p.bytes = L.total;
    p.count = count;
    p.nprep = int32_t(L.xs.size());
    p.act = act;
    p.fmt = items[0].w.fmt;
    p.M = M;
    p.tiles = L.tiles;
    p.prep_entries = int64_t(L.xs.size()) * M;          // preparation workgroups (one per token)
    p.kmax = L.kmax;
    p.prob_table = base + L.prob_off;
    p.prep_table = base + L.prep_off;
    p.map_table = base + L.map_off;
    p.epilogues = 0;
    for (int i = 0; i < count; ++i) p.epilogues |= is_pair(items[i]) ? 1 : 0;
    *plan = p;
    return LL_OK;
}

size_t ll_gemv_plan_bytes(const ll_gemv_item* items, int32_t count, int32_t act, int64_t M) {
    if (!items || count <= 0) return size_t(-1);
    const std::vector<ll_gemv_item_ex> ex = widen(items, count);
    return ll_gemv_plan_bytes_ex(ex.data(), count, act, M);
}

ll_status ll_gemv_plan_init(const ll_gemv_item* items, int32_t count, int32_t act, int64_t M, void* mem, size_t bytes,
                            ll_gemv_plan* plan) {
    if (!items || count <= 0) return ll::fail(LL_EINVAL, "ll_gemv_plan: no items");
    const std::vector<ll_gemv_item_ex> ex = widen(items, count);
    return ll_gemv_plan_init_ex(ex.data(), count, act, M, mem, bytes, plan);
}

size_t ll_gemv_plan_bytes_i8(const ll_gemv_item_i8* items, int32_t count, int64_t M) {
    LayoutI8 L;
    if (plan_layout_i8(items, count, M, L)) return size_t(-1);
    return L.total;
}

ll_status ll_gemv_plan_init_i8(const ll_gemv_item_i8* items, int32_t count, int64_t M, void* mem, size_t bytes,
                               ll_gemv_plan* plan) {
    if (!plan) return ll::fail(LL_EINVAL, "ll_gemv_plan_init_i8: plan is NULL");
    LayoutI8 L;
    ll_status st = plan_layout_i8(items, count, M, L);
    if (st) return st;
    if (!mem || bytes < L.total)
        return ll::failf(LL_EWORKSPACE, "ll_gemv_plan_init_i8: %zu device bytes required", L.total);
    if (!aligned(mem, 16)) return ll::fail(LL_EALIGN, "ll_gemv_plan_init_i8: mem must be 16-byte aligned");
    char* base = static_cast<char*>(mem);
    std::vector<char> host(L.frag_off, 0);
    int32_t* map = reinterpret_cast<int32_t*>(host.data() + L.map_off);
    const std::vector<int64_t> wgs = assign_w1_wgs(items, count, llk::w1_batch_slots(M, L.kmax, L.scv));
    int64_t first = 0;
    for (int i = 0; i < count; ++i) {
        const ll_gemv_item_i8& it = items[i];
        const char* ops = base + L.frag_at[size_t(L.prep_of[size_t(i)])];
        llk::fill_w1_prob(host.data() + L.prob_off + size_t(i) * llk::w1_batch_prob_bytes(), it.w.codes, it.w.scales,
                          ops, it.xs, it.bias, it.y, it.w.N, it.w.K, first, wgs[size_t(i)]);
        for (int64_t g = 0; g < wgs[size_t(i)]; ++g) map[first + g] = i;
        first += wgs[size_t(i)];
    }
    for (size_t j = 0; j < L.xq.size(); ++j)
        llk::fill_w1_prep(host.data() + L.prep_off + j * llk::w1_batch_prep_bytes(), L.xq[j], base + L.frag_at[j], M,
                          L.xk[j], L.blk0[j]);
    st = hip_status(hipMemcpy(mem, host.data(), host.size(), hipMemcpyHostToDevice), "ll_gemv_plan_init_i8");
    if (st) return st;
    ll_gemv_plan p;
    std::memset(&p, 0, sizeof p);
    p.mem = mem;
    p.bytes = L.total;
    p.count = count;
    p.nprep = int32_t(L.xq.size());
    p.act = LL_ACT_I8;
    p.fmt = LL_FMT_W1;
    p.M = M;
    p.tiles = first;                                    // workgroups of the product launch
    p.prep_entries = L.prep_blocks;                     // preparation blocks
    p.kmax = L.kmax;
    p.prob_table = base + L.prob_off;
    p.prep_table = base + L.prep_off;
    p.map_table = base + L.map_off;
    p.flags = L.scv ? 1 : 0;
    *plan = p;
    return LL_OK;
}

ll_status ll_gemv_plan_prepare(const ll_gemv_plan* plan, void* stream) {
    ll_status st = check_plan(plan);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan->act == LL_ACT_I8)
        return hip_status(llk::launch_w1_batch_prep(plan->prep_table, plan->nprep, plan->prep_entries, plan->M, s),
                          "ll_gemv_plan_prepare");
    if (llk::f4_engine(plan->M, plan->kmax))
        return hip_status(llk::launch_f4_batch_prep(plan->prep_table, int(plan->prep_entries), plan->fmt, plan->kmax,
                                                    s),
                          "ll_gemv_plan_prepare");
    return hip_status(llk::launch_planes_batch_prep(plan->prep_table, plan->nprep, plan->fmt, plan->M, s),
                      "ll_gemv_plan_prepare");
}

ll_status ll_gemv_plan_product(const ll_gemv_plan* plan, void* stream) {
    ll_status st = check_plan(plan);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan->act == LL_ACT_I8)
        return hip_status(llk::launch_w1_batch_product(plan->prob_table, plan->map_table, plan->tiles, plan->M,
                                                       plan->kmax, (plan->flags & 1) != 0, s),
                          "ll_gemv_plan_product");
    if (llk::f4_engine(plan->M, plan->kmax))
        return hip_status(llk::launch_f4_batch_product(plan->prob_table, plan->map_table, plan->fmt, plan->tiles,
                                                       plan->kmax, plan->epilogues != 0, plan->M, s),
                          "ll_gemv_plan_product");
    return hip_status(llk::launch_planes_batch_product(plan->prob_table, plan->map_table, plan->fmt, plan->M,
                                                       plan->tiles, s),
                      "ll_gemv_plan_product");
}

ll_status ll_gemv_plan_run(const ll_gemv_plan* plan, void* stream) {
    ll_status st = ll_gemv_plan_prepare(plan, stream);
    if (st) return st;
    return ll_gemv_plan_product(plan, stream);
}

}  // extern "C"
