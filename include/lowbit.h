/*
 * lowbit.h -- C ABI of the packed low-bit BitLinear library for AMD MI355X
 * (gfx950).  The library computes
 *
 *     y[m, n] = scale * sum_k w[n, k] * x[m, k]
 *
 * reading ternary or binary weights directly in their packed layouts.
 *
 * Sources of the operations declared here:
 *   [BL] Hesper API doc "Hesper/Layers/BitLinear": "i2_s Packing Format"
 *        (code table, 128-element / 32-byte groups at shifts 6/4/2/0, one
 *        fp32 scale at the end of the tensor data), "BitLinear Mathematics"
 *        (the product), "High-Level API" (4-byte little-endian scale,
 *        forward(in, out)).
 *   [TQ] Hesper API doc "Hesper/Quantization/TQ2_0": "TQ2_0 Format"
 *        (256-element blocks, 64 packed bytes + fp16 scale = 66 bytes,
 *        codes 0b11/0b00/0b01), "GPU Unpacking Kernel" (packed codes and
 *        fp16 scales as two separate device buffers).
 *   [BG] binary-gemm kernel card: "API" (pack_weights, unpack_weights,
 *        quantize_activation, binary_gemm), "Method" (stored bit
 *        b = (w+1)/2, per-group fp16 scales, dot identity), "Usage"
 *        (from_dense), "Requirements and limits" (K a multiple of 32 and of
 *        the group size).
 *
 * Conventions for every function:
 *   - Matrices are row-major: x is [M, K], y is [M, N], weights are [N, K]
 *     (y = x * W^T).
 *   - Host functions take host pointers; device functions take device
 *     pointers allocated by the caller (for example torch tensors).  The
 *     library never frees, and no device function allocates or
 *     synchronizes: kernels are enqueued on `stream` (a hipStream_t; NULL
 *     means the default stream) and the call returns.
 *   - Every argument is validated on the host before anything is written or
 *     launched.  On error the function returns a negative ll_status, leaves
 *     every output untouched, and ll_last_error() describes the problem.
 *   - Device pointers must be 16-byte aligned (LL_EALIGN otherwise).
 *   - Workspaces.  A device entry point that needs scratch memory takes a
 *     caller-owned device buffer, 16-byte aligned, of at least the size its
 *     ll_*_workspace_size function returns (LL_EWORKSPACE otherwise).  The
 *     first LL_WORKSPACE_COUNTER_BYTES bytes of every workspace hold only
 *     split-K arrival counters: zero-fill the buffer (at least those bytes)
 *     once before its first use.  Every call leaves the counters zero and
 *     writes nothing else there, so one buffer serves calls of any entry
 *     point, format and shape in turn (an M = 8 call followed by an M = 1
 *     call, say).  The rest of the buffer is overwritten by each call.
 *     Calls that can overlap in time (different streams, or a graph replayed
 *     concurrently) must not share a workspace.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LL_ABI_VERSION 5

/* Bytes at the start of every workspace reserved for split-K counters. */
#define LL_WORKSPACE_COUNTER_BYTES 4096

typedef enum {
    LL_OK = 0,
    LL_EINVAL = -1,      /* null pointer, unknown enum, non-positive size */
    LL_ESHAPE = -2,      /* K not a multiple of the format's group/block, M outside the entry point's range */
    LL_EALIGN = -3,      /* a device pointer is not 16-byte aligned */
    LL_ECODE = -4,       /* weight value outside the format's alphabet, or an invalid packed code */
    LL_EWORKSPACE = -5,  /* workspace missing or smaller than ll_*_workspace_size() */
    LL_EHIP = -6,        /* HIP runtime error (no device, launch failure); detail in ll_last_error() */
    LL_ERANGE = -7       /* a size does not fit the kernel's index arithmetic */
} ll_status;

typedef enum {
    LL_FMT_I2S = 1,      /* [BL] ternary, 2-bit codes, one fp32 scale per tensor */
    LL_FMT_TQ2_0 = 2,    /* [TQ] ternary, 256-element blocks, fp16 scale per block */
    LL_FMT_W1 = 3        /* [BG] binary sign bits, fp16 scale per G weights */
} ll_format;

typedef enum {
    LL_ACT_F32 = 1,      /* activations fp32 [M, K] */
    LL_ACT_I8 = 2        /* activations int8 [M, K] with one fp32 scale per token (ll_quantize_act) */
} ll_act;

typedef enum {
    LL_DT_F32 = 1,
    LL_DT_BF16 = 2
} ll_dtype;

/*
 * A packed weight matrix resident in device memory.
 *   LL_FMT_I2S : codes  = N*K/4 packed bytes followed by the 4-byte
 *                         little-endian fp32 scale (exactly the output of
 *                         ll_pack_i2s); scales = NULL.  K % 128 == 0.
 *   LL_FMT_TQ2_0: codes = the 64 code bytes of every block, blocks in
 *                         order (N*K/4 bytes); scales = fp16 [N*K/256], one
 *                         per block in the same order (ll_tq2_split turns
 *                         66-byte blocks into these two arrays).  K % 256 == 0.
 *   LL_FMT_W1  : codes  = uint32 [N, K/32] sign bits (ll_pack_w1);
 *                scales = fp16 [N, K/group].  K % 32 == 0, K % group == 0.
 * group: W1 scale group size G (> 0, multiple of 32); ignored otherwise.
 * Every device entry point takes 1 <= N < 2^31 and 1 <= K <= 2^24, and i2_s
 * K <= 2^20 (its products keep exact int32 sums of whole rows; larger K is
 * LL_ERANGE).
 */
typedef struct {
    int32_t fmt;         /* ll_format */
    int32_t group;
    int64_t N, K;
    const void* codes;
    const void* scales;
} ll_weights;

/* ------------------------------------------------------------------ */
/* Library information                                                  */
/* ------------------------------------------------------------------ */

int ll_abi_version(void);
const char* ll_strerror(int status);
/* Text of the last error raised on the calling thread ("" if none). */
const char* ll_last_error(void);

/* ------------------------------------------------------------------ */
/* Host-side formats (CPU, host pointers, caller-owned buffers)          */
/* ------------------------------------------------------------------ */

/* Bytes of the packed codes of an N x K matrix in format fmt (the i2_s
   count includes its 4-byte tail scale; TQ2_0 counts the 66-byte blocks).
   *scales_bytes (if not NULL) receives the size of the separate scale array
   (0 for i2_s; 2*N*K/256 for the split TQ2_0 device layout; 2*N*K/group for
   W1).  Returns 0 for an invalid shape. */
size_t ll_packed_size(int32_t fmt, int64_t N, int64_t K, int32_t group, size_t* scales_bytes);

/* [BL "i2_s Packing Format"] w: int8 [N,K] in {-1,0,+1}; out: N*K/4 + 4
   bytes.  Code of w is w+1 (-1 -> 0b00, 0 -> 0b01, +1 -> 0b10); element r of
   each 128-element group goes to byte r%32 of the group's 32 bytes at shift
   6 - 2*(r/32); the scale is appended as 4 little-endian bytes.
   LL_ESHAPE if K % 128, LL_ECODE for a value outside {-1,0,1}. */
ll_status ll_pack_i2s(const int8_t* w, int64_t N, int64_t K, float scale, uint8_t* out);
/* Inverse of ll_pack_i2s.  LL_ECODE if a code 0b11 occurs (w is then
   filled anyway, that element as +2). scale may be NULL. */
ll_status ll_unpack_i2s(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, float* scale);

/* [TQ "TQ2_0 Format"] w: int8 [N,K] in {-1,0,+1}; scales: fp16 bits
   [N*K/256] (block order); out: 66*N*K/256 bytes of blocks (64 code bytes,
   then scale_low, scale_high).  Codes 0 -> 0b00, +1 -> 0b01, -1 -> 0b11;
   element e of a block sits in byte e/4 at bits 2*(e%4).
   LL_ESHAPE if K % 256, LL_ECODE for a value outside {-1,0,1}. */
ll_status ll_pack_tq2(const int8_t* w, const uint16_t* scales, int64_t N, int64_t K, uint8_t* out);
/* Inverse of ll_pack_tq2; LL_ECODE if a code 0b10 occurs (decoded as -2). */
ll_status ll_unpack_tq2(const uint8_t* blocks, int64_t N, int64_t K, int8_t* w, uint16_t* scales);
/* [TQ "GPU Unpacking Kernel": separate packed and scale buffers] 66-byte
   blocks -> codes (N*K/4 bytes) + scales (fp16 [N*K/256]). */
ll_status ll_tq2_split(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);

/* [BG "API": pack_weights] w: int8 [N,K]; bit k%32 of word n*(K/32)+k/32
   is 1 where w > 0 (stored bit (w+1)/2; zeros store 0, i.e. -1).
   LL_ESHAPE if K % 32. */
ll_status ll_pack_w1(const int8_t* w, int64_t N, int64_t K, uint32_t* out);
/* [BG "API": unpack_weights] bits -> int8 {-1,+1} [N,K]. */
ll_status ll_unpack_w1(const uint32_t* bits, int64_t N, int64_t K, int8_t* w);
/* [BG "Usage": from_dense, sign + group mean-abs scale] W: fp32 [N,K].
   bits as ll_pack_w1 of sign(W) (W > 0 -> +1); scales[n, g] = fp16 (round
   to nearest even) of mean_{k in g} |W[n,k]| accumulated in fp64.
   LL_ESHAPE unless K % 32 == 0, group > 0 and K % group == 0. */
ll_status ll_w1_from_dense(const float* W, int64_t N, int64_t K, int32_t group, uint32_t* bits, uint16_t* scales);

/* Checks a host copy of packed codes: LL_ECODE for an invalid code (i2_s
   0b11, TQ2_0 0b10; W1 has none), *bad_index (may be NULL) = element index
   n*K+k of the first one, else -1.  For TQ2_0, codes is the split layout. */
ll_status ll_validate(int32_t fmt, const void* codes, int64_t N, int64_t K, int64_t* bad_index);

/* ------------------------------------------------------------------ */
/* Device entry points (gfx950)                                          */
/* ------------------------------------------------------------------ */

/* [BG "API": quantize_activation] Per-token absmax quantization.
   x: device [M,K] fp32 or bf16 (x_dtype); xq: device int8 [M,K];
   xs: device fp32 [M].  For each token: a = max|x|; a == 0 gives s = 0 and
   q = 0; else inv = 127/a (IEEE fp32 division), q = round-half-even(x*inv)
   clamped to [-127,127], s = a/127.  xsum: device int32 [M] receiving
   sum_k q[m,k] (the per-token term of the offset form sum_k w q =
   sum_k (w+1) q - sum_k q), or NULL.  1 <= M, 1 <= K <= 2^20. */
ll_status ll_quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                          int8_t* xq, float* xs, int32_t* xsum, void* stream);

/* Bytes of device workspace ll_bitlinear_gemv needs for these arguments
   (0 when none is needed).  Returns (size_t)-1 for invalid arguments. */
size_t ll_gemv_workspace_size(const ll_weights* w, int32_t act, int64_t M);

/* [BL "Fused BitLinear Kernel", "M=1 Warp-Cooperative" ; BG "API":
   binary_gemm] Decode-size product, 1 <= M <= 16, reading the packed codes
   in the kernel.  act == LL_ACT_F32: x fp32 [M,K], xs unused (NULL); formats
   i2_s and TQ2_0; y = scale * sum_k w*x (i2_s) or sum over blocks of
   s_block * sum w*x (TQ2_0), within 1e-5 * scale * sum|x| (+1e-6) of the
   exact value (x split into five int8 planes per token, exact integer sums,
   fp64 epilogue; up to three tokens per pass over the weights).
   act == LL_ACT_I8: x int8 [M,K], xs fp32 [M] from ll_quantize_act; formats
   i2_s (y = ((float)acc * xs[m]) * scale, acc exact int32, the same bits as
   ll_bitlinear_gemm), TQ2_0 (y = (float)((double)xs[m] * sum_b s_b * acc_b),
   acc_b the exact block sums) and W1 (y = (float)((double)xs[m] *
   sum_g s_g * d_g), d_g the exact per-group integer dot); i2_s and TQ2_0
   take all M tokens in one pass over the weights and need no workspace.
   bias: device fp32 [N] added last, or NULL.  y: device fp32
   [M,N].  workspace: at least ll_gemv_workspace_size(w, act, M) bytes (may
   be NULL when that is 0), under the workspace rules above; with W1 weights
   it holds the prepared activation digits (group sizes other than 128, or
   more than two tokens), and a narrow matrix whose activation operand is
   too large for one workgroup's memory splits K over workgroups, which
   publish partial sums there and count their arrivals in the workspace's
   counter region. */
ll_status ll_bitlinear_gemv(const ll_weights* w, int32_t act, const void* x, const float* xs,
                            int64_t M, const float* bias, float* y,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Prepared batch of decode products                                     */
/* ------------------------------------------------------------------ */

/* [BL "High-Level API" / layer header: PreparedDispatch fast path replayed
   per forward call; "Execute forward pass" for each layer] Many independent
   decode products y_i = W_i x_i (for example every BitLinear of a decode
   step) prepared once and then run with two launches per call: one that
   lays every distinct activation out as matrix-core operands, one that
   walks a device-resident table of all products.  All items share act,
   format and M (1 <= M <= 16); N and K may differ.  Only act == LL_ACT_F32
   with i2_s or TQ2_0 is supported.  Items with the same x pointer and K
   share one activation layout: with every K <= 2^17, twelve balanced base-8
   fp4 digit planes per token, multiplied on the fp4 matrix cores with all M
   tokens in one pass over the weights (two passes for M > 8; y within the
   same tolerance as ll_bitlinear_gemv); otherwise the int8 planes of
   ll_bitlinear_gemv. */
typedef struct {
    ll_weights w;        /* packed weights (device pointers, as for ll_bitlinear_gemv) */
    const void* x;       /* device fp32 [M, K] */
    const float* bias;   /* device fp32 [N] or NULL */
    float* y;            /* device fp32 [M, N] */
} ll_gemv_item;

typedef struct {
    void* mem;           /* device memory given to ll_gemv_plan_init (caller-owned) */
    size_t bytes;
    int32_t count, nprep, act, fmt;
    int64_t M, tiles, prep_entries, kmax;
    void* prob_table;    /* inside mem */
    void* prep_table;    /* inside mem */
    void* map_table;     /* inside mem: product index of every workgroup */
    int32_t epilogues;   /* nonzero when some item has a fused epilogue */
    int32_t flags;       /* launch variant chosen by the init call */
} ll_gemv_plan;

/* Fused epilogues of a prepared product.
   LL_EPI_NONE: y = W x (+ bias).  With M == 1 the bias operand is the
     residual stream of [BL "Fused BitLinear + Residual Add Kernel"] and "M=1
     warp-cooperative kernel with fused residual add": y = residual + W x,
     the add done last in fp32.
   LL_EPI_RELU2_MUL [BL "Fused Gate+Up+ReLU²×Mul M=1 Kernel"]: two products
     of one activation, gate = W x and up = W2 x (each rounded to fp32 as a
     plain product would be), and y = (r * r) * up with r = max(0, gate), two
     fp32 multiplies in that order.  W and W2 must have the same format, N
     and K; M must be 1 (the fp4 engine); bias must be NULL.  The two
     matrices are read in one pass over x's operands. */
typedef enum { LL_EPI_NONE = 0, LL_EPI_RELU2_MUL = 1 } ll_epilogue;

typedef struct {
    ll_weights w;        /* packed weights; the gate for LL_EPI_RELU2_MUL */
    ll_weights w2;       /* LL_EPI_RELU2_MUL: the up weights; ignored otherwise */
    const void* x;       /* device fp32 [M, K] */
    const float* bias;   /* device fp32 [N] or NULL (LL_EPI_NONE only) */
    float* y;            /* device fp32 [M, N] */
    int32_t epilogue;    /* ll_epilogue */
    float norm_eps;      /* RMSNorm epsilon (>= 0), with norm_w */
    const float* norm_w; /* RMSNorm prologue [BL "Fused RMSNorm + BitLinear + Residual Add M=1
                            Kernel"]: device fp32 [K] (16-byte aligned), or NULL.  The product
                            then multiplies xn = (x * rinv) * norm_w, rinv = 1 / sqrt(sum_k x^2 / K
                            + norm_eps) (sum and root in fp64, rinv rounded to fp32, two fp32
                            multiplies; a zero row with norm_eps = 0 gives xn = 0).  M == 1 only. */
} ll_gemv_item_ex;

/* Device bytes ll_gemv_plan_init needs for these items ((size_t)-1 for
   invalid arguments). */
size_t ll_gemv_plan_bytes(const ll_gemv_item* items, int32_t count, int32_t act, int64_t M);
/* Validates every item (same rules and status codes as ll_bitlinear_gemv),
   writes the product and activation tables into mem with a synchronous
   host-to-device copy and fills *plan.  mem (16-byte aligned, at least
   ll_gemv_plan_bytes) must stay allocated, and every pointer in the items
   valid, for as long as the plan is run.  This is the only call here that
   synchronizes. */
ll_status ll_gemv_plan_init(const ll_gemv_item* items, int32_t count, int32_t act, int64_t M,
                            void* mem, size_t bytes, ll_gemv_plan* plan);
/* The same for items with a fused epilogue (ll_gemv_item_ex); plain items
   are LL_EPI_NONE with w2 unused.  An invalid epilogue code, a gated pair
   whose matrices differ in format, N or K, a gated pair with M != 1 or a
   bias is LL_EINVAL (LL_ESHAPE for the shape mismatch); so is a norm with
   M != 1 or a negative or non-finite epsilon.  Items sharing x, K, norm_w
   and norm_eps share one prepared operand. */
size_t ll_gemv_plan_bytes_ex(const ll_gemv_item_ex* items, int32_t count, int32_t act, int64_t M);
ll_status ll_gemv_plan_init_ex(const ll_gemv_item_ex* items, int32_t count, int32_t act, int64_t M,
                               void* mem, size_t bytes, ll_gemv_plan* plan);
/* [BG "Method", "API": binary_gemm; BL "High-Level API": PreparedDispatch]
   A prepared batch of W1A8 products: binary weights with group size 128
   and int8 activations, 1 <= M <= 8, every product as ll_bitlinear_gemv
   computes it (bit-exact: y = (float)((double)xs[m] * sum_g s_g * d_g),
   then + bias).  Items with the same xq pointer and K share one prepared
   operand.  Each item's K must leave the operand of M tokens within the
   streaming product's workgroup memory: (K / 128) * 2M * 144 + 4 (M K / 128
   + 4) + 64 <= 114688 bytes (M = 1: K <= 50,176; M = 8: K <= 6,272), else
   LL_ERANGE.  Validation otherwise as
   ll_bitlinear_gemv (LL_EINVAL for another format or a missing pointer,
   LL_ESHAPE for a group other than 128 or K % 128 != 0, LL_EALIGN for xq
   not 16-byte aligned or xs, y, bias not 4-byte aligned).  Run with
   ll_gemv_plan_run / _prepare / _product like the plans above. */
typedef struct {
    ll_weights w;        /* W1 weights, group 128 (device pointers) */
    const int8_t* xq;    /* device int8 [M, K] */
    const float* xs;     /* device fp32 [M] per-token scales */
    const float* bias;   /* device fp32 [N] or NULL */
    float* y;            /* device fp32 [M, N] */
} ll_gemv_item_i8;
size_t ll_gemv_plan_bytes_i8(const ll_gemv_item_i8* items, int32_t count, int64_t M);
ll_status ll_gemv_plan_init_i8(const ll_gemv_item_i8* items, int32_t count, int64_t M, void* mem, size_t bytes,
                               ll_gemv_plan* plan);
/* Both launches: ll_gemv_plan_prepare, then ll_gemv_plan_product. */
ll_status ll_gemv_plan_run(const ll_gemv_plan* plan, void* stream);
/* Lays out the current contents of every x as operands (inside mem). */
ll_status ll_gemv_plan_prepare(const ll_gemv_plan* plan, void* stream);
/* The products from the last prepared activations; writes every y. */
ll_status ll_gemv_plan_product(const ll_gemv_plan* plan, void* stream);

/* [BL "Subgroup-Matrix Multi-row BitLinear Kernel"; BG "Requirements and
   limits": route prefill elsewhere] Prefill-size product, M >= 1 (meant for
   M > 16), int8 activations with int8 MFMA and exact int32 accumulation.
   Format i2_s: y = ((float)acc * xs[m]) * scale.  xq: device int8 [M,K];
   xs: device fp32 [M]; bias: device fp32 [N] or NULL; y: device fp32 [M,N];
   acc_out: device int32 [M,N] receiving the raw integer dot (or NULL; i2_s
   only).  Format TQ2_0 [TQ "TQ2_0 Format"; with int8 activations]: each
   256-k block's exact int32 dot d_b is scaled by its fp16 scale into fp32,
   y = (sum_b s_b * d_b) * xs[m] (+ bias), within 1e-5 * xs[m] * sum_b |s_b|
   * sum_{k in b} |q_k| (+1e-6) of the exact value; the same result for
   every split of K.  Format W1 [BG "Method"]: with group size 128 and
   M > 16 on the int8 matrix cores, each group's exact int32 dot scaled by
   its fp16 scale into fp32, y = (sum_g s_g * d_g) * xs[m] (+ bias), within
   1e-5 * xs[m] * sum_g |s_g| * sum_{k in g} |q_k| (+1e-6) of the exact
   value and the same for every split of K; other group sizes, and M <= 16,
   as ll_bitlinear_gemv (bit-exact), in passes of up to 16 tokens (8 where
   only a pass of 8 fits the streaming product) that each read the weights
   once.
   workspace: at least ll_gemm_workspace_size(w, M) bytes (NULL allowed
   when that is 0; (size_t)-1 for invalid arguments), under the workspace
   rules above.  It holds the split-K partial tiles of narrow products (all
   formats on the matrix cores) or the prepared operands of the W1 passes,
   and the counters of both. */
size_t ll_gemm_workspace_size(const ll_weights* w, int64_t M);
ll_status ll_bitlinear_gemm(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M,
                            const float* bias, float* y, int32_t* acc_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): the
   product of ll_bitlinear_gemm, with the same arguments, rules and results,
   but no workspace argument.  Its scratch (split-K counters and partial
   tiles, the operands of W1 passes) is a static device array of
   ll_gemm_noalloc_scratch_bytes() bytes (32 MiB), one copy per GPU, held by
   the library from its load until the process ends; the call allocates and
   frees nothing.  A product needing more scratch than that (ll_gemm_
   workspace_size above the limit: W1 passes with very long K) is refused
   with LL_EWORKSPACE before anything is launched.  Every call on a GPU
   shares that GPU's array: calls that overlap in time on one GPU (other
   streams, concurrent graph replays) race and must not be made. */
size_t ll_gemm_noalloc_scratch_bytes(void);
ll_status ll_bitlinear_gemm_noalloc(const ll_weights* w, const int8_t* xq, const float* xs, int64_t M,
                                    const float* bias, float* y, int32_t* acc_out, void* stream);

/* [BG "API": binary_linear(x, wq, wscale, bias, group_size), bf16 in and out]
   One call from bf16 activations to bf16 outputs: per-token int8
   quantization of x (as ll_quantize_act), the int8 product of
   ll_bitlinear_gemm for the format (i2_s, TQ2_0 or W1, any M >= 1), the
   bias added in fp32, and y rounded to bf16 (to nearest, ties to even;
   NaN -> 0x7FC0 with its sign).  x: device bf16 bits [M,K]; bias: device
   fp32 [N] or NULL; y: device bf16 bits [M,N].  The result is the bf16
   rounding of what ll_quantize_act followed by ll_bitlinear_gemm gives.
   workspace: at least ll_binary_linear_workspace_size(w, M) bytes, under
   the workspace rules above (it holds the quantized x with its token scales
   and sums, and the product's scratch).  Two launches on `stream`: the
   quantization, then the product with the bias and the bf16 rounding in its
   epilogue.  The size function returns (size_t)-1 for an unsupported
   format or invalid arguments. */
size_t ll_binary_linear_workspace_size(const ll_weights* w, int64_t M);
ll_status ll_binary_linear(const ll_weights* w, const uint16_t* x, int64_t M, const float* bias, uint16_t* y,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Diagnostics                                                          */
/* ------------------------------------------------------------------ */

/* A plain streaming read of `bytes` (a positive multiple of 16) at device
   pointer p (16-byte aligned) by `blocks` workgroups of 256 threads, each
   16-byte word once: the reference read rate the weight-streaming products
   are compared with.  sink: device uint32 [blocks], overwritten with a fold
   of what each workgroup read. */
ll_status ll_probe_stream_read(const void* p, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWBIT_H */
