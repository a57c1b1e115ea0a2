// Kernel launchers: host functions that enqueue the HIP kernels.  Arguments
// are validated by the C-ABI layer before any launcher is called; launchers
// only pick the kernel variant and grid, and return hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace llk {

// Every device workspace the library is given starts with a region of
// kCounterBytes that holds only split-K arrival counters (int32, one per
// output tile or row block, at most kMaxCounters).  Each call that uses
// counters leaves them zero again, and no call writes anything else there,
// so one workspace zero-filled once serves calls of any shape and format in
// turn.  The launchers take the counter base and the data region (the
// workspace past the counters) as separate pointers.
constexpr size_t kCounterBytes = 4096;
constexpr int64_t kMaxCounters = int64_t(kCounterBytes / 4);

// The static device scratch of the allocation-free entry point: its size,
// and the address of the current device's copy (its counter region cleared
// on `stream` the first time a device asks).
size_t static_scratch_bytes();
hipError_t static_scratch(void** out, hipStream_t stream);

// Diagnostic streaming read of `bytes` (a multiple of 16) by `blocks`
// workgroups; one word per workgroup into sink.
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);

// Raises a kernel's dynamic LDS limit to at least `bytes` on the current
// device.  hipFuncSetAttribute is a host-side call that costs microseconds,
// so each (kernel, device) pair is set once and remembered.
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes);

// xsum: int32 [M] receiving sum_k q[m,k], or NULL
hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, int8_t* xq, float* xs, int32_t* xsum,
                           hipStream_t stream);

// W1A8 product (binary weights, int8 activations), any M (passes of up to 16
// tokens, each reading the weights once); K % 128 == 0, G in {32,64,128,256}.
// ws (w1_workspace bytes) holds the prepared activation operands and, for a
// narrow matrix whose K is split over workgroups, their fp64 partial sums;
// counters: one per row block (zero on entry, left zero).
size_t w1_workspace(int64_t M, int64_t N, int64_t K, int G);
hipError_t launch_w1_gemv(const uint32_t* bits, const uint16_t* scales, int64_t N, int64_t K, int G, const int8_t* xq,
                          const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                          hipStream_t stream, uint16_t* y16 = nullptr);

// Prepared batches of W1 products (G = 128): w1_batch_fits(M, K) for every
// product; one table entry per product (fill_w1_prob, wg0 its first
// workgroup, wgs its workgroups: 1 .. w1_batch_wgs(N), a wave's blocks
// ceil(w1_batch_blocks(N) / (8 wgs))) and per distinct activation
// (fill_w1_prep, blk0 its first of w1_batch_prep_blocks(M, K) blocks,
// operands of w1_batch_operand_bytes(M, K) bytes); scv: every K % 1024 == 0.
// w1_batch_slots: workgroups of the product launch resident at once on the
// current device (0 when it cannot be queried).
bool w1_batch_fits(int64_t M, int64_t K);
int64_t w1_batch_wgs(int64_t N);
int64_t w1_batch_blocks(int64_t N);
int w1_batch_slots(int64_t M, int64_t kmax, bool scv);
int64_t w1_batch_prep_blocks(int64_t M, int64_t K);
size_t w1_batch_operand_bytes(int64_t M, int64_t K);
size_t w1_batch_prob_bytes();
size_t w1_batch_prep_bytes();
void fill_w1_prob(void* dst, const void* bits, const void* scales, const void* ops, const float* xs, const float* bias,
                  float* y, int64_t N, int64_t K, int64_t wg0, int64_t wgs);
void fill_w1_prep(void* dst, const int8_t* xq, void* ops, int64_t M, int64_t K, int64_t blk0);
hipError_t launch_w1_batch_prep(const void* prep_table, int nprep, int64_t blocks, int64_t M, hipStream_t stream);
hipError_t launch_w1_batch_product(const void* prob_table, const void* map, int64_t wgs, int64_t M, int64_t kmax,
                                   bool scv, hipStream_t stream);

// int8-activation prefill product, format i2_s.  ws: gemm_i8_workspace bytes
// of split-K partial tiles and counters one per output tile (zero on entry,
// left zero), or NULL (either) to forbid splits.
size_t gemm_i8_workspace(int64_t M, int64_t N, int64_t K, int fmt);   // fmt: 1 i2_s, 2 TQ2_0, 3 W1
// xsum: sum_k q per token from the quantization (then the kernel skips its
// own row sums), or NULL; y16: bf16 output [M,N] written instead of y, or NULL.
hipError_t launch_gemm_i8_i2s(const uint8_t* codes, int64_t N, int64_t K, const int8_t* xq,
                              const float* xs, int64_t M, const float* bias, float* y,
                              int32_t* acc_out, int32_t* counters, void* ws, hipStream_t stream,
                              const int32_t* xsum = nullptr, uint16_t* y16 = nullptr);
// The same product with W1 weights of group size 128 (bits uint32 [N][K/32],
// scales fp16 [N][K/128]); y = s_tok * sum_g s_g * d_g in fp32 (no acc_out).
hipError_t launch_gemm_i8_w1(const uint32_t* bits, const uint16_t* scales, int64_t N, int64_t K, const int8_t* xq,
                             const float* xs, int64_t M, const float* bias, float* y, int32_t* counters, void* ws,
                             hipStream_t stream, uint16_t* y16 = nullptr);
// The same product with TQ2_0 weights (codes N*K/4 bytes, scales fp16
// [N][K/256]); y = s_tok * sum_b s_b * d_b in fp32 (no acc_out); the same
// workspace size and rules.
hipError_t launch_gemm_i8_tq2(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                              const int8_t* xq, const float* xs, int64_t M, const float* bias, float* y,
                              int32_t* counters, void* ws, hipStream_t stream, uint16_t* y16 = nullptr);

}  // namespace llk

namespace llk {
// fp32-activation decode product, formats i2_s (fmt 1) and TQ2_0 (fmt 2),
// 1 <= M <= 16: activations split into int8 planes (one preparation launch),
// int8 matrix cores with exact int32 accumulation, up to three tokens per
// pass (gemv_planes.hip).  Prepared batches: device tables built by the C-ABI
// layer (ll_gemv_plan_init).
// A single call with M == 1 and K <= 8192 runs fused: each product workgroup
// builds the planes itself from x, so no workspace and no preparation launch.
constexpr int64_t kPlanesMaxM = 16;
bool planes_fused(int64_t M, int64_t K);
size_t planes_workspace(int64_t M, int64_t K);       // single call: 0 when fused
size_t planes_operand_bytes(int64_t M, int64_t K);   // prepared operands of one activation
int64_t planes_batch_rows();
size_t planes_prob_bytes();
size_t planes_prep_bytes();
void fill_planes_prob(void* dst, const void* codes, const void* scales, const void* ws, const float* bias, float* y,
                      int64_t N, int64_t K, int64_t wg0);
void fill_planes_prep(void* dst, const float* x, void* ws, int64_t K);
hipError_t launch_gemv_planes(int fmt, const void* codes, const void* scales, int64_t N, int64_t K, const float* x,
                              int64_t M, const float* bias, float* y, void* ws, hipStream_t stream);
// int8 activations xq [M][K] with per-token scales xs, 1 <= M <= 16, one launch, no workspace
hipError_t launch_gemv_i8_planes(int fmt, const void* codes, const void* scales, int64_t N, int64_t K,
                                 const int8_t* xq, const float* xs, int64_t M, const float* bias, float* y,
                                 hipStream_t stream);
hipError_t launch_planes_batch_prep(const void* prep_table, int nprep, int fmt, int64_t M, hipStream_t stream);
// map: int32 [wgs], the product each workgroup runs
hipError_t launch_planes_batch_product(const void* prob_table, const void* map, int fmt, int64_t M, int64_t wgs,
                                       hipStream_t stream);
}  // namespace llk

namespace llk {
// fp32-activation decode product on the fp4 matrix cores (gemv_fp4.hip),
// formats i2_s (fmt 1) and TQ2_0 (fmt 2): activations as twelve base-8 digit
// planes per token (one preparation launch), weights fed to the MFMAs straight
// from registers, one 16-row MFMA block per token.  Used by prepared batches
// with M <= 16 and every K <= 2^17.
bool f4_engine(int64_t M, int64_t kmax);             // 1 <= M <= 16, every K <= 2^17
int64_t f4_op_stride(int64_t K);                     // bytes between two tokens' prepared digits
size_t f4_operand_bytes(int64_t M, int64_t K);       // prepared digits of one activation (M tokens)
int64_t f4_batch_rows(bool pair, int fmt, int64_t M);   // output rows per workgroup (a gated pair: rows of both)
size_t f4_prob_bytes();
size_t f4_prep_bytes();
int64_t f4_grid(int64_t T);                         // workgroups launched for T logical ones
// codes2 / scales2: the up weights of a gated pair (codes / scales the gate), or NULL;
// ops: token 0's digits, token m's at ops + m f4_op_stride(K)
void fill_f4_prob(void* dst, const void* codes, const void* scales, const void* ops, const float* bias, float* y,
                  int64_t N, int64_t K, int64_t wg0, const void* codes2, const void* scales2, int64_t M);
// one entry per token; norm_w: the RMSNorm weights of an activation normalised in the preparation, or NULL
void fill_f4_prep(void* dst, const float* x, void* ops, int64_t K, const float* norm_w, float eps);
hipError_t launch_f4_batch_prep(const void* prep_table, int nentries, int fmt, int64_t kmax, hipStream_t stream);
// map: int32 [T], the product of each logical workgroup; pairs: the table holds gated pairs
hipError_t launch_f4_batch_product(const void* prob_table, const void* map, int fmt, int64_t T, int64_t kmax,
                                   bool pairs, int64_t M, hipStream_t stream);
}  // namespace llk
