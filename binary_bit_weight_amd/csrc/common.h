// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace llk {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kWave = 64;

// Global-memory views.  Pointers that a kernel reads from a table in memory
// are generic to the compiler, which then emits FLAT instructions; a FLAT
// load also counts against the LDS wait counter, so every LDS wait would
// stall on outstanding weight prefetches.  Loads go through explicitly
// global (address space 1) pointers instead.
typedef __attribute__((address_space(1))) const i32x4 gi32x4;
typedef __attribute__((address_space(1))) const int32_t gint32;
typedef __attribute__((address_space(1))) const f32x4 gf32x4;

// 16-byte global load / store through the vector memory path.
// (C-style casts: they are address-space conversions, which reinterpret_cast
// does not perform.)
__device__ __forceinline__ i32x4 ld16(const void* p) { return *(gi32x4*)p; }
__device__ __forceinline__ void st16(void* p, i32x4 v) { *(__attribute__((address_space(1))) i32x4*)p = v; }
// Streaming (non-temporal) 16-byte load for weights that are read once.
__device__ __forceinline__ i32x4 ld16_stream(const void* p) { return __builtin_nontemporal_load((gi32x4*)p); }
__device__ __forceinline__ int32_t ld32(const void* p) { return *(gint32*)p; }
__device__ __forceinline__ f32x4 ld16f(const void* p) { return *(gf32x4*)p; }
__device__ __forceinline__ uint16_t ld2(const void* p) { return *(__attribute__((address_space(1))) const uint16_t*)p; }

// Buffer loads: a resource (base address, size in bytes) in scalar registers
// plus a per-lane byte offset.  The hardware returns zeros for an offset at or
// past the size, so a resource ending with its array makes every read past the
// array's end a read of zeros.  bytes <= 0 gives an empty resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : bytes >= int64_t(0xFFFFFFFF) ? 0xFFFFFFFFu : uint32_t(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(n), 0x00020000);
}
// 16 bytes, streaming (non-temporal: read once).
__device__ __forceinline__ i32x4 buffer_ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ i32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// 8 bytes into the low half of a 16-byte vector.
__device__ __forceinline__ i32x4 buffer_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return i32x4{int(v[0]), int(v[1]), 0, 0};
}
__device__ __forceinline__ uint16_t buffer_ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buffer_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Butterfly sum / max over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Butterfly sums of N independent values over the 64 lanes of a wave, the N
// shuffles of each step issued together (one LDS-permute wait per step
// instead of one per shuffle).
template <int N>
__device__ __forceinline__ void wave_sum_n(int (&v)[N]) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        int t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = __shfl_xor(v[i], o, kWave);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += t[i];
    }
}

// Device-coherent 32-bit store / load (agent scope): written through, and
// read from, the point of coherence of all XCDs, so a value passed between
// workgroups needs no cache-wide writeback or invalidate.
__device__ __forceinline__ void st_coherent(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_coherent(const int32_t* p) {
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent64(double* p, double v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __double_as_longlong(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_coherent64(const double* p) {
    return __longlong_as_double(__hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<double*>(p)),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Split-K handoff.  A split publishes its partial sums, every wave waits for
// its stores, the workgroup meets at a barrier, and one thread counts the
// split in with arrive_release: an agent-scope release read-modify-write,
// which orders the published partials before the count.  The split that
// reads count + 1 == splits is the last; its threads then take
// acquire_agent (an agent-scope acquire fence, which pairs with every other
// split's release through the counter) before loading the others'
// partials.  Only the last split pays for the acquire (a cache invalidate),
// so the arrivals do not throw away the L2 contents other workgroups are
// still reading.
__device__ __forceinline__ int32_t arrive_release(int32_t* c) {
    return __hip_atomic_fetch_add(c, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// Wait until every vector memory operation of this wave has completed
// (gfx9 s_waitcnt: vmcnt = 0, expcnt and lgkmcnt not waited on).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// fp32 -> bf16 bits, round to nearest with ties to even on the bit pattern
// (add 0x7FFF plus the lowest kept bit, keep the high half; overflow goes to
// infinity); NaN becomes the quiet NaN 0x7FC0 with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t(((u >> 16) & 0x8000u) | 0x7FC0u);
    return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return float(__builtin_bit_cast(_Float16, h));
}

}  // namespace llk
