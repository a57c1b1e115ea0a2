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

// 16-byte global load / store through the vector memory path.
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ void st16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }
// Streaming (non-temporal) 16-byte load for weights that are read once.
__device__ __forceinline__ i32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
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

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return float(__builtin_bit_cast(_Float16, h));
}

}  // namespace llk
