// Diagnostic: a plain streaming read of a device buffer, the reference rate
// the weight-streaming products are compared with (no arithmetic of the
// method).  Every 16-byte word is read once with a non-temporal load; thread
// 0 of each workgroup stores a fold of its own loads into `sink` so the
// loads stay.
#include "common.h"
#include "launch.h"

namespace {

using namespace llk;

// Each workgroup reads 32 KiB contiguous chunks (eight 4 KiB pieces, one
// 16-byte load per thread and piece, all eight in flight), chunks grid-strided:
// the shape that measured fastest among 4 / 8 / 16 loads in flight and
// 1024 / 2048 / 4096 workgroups (about 7.1 TB/s on a 1 GiB buffer).
__global__ void __launch_bounds__(256) stream_read_kernel(const i32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
    constexpr int U = 8;
    uint32_t acc = 0;
    const int64_t chunk = int64_t(gridDim.x) * 256 * U;
    for (int64_t base = int64_t(blockIdx.x) * 256 * U; base < n16; base += chunk) {
        i32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t j = base + int64_t(u) * 256 + threadIdx.x;
            j = j < n16 ? j : n16 - 1;
            v[u] = ld16_stream(p + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= uint32_t(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

namespace llk {

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, static_cast<const i32x4*>(p),
                       int64_t(bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace llk
