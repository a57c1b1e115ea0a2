// Static device scratch for the entry point that allocates nothing
// (ll_bitlinear_gemm_noalloc): a file-scope device array of kScratchBytes,
// one copy per GPU, held from the library's load until the process ends.
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address: the address of the current GPU's copy is taken once per
// device with hipGetSymbolAddress and kept, and only that address is handed
// to kernels.  On a device's first use the counter region at its start is
// cleared by a fill kernel on the caller's stream (no memset node, so the
// call may be captured in a graph); every product leaves its counters zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void __launch_bounds__(256) zero_words(uint32_t* __restrict__ p, int n) {
    const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
    if (i < n) p[i] = 0u;
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace llk {

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(void** out, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        const int words = int(kCounterBytes / 4);
        hipLaunchKernelGGL(zero_words, dim3(unsigned((words + 255) / 256)), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                           words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace llk
