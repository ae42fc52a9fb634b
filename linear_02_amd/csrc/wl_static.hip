// A workspace in a static device array, for wl_linear_static: callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) still get the decode and few-token
// kernels, whose hand-offs need a workspace.
//
// The array is a file-scope __device__ variable: every device the library runs
// on holds its own copy, at its own address, until the process ends. In host
// code the array's name is only a stand-in for the symbol, so its device
// address is looked up once per device with hipGetSymbolAddress and only that
// address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // the array's address on each device once it is set up

}  // namespace

hipError_t static_scratch(hipStream_t stream, void **out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        // The sync area (ticket counters, tagged words) starts at zero; a fill
        // kernel, ordered before the first call's kernels on its stream.
        e = launch_sync_clear(static_cast<unsigned long long *>(p), kSyncBytes / 8, stream);
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace wl
