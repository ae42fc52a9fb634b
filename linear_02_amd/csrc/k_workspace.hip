// Clearing a workspace's sync area (the ticket counters and generation-tagged
// words of the in-launch hand-offs) with a plain fill kernel, so that the
// clear can sit inside a captured HIP graph.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

__global__ __launch_bounds__(256) void sync_clear_kernel(u32x4 *p, size_t n16) {
    const u32x4 z{0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

}  // namespace

hipError_t launch_sync_clear(unsigned long long *sync, size_t n_words, hipStream_t stream) {
    const size_t n16 = n_words / 2;
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(sync_clear_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<u32x4 *>(sync), n16);
    return hipGetLastError();
}

}  // namespace wl
