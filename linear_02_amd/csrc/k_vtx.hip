// V^T x of the low-rank delta for the decode regime: the inner sum over i
// of V[i,k] * x[t,i] in the per-element expansion of the reconstruction formula
// ("In-kernel reconstruction", introduction).
//
// Workgroup (slice, child, token block): the input axis is cut into slices of
// at most kVtxMaxSlice inputs, so that calls with few tokens spread over
// several compute units (and, for larger token blocks, the x slice fits in LDS). Each workgroup writes the
// slice's partial sums; the consuming kernel (launched after this one on the
// same stream) adds the slices in slice order, so the result does not depend
// on scheduling. There is no cross-workgroup communication inside the kernel.
#include "wl_device.h"
#include "wl_kernels.h"
#include "wl_vtx_slice.h"

namespace wl {

namespace {

constexpr int kThreads = kVtxSliceThreads;

template <int TB>
__global__ __launch_bounds__(kThreads) void vtx_kernel(VtxJob job) {
    // Up to two tokens per workgroup: every thread loads its x values straight
    // from global memory together with its V entries (one round trip); more
    // tokens: the x slice is staged in LDS first and shared.
    constexpr bool kStage = TB > 2;
    __shared__ u32x4 xs_raw[kStage ? TB * kVtxMaxSlice / 8 : 1];
    __shared__ float red[kThreads][TB + 1];

    const int slice = blockIdx.x, c = blockIdx.y, tb = blockIdx.z;
    const int tid = threadIdx.x;
    const int t0 = tb * TB;
    const int tn = min(TB, job.T - t0);
    const int i0 = slice * job.slice_len;
    const int len = max(0, min(job.d_in - i0, job.slice_len));

    if constexpr (kStage) {
        // x[t0 .. t0+TB)[i0 .. i0+len) as 16-byte pieces; absent tokens are zero.
        const int nchunk = len >> 3;
        const u32x4 *xg = reinterpret_cast<const u32x4 *>(job.x);
        const int row_chunks = job.d_in >> 3;
        for (int idx = tid; idx < TB * nchunk; idx += kThreads) {
            const int t = idx / nchunk, j = idx - t * nchunk;
            xs_raw[t * (kVtxMaxSlice / 8) + j] =
                t < tn ? xg[(size_t)(t0 + t) * row_chunks + (i0 >> 3) + j] : u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
    }
    const uint16_t *xs = reinterpret_cast<const uint16_t *>(xs_raw);

    const int r = job.r[c];
    if constexpr (kStage) {
        vtx_slice_sums<TB>(job.V[c], r, i0, len, [&](int ic, int t) { return bf16_f(xs[t * kVtxMaxSlice + ic]); },
                           red);
    } else {
        const VtxXGlobal<TB> xg{job.x + (size_t)t0 * job.d_in, job.d_in, i0, tn};
        vtx_slice_sums<TB>(job.V[c], r, i0, len, xg, red);
    }

    // partial[c][slice][t][k]
    float *part = job.partial[c] + (size_t)slice * job.ld_T * r;
    for (int idx = tid; idx < r * tn; idx += kThreads) {
        const int t = idx / r, kk = idx - t * r;
        part[(size_t)(t0 + t) * r + kk] = vtx_slice_total<TB>(red, r, t, kk);
    }
}

}  // namespace

hipError_t launch_vtx(const VtxJob &job, hipStream_t stream) {
    const int tb = job.T >= 8 ? 8 : job.T >= 4 ? 4 : job.T >= 2 ? 2 : 1;
    const dim3 grid(job.n_slices, job.n_ch, (job.T + tb - 1) / tb);
    switch (tb) {
        case 8: hipLaunchKernelGGL(vtx_kernel<8>, grid, dim3(kThreads), 0, stream, job); break;
        case 4: hipLaunchKernelGGL(vtx_kernel<4>, grid, dim3(kThreads), 0, stream, job); break;
        case 2: hipLaunchKernelGGL(vtx_kernel<2>, grid, dim3(kThreads), 0, stream, job); break;
        default: hipLaunchKernelGGL(vtx_kernel<1>, grid, dim3(kThreads), 0, stream, job); break;
    }
    return hipGetLastError();
}

}  // namespace wl
