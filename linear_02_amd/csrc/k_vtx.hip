// V^T x of the low-rank delta: the inner sum over i of V[i,k] * x[t,i] in the
// per-element expansion of the reconstruction equation ("In-kernel
// reconstruction", reconstruction equation). Computed once per call into the
// workspace; every output row's epilogue then reads it.
//
// Workgroup (slice, child, token block): the input axis is cut into slices so
// that decode-sized calls (one token, a few thousand inputs) still spread over
// many compute units. Each workgroup stages its slice of x in LDS, lets thread
// (g, k) sum rows g, g+G, ... of the slice for rank index k, folds the G partial
// sums through LDS and writes them out. The last workgroup of a (child, token
// block) to arrive adds the slice partials in slice order, so the result is
// the same whichever workgroup finishes first. No workgroup ever waits.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void vtx_kernel(VtxJob job) {
    __shared__ u32x4 xs_raw[kVtxTok * kVtxMaxSlice / 8];
    __shared__ float red[kThreads][kVtxTok + 1];
    __shared__ int last;

    const int slice = blockIdx.x, c = blockIdx.y, tb = blockIdx.z;
    const int tid = threadIdx.x;
    const int t0 = tb * kVtxTok;
    const int tn = min(kVtxTok, job.T - t0);
    const int i0 = slice * job.slice_len;
    const int len = max(0, min(job.d_in - i0, job.slice_len));
    const int nchunk = len >> 3;

    // Stage x[t0 .. t0+kVtxTok)[i0 .. i0+len) as 16-byte pieces; absent tokens are zero.
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(job.x);
    const int row_chunks = job.d_in >> 3;
    for (int idx = tid; idx < kVtxTok * nchunk; idx += kThreads) {
        const int t = idx / nchunk, j = idx - t * nchunk;
        xs_raw[t * (kVtxMaxSlice / 8) + j] =
            t < tn ? xg[(size_t)(t0 + t) * row_chunks + (i0 >> 3) + j] : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const uint16_t *xs = reinterpret_cast<const uint16_t *>(xs_raw);

    const int r = job.r[c];
    int rp = 1;
    while (rp < r) rp <<= 1;
    const int k = tid & (rp - 1), g = tid / rp, G = kThreads / rp;
    const uint16_t *__restrict__ V = job.V[c];

    float acc[kVtxTok];
#pragma unroll
    for (int t = 0; t < kVtxTok; ++t) acc[t] = 0.f;
    if (k < r) {
        for (int i = g; i < len; i += G) {
            const float v = bf16_f(V[(size_t)(i0 + i) * r + k]);
#pragma unroll
            for (int t = 0; t < kVtxTok; ++t) acc[t] += v * bf16_f(xs[t * kVtxMaxSlice + i]);
        }
    }
#pragma unroll
    for (int t = 0; t < kVtxTok; ++t) red[tid][t] = acc[t];
    __syncthreads();

    const bool single = job.n_slices == 1;
    float *part = job.partial + ((size_t)(tb * job.n_ch + c) * job.n_slices + slice) * kVtxTok * kMaxRank;
    for (int idx = tid; idx < r * tn; idx += kThreads) {
        const int t = idx / r, kk = idx - t * r;
        float sum = 0.f;
        for (int gg = 0; gg < G; ++gg) sum += red[gg * rp + kk][t];
        if (single)
            job.vtx[c][(size_t)(t0 + t) * r + kk] = sum;
        else
            part[t * kMaxRank + kk] = sum;
    }
    if (single) return;

    // Publish this slice; the last slice of the (child, token block) adds them all.
    __threadfence();
    __syncthreads();
    uint32_t *cnt = job.counter + tb * job.n_ch + c;
    if (tid == 0) last = atomicAdd(cnt, 1u) == (uint32_t)(job.n_slices - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();
    const float *base = job.partial + (size_t)(tb * job.n_ch + c) * job.n_slices * kVtxTok * kMaxRank;
    for (int idx = tid; idx < r * tn; idx += kThreads) {
        const int t = idx / r, kk = idx - t * r;
        float sum = 0.f;
        for (int sl = 0; sl < job.n_slices; ++sl)
            sum += base[((size_t)sl * kVtxTok + t) * kMaxRank + kk];
        job.vtx[c][(size_t)(t0 + t) * r + kk] = sum;
    }
    if (tid == 0) atomicExch(cnt, 0u);
}

}  // namespace

hipError_t launch_vtx(const VtxJob &job, hipStream_t stream) {
    const int n_tb = (job.T + kVtxTok - 1) / kVtxTok;
    hipLaunchKernelGGL(vtx_kernel, dim3(job.n_slices, job.n_ch, n_tb), dim3(kThreads), 0, stream, job);
    return hipGetLastError();
}

}  // namespace wl
