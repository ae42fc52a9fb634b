// Reconstruction fidelity ("What weightless inference costs", "Reconstruction
// fidelity"): the relative Frobenius error
//   ||W - R||_F / ||W||_F
// of a reconstruction R of a weight W, both bf16 with n elements, and 0 when
// ||W||_F is 0 and R equals W, +inf when ||W||_F is 0 and R does not.
//
// A memory-bound reduction. Launch 1: every thread walks 16-byte pieces of both
// matrices with a grid stride and keeps fp64 sums of (w - r)^2 and w^2 (the
// difference and the squares of bf16 values are exact in fp64); each workgroup
// adds its threads' sums in a fixed tree and stores one pair. Launch 2: one
// workgroup adds the pairs in the same fixed way and forms the ratio. The grid
// depends on n only, so the result is the same from run to run.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double bf16_d(uint32_t bits16) { return (double)__uint_as_float(bits16 << 16); }

// Fixed-tree sum of one double per thread over the workgroup; thread 0 gets it.
__device__ __forceinline__ void block_sum2(double &a, double &b, double (*sm)[kThreads]) {
    const int tid = threadIdx.x;
    sm[0][tid] = a;
    sm[1][tid] = b;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (tid < s) {
            sm[0][tid] += sm[0][tid + s];
            sm[1][tid] += sm[1][tid + s];
        }
        __syncthreads();
    }
    a = sm[0][0];
    b = sm[1][0];
}

__global__ __launch_bounds__(kThreads) void frob_partial_kernel(FrobJob job) {
    __shared__ double sm[2][kThreads];
    const int64_t n8 = job.n >> 3;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const u32x4 *W = reinterpret_cast<const u32x4 *>(job.W);
    const u32x4 *R = reinterpret_cast<const u32x4 *>(job.R);
    double num = 0.0, den = 0.0;
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n8; q += stride) {
        const u32x4 w = ldg(W + q), r = ldg(R + q);
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double a = bf16_d(e & 1 ? wv[e >> 1] >> 16 : wv[e >> 1] & 0xFFFFu);
            const double b = bf16_d(e & 1 ? rv[e >> 1] >> 16 : rv[e >> 1] & 0xFFFFu);
            num += (a - b) * (a - b);
            den += a * a;
        }
    }
    // The last n % 8 elements: thread 0 of workgroup 0.
    if (blockIdx.x == 0 && threadIdx.x == 0)
        for (int64_t j = n8 << 3; j < job.n; ++j) {
            const double a = bf16_d(job.W[j]), b = bf16_d(job.R[j]);
            num += (a - b) * (a - b);
            den += a * a;
        }
    block_sum2(num, den, sm);
    if (threadIdx.x == 0) {
        job.part[2 * blockIdx.x] = num;
        job.part[2 * blockIdx.x + 1] = den;
    }
}

__global__ __launch_bounds__(kThreads) void frob_final_kernel(FrobJob job) {
    __shared__ double sm[2][kThreads];
    double num = 0.0, den = 0.0;
    for (int b = threadIdx.x; b < job.n_wg; b += kThreads) {
        num += job.part[2 * b];
        den += job.part[2 * b + 1];
    }
    block_sum2(num, den, sm);
    if (threadIdx.x == 0) job.out[0] = den == 0.0 ? (num == 0.0 ? 0.0 : __builtin_huge_val()) : sqrt(num) / sqrt(den);
}

}  // namespace

int frob_workgroups(int64_t n) {
    const int64_t per_wg = (int64_t)kThreads * 8 * 8;       // about 8 pieces per thread
    const int64_t wg = (n + per_wg - 1) / per_wg;
    return wg < 1 ? 1 : wg > kFrobMaxWorkgroups ? kFrobMaxWorkgroups : (int)wg;
}

hipError_t launch_frob(const FrobJob &job, hipStream_t stream) {
    hipLaunchKernelGGL(frob_partial_kernel, dim3(job.n_wg), dim3(kThreads), 0, stream, job);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(frob_final_kernel, dim3(1), dim3(kThreads), 0, stream, job);
    return hipGetLastError();
}

}  // namespace wl
