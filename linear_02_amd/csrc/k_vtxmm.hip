// V^T x on the matrix cores for the prefill-sized path, in a launch of its own
// (one workgroup of 8 waves per unit; the unit itself is in wl_vtxmm.h):
//   part[c][split][t][k] = sum over the split's inputs i of x[t][i] V_c[i][k]
// (the first factor of the low-rank correction, "In-kernel reconstruction",
// introduction). Its consumer (the GEMM epilogue) adds the splits in split order.
#include "wl_vtxmm.h"

namespace wl {

namespace {

constexpr int kW = 8;                          // waves per workgroup

template <int NV, int RS>
__global__ __launch_bounds__(kW * 64) void vtxmm_kernel(VtxMM job) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[vtx_unit_lds_bytes<kW, NV>()];
    vtxmm_unit<kW, NV, RS>(job, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

template <int NV, int RS>
void launch_one(const VtxMM &job, hipStream_t stream) {
    const dim3 grid((job.T + 31) / 32, job.S, job.n);
    hipLaunchKernelGGL((vtxmm_kernel<NV, RS>), grid, dim3(kW * kWave), 0, stream, job);
}

bool all_rank(const VtxMM &job, int r) {
    for (int c = 0; c < job.n; ++c)
        if (job.r[c] != r) return false;
    return true;
}

}  // namespace

int vtxmm_splits(int d_in, int max_r) {
    // About four blocks per wave.
    (void)max_r;
    const int nkb = (d_in + kVtxKB - 1) / kVtxKB;
    const int per = 4 * kW;
    const int S = (nkb + per - 1) / per;
    return S < 1 ? 1 : S < kVtxMaxSplits ? S : kVtxMaxSplits;
}

hipError_t launch_vtxmm(const VtxMM &job, hipStream_t stream) {
    int max_r = 0;
    for (int c = 0; c < job.n; ++c) max_r = job.r[c] > max_r ? job.r[c] : max_r;
    if (max_r <= 32) {
        if (all_rank(job, 32)) launch_one<1, 32>(job, stream);
        else launch_one<1, 0>(job, stream);
    } else {
        if (all_rank(job, 64)) launch_one<2, 64>(job, stream);
        else launch_one<2, 0>(job, stream);
    }
    return hipGetLastError();
}

}  // namespace wl
