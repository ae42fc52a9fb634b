// The effective weight of the precompute-outside path ("Serve and generate
// with weightless", setting the fast path on NVIDIA; the "What weightless
// inference costs" page writes the same matrix as diag(s) W0 + U V^T):
//
//   W_eff[o,i] = bf16( s[o] * W0[o,i] + sum_k U[o,k] V[i,k] )
//
// The low-rank product U V^T is a contraction over the rank only (K = r <= 64),
// done on the matrix cores: A = U (rows o, contiguous in k) and B = V (columns
// i, contiguous in k) both load straight from global memory as 16-byte pieces.
// The fp32 result is combined with the s-scaled W0 element and rounded once.
// Each wave owns a 32-row x 64-column tile (two 32x32 MFMA outputs), so every
// W0/W_eff row segment it touches is 128 contiguous bytes.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int TM = 128, TN = 64;   // workgroup tile: rows o x columns i

__device__ __forceinline__ u32x4 load8(const uint16_t *p, int row, int ld, int k0, int r, bool ok) {
    // bf16 row[k0 .. k0+8) of a [*][r] matrix, zero past r or when !ok.
    u32x4 v{0u, 0u, 0u, 0u};
    if (!ok) return v;
    if ((r & 7) == 0) {
        if (k0 < r) v = *reinterpret_cast<const u32x4 *>(p + (size_t)row * ld + k0);
        return v;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = k0 + e < r ? p[(size_t)row * ld + k0 + e] : 0u;
        v[e >> 1] |= b << (16 * (e & 1));
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void weff_kernel(Weff w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int fr = lane & 31, fk = lane >> 5;
    const int o0 = blockIdx.y * TM + wave * 32;
    const int i0 = blockIdx.x * TN;
    if (o0 >= w.d_out) return;

    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    for (int k0 = 0; k0 < w.r; k0 += 16) {
        const int kb = k0 + 8 * fk;
        const u32x4 a = load8(w.U, o0 + fr, w.r, kb, w.r, o0 + fr < w.d_out);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = i0 + j * 32 + fr;
            const u32x4 b = load8(w.V, i, w.r, kb, w.r, i < w.d_in);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
        }
    }

    // Lane (fr, fk) of output tile j holds column i = i0 + 32j + fr, rows
    // o0 + 8*(e/4) + 4*fk + (e%4).
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int o = o0 + 8 * (e >> 2) + 4 * fk + (e & 3);
        if (o >= w.d_out) continue;
        const float sv = w.s ? w.s[o] : 1.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = i0 + j * 32 + fr;
            if (i < w.d_in) {
                const size_t idx = (size_t)o * w.d_in + i;
                w.W_eff[idx] = f_bf16(sv * bf16_f(w.W0[idx]) + acc[j][e]);
            }
        }
    }
}

}  // namespace

hipError_t launch_weff(const Weff &w, hipStream_t stream) {
    const dim3 grid((w.d_in + TN - 1) / TN, (w.d_out + TM - 1) / TM);
    hipLaunchKernelGGL(weff_kernel, grid, dim3(kThreads), 0, stream, w);
    return hipGetLastError();
}

}  // namespace wl
