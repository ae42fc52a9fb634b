// V^T x over one slice of the input axis, by one workgroup of 256 threads:
//   partial[t][k] = sum over the slice's inputs i of V[i][k] * x[t][i]
// (the inner sum over i in the per-element expansion of the reconstruction
// formula, "In-kernel reconstruction", introduction). Shared by the V^T x
// launch and by the decode kernel's producer and fallback paths, so every one
// of them forms the same sums in the same order and gets the same bits.
#pragma once

#include "wl_device.h"

namespace wl {

constexpr int kVtxSliceThreads = 256;

// Per-thread sums, then stored to red[tid][t]. Thread (g, k), with rp the
// smallest power of two >= r and G = 256 / rp, sums rows g, g + G, ... of the
// slice for rank column k; the loads of 16 rows are issued before any of them
// is used. Every address is valid (rows clamped into the slice) and the values
// are masked afterwards, so the 16 rows' loads are all in flight at once.
// x_at(ic, t) returns x[t][i0 + ic] as fp32 (0 for absent tokens).
// Ends with a barrier; begins with one, so red may be reused right away.
template <int TB, class XAt>
__device__ __forceinline__ void vtx_slice_sums(const uint16_t *__restrict__ V, int r, int i0, int len, XAt x_at,
                                               float (*red)[TB + 1]) {
    const int tid = threadIdx.x;
    int rp = 1;
    while (rp < r) rp <<= 1;
    const int k = tid & (rp - 1), g = tid / rp, G = kVtxSliceThreads / rp;
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.f;
    if (k < r) {
        for (int ib = g; ib < len; ib += 16 * G) {
            float v[16], xv[16][TB];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int i = ib + u * G;
                const bool in = i < len;
                const int ic = min(i, len - 1);
                const float vv = bf16_f(V[(size_t)(i0 + ic) * r + k]);
                v[u] = in ? vv : 0.f;
#pragma unroll
                for (int t = 0; t < TB; ++t) xv[u][t] = x_at(ic, t);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int t = 0; t < TB; ++t) acc[t] += v[u] * xv[u][t];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TB; ++t) red[tid][t] = acc[t];
    __syncthreads();
}

// The slice's partial sum for (t, kk) after vtx_slice_sums: the G group sums
// of column kk added in group order.
template <int TB>
__device__ __forceinline__ float vtx_slice_total(const float (*red)[TB + 1], int r, int t, int kk) {
    int rp = 1;
    while (rp < r) rp <<= 1;
    const int G = kVtxSliceThreads / rp;
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += red[gg * rp + kk][t];
    return sum;
}

// x values of up to two tokens read straight from global memory: x points at
// the first token's row, tn tokens present.
template <int TB>
struct VtxXGlobal {
    const uint16_t *x;
    int d_in, i0, tn;
    __device__ __forceinline__ float operator()(int ic, int t) const {
        const float xx = bf16_f(x[(size_t)min(t, tn - 1) * d_in + i0 + ic]);
        return t < tn ? xx : 0.f;
    }
};

}  // namespace wl
