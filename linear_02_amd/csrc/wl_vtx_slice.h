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

// Thread (g, k), with rp the smallest power of two >= r and G = 256 / rp, sums
// rows g, g + G, ... of the slice for rank column k; the loads of 16 rows are
// issued before any of them is used. Every address is valid (rows clamped into
// the slice) and the values are masked afterwards, so the 16 rows' loads are
// all in flight at once. The groups of one wave are then added by an xor
// butterfly over the lanes of column k (a + b = b + a, so every lane ends with
// the same bits), and the wave sums stored to red for vtx_slice_total, which
// adds the four waves in order.
// x_at(ic, t) returns x[t][i0 + ic] as fp32 (0 for absent tokens).
// issued() runs once in every thread, right after the first 16 rows' loads are
// issued (a caller's own memory operation issued there overlaps them).
// Ends with a barrier; begins with one, so red may be reused right away.
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};
template <int TB, class XAt, class Hook = NoHook>
__device__ __forceinline__ void vtx_slice_sums(const uint16_t *__restrict__ V, int r, int i0, int len, XAt x_at,
                                               float (*red)[TB + 1], Hook issued = Hook()) {
    const int tid = threadIdx.x;
    int rp = 1;
    while (rp < r) rp <<= 1;
    const int k = tid & (rp - 1), g = tid / rp, G = kVtxSliceThreads / rp;
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.f;
    auto rows16 = [&](int ib, bool first) {
        float v[16], xv[16][TB];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = ib + u * G;
            const bool in = i < len;
            const int ic = min(i, len - 1);
            const float vv = bf16_f(ldg(V + (size_t)(i0 + ic) * r + k));
            v[u] = in ? vv : 0.f;
#pragma unroll
            for (int t = 0; t < TB; ++t) xv[u][t] = x_at(ic, t);
        }
        if (first) issued();
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int t = 0; t < TB; ++t) acc[t] += v[u] * xv[u][t];
    };
    // The first 16 rows outside the loop: a loop header makes the compiler wait
    // for every earlier memory operation (a caller's atomic, say) before these
    // loads are issued.
    if (k < r && g < len) {
        rows16(g, true);
        for (int ib = g + 16 * G; ib < len; ib += 16 * G) rows16(ib, false);
    } else {
        issued();
    }
    for (int off = rp; off < kWave; off <<= 1)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[t] += __shfl_xor(acc[t], off);
    __syncthreads();
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    float *r1 = &red[0][0];   // [4 waves][64 columns][TB] within red
    if (lane < rp)
#pragma unroll
        for (int t = 0; t < TB; ++t) r1[(wave * kWave + lane) * TB + t] = acc[t];
    __syncthreads();
}

// The slice's partial sum for (t, kk) after vtx_slice_sums: the four wave sums
// of column kk added in wave order.
template <int TB>
__device__ __forceinline__ float vtx_slice_total(const float (*red)[TB + 1], int r, int t, int kk) {
    (void)r;
    const float *r1 = &red[0][0];
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kVtxSliceThreads / kWave; ++w) sum += r1[(w * kWave + kk) * TB + t];
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
