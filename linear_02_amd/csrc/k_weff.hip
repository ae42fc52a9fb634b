// The effective weight of the precompute-outside path ("Serve and generate
// with weightless", setting the fast path on NVIDIA; the "What weightless
// inference costs" page writes the same matrix as diag(s) W0 + U V^T):
//
//   W_eff[o,i] = bf16( s[o] * W0[o,i] + sum_k U[o,k] V[i,k] )
//
// The low-rank product U V^T is a contraction over the rank only (K = r <= 64),
// done on the matrix cores: A = U (rows o, contiguous in k) and B = V (columns
// i, contiguous in k) both load straight from global memory as 16-byte pieces.
// The kernel is bound by memory traffic (W0 read and W_eff written, 2 bytes each
// per element), so the fp32 product goes through LDS to be read back along rows:
// every lane then reads W0 and writes W_eff in 16-byte pieces, 256 contiguous
// bytes per 16 lanes. The W0 pieces are loaded before the products start.
// Several projections (a layer's seven) can share one launch, each workgroup
// taking one tile of one of them: a launch costs several microseconds whatever
// its size, so one per projection spent most of a layer's time on them.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int TM = 128, TN = 128;             // workgroup tile: rows o x columns i
constexpr int LDT = TN + 4;                   // fp32 row stride of the staged product
constexpr int kChunks = TM * TN / 8 / kThreads;   // 16-byte pieces per thread

__device__ __forceinline__ u32x4 load8(const uint16_t *p, int row, int ld, int k0, int r, bool ok) {
    // bf16 row[k0 .. k0+8) of a [*][r] matrix, zero past r or when !ok.
    u32x4 v{0u, 0u, 0u, 0u};
    if (!ok) return v;
    if ((r & 7) == 0) {
        if (k0 < r) v = ldg(reinterpret_cast<const u32x4 *>(p + (size_t)row * ld + k0));
        return v;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = k0 + e < r ? p[(size_t)row * ld + k0 + e] : 0u;
        v[e >> 1] |= b << (16 * (e & 1));
    }
    return v;
}

// One 128 x 128 tile: rows [by * TM, +TM), columns [bx * TN, +TN).
__device__ __forceinline__ void weff_tile(const Weff &w, int bx, int by, float *prod) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 31, fk = lane >> 5;
    const int ob = by * TM, ib = bx * TN;
    const int nch = w.d_in >> 3;

    // This thread's pieces: row ob + c / 16, columns ib + 8 * (c % 16), c = tid + 256 m.
    u32x4 w0[kChunks];
#pragma unroll
    for (int m = 0; m < kChunks; ++m) {
        const int c = tid + m * kThreads, o = min(ob + c / 16, w.d_out - 1), j = min((ib >> 3) + c % 16, nch - 1);
        w0[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w.W0) + (size_t)o * nch + j);
    }

    if (w.r > 0) {
        // Wave: rows ob + 32 * wave .. +32, all TN columns (four 32x32 outputs).
        f32x16 acc[TN / 32];
#pragma unroll
        for (int j = 0; j < TN / 32; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        // All U and V pieces (at most kMaxRank / 16 steps) are loaded before the products.
        constexpr int kSteps = kMaxRank / 16;
        const int o = ob + wave * 32 + fr;
        u32x4 a[kSteps], b[kSteps][TN / 32];
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int kb = 16 * q + 8 * fk;
            a[q] = load8(w.U, o, w.r, kb, w.r, o < w.d_out && 16 * q < w.r);
#pragma unroll
            for (int j = 0; j < TN / 32; ++j) {
                const int i = ib + j * 32 + fr;
                b[q][j] = load8(w.V, i, w.r, kb, w.r, i < w.d_in && 16 * q < w.r);
            }
        }
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            if (16 * q >= w.r) break;
#pragma unroll
            for (int j = 0; j < TN / 32; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[q]),
                                                                __builtin_bit_cast(bf16x8, b[q][j]), acc[j], 0, 0, 0);
        }
        // Lane (fr, fk) of output j holds column 32j + fr, rows 8*(e/4) + 4*fk + (e%4).
        // The empty asm statements keep these stores apart: this compiler merges
        // them into paired LDS stores with wrong offsets for this row stride.
        float *base = prod + (wave * 32 + 4 * fk) * LDT + fr;
#pragma unroll
        for (int j = 0; j < TN / 32; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                base[(8 * (e >> 2) + (e & 3)) * LDT + j * 32] = acc[j][e];
                asm volatile("" ::: "memory");
            }
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < kChunks; ++m) {
        const int c = tid + m * kThreads, ol = c / 16, jl = c % 16;
        const int o = ob + ol, j = (ib >> 3) + jl;
        if (o >= w.d_out || j >= nch) continue;
        float lr[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (w.r > 0) {
            const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&prod[ol * LDT + 8 * jl]);
            const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&prod[ol * LDT + 8 * jl + 4]);
            lr[0] = p0.x; lr[1] = p0.y; lr[2] = p0.z; lr[3] = p0.w;
            lr[4] = p1.x; lr[5] = p1.y; lr[6] = p1.z; lr[7] = p1.w;
        }
        const float sv = w.s ? ldg(w.s + o) : 1.0f;
        const uint32_t wv[4] = {w0[m].x, w0[m].y, w0[m].z, w0[m].w};
        uint32_t out[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v0 = sv * bf16_f(wv[q] & 0xFFFFu) + lr[2 * q];
            const float v1 = sv * bf16_f(wv[q] >> 16) + lr[2 * q + 1];
            out[q] = (uint32_t)f_bf16(v0) | ((uint32_t)f_bf16(v1) << 16);
        }
        // Streaming stores: W_eff is written once and not read back here (11 %
        // faster over a layer's projections than plain stores).
        __builtin_nontemporal_store(u32x4{out[0], out[1], out[2], out[3]},
                                    reinterpret_cast<u32x4 *>(w.W_eff) + (size_t)o * nch + j);
    }
}

__global__ __launch_bounds__(kThreads) void weff_kernel(Weff w) {
    __shared__ float prod[TM * LDT];
    weff_tile(w, blockIdx.x, blockIdx.y, prod);
}

// Several projections in one launch: workgroup b belongs to the first entry p
// with b < tiles_end[p], and takes that entry's tile b - tiles_end[p - 1]
// (column tiles fastest), with the same arithmetic as the one-projection kernel.
__global__ __launch_bounds__(kThreads) void weff_batch_kernel(WeffBatch bt) {
    __shared__ float prod[TM * LDT];
    const int b = blockIdx.x;
    int p = 0;
    while (p < bt.n - 1 && b >= bt.tiles_end[p]) ++p;
    const int t = b - (p > 0 ? bt.tiles_end[p - 1] : 0);
    const Weff &w = bt.w[p];
    const int gx = (w.d_in + TN - 1) / TN;
    weff_tile(w, t % gx, t / gx, prod);
}

}  // namespace

hipError_t launch_weff(const Weff &w, hipStream_t stream) {
    const dim3 grid((w.d_in + TN - 1) / TN, (w.d_out + TM - 1) / TM);
    hipLaunchKernelGGL(weff_kernel, grid, dim3(kThreads), 0, stream, w);
    return hipGetLastError();
}

int weff_tiles(int d_in, int d_out) { return ((d_in + TN - 1) / TN) * ((d_out + TM - 1) / TM); }

hipError_t launch_weff_batch(const WeffBatch &bt, hipStream_t stream) {
    if (bt.n < 1) return hipSuccess;
    hipLaunchKernelGGL(weff_batch_kernel, dim3(bt.tiles_end[bt.n - 1]), dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

}  // namespace wl
