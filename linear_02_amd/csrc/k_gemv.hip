// Decode-sized projections (one to a few tokens per pass). Here the W0 stream
// is nearly all of the memory traffic, so the kernel is built around reading
// W0 once at full HBM rate:
//   * each wave owns R consecutive output rows at a time (a task) and walks
//     them with its 64 lanes side by side, 16 bytes per lane per load, so one
//     wave-wide load covers 1 KiB of a row and NB loads per row are in flight;
//   * the tokens of the pass sit in LDS, read once per 16-byte piece and
//     reused across the R rows;
//   * products go through v_dot2c_f32_bf16 into fp32 accumulators;
//   * workgroups loop over tasks (grid-stride), so x is staged once per
//     workgroup, not once per row.
// Epilogue ("In-kernel reconstruction", per-element expansion of the
// reconstruction equation): lane k < r adds U[o,k] * vtx[t,k] to its share of
// the s[o]-scaled row sum, so one wave reduction yields
//   y[t,o] = s[o] * sum_i W0[o,i] x[t,i] + sum_k U[o,k] vtx[t,k],
// which is rounded once to bf16. Pair mode (gate/up of the MLP) streams the
// gate row and the up row together and writes bf16(gelu_tanh(g) * u).
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ const Child &child_of(const Gemv &g, int row) {
    if (g.n_ch > 2 && row >= g.ch[2].col0) return g.ch[2];
    if (g.n_ch > 1 && row >= g.ch[1].col0) return g.ch[1];
    return g.ch[0];
}

// s[o] * acc + sum_k U[o,k] vtx[t,k], summed over the wave; valid in every lane.
__device__ __forceinline__ float finish_row(const Child &c, int o, int tok, float acc, int lane) {
    float v = (c.s ? c.s[o] : 1.0f) * acc;
    if (lane < c.r) v += bf16_f(c.U[(size_t)o * c.r + lane]) * c.vtx[(size_t)tok * c.r + lane];
    return wave_sum(v);
}

template <int TT, int R, int P, int NB>
__global__ __launch_bounds__(kThreads) void gemv_kernel(Gemv g, int t0) {
    extern __shared__ u32x4 xs[];   // [TT][nch] 16-byte pieces of x
    const int nch = g.d_in >> 3;
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(g.x);
        for (int idx = threadIdx.x; idx < TT * nch; idx += kThreads) {
            const int t = idx / nch;
            xs[idx] = t0 + t < g.T ? src[(size_t)(t0 + t) * nch + (idx - t * nch)] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int n_task = (g.rows + R - 1) / R;
    for (int task = blockIdx.x * kWaves + (threadIdx.x >> 6); task < n_task; task += gridDim.x * kWaves) {
        const int row0 = task * R;
        const u32x4 *w[R][P];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = min(row0 + j, g.rows - 1);   // rows past the end re-read the last row
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const Child &c = P == 2 ? g.ch[p] : child_of(g, row);
                w[j][p] = reinterpret_cast<const u32x4 *>(c.W0 + (size_t)(row - c.col0) * g.d_in);
            }
        }
        float acc[R][P][TT];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int t = 0; t < TT; ++t) acc[j][p][t] = 0.f;

        for (int c0 = lane; c0 < nch; c0 += kWave * NB) {
            u32x4 wv[NB][R][P];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int cc = c0 + kWave * u;
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        wv[u][j][p] = cc < nch ? __builtin_nontemporal_load(w[j][p] + cc) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int cc = c0 + kWave * u;
                if (cc < nch) {
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const u32x4 xv = xs[t * nch + cc];
#pragma unroll
                        for (int j = 0; j < R; ++j)
#pragma unroll
                            for (int p = 0; p < P; ++p) acc[j][p][t] = dot8(wv[u][j][p], xv, acc[j][p][t]);
                    }
                }
            }
        }

#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = row0 + j;
            if (row >= g.rows) break;                       // wave-uniform
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const int tok = t0 + t;
                if (tok >= g.T) break;                      // wave-uniform
                float out;
                if (P == 2) {
                    const float gv = finish_row(g.ch[0], row, tok, acc[j][0][t], lane);
                    const float uv = finish_row(g.ch[1], row, tok, acc[j][P - 1][t], lane);
                    out = gelu_tanh(gv) * uv;
                } else {
                    const Child &c = child_of(g, row);
                    out = finish_row(c, row - c.col0, tok, acc[j][0][t], lane);
                }
                if (lane == 0) g.y[(size_t)tok * g.ldy + row] = f_bf16(out);
            }
        }
    }
}

template <int TT, int R, int P, int NB>
hipError_t launch_tt(const Gemv &g, int t0, int n_cu, hipStream_t stream) {
    const int n_task = (g.rows + R - 1) / R;
    const size_t lds = (size_t)TT * g.d_in * sizeof(uint16_t);
    const int per_cu = lds <= 16384 ? 4 : lds <= 32768 ? 3 : 2;
    int blocks = (n_task + kWaves - 1) / kWaves;
    if (blocks > n_cu * per_cu) blocks = n_cu * per_cu;
    hipLaunchKernelGGL((gemv_kernel<TT, R, P, NB>), dim3(blocks), dim3(kThreads), lds, stream, g, t0);
    return hipGetLastError();
}

template <int R, int P, int NB>
hipError_t launch_all(const Gemv &g, int n_cu, hipStream_t stream) {
    for (int t0 = 0; t0 < g.T;) {
        const int left = g.T - t0;
        int tt = left >= 4 ? 4 : left >= 2 ? 2 : 1;
        while (tt > 1 && tt * g.d_in > kGemvMaxStaged) tt >>= 1;
        hipError_t e;
        if (tt == 4)
            e = launch_tt<4, R, P, NB>(g, t0, n_cu, stream);
        else if (tt == 2)
            e = launch_tt<2, R, P, NB>(g, t0, n_cu, stream);
        else
            e = launch_tt<1, R, P, NB>(g, t0, n_cu, stream);
        if (e != hipSuccess) return e;
        t0 += tt;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv(const Gemv &g, int n_cu, hipStream_t stream) {
    if (g.pair) return launch_all<1, 2, 4>(g, n_cu, stream);
    return launch_all<2, 1, 4>(g, n_cu, stream);
}

}  // namespace wl
