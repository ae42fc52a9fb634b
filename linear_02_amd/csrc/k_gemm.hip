// Matrix-core path for larger token counts (prefill-sized calls).
//
//   m[t,o]  = sum_i x[t,i] W0[o,i]                  bf16 x bf16 -> fp32 on MFMA
//   y[t,o]  = bf16( s[o] * m[t,o] + sum_k vtx[t,k] U[o,k] )
//
// ("In-kernel reconstruction", reconstruction equation and its GEMM form:
// s scales the W0 product, the rank-r term is added unscaled.)
//
// Both operands are contiguous along the input axis (x[T][d_in], W0[d_out][d_in]),
// so tiles go straight from global memory into LDS as 16-byte pieces without
// any transpose. A workgroup owns a 128-token x 128-output tile; its four waves
// each own 64 x 64 of it as a 2 x 2 grid of 32x32x16 bf16 MFMAs. The input
// axis is walked 32 at a time through double-buffered LDS tiles.
//
// Epilogue: the accumulators are scaled by s[o] (one column per lane in the
// 32x32 output layout), then the rank-r term runs on the matrix cores as a few
// extra K steps with A = vtx and B = U. vtx (the sum, in slice order, of the
// V^T x slice partials written by the preceding launch) is fp32; it is split into a bf16
// head and a bf16 remainder (vtx = hi + lo up to about 2^-16 relative) and both
// go through the MFMA, so the rank term keeps close to fp32 accuracy. Results
// are rounded once to bf16. Pair mode (the MLP's gate/up) keeps two
// accumulator sets over the same x tile and writes bf16(gelu_tanh(g) * u).
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDC = BK / 8 + 1;          // 16-byte pieces per LDS row (one of padding)

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = (uint32_t)f_bf16(v[2 * j]) | ((uint32_t)f_bf16(v[2 * j + 1]) << 16);
    return r;
}

// Tile coordinates of workgroup blockIdx.x over the children's output tiles.
__device__ __forceinline__ int tile_child(const Gemm &g, int bx, int &n0) {
    int c = 0;
    int left = bx;
    for (; c < g.n_ch - 1; ++c) {
        const int nt = (g.ch[c].d_out + BN - 1) / BN;
        if (left < nt) break;
        left -= nt;
    }
    n0 = left * BN;
    return c;
}

template <int P>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Gemm g) {
    __shared__ u32x4 As[2][BM * LDC];
    __shared__ u32x4 Bs[2][P][BN * LDC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    int n0;
    const int cidx = P == 2 ? 0 : tile_child(g, blockIdx.x, n0);
    if (P == 2) n0 = blockIdx.x * BN;
    const Child &C0 = P == 2 ? g.ch[0] : (cidx == 0 ? g.ch[0] : cidx == 1 ? g.ch[1] : g.ch[2]);
    const int d_out = C0.d_out;
    const int m0 = blockIdx.y * BM;
    const int d_in = g.d_in, nch = d_in >> 3;
    const int nk = (d_in + BK - 1) / BK;

    const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
    const u32x4 *wg[P];
#pragma unroll
    for (int p = 0; p < P; ++p) wg[p] = reinterpret_cast<const u32x4 *>((P == 2 ? g.ch[p] : C0).W0);

    // Global -> register staging: two 16-byte pieces per thread per operand tile.
    u32x4 ra[2], rb[2][P];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = tid + kThreads * h;
            const int row = q >> 2, kc = kt * (BK / 8) + (q & 3);
            const bool kin = kc < nch;
            ra[h] = (kin && m0 + row < g.T) ? xg[(size_t)(m0 + row) * nch + kc] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int p = 0; p < P; ++p)
                rb[h][p] = (kin && n0 + row < d_out) ? __builtin_nontemporal_load(wg[p] + (size_t)(n0 + row) * nch + kc)
                                                     : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = tid + kThreads * h;
            const int row = q >> 2, kc = q & 3;
            As[buf][row * LDC + kc] = ra[h];
#pragma unroll
            for (int p = 0; p < P; ++p) Bs[buf][p][row * LDC + kc] = rb[h][p];
        }
    };

    f32x16 acc[P][2][2];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[p][i][j][e] = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int fr = lane & 31, fk = lane >> 5;   // fragment row / column, K half
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int kc = 2 * s + fk;
            u32x4 a[2], b[P][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = As[buf][(wm * 64 + i * 32 + fr) * LDC + kc];
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int j = 0; j < 2; ++j) b[p][j] = Bs[buf][p][(wn * 64 + j * 32 + fr) * LDC + kc];
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[p][i][j] = mfma(a[i], b[p][j], acc[p][i][j]);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue. Lane (fr, fk) of output tile (i, j) holds column o = n0 + wn*64 + j*32 + fr
    // and rows m0 + wm*64 + i*32 + 8*(e/4) + 4*fk + (e%4), e = 0..15.
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const Child &C = P == 2 ? g.ch[p] : C0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int o = n0 + wn * 64 + j * 32 + fr;
            const float sv = (C.s && o < d_out) ? C.s[o] : 1.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[p][i][j] *= sv;
        }
        const int r = C.r;
        for (int k0 = 0; k0 < r; k0 += 16) {
            const int kb = k0 + 8 * fk;
            u32x4 ahi[2], alo[2], bu[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int t = m0 + wm * 64 + i * 32 + fr;
                float hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v = 0.f;
                    if (t < g.T && kb + e < r)
                        for (int sl = 0; sl < C.vtx_slices; ++sl)
                            v += C.vtx[((size_t)sl * g.T + t) * r + kb + e];
                    hi[e] = bf16_f(f_bf16(v));
                    lo[e] = v - hi[e];
                }
                ahi[i] = pack8(hi);
                alo[i] = pack8(lo);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int o = n0 + wn * 64 + j * 32 + fr;
                float u[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u[e] = (o < d_out && kb + e < r) ? bf16_f(C.U[(size_t)o * r + kb + e]) : 0.f;
                bu[j] = pack8(u);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[p][i][j] = mfma(ahi[i], bu[j], acc[p][i][j]);
                    acc[p][i][j] = mfma(alo[i], bu[j], acc[p][i][j]);
                }
        }
    }

    const int col0 = P == 2 ? 0 : C0.col0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int o = n0 + wn * 64 + j * 32 + fr;
        if (o >= d_out) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
                if (t < g.T) {
                    const float v = P == 2 ? gelu_tanh(acc[0][i][j][e]) * acc[P - 1][i][j][e] : acc[0][i][j][e];
                    g.y[(size_t)t * g.ldy + col0 + o] = f_bf16(v);
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm(const Gemm &g, hipStream_t stream) {
    int ntiles = 0;
    if (g.pair)
        ntiles = (g.ch[0].d_out + BN - 1) / BN;
    else
        for (int c = 0; c < g.n_ch; ++c) ntiles += (g.ch[c].d_out + BN - 1) / BN;
    const dim3 grid(ntiles, (g.T + BM - 1) / BM);
    if (g.pair)
        hipLaunchKernelGGL(gemm_kernel<2>, grid, dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

}  // namespace wl
