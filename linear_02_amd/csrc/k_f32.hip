// The fp32 variant of every operation: W0, U, V, x, y (and the MLP's h, and
// W_eff) in IEEE binary32, s fp32 as always. The custom-op description on the
// "In-kernel reconstruction" page says the op also supports float32; the
// arithmetic is the same reconstruction formula, accumulated in fp32 and never
// rounded below fp32.
//
// Launches of one projection (children share x):
//   1. f32_vtx_part_kernel   part[c][slice][t][k] = sum over the slice's inputs i of V_c[i][k] x[t][i]
//   2. f32_vtx_sum_kernel    vtx[c][t][k] = the slices of part added in slice order
//   3. f32_gemv_kernel (T <= 8: one wave per output row, W0 rows streamed as
//      16-byte pieces) or f32_gemm_kernel (matrix cores, v_mfma_f32_32x32x2_f32,
//      128-token tiles through LDS), both ending with
//      y[t][col0 + o] = s[o] * m[t][o] + sum_k U[o][k] vtx[t][k]
//      (pair mode: h[t][o] = gelu_tanh(gate) * up).
// Launches 1-2 are skipped when no child has a rank term. Every sum runs in a
// fixed order, so results repeat bit for bit.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum_f32(float v) {
    // Butterfly over the 64 lanes: every lane ends with the same, fixed-order sum.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---- V^T x ---------------------------------------------------------------------
// Slice partials. A workgroup of 64 rank lanes x 4 groups takes one slice of
// kF32VtxSlice inputs and the slice of x for its tokens in LDS (zeros past the
// slice's end and past T).
//   FEW (T <= 4): the four groups split the slice's inputs; each thread loads
//     its 64 V values at once (one memory round trip) and sums every token; the
//     groups' sums are added in group order through LDS.
//   else: the groups split kVtxTokMany tokens; each thread streams the slice's
//     V values sixteen at a time and keeps its tokens' sums.
// Every sum runs in input order within a thread, then in a fixed order.
constexpr int kVtxTokMany = 32;

template <bool FEW>
__global__ __launch_bounds__(256) void f32_vtx_part_kernel(F32Vtx job) {
    constexpr int NTOK = FEW ? 4 : kVtxTokMany;           // tokens of a workgroup
    __shared__ float xs[NTOK][kF32VtxSlice];
    __shared__ float red[FEW ? 4 * 4 * 64 : 1];
    const int c = blockIdx.z, slice = blockIdx.x;
    const int r = c == 0 ? job.r[0] : c == 1 ? job.r[1] : job.r[2];
    const float *V = c == 0 ? job.V[0] : c == 1 ? job.V[1] : job.V[2];
    float *part = c == 0 ? job.part[0] : c == 1 ? job.part[1] : job.part[2];
    const int tid = threadIdx.x, k = tid & 63, grp = tid >> 6;
    const int i0 = slice * kF32VtxSlice, len = min(job.d_in - i0, kF32VtxSlice);
    const int t0 = blockIdx.y * NTOK;
    for (int e = tid; e < NTOK * kF32VtxSlice; e += 256) {
        const int tt = e / kF32VtxSlice, i = e % kF32VtxSlice, t = t0 + tt;
        xs[tt][i] = (i < len && t < job.T) ? job.x[(size_t)t * job.d_in + i0 + i] : 0.f;
    }
    __syncthreads();
    const int kc = min(k, r - 1);   // lanes past r compute a copy of column r - 1 and store nothing
    if constexpr (FEW) {
        constexpr int Q = kF32VtxSlice / 4;
        float v[Q], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < Q; ++u) v[u] = V[(size_t)(i0 + min(grp * Q + u, len - 1)) * r + kc];
#pragma unroll
        for (int u = 0; u < Q; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = fmaf(v[u], xs[t][grp * Q + u], acc[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) red[(grp * 4 + t) * 64 + k] = acc[t];
        __syncthreads();
        if (grp == 0 && k < r) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float a = ((red[t * 64 + k] + red[(4 + t) * 64 + k]) + red[(8 + t) * 64 + k]) +
                                red[(12 + t) * 64 + k];
                if (t0 + t < job.T) part[((size_t)slice * job.T + t0 + t) * r + k] = a;
            }
        }
    } else {
        constexpr int PT = NTOK / 4;   // tokens per thread: grp, grp + 4, ...
        float acc[PT];
#pragma unroll
        for (int j = 0; j < PT; ++j) acc[j] = 0.f;
        for (int i = 0; i < kF32VtxSlice; i += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = V[(size_t)(i0 + min(i + u, len - 1)) * r + kc];
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int j = 0; j < PT; ++j) acc[j] = fmaf(v[u], xs[grp + 4 * j][i + u], acc[j]);
        }
        if (k < r) {
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                const int t = t0 + grp + 4 * j;
                if (t < job.T) part[((size_t)slice * job.T + t) * r + k] = acc[j];
            }
        }
    }
}

// vtx[c][t][k]: one wave per element, lane j adding slices j, j + 64, ... in order,
// then a butterfly over the lanes.
__global__ __launch_bounds__(256) void f32_vtx_sum_kernel(F32Vtx job) {
    const int c = blockIdx.y, lane = threadIdx.x & 63;
    const int r = c == 0 ? job.r[0] : c == 1 ? job.r[1] : job.r[2];
    const float *part = c == 0 ? job.part[0] : c == 1 ? job.part[1] : job.part[2];
    float *vtx = c == 0 ? job.vtx[0] : c == 1 ? job.vtx[1] : job.vtx[2];
    const size_t n = (size_t)job.T * r, e = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= n) return;   // wave-uniform
    float a = 0.f;
    for (int s = lane; s < job.n_slices; s += 64) a += part[(size_t)s * n + e];
    a = wave_sum_f32(a);
    if (lane == 0) vtx[e] = a;
}

// ---- few tokens: one wave per output row (P = 2: one row of gate and of up) ----
template <int P, int TT>
__global__ __launch_bounds__(256) void f32_gemv_kernel(F32Proj g) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * 4 + wave;
    int rows = 0;
    if (P == 2)
        rows = g.ch[0].d_out;
    else
        for (int c = 0; c < g.n_ch; ++c) rows += g.ch[c].d_out;
    if (row >= rows) return;   // wave-uniform; the kernel has no barrier
    int c0 = 0, o = row;
    if (P == 1)
        while (c0 < g.n_ch - 1 && o >= g.ch[c0].d_out) o -= g.ch[c0++].d_out;
    const F32Child *ch[P];
#pragma unroll
    for (int p = 0; p < P; ++p) ch[p] = &g.ch[P == 2 ? p : c0];

    const int T = g.T, n4 = g.d_in >> 2;
    const f32x4v *xg = reinterpret_cast<const f32x4v *>(g.x);
    const f32x4v *wr[P];
#pragma unroll
    for (int p = 0; p < P; ++p) wr[p] = reinterpret_cast<const f32x4v *>(ch[p]->W0) + (size_t)o * n4;
    float acc[P][TT];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[p][t] = 0.f;
#pragma unroll 8
    for (int q = lane; q < n4; q += 64) {
        f32x4v w[P];
#pragma unroll
        for (int p = 0; p < P; ++p) w[p] = __builtin_nontemporal_load(wr[p] + q);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const f32x4v xv = xg[(size_t)min(t, T - 1) * n4 + q];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                float a = acc[p][t];
                a = fmaf(w[p].x, xv.x, a);
                a = fmaf(w[p].y, xv.y, a);
                a = fmaf(w[p].z, xv.z, a);
                a = fmaf(w[p].w, xv.w, a);
                acc[p][t] = a;
            }
        }
    }
    float out[P][TT];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const F32Child &C = *ch[p];
        const float sv = C.s ? C.s[o] : 1.0f;
        const float u = lane < C.r ? C.U[(size_t)o * C.r + lane] : 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float m = wave_sum_f32(acc[p][t]);
            float rk = 0.f;
            if (C.r > 0) {
                const float v = lane < C.r ? C.vtx[(size_t)min(t, T - 1) * C.r + lane] : 0.f;
                rk = wave_sum_f32(u * v);
            }
            out[p][t] = fmaf(sv, m, rk);
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
        if (lane == t && t < T)
            g.y[(size_t)t * g.ldy + ch[0]->col0 + o] = P == 2 ? gelu_tanh(out[0][t]) * out[P - 1][t] : out[0][t];
}

// ---- many tokens: matrix cores -------------------------------------------------
// Workgroup tile: 128 tokens x 128 output columns (P = 2: 64 of gate and the same
// 64 of up), four waves of 64 x 64 (P = 2: 64 x 32 per child), input axis in
// steps of 16 through two LDS buffers (rows padded to 20 floats: the fragment
// reads of 32 rows are then free of bank conflicts). MFMA step s of a 16-input
// block pairs input s (lanes 0-31) with input 8 + s (lanes 32-63) in both
// operands, so each lane's eight inputs of a block are contiguous in LDS.
constexpr int kBM = 128, kBK = 16, kLdsRow = kBK + 4;

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int P>
__global__ __launch_bounds__(256) void f32_gemm_kernel(F32Proj g) {
    constexpr int BN = kBM / P;          // output columns per child
    constexpr int TN = 2 / P;            // 32-column blocks per wave and child
    __shared__ __attribute__((aligned(16))) float As[2][kBM][kLdsRow];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBM][kLdsRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int fr = lane & 31, fh = lane >> 5;

    const int n_mt = (g.T + kBM - 1) / kBM;
    const int mt = blockIdx.x % n_mt, nt = blockIdx.x / n_mt;
    int cidx = 0, n0 = nt * BN;
    if (P == 1) {
        int left = nt;
        while (cidx < g.n_ch - 1 && left >= (g.ch[cidx].d_out + BN - 1) / BN) left -= (g.ch[cidx++].d_out + BN - 1) / BN;
        n0 = left * BN;
    }
    const F32Child *ch[P];
#pragma unroll
    for (int p = 0; p < P; ++p) ch[p] = &g.ch[P == 2 ? p : cidx];
    const int d_out = ch[0]->d_out, m0 = mt * kBM, d_in = g.d_in, T = g.T;

    // Tile loads: thread q = h*256 + tid takes row q / 4, 16-byte piece q % 4.
    const f32x4v zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4v ra[2], rb[2];
    auto load = [&](int k0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = h * 256 + tid, row = q >> 2, k = k0 + 4 * (q & 3);
            const bool kin = k < d_in;
            const int kc = kin ? k : 0;
            const f32x4v a = *reinterpret_cast<const f32x4v *>(g.x + (size_t)min(m0 + row, T - 1) * d_in + kc);
            ra[h] = kin ? a : zero4;
            const int p = row / BN, o = min(n0 + row % BN, d_out - 1);
            const float *w = (P == 2 && p == 1) ? ch[P - 1]->W0 : ch[0]->W0;
            const f32x4v b = *reinterpret_cast<const f32x4v *>(w + (size_t)o * d_in + kc);
            rb[h] = kin ? b : zero4;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = h * 256 + tid, row = q >> 2, pc = q & 3;
            *reinterpret_cast<f32x4v *>(&As[buf][row][4 * pc]) = ra[h];
            *reinterpret_cast<f32x4v *>(&Bs[buf][row][4 * pc]) = rb[h];
        }
    };

    f32x16 acc[P][2][TN];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[p][i][j][e] = 0.f;

    // One 16-input block from LDS buffer `buf` into the accumulators of children [p_lo, p_hi).
    auto compute = [&](int buf, int p_lo, int p_hi) {
        float a[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float *src = &As[buf][wm * 64 + i * 32 + fr][8 * fh];
            const f32x4v lo = *reinterpret_cast<const f32x4v *>(src), hi = *reinterpret_cast<const f32x4v *>(src + 4);
            a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
            a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (p < p_lo || p >= p_hi) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float *src = &Bs[buf][p * BN + wn * (BN / 2) + j * 32 + fr][8 * fh];
                const f32x4v lo = *reinterpret_cast<const f32x4v *>(src), hi = *reinterpret_cast<const f32x4v *>(src + 4);
                const float b[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int s = 0; s < 8; ++s)
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[p][i][j] = mfma_f32(a[i][s], b[s], acc[p][i][j]);
            }
        }
    };

    const int nk = (d_in + kBK - 1) / kBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load((kt + 1) * kBK);
        compute(kt & 1, 0, P);
        if (kt + 1 < nk) store((kt + 1) & 1);
        __syncthreads();
    }

    // Scale by s, then the rank term as further 16-wide steps over (vtx, U).
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const F32Child &C = *ch[p];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int o = n0 + wn * (BN / 2) + j * 32 + fr;
            const float sv = C.s ? C.s[min(o, d_out - 1)] : 1.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[p][i][j] *= sv;
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const F32Child &C = *ch[p];
        const int r = C.r;
        for (int k0 = 0; k0 < r; k0 += kBK) {
            // A: vtx rows of the tile's tokens; B: U rows of this child's columns.
            for (int e = tid; e < kBM * kBK; e += 256) {
                const int row = e / kBK, kk = e % kBK, k = k0 + kk;
                const bool ok = k < r;
                As[0][row][kk] = ok ? C.vtx[(size_t)min(m0 + row, T - 1) * r + min(k, r - 1)] : 0.f;
            }
            for (int e = tid; e < BN * kBK; e += 256) {
                const int row = e / kBK, kk = e % kBK, k = k0 + kk;
                const bool ok = k < r;
                Bs[0][p * BN + row][kk] = ok ? C.U[(size_t)min(n0 + row, d_out - 1) * r + min(k, r - 1)] : 0.f;
            }
            __syncthreads();
            compute(0, p, p + 1);
            __syncthreads();
        }
    }

    // Lane (fr, fh) of block (i, j): column o = n0 + wn*(BN/2) + j*32 + fr, token rows
    // m0 + wm*64 + i*32 + 8*(e/4) + 4*fh + (e%4).
    const int col0 = ch[0]->col0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int o = n0 + wn * (BN / 2) + j * 32 + fr;
        if (o >= d_out) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                if (t < T) {
                    const float v = P == 2 ? gelu_tanh(acc[0][i][j][e]) * acc[P - 1][i][j][e] : acc[0][i][j][e];
                    g.y[(size_t)t * g.ldy + col0 + o] = v;
                }
            }
    }
}

// ---- W_eff[o][i] = s[o] W0[o][i] + sum_k U[o][k] V[i][k], fp32 ---------------------
// Workgroup: 256 consecutive columns i (one per thread, V[i][:] in registers) x
// kWeffRows rows o (U rows and s in LDS). Every W0 load of the workgroup is
// issued before any product, and the products run rank step outer, row inner:
// kWeffRows independent sums per thread instead of one dependent chain per row
// (64 rows per workgroup, row after row, took 241 µs for a layer's seven
// projections, the small ones bound by a single wave's chain).
constexpr int kWeffRows = 32;
template <int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void f32_weff_kernel(WeffF32 w) {
    __shared__ __attribute__((aligned(16))) float Us[kMaxRank][kWeffRows];   // [k][row]
    __shared__ float ss[kWeffRows];
    const int tid = threadIdx.x, i = blockIdx.x * 256 + tid, o0 = blockIdx.y * kWeffRows;
    const int r = w.r, rows = min(kWeffRows, w.d_out - o0);
    constexpr int RB1 = RB > 0 ? RB : 1;   // (no iteration when RB = 0)
    for (int e = tid; e < kWeffRows * RB; e += 256) {
        const int row = e / RB1, k = e % RB1;
        Us[k][row] = (row < rows && k < r) ? w.U[(size_t)(o0 + row) * r + k] : 0.f;
    }
    if (tid < kWeffRows) ss[tid] = (tid < rows && w.s) ? w.s[o0 + tid] : 1.0f;
    const int ic = min(i, w.d_in - 1);
    float w0[kWeffRows];
#pragma unroll
    for (int j = 0; j < kWeffRows; ++j)
        w0[j] = __builtin_nontemporal_load(w.W0 + (size_t)(o0 + min(j, rows - 1)) * w.d_in + ic);
    float v[RB1];
    v[0] = 0.f;
    if (RB == 0) {
        // no rank term: V is not read (it may be null)
    } else if ((r & 3) == 0) {
        // V[i][:] as 16-byte pieces (rows 16-byte aligned), masked past r
#pragma unroll
        for (int k = 0; k < RB1; k += 4) {
            const f32x4 p4 = *reinterpret_cast<const f32x4 *>(w.V + (size_t)ic * r + min(k, r - 4));
            v[k] = k < r ? p4.x : 0.f;
            if (k + 1 < RB1) v[k + 1] = k < r ? p4.y : 0.f;
            if (k + 2 < RB1) v[k + 2] = k < r ? p4.z : 0.f;
            if (k + 3 < RB1) v[k + 3] = k < r ? p4.w : 0.f;
        }
    } else {
#pragma unroll
        for (int k = 0; k < RB1; ++k) v[k] = k < r ? w.V[(size_t)ic * r + min(k, r - 1)] : 0.f;
    }
    __syncthreads();
    float d[kWeffRows];
#pragma unroll
    for (int j = 0; j < kWeffRows; ++j) d[j] = 0.f;
#pragma unroll 4
    for (int k = 0; k < RB; ++k) {
        float uk[kWeffRows];
#pragma unroll
        for (int q = 0; q < kWeffRows / 4; ++q) {
            const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&Us[k][4 * q]);
            uk[4 * q] = u4.x;
            uk[4 * q + 1] = u4.y;
            uk[4 * q + 2] = u4.z;
            uk[4 * q + 3] = u4.w;
        }
#pragma unroll
        for (int j = 0; j < kWeffRows; ++j) d[j] = fmaf(uk[j], v[k], d[j]);
    }
    if (i >= w.d_in) return;
#pragma unroll
    for (int j = 0; j < kWeffRows; ++j)
        if (j < rows) __builtin_nontemporal_store(fmaf(ss[j], w0[j], d[j]), w.W_eff + (size_t)(o0 + j) * w.d_in + i);
}

}  // namespace

int f32_vtx_slices(int d_in) { return (d_in + kF32VtxSlice - 1) / kF32VtxSlice; }

hipError_t launch_f32_vtx(const F32Vtx &job, hipStream_t stream) {
    if (job.n_ch == 0) return hipSuccess;
    int max_r = 0;
    for (int c = 0; c < job.n_ch; ++c) max_r = job.r[c] > max_r ? job.r[c] : max_r;
    if (job.T <= 4)
        hipLaunchKernelGGL(f32_vtx_part_kernel<true>, dim3(job.n_slices, 1, job.n_ch), dim3(256), 0, stream, job);
    else
        hipLaunchKernelGGL(f32_vtx_part_kernel<false>,
                           dim3(job.n_slices, (job.T + kVtxTokMany - 1) / kVtxTokMany, job.n_ch), dim3(256), 0,
                           stream, job);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(f32_vtx_sum_kernel, dim3((unsigned)(((size_t)job.T * max_r + 3) / 4), job.n_ch), dim3(256), 0,
                       stream, job);
    return hipGetLastError();
}

hipError_t launch_f32_gemv(const F32Proj &g, hipStream_t stream) {
    int rows = 0;
    if (g.pair)
        rows = g.ch[0].d_out;
    else
        for (int c = 0; c < g.n_ch; ++c) rows += g.ch[c].d_out;
    const dim3 grid((rows + 3) / 4), block(256);
#define WL_F32_GEMV(PP, TTT) hipLaunchKernelGGL((f32_gemv_kernel<PP, TTT>), grid, block, 0, stream, g)
    if (g.pair) {
        if (g.T <= 1) WL_F32_GEMV(2, 1);
        else if (g.T <= 2) WL_F32_GEMV(2, 2);
        else if (g.T <= 4) WL_F32_GEMV(2, 4);
        else WL_F32_GEMV(2, 8);
    } else {
        if (g.T <= 1) WL_F32_GEMV(1, 1);
        else if (g.T <= 2) WL_F32_GEMV(1, 2);
        else if (g.T <= 4) WL_F32_GEMV(1, 4);
        else WL_F32_GEMV(1, 8);
    }
#undef WL_F32_GEMV
    return hipGetLastError();
}

hipError_t launch_f32_gemm(const F32Proj &g, hipStream_t stream) {
    const int bn = g.pair ? kBM / 2 : kBM;
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + bn - 1) / bn;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + bn - 1) / bn;
    const int total = n_nt * ((g.T + kBM - 1) / kBM);
    if (g.pair)
        hipLaunchKernelGGL(f32_gemm_kernel<2>, dim3(total), dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL(f32_gemm_kernel<1>, dim3(total), dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_weff_f32(const WeffF32 &w, hipStream_t stream) {
    const dim3 grid((w.d_in + 255) / 256, (w.d_out + kWeffRows - 1) / kWeffRows), block(256);
    if (w.r == 0) hipLaunchKernelGGL(f32_weff_kernel<0>, grid, block, 0, stream, w);
    else if (w.r <= 8) hipLaunchKernelGGL(f32_weff_kernel<8>, grid, block, 0, stream, w);
    else if (w.r <= 16) hipLaunchKernelGGL(f32_weff_kernel<16>, grid, block, 0, stream, w);
    else if (w.r <= 32) hipLaunchKernelGGL(f32_weff_kernel<32>, grid, block, 0, stream, w);
    else hipLaunchKernelGGL(f32_weff_kernel<64>, grid, block, 0, stream, w);
    return hipGetLastError();
}

}  // namespace wl
