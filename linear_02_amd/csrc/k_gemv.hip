// Decode-sized projections (one to eight tokens per pass), one launch per pass.
//
// At these token counts W0 is nearly all of the memory traffic (2 bytes per
// multiply-add), and every dependent global round trip costs on the order of a
// microsecond. So each launch issues all of its loads up front and then only
// computes:
//
// V^T x ("In-kernel reconstruction", introduction: the inner sum over i of
//   V[i,k] x[t,i]) reaches the epilogue in one of two ways.
//   * Redundant (small V, at most 2 tokens): every workgroup reads all of V
//     (from L2 after the first workgroup) with 16-byte loads issued before the
//     W0 stream, and reduces it itself after the stream. Each wave owns one
//     unit (a 16-byte column of V, or a part of one), its lanes walk the rows,
//     and a wave sum per rank entry finishes the unit; units of one column are
//     added in part order. No workgroup depends on another.
//   * Slice partials (otherwise): a V^T x launch just before this one wrote
//     per-slice partial sums; they are loaded before the W0 stream and added in
//     fixed groups of 16 slices, group sums in order, the same association in
//     every workgroup and for a child computed alone or with Q/K/V siblings.
// W0 x. A workgroup owns a few consecutive output rows; each of its four waves
//   streams R rows (or one segment of a long row) with its 64 lanes side by
//   side, 16 bytes per lane per load and up to 8 loads per row in flight. Each
//   lane keeps the matching 16-byte pieces of the tokens in registers (no LDS
//   staging, no barrier before the stream) and multiplies on v_dot2c_f32_bf16
//   into fp32. The epilogue operands (U rows, s) are also loaded up front.
// Loads are written so that the compiler can keep them in flight together:
//   every address is valid (indices clamped, a valid stand-in pointer where a
//   tensor is absent) and the value is masked afterwards, and per-child fields
//   are chosen with selects rather than by indexing the kernel-argument array
//   with a per-lane index (which becomes a chain of dependent vector loads).
// Epilogue. The wave sums (DPP butterflies) meet in LDS; the rank term
//   sum_k U[o,k] vtx[t,k] of each output is one wave's sum (lane k takes one
//   product); then one thread per (row, token) forms
//     y[t,o] = s[o] * (W0 x)[t,o] + sum_k U[o,k] vtx[t,k]
//   adding row segments in order, and rounds once to bf16. Pair mode (gate/up
//   of the MLP) streams the gate row and the up row together and writes
//   bf16(gelu_tanh(g) * u).
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxRowsG = 8;                 // rows per workgroup: (4 / nseg) * R <= 8
constexpr int kUPerThread = kMaxRowsG * 2 * kMaxRank / kThreads;
constexpr int kGroup = 16;                   // slices per group in the partial sums

__device__ __forceinline__ int child_index(const GemvF &g, int row) {
    if (g.n_ch > 2 && row >= g.ch[2].col0) return 2;
    if (g.n_ch > 1 && row >= g.ch[1].col0) return 1;
    return 0;
}

// Per-child fields chosen by a per-lane child index ci. Indexing the
// kernel-argument array with a per-lane index becomes a dependent vector load,
// and a chain of selects over the three values is turned by the compiler into
// a table in scratch memory; a sum of masked differences is neither.
template <class T>
__device__ __forceinline__ T blend3(int ci, T a, T b, T c) {
    return a + (ci > 0 ? b - a : T(0)) + (ci > 1 ? c - b : T(0));
}
struct ChFields {
    uint64_t U0, U1, U2, s0, s1, s2;
    int r0, r1, r2, c1, c2;   // ranks; first rows of children 1 and 2 (absent children are host-zeroed)
    __device__ __forceinline__ explicit ChFields(const GemvF &g)
        : U0((uint64_t)g.ch[0].U), U1((uint64_t)g.ch[1].U), U2((uint64_t)g.ch[2].U),
          s0((uint64_t)g.ch[0].s), s1((uint64_t)g.ch[1].s), s2((uint64_t)g.ch[2].s),
          r0(g.ch[0].r), r1(g.ch[1].r), r2(g.ch[2].r), c1(g.ch[1].col0), c2(g.ch[2].col0) {}
    __device__ __forceinline__ int r(int ci) const { return blend3(ci, r0, r1, r2); }
    __device__ __forceinline__ int col0(int ci) const { return blend3(ci, 0, c1, c2); }
    __device__ __forceinline__ const uint16_t *U(int ci) const {
        return reinterpret_cast<const uint16_t *>(blend3(ci, U0, U1, U2));
    }
    __device__ __forceinline__ const float *s(int ci) const {
        return reinterpret_cast<const float *>(blend3(ci, s0, s1, s2));
    }
};
__device__ __forceinline__ int ch_r(const GemvF &g, int ci) { return blend3(ci, g.ch[0].r, g.ch[1].r, g.ch[2].r); }

// Rank entries of all children flattened: item -> (child, token, k), item < total.
__device__ __forceinline__ int vtx_items(const GemvF &g, int tt) {
    return tt * (g.ch[0].r + (g.n_ch > 1 ? g.ch[1].r : 0) + (g.n_ch > 2 ? g.ch[2].r : 0));
}
__device__ __forceinline__ void vtx_item(const GemvF &g, int tt, int item, int &c, int &t, int &k) {
    const int n0 = tt * g.ch[0].r, n1 = g.n_ch > 1 ? tt * g.ch[1].r : 0;
    c = 0;
    if (g.n_ch > 1 && item >= n0) {
        item -= n0;
        c = 1;
        if (g.n_ch > 2 && item >= n1) {
            item -= n1;
            c = 2;
        }
    }
    const int r = max(ch_r(g, c), 1);
    t = item / r;
    k = item - t * r;
}

__device__ __forceinline__ float group_sum(const float *base, int stride, int s0, int s1) {
    float v[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) v[u] = base[(size_t)min(s0 + u, s1 - 1) * stride];
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) sum += s0 + u < s1 ? v[u] : 0.f;
    return sum;
}

// Slice partials, split mapping (items * groups <= threads): thread (item,
// group) loads one group of slices before the W0 stream (every address valid,
// the count of real slices kept in n) and adds them after it.
template <int TT>
__device__ __forceinline__ void gather_issue(const GemvF &g, int n_items, int n_groups, float (&v)[kGroup], int &n) {
    int item = threadIdx.x / n_groups;
    const int grp = threadIdx.x - item * n_groups;
    const bool ok = item < n_items;
    item = ok ? item : 0;
    int c, t, k;
    vtx_item(g, TT, item, c, t, k);
    const int r = ch_r(g, c);
    const float *base = g.partial + (size_t)c * kGemvPartialPerChild + t * r + k;
    const int s0 = grp * kGroup, s1 = min(g.S, s0 + kGroup);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) v[u] = ldg(base + (size_t)min(s0 + u, s1 - 1) * (TT * r));
    n = ok ? s1 - s0 : 0;
}
__device__ __forceinline__ float gather_finish(const float (&v)[kGroup], int n) {
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) sum += u < n ? v[u] : 0.f;
    return sum;
}

// Slice partials, full mapping: thread per item, groups in order, into vs.
template <int TT>
__device__ void gather_full(const GemvF &g, int n_items, float (*vs)[TT][kMaxRank]) {
    for (int item = threadIdx.x; item < n_items; item += kThreads) {
        int c, t, k;
        vtx_item(g, TT, item, c, t, k);
        const int r = ch_r(g, c);
        const float *base = g.partial + (size_t)c * kGemvPartialPerChild + t * r + k;
        float sum = 0.f;
        for (int s0 = 0; s0 < g.S; s0 += kGroup) sum += group_sum(base, TT * r, s0, min(g.S, s0 + kGroup));
        vs[c][t][k] = sum;
    }
}

// Redundant V^T x: this lane's 16-byte pieces of its wave's unit, and the
// matching tokens, loaded before the W0 stream.
//   r >= 8: piece j is V[j][kc*8 .. kc*8+8), token value x[t][j]
//   r == 4: piece j is rows 2j and 2j+1 of V (4 entries each), x[t][2j .. 2j+1]
template <int TT>
struct RedLoads {
    u32x4 v[kRedMaxPieces];
    uint32_t x[kRedMaxPieces][TT];
};

template <int TT>
__device__ __forceinline__ void red_issue(const GemvF &g, RedLoads<TT> &rl, int wave, int lane) {
    if (wave >= g.red_units) return;
    const Child &c = g.ch[g.red_c[wave]];
    const int r = c.r, lo = g.red_lo[wave], hi = g.red_hi[wave], kc = g.red_kc[wave];
#pragma unroll
    for (int m = 0; m < kRedMaxPieces; ++m) {
        const int j = lo + lane + kWave * m;
        const bool in = j < hi;
        const int jc = in ? j : lo;   // a valid piece; the value is dropped below
        const u32x4 v = *reinterpret_cast<const u32x4 *>(r >= 8 ? c.V + (size_t)jc * r + kc * 8 : c.V + (size_t)jc * 8);
        rl.v[m] = in ? v : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const bool tin = in && g.t0 + t < g.T;
            const uint16_t *xt = g.x + (size_t)min(g.t0 + t, g.T - 1) * g.d_in;
            const uint32_t xv = r >= 8 ? (uint32_t)xt[jc] : *reinterpret_cast<const uint32_t *>(xt + 2 * jc);
            rl.x[m][t] = tin ? xv : 0u;
        }
    }
}

// Reduce the loaded pieces: lane 63 of the wave ends with the unit's sums for
// its 8 rank slots, stored to upart[wave][slot][t].
template <int TT>
__device__ __forceinline__ void red_reduce(const GemvF &g, const RedLoads<TT> &rl, int wave, int lane,
                                           float (*upart)[8][TT]) {
    if (wave >= g.red_units) return;
    const int r = g.ch[g.red_c[wave]].r;
    float acc[8][TT];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[e][t] = 0.f;
#pragma unroll
    for (int m = 0; m < kRedMaxPieces; ++m) {
        const u32x4 v = rl.v[m];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const uint32_t xv = rl.x[m][t];
            const float x0 = bf16_f(xv & 0xFFFFu);
            const float x1 = r >= 8 ? x0 : bf16_f(xv >> 16);   // r == 4: second row of the piece
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ve = bf16_f(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu);
                acc[e][t] += ve * (e < 4 ? x0 : x1);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float s = wave_sum(acc[e][t]);
            if (lane == kWave - 1) upart[wave][e][t] = s;
        }
}

template <int TT, int R, int P, bool RED>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvF g) {
    constexpr int NB0 = (TT <= 2 ? 8 : TT == 4 ? 4 : 2) / (R * P);
    constexpr int NB = NB0 > 0 ? NB0 : 1;       // 16-byte loads per row per lane per batch
    constexpr bool RED_OK = RED && TT <= kRedMaxTok;
    __shared__ float mbuf[kWaves][R][P][TT];
    __shared__ float vs[kMaxChildren][TT][kMaxRank];
    __shared__ float ulds[kMaxRowsG][P][kMaxRank];
    __shared__ float slds[kMaxRowsG][P];
    __shared__ float gsum[kThreads];
    __shared__ float upart[kWaves][8][TT];
    __shared__ float rterm[kMaxRowsG][P][TT];

    // The wave index is uniform: keep it (and what derives from it) in scalar registers.
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = g.d_in >> 3;
    const int nseg = g.nseg;
    const int rows_g = (kWaves / nseg) * R;
    const int rowbase = blockIdx.x * rows_g;
    const bool red = RED_OK && g.vmode == kVtxRedundant;
    const bool parts = g.vmode == kVtxPartials;

    // ---- everything the epilogue needs, issued before the stream ----
    const ChFields cf(g);
    RedLoads<RED_OK ? TT : 1> rl;
    if constexpr (RED_OK)
        if (red) red_issue<TT>(g, rl, wave, lane);
    float upre[kUPerThread];
#pragma unroll
    for (int u = 0; u < kUPerThread; ++u) {
        const int item = tid + u * kThreads;          // (jr, p, k) over [kMaxRowsG][P][64]
        const int jr = item / (P * kMaxRank), p = (item / kMaxRank) % P, k = item % kMaxRank;
        const int row = rowbase + jr;
        const int ci = P == 2 ? p : child_index(g, min(row, g.rows - 1));
        const int r = cf.r(ci);
        const bool ok = jr < rows_g && row < g.rows && k < r;
        const uint16_t *src = ok ? cf.U(ci) + (size_t)(row - cf.col0(ci)) * r + k : g.x;
        const float v = bf16_f(ldg(src));
        upre[u] = ok ? v : 0.f;
    }
    float spre;
    {
        const int jr = min(tid / P, rows_g - 1), p = tid % P;
        const int row = min(rowbase + jr, g.rows - 1);
        const int ci = P == 2 ? p : child_index(g, row);
        const float *sp = cf.s(ci);
        const float v = ldg(sp ? sp + (row - cf.col0(ci)) : reinterpret_cast<const float *>(g.x));
        spre = sp ? v : 1.f;
    }
    const int n_items = g.vmode != kVtxNone ? vtx_items(g, TT) : 0;
    const int n_groups = (g.S + kGroup - 1) / kGroup;
    const bool split = n_items * n_groups <= kThreads;
    float gv[kGroup];
    int gn = 0;
    if (parts && split) gather_issue<TT>(g, n_items, n_groups, gv, gn);

    // ---- W0 x ----
    {
        const int seg = wave % nseg, rb = wave / nseg;
        const int row0 = rowbase + rb * R;
        const int seg_len = (nch + nseg - 1) / nseg;
        const int c_lo = seg * seg_len, c_hi = min(nch, c_lo + seg_len);
        const u32x4 *w[R][P];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = min(row0 + j, g.rows - 1);   // rows past the end re-read the last row
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const Child &c = g.ch[P == 2 ? p : child_index(g, row)];
                w[j][p] = reinterpret_cast<const u32x4 *>(c.W0 + (size_t)(row - c.col0) * g.d_in);
            }
        }
        const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
        float acc[R][P][TT];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int t = 0; t < TT; ++t) acc[j][p][t] = 0.f;

        for (int c0 = c_lo + lane; c0 < c_hi; c0 += kWave * NB) {
            u32x4 wv[NB][R][P], xv[NB][TT];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int cc = c0 + kWave * u;
                const bool in = cc < c_hi;
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        wv[u][j][p] = in ? __builtin_nontemporal_load(w[j][p] + cc) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int t = 0; t < TT; ++t)
                    xv[u][t] = (in && g.t0 + t < g.T) ? xg[(size_t)(g.t0 + t) * nch + cc] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < NB; ++u)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int j = 0; j < R; ++j)
#pragma unroll
                        for (int p = 0; p < P; ++p) acc[j][p][t] = dot8(wv[u][j][p], xv[u][t], acc[j][p][t]);
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const float v = wave_sum(acc[j][p][t]);
                    if (lane == 0) mbuf[wave][j][p][t] = v;
                }
    }

    // ---- epilogue ----
#pragma unroll
    for (int u = 0; u < kUPerThread; ++u) {
        const int item = tid + u * kThreads;
        if (item < kMaxRowsG * P * kMaxRank) (&ulds[0][0][0])[item] = upre[u];
    }
    if (tid < rows_g * P) (&slds[0][0])[tid] = spre;
    if constexpr (RED_OK)
        if (red) red_reduce<TT>(g, rl, wave, lane, upart);
    if (parts) {
        if (split)
            gsum[tid] = gather_finish(gv, gn);
        else
            gather_full<TT>(g, n_items, vs);
    }
    __syncthreads();
    if (parts && split)
        for (int item = tid; item < n_items; item += kThreads) {
            float sum = 0.f;
            for (int j = 0; j < n_groups; ++j) sum += gsum[item * n_groups + j];
            int c, t, k;
            vtx_item(g, TT, item, c, t, k);
            vs[c][t][k] = sum;
        }
    if (red)
        for (int item = tid; item < n_items; item += kThreads) {
            // Units of the column holding (c, k), in part order.
            int c, t, k;
            vtx_item(g, TT, item, c, t, k);
            const bool wide = ch_r(g, c) >= 8;
            const int kc = wide ? k >> 3 : 0, e = wide ? (k & 7) : k;
            float sum = 0.f;
            for (int u = 0; u < g.red_units; ++u)
                if (g.red_c[u] == c && g.red_kc[u] == kc)
                    sum += wide ? upart[u][e][t] : upart[u][e][t] + upart[u][e + 4][t];
            vs[c][t][k] = sum;
        }
    __syncthreads();

    // Rank term of each (row, p, token): one wave per output, lane k takes
    // U[o,k] vtx[t,k], and a wave sum (fixed butterfly order) adds them.
    if (n_items > 0) {
        const int n_out = rows_g * P * TT;
        for (int oi = wave; oi < n_out; oi += kWaves) {
            const int jr = oi / (P * TT), p = (oi / TT) % P, t = oi % TT;
            const int row = min(rowbase + jr, g.rows - 1);
            const int ci = P == 2 ? p : child_index(g, row);
            const int r = ch_r(g, ci);
            const float prod = lane < r ? ulds[jr][p][lane] * vs[ci][t][lane] : 0.f;
            const float sum = wave_sum(prod);
            if (lane == 0) rterm[jr][p][t] = sum;
        }
        __syncthreads();
    }

    for (int idx = tid; idx < rows_g * TT; idx += kThreads) {
        const int jr = idx / TT, t = idx - jr * TT;
        const int rbi = jr / R, j = jr - rbi * R;
        const int row = rowbase + jr;
        const int tok = g.t0 + t;
        if (row >= g.rows || tok >= g.T) continue;
        float val[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float m = 0.f;
            for (int sg = 0; sg < nseg; ++sg) m += mbuf[rbi * nseg + sg][j][p][t];
            val[p] = slds[jr][p] * m + (n_items > 0 ? rterm[jr][p][t] : 0.f);
        }
        const float out = P == 2 ? gelu_tanh(val[0]) * val[P - 1] : val[0];
        g.y[(size_t)tok * g.ldy + row] = f_bf16(out);
    }
}

template <int TT, int R, int P, bool RED>
hipError_t launch_tt(const GemvF &g, int n_wg, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_kernel<TT, R, P, RED>), dim3(n_wg), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

template <int R, int P>
hipError_t launch_r(const GemvF &g, int tt, int n_wg, hipStream_t stream) {
    const bool red = g.vmode == kVtxRedundant;
    switch (tt) {
        case 8: return launch_tt<8, R, P, false>(g, n_wg, stream);
        case 4: return launch_tt<4, R, P, false>(g, n_wg, stream);
        case 2: return red ? launch_tt<2, R, P, true>(g, n_wg, stream) : launch_tt<2, R, P, false>(g, n_wg, stream);
        default: return red ? launch_tt<1, R, P, true>(g, n_wg, stream) : launch_tt<1, R, P, false>(g, n_wg, stream);
    }
}

}  // namespace

// Slices of the input axis for the V^T x launch: about 128 inputs each, at most
// kGemvMaxSlices. They depend on d_in only, so a child's vtx is summed in the
// same order whether it is computed alone or with Q/K/V siblings.
int gemv_slice_len(int d_in) {
    int S = (d_in + 127) / 128;
    if (S > kGemvMaxSlices) S = kGemvMaxSlices;
    return ((d_in + S - 1) / S + 7) / 8 * 8;
}

// Tokens per pass: the smallest power of two covering T, at most kGemvMaxTok.
// 0 when d_in is beyond what the decode kernel supports.
int gemv_tokens_per_pass(int d_in, int T) {
    if (d_in > kGemvMaxDin) return 0;
    int tt = 1;
    while (tt < T && tt < kGemvMaxTok) tt *= 2;
    return tt;
}

GemvPlan gemv_plan(const GemvF &g, int tt, bool allow_redundant) {
    GemvPlan p;
    const int nch = g.d_in / 8;
    p.nseg = nch <= 640 ? 1 : nch <= 1280 ? 2 : 4;
    p.R = (p.nseg == 1 && nch <= 256) ? 2 : 1;
    const int rows_g = (kWaves / p.nseg) * p.R;
    p.n_wg = (g.rows + rows_g - 1) / rows_g;
    p.slice_len = gemv_slice_len(g.d_in);
    int sum_r = 0;
    for (int c = 0; c < g.n_ch; ++c) sum_r += g.ch[c].r;
    p.S = sum_r > 0 ? (g.d_in + p.slice_len - 1) / p.slice_len : 0;
    p.vmode = sum_r > 0 ? kVtxPartials : kVtxNone;
    if (sum_r == 0 || !allow_redundant || tt > kRedMaxTok) return p;

    // Redundant V^T x: every child's rank must be 4 or a multiple of 8, the
    // columns (16-byte wide, or one for r == 4) at most one per wave, each
    // lane's share of its unit within kRedMaxPieces pieces, and the re-reads of
    // V by all workgroups within kRedMaxTraffic bytes (measured: beyond a few MB
    // they cost more than a separate V^T x launch).
    if ((long long)p.n_wg * g.d_in * sum_r * 2 > kRedMaxTraffic) return p;
    int cols = 0;
    for (int c = 0; c < g.n_ch; ++c) {
        const int r = g.ch[c].r;
        if (r == 0) continue;
        if (r != 4 && r % 8) return p;
        cols += r >= 8 ? r / 8 : 1;
    }
    if (cols > kWaves) return p;
    const int parts = cols == 1 ? 4 : cols == 2 ? 2 : 1;
    int u = 0;
    for (int c = 0; c < g.n_ch; ++c) {
        const int r = g.ch[c].r;
        if (r == 0) continue;
        const int pieces = r >= 8 ? g.d_in : g.d_in / 2;
        const int per = (pieces + parts - 1) / parts;
        if ((per + kWave - 1) / kWave > kRedMaxPieces) return p;
        for (int kc = 0; kc < (r >= 8 ? r / 8 : 1); ++kc)
            for (int q = 0; q < parts; ++q) {
                p.red_c[u] = c;
                p.red_kc[u] = kc;
                p.red_lo[u] = q * per;
                p.red_hi[u] = min(pieces, (q + 1) * per);
                ++u;
            }
    }
    p.red_units = u;
    p.vmode = kVtxRedundant;
    return p;
}

hipError_t launch_gemv(const GemvF &g, const GemvPlan &plan, int tt, hipStream_t stream) {
    GemvF a = g;
    a.nseg = plan.nseg;
    a.S = plan.S;
    a.vmode = plan.vmode;
    a.red_units = plan.red_units;
    for (int u = 0; u < kWaves; ++u) {
        a.red_c[u] = plan.red_c[u];
        a.red_kc[u] = plan.red_kc[u];
        a.red_lo[u] = plan.red_lo[u];
        a.red_hi[u] = plan.red_hi[u];
    }
    if (g.pair) {
        if (plan.R == 2) return launch_r<2, 2>(a, tt, plan.n_wg, stream);
        return launch_r<1, 2>(a, tt, plan.n_wg, stream);
    }
    if (plan.R == 2) return launch_r<2, 1>(a, tt, plan.n_wg, stream);
    return launch_r<1, 1>(a, tt, plan.n_wg, stream);
}

}  // namespace wl
