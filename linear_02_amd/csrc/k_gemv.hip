// Decode-sized projections (one to eight tokens per pass), one launch per pass.
//
// At these token counts W0 is nearly all of the memory traffic (2 bytes per
// multiply-add), and every dependent global round trip costs on the order of a
// microsecond. So each launch issues all of its loads up front and then only
// computes:
//
// V^T x ("In-kernel reconstruction", introduction: the inner sum over i of
//   V[i,k] x[t,i]) reaches the epilogue as per-slice partial sums, added in
//   fixed groups of 16 slices, group sums in order: the same association in
//   every workgroup and for a child computed alone or with Q/K/V siblings. The
//   partials come from one of two places:
//     - In-launch (at most 4 tokens per pass): the first workgroups of this
//       launch are producers, one per (child, slice), each computing its slice
//       as the V^T x launch would. Each partial is stored as one 64-bit word,
//       the launch's tag (generation + 1, from a ticket counter) beside the
//       fp32 value, by a single device-scope atomic store. The other
//       workgroups take the same tag at their start, stream W0, then read the
//       words with device-scope atomic loads and read again any word still
//       without their tag. A word with the right tag holds the right value,
//       so no fence or flag is needed (a release fence writes back the whole
//       L2 on this chip and cost more than the separate launch it replaces).
//       Producers come first in the grid, so they are dispatched before any
//       workgroup waits for them, and each wait is bounded: a workgroup whose
//       wait runs out computes every slice itself in the same order, and gets
//       the same bits.
//     - A V^T x launch just before this one; the partials are then loaded
//       before the W0 stream.
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
// Epilogue. The wave sums (DPP butterflies) meet in LDS with U and s; then one
//   thread per (row, token) forms
//     y[t,o] = s[o] * (W0 x)[t,o] + sum_k U[o,k] vtx[t,k]
//   adding row segments in order and the rank term as four interleaved partial
//   sums (k mod 4) added pairwise, and rounds once to bf16. The steps after
//   the stream are few and short: each is a chain of dependent instructions of
//   a single wave, so each barrier-separated step costs a few tenths of a
//   microsecond. Pair mode (gate/up of the MLP) streams the gate row and the up
//   row together and writes bf16(gelu_tanh(g) * u).
#include "wl_device.h"
#include "wl_kernels.h"
#include "wl_vtx_slice.h"
#include "wl_handoff.h"

namespace wl {

namespace {

constexpr int kThreads = kHThreads;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxRowsG = 8;                 // rows per workgroup: (4 / nseg) * R <= 8
constexpr int kUPerThread = kMaxRowsG * 2 * kMaxRank / kThreads;
#ifndef WL_ONE_LEVEL_MAX_READS
#define WL_ONE_LEVEL_MAX_READS 4096
#endif
constexpr long long kOneLevelMaxReads = WL_ONE_LEVEL_MAX_READS;   // in-launch hand-off, see gemv_plan

template <int TT, int R, int P>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvF g) {
    constexpr int NB0 = (TT <= 2 ? 8 : TT == 4 ? 4 : 2) / (R * P);
    constexpr int NB = NB0 > 0 ? NB0 : 1;       // 16-byte loads per row per lane per batch
    constexpr bool INL = TT <= kInLaunchMaxTok;  // in-launch hand-off
    __shared__ float mbuf[kWaves][R][P][TT];
    __shared__ float vred[INL ? kThreads : 1][TT + 1];             // producer / fallback slice sums
    __shared__ float fgs[INL ? kMaxChildren * TT * kMaxRank : 1];  // fallback group sums
    __shared__ uint32_t tag_lds;
    __shared__ u32x4 xstage[INL && TT > 2 ? TT * kXStageMax / 8 : 1];   // producer / fallback x slice
    __shared__ __attribute__((aligned(16))) float vs[kMaxChildren][TT][kMaxRank];
    __shared__ __attribute__((aligned(16))) float ulds[kMaxRowsG][P][kMaxRank];
    __shared__ float slds[kMaxRowsG][P];
    __shared__ float gsum[kThreads];

    // The wave index is uniform: keep it (and what derives from it) in scalar registers.
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = g.d_in >> 3;
    const int nseg = g.nseg;
    const int rows_g = (kWaves / nseg) * R;
    const bool parts = g.vmode == kVtxPartials;
    const bool inl = INL && g.vmode == kVtxInLaunch;
    unsigned long long ticket;   // thread 0 of an in-launch projection workgroup only
    if constexpr (INL) {
        if (inl) {
            if ((int)blockIdx.x < g.n_prod) {
                vtx_produce<TT>(g, vred, xstage, &tag_lds, gsum, vs);
                return;
            }
            if (tid == 0) ticket = take_ticket(g);   // used after the stream
        }
    }
    const int rowbase = ((int)blockIdx.x - g.n_prod) * rows_g;

    // ---- everything the epilogue needs, issued before the stream ----
    const ChFields cf(g);
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

    // ---- epilogue operands into LDS (loaded before the stream) ----
#pragma unroll
    for (int u = 0; u < kUPerThread; ++u) {
        const int item = tid + u * kThreads;
        if (item < kMaxRowsG * P * kMaxRank) (&ulds[0][0][0])[item] = upre[u];
    }
    if (tid < rows_g * P) (&slds[0][0])[tid] = spre;
    // Split mapping with one group of slices: thread `item` holds its entry's
    // whole sum and writes it into vs itself. Its (child, token, rank), worked
    // out while the words may still be on their way.
    const bool own_entry = split && n_groups == 1;
    int vc = 0, vt = 0, vk = 0;
    if (own_entry) vtx_item(g, TT, min(tid, max(n_items - 1, 0)), vc, vt, vk);

    // ---- V^T x from this launch's producers ----
    bool have = false, fallback = false;
    if constexpr (INL) {
        if (inl) {
            if (tid == 0) tag_lds = ticket_tag(ticket);
            __syncthreads();
            const int retries = g.spin_limit - 1;   // spin_limit reads in all; 0: none
            const bool got = g.spin_limit > 0 &&
                             (g.two_level ? gather_final<TT>(g, n_items, tag_lds, retries, vs)
                              : split     ? gather_tagged_split<TT>(g, n_items, n_groups, tag_lds, retries, gv, gn)
                                          : gather_tagged_full<TT>(g, n_items, tag_lds, retries, vs));
            fallback = __syncthreads_or(!got);
            have = !fallback;
            if (fallback && tid == 0)
                __hip_atomic_fetch_add(g.sync + kSyncFallbackWord, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- V^T x into vs: each entry is 0 + its group sums in order ----
    const bool sums = (parts || (have && !g.two_level)) && split;
    if (sums) {
        const float v = gather_finish(gv, gn);
        if (!own_entry)
            gsum[tid] = v;
        else if (tid < n_items)
            vs[vc][vt][vk] = 0.f + v;
    } else if (parts) {
        gather_full(g, n_items, vs);
    }
    if constexpr (INL)
        if (fallback) vtx_fallback<TT>(g, n_items, vs, vred, xstage, fgs);
    __syncthreads();
    if (sums && !own_entry) {
        for (int item = tid; item < n_items; item += kThreads) {
            float sum = 0.f;
            for (int j = 0; j < n_groups; ++j) sum += gsum[item * n_groups + j];
            int c, t, k;
            vtx_item(g, TT, item, c, t, k);
            vs[c][t][k] = sum;
        }
        __syncthreads();
    }

    // ---- outputs ----
    // One thread per (row, token): the row segments in order, scaled by s, plus
    // the rank term sum_k U[o,k] vtx[t,k] as four interleaved partial sums (k
    // mod 4) added pairwise; one RNE cast to bf16.
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
            float rt = 0.f;
            if (n_items > 0) {
                const int ci = P == 2 ? p : child_index(g, row);
                const int r = ch_r(g, ci);
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
                for (int k0 = 0; k0 < r; k0 += 4) {
                    // U past r is zero (masked at its load); vs past r was never written
                    const f32x4 u = *reinterpret_cast<const f32x4 *>(&ulds[jr][p][k0]);
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(&vs[ci][t][k0]);
                    a0 += u.x * v.x;
                    a1 += u.y * (k0 + 1 < r ? v.y : 0.f);
                    a2 += u.z * (k0 + 2 < r ? v.z : 0.f);
                    a3 += u.w * (k0 + 3 < r ? v.w : 0.f);
                }
                rt = (a0 + a1) + (a2 + a3);
            }
            val[p] = slds[jr][p] * m + rt;
        }
        const float out = P == 2 ? gelu_tanh_bf16out(val[0]) * val[P - 1] : val[0];
        g.y[(size_t)tok * g.ldy + row] = f_bf16(out);
    }
}

template <int TT, int R, int P>
hipError_t launch_tt(const GemvF &g, int n_wg, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_kernel<TT, R, P>), dim3(n_wg), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

template <int R, int P>
hipError_t launch_r(const GemvF &g, int tt, int n_wg, hipStream_t stream) {
    switch (tt) {
        case 8: return launch_tt<8, R, P>(g, n_wg, stream);
        case 4: return launch_tt<4, R, P>(g, n_wg, stream);
        case 2: return launch_tt<2, R, P>(g, n_wg, stream);
        default: return launch_tt<1, R, P>(g, n_wg, stream);
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

// V^T x at 1 to 4 tokens per pass comes from producer workgroups of the same
// launch (measured faster than every workgroup reading a small V itself, by
// about 1 µs, and than a separate launch), unless allow_inlaunch is false; then,
// and above 2 tokens, from a V^T x launch just before.
GemvPlan gemv_plan(const GemvF &g, int tt, bool allow_inlaunch) {
    GemvPlan p;
    const int nch = g.d_in / 8;
    p.nseg = nch <= 640 ? 1 : nch <= 1280 ? 2 : 4;
    p.R = (p.nseg == 1 && nch <= 256) ? 2 : 1;
    const int rows_g = (kWaves / p.nseg) * p.R;
    p.n_wg = (g.rows + rows_g - 1) / rows_g;
    p.slice_len = gemv_slice_len(g.d_in);
    int sum_r = 0, n_v = 0;
    for (int c = 0; c < g.n_ch; ++c) {
        sum_r += g.ch[c].r;
        n_v += g.ch[c].r > 0;
    }
    p.S = sum_r > 0 ? (g.d_in + p.slice_len - 1) / p.slice_len : 0;
    p.vmode = sum_r > 0 ? kVtxPartials : kVtxNone;
    if (sum_r == 0 || !allow_inlaunch || tt > kInLaunchMaxTok) return p;
    p.vmode = kVtxInLaunch;
    p.n_prod = p.S * n_v;
    // One level: every projection workgroup reads the words of every slice,
    // device-scope reads that miss L2 and all fall on the same few lines.
    // Measured on the Gemma-3-1B-shaped layer at ranks 4, 16 and 32, 1 and 2
    // tokens: one level is faster for Q/K/V and O (1,152 to 1,728 workgroup x
    // slice reads per launch), two levels for gate/up and down (7,776 and
    // 31,104), whatever the bytes read.
    p.two_level = (long long)p.n_wg * p.S > kOneLevelMaxReads;
    return p;
}

hipError_t launch_gemv(const GemvF &g, const GemvPlan &plan, int tt, hipStream_t stream) {
    GemvF a = g;
    a.nseg = plan.nseg;
    a.S = plan.S;
    a.vmode = plan.vmode;
    a.n_prod = plan.vmode == kVtxInLaunch ? plan.n_prod : 0;
    a.two_level = plan.two_level;
    a.slice_len = plan.slice_len;
    const int n_wg = plan.n_wg + a.n_prod;   // producers first
    if (g.pair) {
        if (plan.R == 2) return launch_r<2, 2>(a, tt, n_wg, stream);
        return launch_r<1, 2>(a, tt, n_wg, stream);
    }
    if (plan.R == 2) return launch_r<2, 1>(a, tt, n_wg, stream);
    return launch_r<1, 1>(a, tt, n_wg, stream);
}

}  // namespace wl
