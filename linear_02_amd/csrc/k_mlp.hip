// The MLP at decode sizes (one to four tokens per pass) in one launch
// ("In-kernel reconstruction", the custom-op path: the fused MLP op runs gate,
// up, the activation and down as one operation).
//
// The down projection's input h is the whole gate/up result, so a launch that
// splits down by output rows needs every workgroup to wait for every other's
// h. This kernel splits down along its input axis instead: the intermediate
// axis is cut into slices of W rows, and the workgroup of slice j
//   1. streams the W gate rows and W up rows of its slice (all d_model inputs)
//      and forms h[t][i] = bf16(gelu_tanh(gate) * up) for i in the slice, with
//      the gate/up rank terms from V^T x slices that producer workgroups of the
//      same launch hand over (wl_handoff.h);
//   2. forms the slice's share of down for every output o,
//        p_j[t][o] = s[o] * sum_{i in j} W0[o][i] h[t][i]
//                    + sum_k U[o][k] * sum_{i in j} V[i][k] h[t][i],
//      which is the per-element expansion of the reconstruction formula
//      ("In-kernel reconstruction", introduction) restricted to the slice's
//      inputs: the formula is linear in h, so the slices' shares add up to it;
//   3. stores p_j as 64-bit words tagged with the launch's generation, then, for
//      its groups of 8 outputs, reads every slice's words, adds them in slice
//      order and rounds once to bf16.
// Only the partial outputs cross workgroups (and V^T x of gate/up); h never
// leaves the workgroup that made it. Every wait is bounded: a workgroup whose
// wait runs out computes what it waited for with the same arithmetic, so the
// result does not depend on timing.
//
// Memory: the gate/up rows (2 W d_model bf16) are read by 16-lane row groups,
// 16 bytes per lane, every load of a batch issued before any is used; the
// slice's down columns (d_out rows x W inputs) follow into registers and stream
// while V^T x is gathered and h formed. The down U rows and s, the same for
// every slice, come from L2. Direct-to-LDS loads (the slice's small operands)
// only target the first 64 KiB of LDS: their LDS address is taken from a
// 16-bit field.
#include "wl_device.h"
#include "wl_kernels.h"
#include "wl_vtx_slice.h"
#include "wl_handoff.h"

namespace wl {

namespace {

constexpr int kThreads = kHThreads;
constexpr int kWaves = kThreads / kWave;
constexpr int kUB = 9;      // 16-byte loads per lane per gate/up row in one batch
constexpr int kPB = kMlpDownBytes / 16 / kThreads;   // down passes (kThreads pieces each) at most

// 16-byte load through the global address space, not kept in the caches
// (each W0 element is used once per launch).
__device__ __forceinline__ u32x4 ld_stream(const uint16_t *p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)p);
}

// Sum over the aligned groups of L lanes (L = 2, 4, 8 or 16, within a DPP row);
// every lane of a group ends with the group's sum, in the same bits.
template <int L>
__device__ __forceinline__ float group_sum_lanes(float v) {
    if constexpr (L >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (L >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (L >= 16) v += dpp<0x140>(v);  // row_mirror
    return v;
}

// One 16-byte piece per lane of a contiguous region of n16 pieces copied into
// LDS, the wave's 64 lanes side by side (the destination is padded to whole
// waves' worth of pieces; lanes past the end reload the last piece).
__device__ __forceinline__ void copy_to_lds(const uint16_t *src, int n16, u32x4 *dst) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
    for (int m = wave * kWave; m < n16; m += kThreads)
        lds_dma16(s + min(m + lane, n16 - 1), dst + m);
}

// Slice j's workgroup index mapping: slice workgroups on one XCD (workgroup b
// runs on XCD b % 8) take consecutive slices, so that slices sharing a
// 128-byte line of a down row are read through the same L2.
__device__ __forceinline__ int slice_of_block(int b, int n_prod, int NS) {
    const int x = b % 8;
    int base = 0, first = 0;
    for (int xx = 0; xx <= x; ++xx) {
        first = n_prod + ((xx - n_prod % 8) % 8 + 8) % 8;
        const int cnt = first < n_prod + NS ? (n_prod + NS - first + 7) / 8 : 0;
        if (xx < x) base += cnt;
    }
    return base + (b - first) / 8;
}

template <int TT, int W>
struct Lds {
    // direct-to-LDS targets first (within the first 64 KiB)
    u32x4 ug[W * kMaxRank / 8];                         // gate U rows of the slice, bf16 [W][r]
    u32x4 uu[W * kMaxRank / 8];                         // up U rows
    u32x4 vd[W * kMaxRank / 8];                         // down V rows of the slice, bf16 [W][rd]
    float vred[kThreads][TT + 1];                       // producer / fallback slice sums
    u32x4 xstage[TT > 2 ? TT * kXStageMax / 8 : 1];     // producer / fallback x slice
    float gsum[kThreads];
    float vs[kMaxChildren][TT][kMaxRank];               // gate / up V^T x
    float fgs[kMaxChildren * TT * kMaxRank];            // fallback group sums
    float ml[2][W][TT];                                 // gate / up W0 x
    float val[2][W][TT];                                // gate / up values
    float sl[2][W];                                     // gate / up s
    alignas(16) uint16_t h[TT][W];                      // bf16 h of the slice
    float vj[TT][kMaxRank];                             // sum over the slice of V_d[i][k] h[t][i]
    float red[32][kMlpGroup];                           // reduction of the partial outputs
    uint32_t tag;
    int miss, need;
};

// ---- step 1: gate/up of slice j into h ----

// W0 x of the slice's 2 W gate/up rows into ml. Wave q takes slice rows
// [q W/4, (q+1) W/4); a step covers 2 slice rows x {gate, up}, one per 16-lane
// row group; each lane takes the row's 16-byte pieces l16, l16 + 16, ... and
// the matching pieces of x (from L2). The loads of UB pieces x SB steps are
// issued before any is used. issued() runs once in every thread, right after
// the first batch's loads are issued (the first batch is peeled out of the
// loops, so that what issued() does stays straight-line code). The caller
// ends it with a barrier.
template <int TT, int W>
struct GateUp {
    static constexpr int STEPS = W / 8;
    static constexpr int SB = STEPS < 4 ? STEPS : 4;
    // A batch (SB x UB pieces of W0, UB x TT of x) keeps about 45 loads in
    // flight per lane.
    static constexpr int UB = 45 / (SB + TT) < kUB ? 45 / (SB + TT) : kUB;
    u32x4 wv[SB][UB], xv[UB][TT];
    float acc[SB][TT];
};

template <int TT, int W>
__device__ __forceinline__ void gu_issue(const MlpDec &a, int i0, int wj, int sb, int ub, GateUp<TT, W> &b) {
    using B = GateUp<TT, W>;
    const int lane = threadIdx.x & (kWave - 1), q = threadIdx.x / kWave;
    const int rho = lane >> 4, l16 = lane & 15;
    const int D = a.gu.d_in, nch = D >> 3;
    const int tn = min(TT, a.gu.T - a.gu.t0);
    const uint16_t *Wrow = (rho & 1) ? a.gu.ch[1].W0 : a.gu.ch[0].W0;
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(a.gu.x + (size_t)a.gu.t0 * D);
#pragma unroll
    for (int st = 0; st < B::SB; ++st) {
        const int i = q * (W / 4) + 2 * (sb + st) + (rho >> 1);
        const uint16_t *base = Wrow + (size_t)(i0 + min(i, wj - 1)) * D;
#pragma unroll
        for (int u = 0; u < B::UB; ++u) b.wv[st][u] = ld_stream(base + 8 * min(l16 + 16 * (ub + u), nch - 1));
    }
#pragma unroll
    for (int u = 0; u < B::UB; ++u) {
        const int ch = min(l16 + 16 * (ub + u), nch - 1);
#pragma unroll
        for (int t = 0; t < TT; ++t) b.xv[u][t] = ldg(xg + (size_t)min(t, tn - 1) * nch + ch);
    }
}

template <int TT, int W>
__device__ __forceinline__ void gu_compute(const MlpDec &a, int ub, GateUp<TT, W> &b) {
    using B = GateUp<TT, W>;
    const int l16 = threadIdx.x & 15, nch = a.gu.d_in >> 3;
    // Pieces past the row's end were loaded from its last piece; their x is
    // zeroed (a select, not a branch), so they add nothing.
#pragma unroll
    for (int u = 0; u < B::UB; ++u) {
        const bool in = l16 + 16 * (ub + u) < nch;
#pragma unroll
        for (int t = 0; t < TT; ++t) b.xv[u][t] = in ? b.xv[u][t] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < B::UB; ++u)
#pragma unroll
        for (int st = 0; st < B::SB; ++st)
#pragma unroll
            for (int t = 0; t < TT; ++t) b.acc[st][t] = dot8(b.wv[st][u], b.xv[u][t], b.acc[st][t]);
}

template <int TT, int W>
__device__ __forceinline__ void gu_finish(int sb, GateUp<TT, W> &b, Lds<TT, W> &s) {
    using B = GateUp<TT, W>;
    const int lane = threadIdx.x & (kWave - 1), q = threadIdx.x / kWave;
    const int rho = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int st = 0; st < B::SB; ++st) {
        const int i = q * (W / 4) + 2 * (sb + st) + (rho >> 1);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float v = group_sum_lanes<16>(b.acc[st][t]);
            if (l16 == 0) s.ml[rho & 1][i][t] = v;
        }
    }
}

template <int TT, int W, class Hook>
__device__ __forceinline__ void gateup_stream(const MlpDec &a, int i0, int wj, Lds<TT, W> &s, Hook issued) {
    using B = GateUp<TT, W>;
    const int nu = ((a.gu.d_in >> 3) + 15) >> 4;
    {
        B b;
        gu_issue<TT, W>(a, i0, wj, 0, 0, b);
        __builtin_amdgcn_sched_barrier(0);
        issued();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < B::SB; ++st)
#pragma unroll
            for (int t = 0; t < TT; ++t) b.acc[st][t] = 0.f;
        gu_compute<TT, W>(a, 0, b);
        for (int ub = B::UB; ub < nu; ub += B::UB) {
            gu_issue<TT, W>(a, i0, wj, 0, ub, b);
            gu_compute<TT, W>(a, ub, b);
        }
        gu_finish<TT, W>(0, b, s);
    }
    for (int sb = B::SB; sb < B::STEPS; sb += B::SB) {
        B b;
#pragma unroll
        for (int st = 0; st < B::SB; ++st)
#pragma unroll
            for (int t = 0; t < TT; ++t) b.acc[st][t] = 0.f;
        for (int ub = 0; ub < nu; ub += B::UB) {
            gu_issue<TT, W>(a, i0, wj, sb, ub, b);
            gu_compute<TT, W>(a, ub, b);
        }
        gu_finish<TT, W>(sb, b, s);
    }
}

// h of the slice from ml, the gate/up scales, U rows (LDS) and V^T x (vs):
// thread (p, i) forms gate or up of slice row i for every token, rank term
// summed over k in order; then thread (i, t) rounds h. Ends with a barrier.
template <int TT, int W>
__device__ __forceinline__ void form_h(const MlpDec &a, int wj, Lds<TT, W> &s) {
    const int tid = threadIdx.x;
    if (tid < 2 * W) {
        const int p = tid / W, i = tid % W;
        const int r = p ? a.gu.ch[1].r : a.gu.ch[0].r;
        const uint16_t *U = reinterpret_cast<const uint16_t *>(p ? s.uu : s.ug);
        float rt[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) rt[t] = 0.f;
        for (int k = 0; k < r; ++k) {
            const float uk = bf16_f(U[min(i, wj - 1) * r + k]);
#pragma unroll
            for (int t = 0; t < TT; ++t) rt[t] += uk * s.vs[p][t][k];
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) s.val[p][i][t] = s.sl[p][i] * s.ml[p][i][t] + rt[t];
    }
    __syncthreads();
    for (int idx = tid; idx < W * TT; idx += kThreads) {
        const int i = idx / TT, t = idx % TT;
        const float hv = i < wj ? gelu_tanh(s.val[0][i][t]) * s.val[1][i][t] : 0.f;
        s.h[t][i] = f_bf16(hv);
    }
    __syncthreads();
}

// vj[t][k] = sum over the slice's rows i (in order) of V_d[i][k] h[t][i].
template <int TT, int W>
__device__ __forceinline__ void form_vj(const MlpDec &a, int wj, Lds<TT, W> &s) {
    const int tid = threadIdx.x, rd = a.rd;
    const uint16_t *V = reinterpret_cast<const uint16_t *>(s.vd);
    for (int idx = tid; idx < TT * rd; idx += kThreads) {
        const int t = idx / rd, k = idx % rd;
        float acc = 0.f;
        for (int i = 0; i < wj; ++i) acc += bf16_f(V[i * rd + k]) * bf16_f(s.h[t][i]);
        s.vj[t][k] = acc;
    }
    __syncthreads();
}

// ---- step 2: the slice's share of down ----

// Lane (ro, c) of wave q takes down row o = pass * 4 RW + q * RW + ro of a
// pass and the slice's 16-byte piece c (inputs i0 + 8c .. i0 + 8c + 7).
template <int W>
struct DownLane {
    static constexpr int L = W / 8, RW = kWave / L;
    int c, ro, q;
    __device__ __forceinline__ DownLane() {
        const int lane = threadIdx.x & (kWave - 1);
        c = lane % L;
        ro = lane / L;
        q = threadIdx.x / kWave;
    }
    __device__ __forceinline__ int row(int pass) const { return pass * (kWaves * RW) + q * RW + ro; }
};

// The lane's piece of down row o from global memory (row and piece clamped).
template <int W>
__device__ __forceinline__ u32x4 load_down_piece(const MlpDec &a, int i0, int wj, int o) {
    const DownLane<W> dl;
    const int oc = min(o, a.D - 1), cc = min(dl.c, wj / 8 - 1);
    return ld_stream(a.W0d + (size_t)oc * a.F + i0 + 8 * cc);
}

// U_d[o][k] for the lane's rank entries: piece c of the row (entries 8c ..
// 8c + 7) when rd is a multiple of 8 (rd <= 8 L), else (rd <= L) entry c.
__device__ __forceinline__ u32x4 load_u_piece(const MlpDec &a, int c, int o) {
    const int rd = a.rd, oc = min(o, a.D - 1);
    const uint16_t *row = a.Ud + (size_t)oc * rd;
    if (rd % 8 == 0) return ldg(reinterpret_cast<const u32x4 *>(row) + min(c, rd / 8 - 1));
    return u32x4{ldg(row + min(c, rd - 1)), 0u, 0u, 0u};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_f(w & 0xFFFFu); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_f(w >> 16); }

// The lane's share of the rank term of token t (products added in k order).
template <int TT, int W>
__device__ __forceinline__ float lane_rank_term(const MlpDec &a, u32x4 u, const Lds<TT, W> &s, int t) {
    const DownLane<W> dl;
    const int rd = a.rd;
    float acc = 0.f;
    if (rd % 8 == 0) {
        if (8 * dl.c < rd) {
            const float *v = &s.vj[t][8 * dl.c];
            acc += bf16_lo(u.x) * v[0];
            acc += bf16_hi(u.x) * v[1];
            acc += bf16_lo(u.y) * v[2];
            acc += bf16_hi(u.y) * v[3];
            acc += bf16_lo(u.z) * v[4];
            acc += bf16_hi(u.z) * v[5];
            acc += bf16_lo(u.w) * v[6];
            acc += bf16_hi(u.w) * v[7];
        }
    } else if (dl.c < rd) {
        acc += bf16_lo(u.x) * s.vj[t][dl.c];
    }
    return acc;
}

// p_j[t][o] of one down row, on every lane of the row's L-lane group:
// s[o] * (W0 h over the slice) + (U over the rank entries).
template <int TT, int W>
__device__ __forceinline__ void down_row(const MlpDec &a, int wj, u32x4 wd, u32x4 u, float so, const Lds<TT, W> &s,
                                         float (&p)[TT]) {
    constexpr int L = W / 8;
    const DownLane<W> dl;
    const bool in = 8 * dl.c < wj;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const u32x4 hv = reinterpret_cast<const u32x4 *>(s.h[t])[dl.c];
        const float m = group_sum_lanes<L>(in ? dot8(wd, hv, 0.f) : 0.f);
        const float rt = a.rd > 0 ? group_sum_lanes<L>(lane_rank_term<TT, W>(a, u, s, t)) : 0.f;
        p[t] = so * m + rt;
    }
}

__device__ __forceinline__ unsigned long long *part_word(const MlpDec &a, int q, int j, int t, int tt, int oo) {
    return a.part + (((size_t)q * a.NS + j) * tt + t) * kMlpGroup + oo;
}

// The lane's down rows (every pass): W0 pieces of the slice, U pieces, s.
struct DownRows {
    u32x4 wd[kPB];
    u32x4 u[kPB];
    float so[kPB];
};
template <int W>
__device__ __forceinline__ void load_down_w0(const MlpDec &a, int i0, int wj, DownRows &b) {
    const DownLane<W> dl;
#pragma unroll
    for (int m = 0; m < kPB; ++m) b.wd[m] = load_down_piece<W>(a, i0, wj, dl.row(m));
}
template <int W>
__device__ __forceinline__ void load_down_us(const MlpDec &a, DownRows &b) {
    const DownLane<W> dl;
#pragma unroll
    for (int m = 0; m < kPB; ++m) {
        const int o = min(dl.row(m), a.D - 1);
        b.u[m] = a.rd > 0 ? load_u_piece(a, dl.c, o) : u32x4{0u, 0u, 0u, 0u};
        b.so[m] = a.sd ? ldg(a.sd + o) : 1.f;
    }
}

// Every down row of slice j as tagged words.
template <int TT, int W>
__device__ __forceinline__ void down_all_rows(const MlpDec &a, int j, int wj, const DownRows &b, const Lds<TT, W> &s,
                                              unsigned long long tag) {
    const DownLane<W> dl;
    const int tn = min(TT, a.gu.T - a.gu.t0);
#pragma unroll
    for (int m = 0; m < kPB; ++m) {
        const int o = dl.row(m);
        if (o - dl.ro >= a.D) break;   // wave-uniform: no row of this pass exists
        float p[TT];
        down_row<TT, W>(a, wj, b.wd[m], b.u[m], b.so[m], s, p);
        if (dl.c == 0 && o < a.D) {
            const int q = o / kMlpGroup, oo = o % kMlpGroup;
            for (int t = 0; t < tn; ++t)
                __hip_atomic_store(part_word(a, q, j, t, TT, oo), tag | __float_as_uint(p[t]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// p_j for the rows of output group q only (a reducer computing a slice whose
// words did not come): wave 0, rows 8q .. 8q + 7, the same per-row arithmetic.
template <int TT, int W>
__device__ __forceinline__ void down_group_rows(const MlpDec &a, int j, int q, int i0, int wj, const Lds<TT, W> &s,
                                                unsigned long long tag) {
    constexpr int RW = kWave / (W / 8);
    const DownLane<W> dl;
    const int tn = min(TT, a.gu.T - a.gu.t0);
    if (dl.q != 0) return;
    for (int r0 = 0; r0 < kMlpGroup; r0 += RW) {
        const int o = q * kMlpGroup + r0 + dl.ro;
        const bool mine = r0 + dl.ro < kMlpGroup;
        const u32x4 wd = load_down_piece<W>(a, i0, wj, o);
        const u32x4 u = a.rd > 0 ? load_u_piece(a, dl.c, o) : u32x4{0u, 0u, 0u, 0u};
        const float so = a.sd ? ldg(a.sd + min(o, a.D - 1)) : 1.f;
        float p[TT];
        down_row<TT, W>(a, wj, wd, u, so, s, p);
        if (dl.c == 0 && mine && o < a.D)
            for (int t = 0; t < tn; ++t)
                __hip_atomic_store(part_word(a, q, j, t, TT, o % kMlpGroup), tag | __float_as_uint(p[t]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Slice j's small operands: gate/up U rows and down V rows into LDS by
// direct-to-LDS copies (the caller waits, wait_vm<0> and a barrier, before
// using them); the thread's gate/up s value (threads below 2 W) is returned,
// to be written to LDS with put_scale once it has arrived.
template <int TT, int W>
__device__ __forceinline__ float stage_slice(const MlpDec &a, int i0, int wj, Lds<TT, W> &s) {
    const int rg = a.gu.ch[0].r, ru = a.gu.ch[1].r, rd = a.rd;
    if (rg > 0) copy_to_lds(a.gu.ch[0].U + (size_t)i0 * rg, wj * rg / 8, s.ug);
    if (ru > 0) copy_to_lds(a.gu.ch[1].U + (size_t)i0 * ru, wj * ru / 8, s.uu);
    if (rd > 0) copy_to_lds(a.Vd + (size_t)i0 * rd, wj * rd / 8, s.vd);
    const int tid = threadIdx.x, p = (tid / W) & 1, i = tid % W;
    const float *sp = p ? a.gu.ch[1].s : a.gu.ch[0].s;
    const float *sg = sp ? sp + i0 + min(i, wj - 1) : reinterpret_cast<const float *>(a.gu.x);
    const float v = ldg(sg);
    return sp ? v : 1.f;
}
template <int TT, int W>
__device__ __forceinline__ void put_scale(float v, Lds<TT, W> &s) {
    const int tid = threadIdx.x;
    if (tid < 2 * W) s.sl[tid / W][tid % W] = v;
}

// Gate/up V^T x of the pass from this launch's producers (or computed here
// when the wait runs out), into s.vs: one thread per (child, token, k) item
// reads that item's tagged slice words, groups of 16 slices in order. (The
// split mapping of the decode GEMV, thread per (item, group), computed wrong
// sums at four tokens per pass when compiled into this kernel, with other
// loads' registers live across it; it is not used here.) Ends with a barrier.
template <int TT, int W>
__device__ __forceinline__ void gather_gateup_vtx(const MlpDec &a, Lds<TT, W> &s) {
    const GemvF &g = a.gu;
    const int tid = threadIdx.x;
    const int n_items = vtx_items(g, TT);
    if (n_items == 0) return;
    const int retries = g.spin_limit - 1;
    const bool got = g.spin_limit > 0 && gather_tagged_full<TT>(g, n_items, s.tag, retries, s.vs);
    const bool fallback = __syncthreads_or(!got);
    if (fallback) {
        if (tid == 0)
            __hip_atomic_fetch_add(g.sync + kSyncFallbackWord, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        vtx_fallback<TT>(g, n_items, s.vs, s.vred, s.xstage, s.fgs);
    }
    __syncthreads();
}

// ---- step 3: the sums over slices ----

// Thread (js, oo) reads slices js, js + 32, ... of output 8q + oo, token t, and
// adds them in order. A word without this launch's tag is read again, at most
// `retries` more times; outputs past d_out count as present. False when a wait
// ran out.
template <int TT, int W>
__device__ __forceinline__ bool reduce_poll(const MlpDec &a, int q, int t, uint32_t tag, int retries, float &sum) {
    const int tid = threadIdx.x, oo = tid % kMlpGroup, js = tid / kMlpGroup;
    const bool real = q * kMlpGroup + oo < a.D;
    constexpr int M = kMlpMaxSlices / 32;
    unsigned long long w[M];
    bool ok = false;
    for (int spin = 0;; ++spin) {
        bool ready = true;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int jj = min(js + 32 * m, a.NS - 1);
            w[m] = ld_word(part_word(a, q, jj, t, TT, oo));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) ready = ready && (!real || js + 32 * m >= a.NS || word_is(w[m], tag));
        if (ready) {
            ok = true;
            break;
        }
        if (spin >= retries) break;
    }
    sum = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m)
        if (js + 32 * m < a.NS) sum += word_value(w[m]);
    return ok;
}

template <int TT, int W>
__global__ __launch_bounds__(kThreads) void mlp_dec_kernel(MlpDec a) {
    __shared__ Lds<TT, W> s;
    const GemvF &g = a.gu;
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < g.n_prod) {
        vtx_produce<TT>(g, s.vred, s.xstage, &s.tag, s.gsum, s.vs);
        return;
    }
    const int j = slice_of_block(blockIdx.x, g.n_prod, a.NS);
    const int i0 = j * W, wj = min(W, a.F - i0);
    const int tn = min(TT, g.T - g.t0);

    // Issue order: the first gate/up batch (and its x), the ticket, the slice's
    // down columns into LDS; they stream while gate/up is reduced.
    // Issue order per wave: the first gate/up batch (and its x), the ticket
    // (thread 0); once the wave's gate/up loads are used, the slice's down
    // columns (into the registers the gate/up batch held), the small operands
    // and the down U / s, all in flight while V^T x is gathered.
    unsigned long long ticket;   // thread 0 only; left undefined elsewhere, so that no copy
                                 // of the atomic's result (and no wait for it) is needed here
    gateup_stream<TT, W>(a, i0, wj, s, [&]() {
        if (tid == 0) ticket = take_ticket(g);
        if (blockIdx.x == 0) advance_empty_copies(g);
    });
    DownRows dr;
    load_down_w0<W>(a, i0, wj, dr);
    __syncthreads();
    if (tid == 0) s.tag = ticket_tag(ticket);
    const float sv = stage_slice<TT, W>(a, i0, wj, s);
    load_down_us<W>(a, dr);
    __syncthreads();
    gather_gateup_vtx<TT, W>(a, s);
    wait_vm<0>();
    put_scale<TT, W>(sv, s);
    __syncthreads();
    form_h<TT, W>(a, wj, s);
    if (a.rd > 0) form_vj<TT, W>(a, wj, s);
    const uint32_t tag32 = s.tag;
    const unsigned long long tag = (unsigned long long)tag32 << 32;
    down_all_rows<TT, W>(a, j, wj, dr, s, tag);

    // ---- sums over slices for this workgroup's output groups ----
    const int retries = g.spin_limit - 1;
    const int oo = tid % kMlpGroup, js = tid / kMlpGroup;
    for (int q = j; q < a.NG; q += a.NS) {
        for (int t = 0; t < tn; ++t) {
            float sum = 0.f;
            const bool ok = g.spin_limit > 0 && reduce_poll<TT, W>(a, q, t, tag32, retries, sum);
            if (tid == 0) s.miss = 0;
            __syncthreads();
            if (!ok) atomicOr(&s.miss, 1);
            __syncthreads();
            if (s.miss) {
                // Compute the words of this group that are not there (every
                // slice's when the wait is switched off), one slice at a time
                // with the slice workgroups' arithmetic, then read them back.
                for (int jj = 0; jj < a.NS; ++jj) {
                    if (tid == 0) s.need = g.spin_limit == 0;
                    __syncthreads();
                    if (js == jj % 32 && q * kMlpGroup + oo < a.D &&
                        !word_is(ld_word(part_word(a, q, jj, t, TT, oo)), tag32))
                        atomicOr(&s.need, 1);
                    __syncthreads();
                    const bool need = s.need;
                    __syncthreads();   // every thread has read s.need before thread 0 resets it
                    if (!need) continue;
                    const int j0 = jj * W, wjj = min(W, a.F - j0);
                    const float svj = stage_slice<TT, W>(a, j0, wjj, s);
                    wait_vm<0>();
                    put_scale<TT, W>(svj, s);
                    __syncthreads();
                    gateup_stream<TT, W>(a, j0, wjj, s, []() {});
                    __syncthreads();
                    form_h<TT, W>(a, wjj, s);
                    if (a.rd > 0) form_vj<TT, W>(a, wjj, s);
                    down_group_rows<TT, W>(a, jj, q, j0, wjj, s, tag);
                    __syncthreads();
                }
                reduce_poll<TT, W>(a, q, t, tag32, kSpinLimit, sum);
            }
            s.red[js][oo] = sum;
            __syncthreads();
            if (tid < kMlpGroup) {
                const int o = q * kMlpGroup + tid;
                float y = 0.f;
                for (int jj = 0; jj < 32; ++jj) y += s.red[jj][tid];
                if (o < a.D) a.y[(size_t)(g.t0 + t) * a.D + o] = f_bf16(y);
            }
            __syncthreads();
        }
    }
    if (blockIdx.x == 0 && tid == 0) sweep_tagged(g.sync, ticket, tag32);
}

template <int TT>
hipError_t launch_w(const MlpDec &a, int W, int grid, hipStream_t stream) {
    switch (W) {
        case 32: hipLaunchKernelGGL((mlp_dec_kernel<TT, 32>), dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 64: hipLaunchKernelGGL((mlp_dec_kernel<TT, 64>), dim3(grid), dim3(kThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL((mlp_dec_kernel<TT, 128>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace

// Slice width W: the smallest of 32, 64, 128 that keeps the slices within
// kMlpMaxSlices, holds the down rank in one 16-byte piece per lane (rd a
// multiple of 8 up to W, or rd up to W / 8) and keeps the slice's down columns
// within the LDS block.
MlpPlan mlp_dec_plan(int d_model, int F, int d_out, int r_gate, int r_up, int r_down, int T) {
    MlpPlan p;
    const int tt = gemv_tokens_per_pass(d_model, T);
    if (tt == 0 || tt > kInLaunchMaxTok) return p;
    int W = 0;
    for (int w = 32; w <= 128 && W == 0; w *= 2) {
        const bool rank_ok = r_down % 8 == 0 ? r_down <= w : r_down <= w / 8;
        if ((F + w - 1) / w <= kMlpMaxSlices && rank_ok && (size_t)d_out * (w / 8) * 16 <= (size_t)kMlpDownBytes)
            W = w;
    }
    if (W == 0) return p;
    const int NS = (F + W - 1) / W;
    const int NG = (d_out + kMlpGroup - 1) / kMlpGroup;
    if ((size_t)NG * NS * tt * kMlpGroup > kSyncPartWords) return p;
    p.tt = tt;
    p.W = W;
    p.NS = NS;
    p.NG = NG;
    p.slice_len = gemv_slice_len(d_model);
    const int n_v = (r_gate > 0) + (r_up > 0);
    p.S = n_v > 0 ? (d_model + p.slice_len - 1) / p.slice_len : 0;
    p.n_prod = p.S * n_v;
    return p;
}

hipError_t launch_mlp_dec(const MlpDec &a, const MlpPlan &p, hipStream_t stream) {
    MlpDec b = a;
    b.gu.S = p.S;
    b.gu.slice_len = p.slice_len;
    b.gu.n_prod = p.n_prod;
    b.gu.vmode = p.n_prod > 0 ? kVtxInLaunch : kVtxNone;
    b.gu.two_level = 0;
    b.NS = p.NS;
    b.NG = p.NG;
    const int grid = p.n_prod + p.NS;
    switch (p.tt) {
        case 4: return launch_w<4>(b, p.W, grid, stream);
        case 2: return launch_w<2>(b, p.W, grid, stream);
        default: return launch_w<1>(b, p.W, grid, stream);
    }
}

}  // namespace wl
