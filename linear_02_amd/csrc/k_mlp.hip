// The MLP at decode sizes (one to four tokens per pass) in one launch
// ("In-kernel reconstruction", the custom-op path: the fused MLP op runs gate,
// up, the activation and down as one operation).
//
// The down projection's input h is the whole gate/up result, so a launch that
// splits down by output rows needs every workgroup to wait for every other's
// h. This kernel splits down along its input axis instead. The intermediate
// axis is cut into slices of 64 rows; the P workgroups of slice j each
//   1. stream their 64 / P gate rows and up rows (all d_model inputs) and form
//      h[t][i] = bf16(gelu_tanh(gate) * up) for those rows, the gate/up rank
//      terms from V^T x slices that producer workgroups of the same launch hand
//      over (wl_handoff.h); the slice's workgroups then exchange their h rows
//      as tagged words, so each holds the slice's whole h;
//   2. form the slice's share of down for their d_out / P output rows o,
//        p_j[t][o] = s[o] * sum_{i in j} W0[o][i] h[t][i]
//                    + sum_k U[o][k] * sum_{i in j} V[i][k] h[t][i],
//      the per-element expansion of the reconstruction formula ("In-kernel
//      reconstruction", introduction) restricted to the slice's inputs: the
//      formula is linear in h, so the slices' shares add up to it;
//   3. store p_j as 64-bit words tagged with the launch's generation, then, for
//      their groups of 8 outputs, read every slice's words, add them in slice
//      order and round once to bf16.
// Every wait is bounded: a workgroup whose wait runs out computes what it
// waited for with the same arithmetic, so the result does not depend on
// timing.
//
// Memory (measured: reading 64-byte pieces of each down row streams at less
// than half the rate of whole 128-byte lines, hence slices of 64 inputs shared
// by P workgroups): the gate/up rows are read by 16-lane row groups, 16 bytes
// per lane, in batches of row steps whose loads are all issued before any is
// used (at one token per pass one batch holds the part's rows); the
// workgroup's down rows (128-byte pieces, 8 lanes per row) go into registers,
// right behind the first batch at two or four tokens, once the gate/up rows
// are in at one token (the faster order for each, measured). The down U rows
// and s, the same for every slice, come from L2. Direct-to-LDS loads are kept
// to the slice's small operands. The down rows of a part are computed as one
// branch-free block (every pass, then the stores), so that their independent
// chains interleave.
#include "wl_device.h"
#include "wl_kernels.h"
#include "wl_vtx_slice.h"
#include "wl_handoff.h"

namespace wl {

namespace {

constexpr int kThreads = kHThreads;
constexpr int kWaves = kThreads / kWave;
constexpr int kW = kMlpSlice;             // slice rows = down inputs per slice
constexpr int kL = kW / 8;                // lanes per down row (one 16-byte piece each)
constexpr int kRW = kWave / kL;           // down rows per wave per pass
constexpr int kPB = kMlpDownPasses;       // down passes per workgroup (kWaves x kRW rows each)
constexpr int kUB = 9;                    // 16-byte pieces per lane per gate/up row in one batch
template <int TT>
constexpr int kSB = TT == 1 ? 4 : 2;      // gate/up row steps (4 rows each) per batch
constexpr int kEarlyWords = 16;           // tagged V^T x words per thread read ahead
constexpr int kRedPitch = 36;             // row of the slice-sum reduction in LDS (32 lanes, padded: no bank conflicts, 16-byte rows)

// 16-byte load through the global address space, not kept in the caches
// (each W0 element is used once per launch).
__device__ __forceinline__ u32x4 ld_stream(const uint16_t *p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)p);
}

// A read of LDS through an explicit LDS pointer: a pointer into the LDS struct
// that passes through a select or a cast is otherwise read with flat
// instructions, which also wait on the global-memory counter.
template <class T>
__device__ __forceinline__ T lds_ld(const T *p) {
    return *(const __attribute__((address_space(3))) T *)p;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_f(w & 0xFFFFu); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_f(w >> 16); }

// Sum over aligned groups of L lanes (L = 2, 4, 8 or 16, within a DPP row);
// every lane of a group ends with the group's sum, in the same bits.
template <int L>
__device__ __forceinline__ float group_sum_lanes(float v) {
    if constexpr (L >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (L >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (L >= 16) v += dpp<0x140>(v);  // row_mirror
    return v;
}

// A contiguous region of n16 16-byte pieces copied into LDS by direct-to-LDS
// loads, the wave's 64 lanes side by side (the destination is padded to whole
// waves' worth of pieces; lanes past the end reload the last piece).
__device__ __forceinline__ void copy_to_lds(const uint16_t *src, int n16, u32x4 *dst) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
    for (int m = wave * kWave; m < n16; m += kThreads) lds_dma16(s + min(m + lane, n16 - 1), dst + m);
}

template <int TT>
struct Lds {
    // direct-to-LDS targets, each padded by one wave's worth of pieces (a copy
    // writes whole waves' worth)
    u32x4 ug[kW * kMaxRank / 8 + kWave];                // gate U rows of the slice, bf16 [64][r] (slice-local rows)
    u32x4 uu[kW * kMaxRank / 8 + kWave];                // up U rows
    u32x4 vd[kW * kMaxRank / 8 + kWave];                // down V rows of the slice, bf16 [64][rd]
    float vred[kThreads][TT + 1];                       // producer / fallback slice sums
    u32x4 xstage[TT > 2 ? TT * kXStageMax / 8 : 1];     // producer / fallback x slice
    float gsum[kThreads];
    alignas(16) float vs[kMaxChildren][TT][kMaxRank];   // gate / up V^T x
    float fgs[kMaxChildren * TT * kMaxRank];            // fallback group sums
    float ml[2][kW][TT];                                // gate / up W0 x (slice-local rows)
    float val[2][kW][TT];                               // gate / up values
    float sl[2][kW];                                    // gate / up s
    alignas(16) uint16_t h[TT][kW];                     // bf16 h of the slice
    float vj[TT][kMaxRank];                             // sum over the slice of V_d[i][k] h[t][i]
    float vjp[kThreads];                                // its row-group sums
    alignas(16) float red[kMlpGroup][kRedPitch];        // reduction of the partial outputs, [output][slice lane]
    uint32_t tag;
    int miss, need;
};

// A part of slice j: slice-local rows [r0, r0 + n) of the intermediate axis
// (rows i0 + r0 ..); n is the part's rows that exist (the last slice may be
// short, and a part of it empty).
struct Part {
    int j, p, i0, wj, r0, n;   // slice, part, first row of the slice, rows of the slice, part's first row, its rows
};
__device__ __forceinline__ Part make_part(const MlpDec &a, int j, int p) {
    Part q;
    q.j = j;
    q.p = p;
    q.i0 = j * kW;
    q.wj = min(kW, a.F - q.i0);
    q.r0 = p * a.WR;
    q.n = max(0, min(a.WR, q.wj - q.r0));
    return q;
}

// ---- step 1: gate/up rows of a part ----

// Wave q takes slice-local rows r0 + q WR/4 .. + WR/4 of gate and of up; a
// step covers 2 rows x {gate, up}, one per 16-lane row group; each lane takes
// the row's 16-byte pieces l16, l16 + 16, ... and the matching pieces of x
// (from L2).
template <int TT>
struct GateUp {
    u32x4 wv[kSB<TT>][kUB], xv[kUB][TT];
    float acc[kSB<TT>][TT];
};

template <int TT>
__device__ __forceinline__ void gu_issue(const MlpDec &a, const Part &pt, int sb, int ub, GateUp<TT> &b) {
    const int lane = threadIdx.x & (kWave - 1), q = threadIdx.x / kWave;
    const int rho = lane >> 4, l16 = lane & 15;
    const int D = a.gu.d_in, nch = D >> 3;
    const int tn = min(TT, a.gu.T - a.gu.t0);
    const uint16_t *Wrow = (rho & 1) ? a.gu.ch[1].W0 : a.gu.ch[0].W0;
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(a.gu.x + (size_t)a.gu.t0 * D);
    const int nr = max(pt.n, 1);
#pragma unroll
    for (int st = 0; st < kSB<TT>; ++st) {
        const int i = q * (a.WR / 4) + 2 * (sb + st) + (rho >> 1);
        const uint16_t *base = Wrow + (size_t)(pt.i0 + pt.r0 + min(i, nr - 1)) * D;
#pragma unroll
        for (int u = 0; u < kUB; ++u) b.wv[st][u] = ld_stream(base + 8 * min(l16 + 16 * (ub + u), nch - 1));
    }
#pragma unroll
    for (int u = 0; u < kUB; ++u) {
        const int ch = min(l16 + 16 * (ub + u), nch - 1);
#pragma unroll
        for (int t = 0; t < TT; ++t) b.xv[u][t] = ldg(xg + (size_t)min(t, tn - 1) * nch + ch);
    }
}

template <int TT>
__device__ __forceinline__ void gu_compute(const MlpDec &a, int ub, GateUp<TT> &b) {
    const int l16 = threadIdx.x & 15, nch = a.gu.d_in >> 3;
    // Pieces past the row's end were loaded from its last piece; their x is
    // zeroed (a select, not a branch), so they add nothing.
#pragma unroll
    for (int u = 0; u < kUB; ++u) {
        const bool in = l16 + 16 * (ub + u) < nch;
#pragma unroll
        for (int t = 0; t < TT; ++t) b.xv[u][t] = in ? b.xv[u][t] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUB; ++u)
#pragma unroll
        for (int st = 0; st < kSB<TT>; ++st)
#pragma unroll
            for (int t = 0; t < TT; ++t) b.acc[st][t] = dot8(b.wv[st][u], b.xv[u][t], b.acc[st][t]);
}

template <int TT>
__device__ __forceinline__ void gu_finish(const MlpDec &a, const Part &pt, int sb, GateUp<TT> &b, Lds<TT> &s) {
    const int lane = threadIdx.x & (kWave - 1), q = threadIdx.x / kWave;
    const int rho = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int st = 0; st < kSB<TT>; ++st) {
        const int i = q * (a.WR / 4) + 2 * (sb + st) + (rho >> 1);
        const bool real = sb + st < a.WR / 8 && i < pt.n;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float v = group_sum_lanes<16>(b.acc[st][t]);
            if (l16 == 0 && real) s.ml[rho & 1][pt.r0 + i][t] = v;
        }
    }
}

template <int TT>
__device__ __forceinline__ void gu_zero(GateUp<TT> &b) {
#pragma unroll
    for (int st = 0; st < kSB<TT>; ++st)
#pragma unroll
        for (int t = 0; t < TT; ++t) b.acc[st][t] = 0.f;
}

// W0 x of a part's gate/up rows into ml, in batches of kSB<TT> row steps.
// first_issued() runs in every thread right after the first batch's loads are
// issued, last_issued() right after the last batch's (both after the one batch
// when there is only one). The first and last batches are peeled out of the
// loop, so the hooks are straight-line code and the waits of each batch count
// exactly the loads issued after it. The caller ends it with a barrier.
// ONE: the part has a single batch (4 or 8 workgroups per slice), fixed at
// compile time so that each kernel has one code path (two paths would be merged
// with register copies that wait for the last hook's loads).
template <int TT, bool ONE, class Hook1, class HookLast>
__device__ __forceinline__ void gateup_rows(const MlpDec &a, const Part &pt, Lds<TT> &s, Hook1 first_issued,
                                            HookLast last_issued) {
    const int nu = ((a.gu.d_in >> 3) + 15) >> 4;
    const int steps = a.WR / 8;
    const int nb = ONE ? 1 : (steps + kSB<TT> - 1) / kSB<TT>;
    auto batch = [&](int sb, auto &&hook) {
        GateUp<TT> b;
        gu_zero<TT>(b);
        gu_issue<TT>(a, pt, sb, 0, b);
        __builtin_amdgcn_sched_barrier(0);
        hook();
        __builtin_amdgcn_sched_barrier(0);
        gu_compute<TT>(a, 0, b);
        for (int ub = kUB; ub < nu; ub += kUB) {
            gu_issue<TT>(a, pt, sb, ub, b);
            gu_compute<TT>(a, ub, b);
        }
        gu_finish<TT>(a, pt, sb, b, s);
    };
    if constexpr (ONE) {
        batch(0, [&]() {
            first_issued();
            last_issued();
        });
        return;
    }
    batch(0, first_issued);
    for (int sb = kSB<TT>; sb < (nb - 1) * kSB<TT>; sb += kSB<TT>) batch(sb, []() {});
    batch((nb - 1) * kSB<TT>, last_issued);
}

// The part's gate/up U rows into LDS (direct-to-LDS), and the thread's gate/up
// s value (threads below 2 x 64: gate or up of slice-local row tid % 64),
// returned to be written with put_scale once it has arrived. The caller waits
// (wait_vm<0>, barrier) before using the U rows.
template <int TT>
__device__ __forceinline__ float stage_part(const MlpDec &a, const Part &pt, Lds<TT> &s) {
    const int rg = a.gu.ch[0].r, ru = a.gu.ch[1].r;
    if (pt.n > 0) {
        if (rg > 0) copy_to_lds(a.gu.ch[0].U + (size_t)(pt.i0 + pt.r0) * rg, pt.n * rg / 8, s.ug + pt.r0 * rg / 8);
        if (ru > 0) copy_to_lds(a.gu.ch[1].U + (size_t)(pt.i0 + pt.r0) * ru, pt.n * ru / 8, s.uu + pt.r0 * ru / 8);
    }
    const int tid = threadIdx.x, p = (tid / kW) & 1, i = tid % kW;
    const float *sp = p ? a.gu.ch[1].s : a.gu.ch[0].s;
    const float *sg = sp ? sp + pt.i0 + min(i, pt.wj - 1) : reinterpret_cast<const float *>(a.gu.x);
    const float v = ldg(sg);
    return sp ? v : 1.f;
}
template <int TT>
__device__ __forceinline__ void put_scale(float v, Lds<TT> &s) {
    const int tid = threadIdx.x;
    if (tid < 2 * kW) s.sl[tid / kW][tid % kW] = v;
}
// The slice's down V rows into LDS (direct-to-LDS).
template <int TT>
__device__ __forceinline__ void stage_vd(const MlpDec &a, const Part &pt, Lds<TT> &s) {
    if (a.rd > 0) copy_to_lds(a.Vd + (size_t)pt.i0 * a.rd, pt.wj * a.rd / 8, s.vd);
}

// h of a part's rows from ml, s, U rows (LDS) and V^T x (vs): thread (p, i)
// forms gate or up of a row for every token, rank term summed over k in order;
// then thread (i, t) rounds h. Ends with a barrier.
template <int TT>
__device__ __forceinline__ void form_h(const MlpDec &a, const Part &pt, Lds<TT> &s) {
    const int tid = threadIdx.x;
    if (tid < 2 * kW) {
        const int p = tid / kW, i = tid % kW;
        if (i >= pt.r0 && i < pt.r0 + pt.n) {
            const int r = p ? a.gu.ch[1].r : a.gu.ch[0].r;
            const uint16_t *U = reinterpret_cast<const uint16_t *>(p ? s.uu : s.ug);
            float rt[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) rt[t] = 0.f;
            if (r % 8 == 0) {
                // 16-byte reads of the U row and of V^T x, products still added in k order
                const u32x4 *Ur = reinterpret_cast<const u32x4 *>(U + i * r);
                for (int k8 = 0; k8 < r / 8; ++k8) {
                    const u32x4 u = lds_ld(Ur + k8);
                    const float uk[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const f32x4 v0 = lds_ld(reinterpret_cast<const f32x4 *>(&s.vs[p][t][8 * k8]));
                        const f32x4 v1 = lds_ld(reinterpret_cast<const f32x4 *>(&s.vs[p][t][8 * k8 + 4]));
                        rt[t] += uk[0] * v0.x;
                        rt[t] += uk[1] * v0.y;
                        rt[t] += uk[2] * v0.z;
                        rt[t] += uk[3] * v0.w;
                        rt[t] += uk[4] * v1.x;
                        rt[t] += uk[5] * v1.y;
                        rt[t] += uk[6] * v1.z;
                        rt[t] += uk[7] * v1.w;
                    }
                }
            } else {
                for (int k = 0; k < r; ++k) {
                    const float uk = bf16_f(lds_ld(U + i * r + k));
#pragma unroll
                    for (int t = 0; t < TT; ++t) rt[t] += uk * s.vs[p][t][k];
                }
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) s.val[p][i][t] = s.sl[p][i] * s.ml[p][i][t] + rt[t];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kW * TT; idx += kThreads) {
        const int i = idx / TT, t = idx % TT;
        if (i >= pt.r0 && i < pt.r0 + pt.n) s.h[t][i] = f_bf16(gelu_tanh_bf16out(s.val[0][i][t]) * s.val[1][i][t]);
    }
    __syncthreads();
}

// ---- the exchange of h between the slice's workgroups ----

// Word (j, i / 2, t): the tag beside the bf16 pair h[t][i], h[t][i + 1].
__device__ __forceinline__ unsigned long long *hx_word(const MlpDec &a, int j, int i2, int t, int tt) {
    return a.hx + ((size_t)j * (kW / 2) + i2) * tt + t;
}
template <int TT>
__device__ __forceinline__ void publish_h(const MlpDec &a, const Part &pt, const Lds<TT> &s, unsigned long long tag) {
    const int tn = min(TT, a.gu.T - a.gu.t0);
    for (int idx = threadIdx.x; idx < (pt.n / 2) * tn; idx += kThreads) {
        const int i2 = pt.r0 / 2 + idx / tn, t = idx % tn;
        const uint32_t v = (uint32_t)s.h[t][2 * i2] | ((uint32_t)s.h[t][2 * i2 + 1] << 16);
        __hip_atomic_store(hx_word(a, pt.j, i2, t, TT), tag | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
// The other parts' h rows of the slice from their words: thread per word,
// read again while it lacks the tag, at most `retries` more times. False when
// some wait ran out (the h rows stay incomplete).
template <int TT>
__device__ __forceinline__ bool fetch_h(const MlpDec &a, const Part &pt, Lds<TT> &s, uint32_t tag, int retries) {
    const int tn = min(TT, a.gu.T - a.gu.t0);
    bool ok = true;
    for (int idx = threadIdx.x; idx < (pt.wj / 2) * tn; idx += kThreads) {
        const int i2 = idx / tn, t = idx % tn;
        if (2 * i2 >= pt.r0 && 2 * i2 < pt.r0 + pt.n) continue;   // this part's own rows
        unsigned long long w = 0;
        bool got = false;
        for (int spin = 0; spin <= retries; ++spin) {
            w = ld_word(hx_word(a, pt.j, i2, t, TT));
            if (word_is(w, tag)) {
                got = true;
                break;
            }
        }
        if (got) {
            s.h[t][2 * i2] = (uint16_t)(w & 0xFFFFu);
            s.h[t][2 * i2 + 1] = (uint16_t)((w >> 16) & 0xFFFFu);
        }
        ok = ok && got;
    }
    return ok;
}

// vj[t][k] = sum over the slice's rows i of V_d[i][k] h[t][i]. Thread (g, t, k)
// adds the products of row group g (64 / G consecutive rows, in row order;
// rows past the slice's end add +0), then thread (t, k) adds the G group sums
// in group order. Ends with a barrier.
template <int TT>
__device__ __forceinline__ void form_vj(const MlpDec &a, const Part &pt, Lds<TT> &s) {
    const int rd = a.rd, n = TT * rd, tid = threadIdx.x;
    const int G = n <= kThreads / 8 ? 8 : n <= kThreads / 4 ? 4 : n <= kThreads / 2 ? 2 : 1;
    const int R = kW / G;
    const uint16_t *V = reinterpret_cast<const uint16_t *>(s.vd);
    if (tid < G * n) {
        const int g = tid / n, item = tid % n, t = item / rd, k = item % rd;
        float acc = 0.f;
        // R is a multiple of 8: eight rows' reads, then their products added
        // in row order.
        for (int u0 = 0; u0 < R; u0 += 8) {
            uint16_t vv[8], hh[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int ic = min(g * R + u0 + u, pt.wj - 1);
                vv[u] = lds_ld(V + ic * rd + k);
                hh[u] = lds_ld(&s.h[t][ic]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                // a product of two bf16 values is exact in fp32
                const float v = bf16_f(vv[u]) * bf16_f(hh[u]);
                acc += g * R + u0 + u < pt.wj ? v : 0.f;
            }
        }
        s.vjp[tid] = acc;
    }
    __syncthreads();
    if (tid < n) {
        // the G <= 8 group sums read together, added in group order
        float gv[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) gv[g] = lds_ld(&s.vjp[min(g, G - 1) * n + tid]);
        float acc = gv[0];
#pragma unroll
        for (int g = 1; g < 8; ++g) acc = g < G ? acc + gv[g] : acc;
        s.vj[tid / rd][tid % rd] = acc;
    }
    __syncthreads();
}

// ---- step 2: the slice's share of down ----

// Lane (ro, c) of wave q takes down row o = o0 + pass * 4 kRW + q * kRW + ro
// of a pass and the slice's 16-byte piece c (inputs i0 + 8c .. i0 + 8c + 7).
struct DownLane {
    int c, ro, q;
    __device__ __forceinline__ DownLane() {
        const int lane = threadIdx.x & (kWave - 1);
        c = lane % kL;
        ro = lane / kL;
        q = threadIdx.x / kWave;
    }
    __device__ __forceinline__ int row(int o0, int pass) const { return o0 + pass * (kWaves * kRW) + q * kRW + ro; }
};

// The down operands (W0, U and s of down) each span less than 4 GiB (the plan
// bounds d_out by the rows the parts hold and the intermediate axis by the
// slices), so their offsets are formed in 32 bits and added to the uniform base.
static_assert((unsigned long long)kMlpDownPasses * kWaves * kRW * 8 * kMlpMaxSlices * kW * 2 < (1ull << 32),
              "down W0 offsets fit 32 bits");
template <class T, class B>
__device__ __forceinline__ const T *at_byte(const B *base, uint32_t bytes) {
    return reinterpret_cast<const T *>(reinterpret_cast<const unsigned char *>(base) + bytes);
}

// The lane's piece of down row o (row and piece clamped into the tensor).
__device__ __forceinline__ u32x4 load_down_piece(const MlpDec &a, const Part &pt, int o) {
    const DownLane dl;
    const uint32_t e = (uint32_t)min(o, a.D - 1) * (uint32_t)a.F + (uint32_t)(pt.i0 + 8 * min(dl.c, pt.wj / 8 - 1));
    return ld_stream(at_byte<uint16_t>(a.W0d, 2u * e));
}

// The lane's rank slots e = 0..SL-1. SL = 4 (rd a multiple of 4, at most 32):
// k = 4c + e. SL = 8: k = 8c + e when rd is a multiple of 8, else (rd < 8) slot
// 0 is k = c. Slots without an entry below rd hold zero, in U and in vj alike,
// so every lane runs the same SL products.
template <int SL>
__device__ __forceinline__ bool rank_slot(int rd, int c, int e, int &k) {
    if (SL == 4) {
        k = 4 * c + e;
        return k < rd;
    }
    if (rd % 8 == 0) {
        k = 8 * c + e;
        return k < rd;
    }
    k = c;
    return e == 0 && c < rd;
}
// Slots per lane for a down rank rd: four where the row's ranks fit four per
// lane (half the products and U bytes of eight), else eight.
__host__ __device__ constexpr int rank_slots(int rd) { return rd % 4 == 0 && rd <= 4 * kL ? 4 : 8; }

// U_d[o][k] for the lane's rank slots (rd > 0): with SL = 4 the 8-byte piece
// c of the row (in the low half); with SL = 8 the 16-byte piece c when rd is
// a multiple of 8, else entry c in the low half of the first word. The piece
// or entry is clamped into the row, so slots past rd hold copies that
// down_row masks out (the mask is applied where the value is used, so that no
// load has to have arrived when the next is issued).
template <int SL>
__device__ __forceinline__ u32x4 load_u_piece(const MlpDec &a, int c, int o) {
    const int rd = a.rd;
    const uint16_t *row = a.Ud + (size_t)min(o, a.D - 1) * rd;
    if (SL == 4) {
        const u32x2 v = ldg(reinterpret_cast<const u32x2 *>(row) + min(c, rd / 4 - 1));
        return u32x4{v.x, v.y, 0u, 0u};
    }
    if (rd % 8 == 0) return ldg(reinterpret_cast<const u32x4 *>(row) + min(c, rd / 8 - 1));
    return u32x4{(uint32_t)ldg(row + min(c, rd - 1)), 0u, 0u, 0u};
}

// What every down row of the lane uses: its 16-byte piece of h and its vj
// slots, per token.
template <int TT, int SL>
struct DownIn {
    u32x4 h[TT];
    float v[TT][SL];
    bool uok;   // the lane has rank slots below rd
};
template <int TT, int SL>
__device__ __forceinline__ void load_down_in(const MlpDec &a, const Lds<TT> &s, DownIn<TT, SL> &d) {
    const DownLane dl;
    int k0;
    d.uok = rank_slot<SL>(a.rd, dl.c, 0, k0);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        d.h[t] = lds_ld(reinterpret_cast<const u32x4 *>(s.h[t]) + dl.c);
#pragma unroll
        for (int e = 0; e < SL; ++e) {
            int k;
            const bool ok = rank_slot<SL>(a.rd, dl.c, e, k);
            const float v = lds_ld(&s.vj[t][min(k, kMaxRank - 1)]);
            d.v[t][e] = ok ? v : 0.f;
        }
    }
}

// p_j[t][o] of one down row, on every lane of the row's kL-lane group: the sum
// over the group's lanes of s[o] * (W0 h over the lane's 8 inputs) + (U vj over
// the lane's rank slots).
template <int TT, int SL>
__device__ __forceinline__ void down_row(const Part &pt, u32x4 wd, u32x4 u, float so, const DownIn<TT, SL> &d,
                                         float (&p)[TT]) {
    const DownLane dl;
    const bool in = 8 * dl.c < pt.wj;
    const uint32_t uw[4] = {d.uok ? u.x : 0u, d.uok ? u.y : 0u, d.uok ? u.z : 0u, d.uok ? u.w : 0u};
    float uk[SL];
#pragma unroll
    for (int e = 0; e < SL; ++e) uk[e] = e & 1 ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        float rt = 0.f;
#pragma unroll
        for (int e = 0; e < SL; ++e) rt += uk[e] * d.v[t][e];
        float m = dot8(wd, d.h[t], 0.f);
        m = in ? m : 0.f;   // a select, not a branch (a lane past a ragged slice's end)
        p[t] = group_sum_lanes<kL>(so * m + rt);
    }
}

__device__ __forceinline__ unsigned long long *part_word(const MlpDec &a, int q, int j, int t, int tt, int oo) {
    return a.part + ((q * a.NS + j) * tt + t) * kMlpGroup + oo;   // below 2^20 words
}

// The part's down rows (every pass): W0 pieces of the slice, U pieces, s.
struct DownRows {
    u32x4 wd[kPB];
    u32x4 u[kPB];
    float so[kPB];
};
__device__ __forceinline__ void load_down_w0(const MlpDec &a, const Part &pt, int o0, DownRows &b) {
    const DownLane dl;
    // load_down_piece for the rows of every pass, the clamped row offsets formed
    // as in load_down_us
    const uint32_t ob = (uint32_t)dl.row(o0, 0), last = (uint32_t)(a.D - 1), step = kWaves * kRW, F = (uint32_t)a.F;
    const uint32_t col = (uint32_t)(pt.i0 + 8 * min(dl.c, pt.wj / 8 - 1));
#pragma unroll
    for (int m = 0; m < kPB; ++m) b.wd[m] = ld_stream(at_byte<uint16_t>(a.W0d, 2u * (min((ob + m * step) * F, last * F) + col)));
}
// One wave-uniform branch each for the U layout and for s, outside the row
// loops, so that every load of a loop is issued before any is waited for.
template <int SL>
__device__ __forceinline__ void load_down_us(const MlpDec &a, int o0, DownRows &b) {
    const DownLane dl;
    const int rd = a.rd;
    // Row of pass m: min(o_0 + m kWaves kRW, D - 1), whose offsets are the
    // clamped multiples min((o_0 + m kWaves kRW) rd, (D - 1) rd): one product per
    // lane, then additions.
    const uint32_t ob = (uint32_t)dl.row(o0, 0), last = (uint32_t)(a.D - 1), step = kWaves * kRW;
    if (SL == 4 && rd > 0) {
        const uint32_t piece = 4u * (uint32_t)min(dl.c, rd / 4 - 1);
#pragma unroll
        for (int m = 0; m < kPB; ++m) {
            const uint32_t e = min((ob + m * step) * (uint32_t)rd, last * (uint32_t)rd) + piece;
            const u32x2 v = ldg(at_byte<u32x2>(a.Ud, 2u * e));
            b.u[m] = u32x4{v.x, v.y, 0u, 0u};
        }
    } else if (rd > 0 && rd % 8 == 0) {
        const uint32_t piece = 8u * (uint32_t)min(dl.c, rd / 8 - 1);
#pragma unroll
        for (int m = 0; m < kPB; ++m) {
            const uint32_t e = min((ob + m * step) * (uint32_t)rd, last * (uint32_t)rd) + piece;
            b.u[m] = ldg(at_byte<u32x4>(a.Ud, 2u * e));
        }
    } else if (rd > 0) {
        const uint32_t k = (uint32_t)min(dl.c, rd - 1);
#pragma unroll
        for (int m = 0; m < kPB; ++m) {
            const uint32_t e = min((ob + m * step) * (uint32_t)rd, last * (uint32_t)rd) + k;
            b.u[m] = u32x4{(uint32_t)ldg(at_byte<uint16_t>(a.Ud, 2u * e)), 0u, 0u, 0u};
        }
    } else {
#pragma unroll
        for (int m = 0; m < kPB; ++m) b.u[m] = u32x4{0u, 0u, 0u, 0u};
    }
    if (a.sd) {
#pragma unroll
        for (int m = 0; m < kPB; ++m) b.so[m] = ldg(at_byte<float>(a.sd, 4u * min(ob + m * step, last)));
    } else {
#pragma unroll
        for (int m = 0; m < kPB; ++m) b.so[m] = 1.f;
    }
}

// The part's down rows [o0, o1) of slice j as tagged words.
template <int TT, int SL>
__device__ __forceinline__ void down_part_rows(const MlpDec &a, const Part &pt, int o0, int o1, const DownRows &b,
                                               const DownIn<TT, SL> &d, unsigned long long tag) {
    static_assert(kRW == kMlpGroup, "a wave's rows of one pass are one output group");
    const DownLane dl;
    const int tn = min(TT, a.gu.T - a.gu.t0);
    // o0 is a multiple of 8, so the lane's row of pass m is entry ro of output
    // group o0 / 8 + kWaves m + q: its words lie a fixed stride apart per pass.
    unsigned long long *w = part_word(a, o0 / kMlpGroup + dl.q, pt.j, 0, TT, dl.ro);
    const int pass_words = kWaves * a.NS * TT * kMlpGroup;
    // Every pass first, as one block without branches (rows past o1 read
    // clamped pieces and are not stored), so that the passes' independent
    // chains interleave; then the stores.
    float p[kPB][TT];
#pragma unroll
    for (int m = 0; m < kPB; ++m) down_row<TT, SL>(pt, b.wd[m], b.u[m], b.so[m], d, p[m]);
#pragma unroll
    for (int m = 0; m < kPB; ++m) {
        const int o = dl.row(o0, m);
        if (dl.c == 0 && o < o1) {
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (t < tn)
                    __hip_atomic_store(w + m * pass_words + t * kMlpGroup, tag | __float_as_uint(p[m][t]),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// p_j for the rows of output group q only (a reducer computing a slice whose
// words did not come): wave 0, rows 8q .. 8q + 7 (one pass of kRW = 8 rows),
// the same per-row arithmetic.
template <int TT, int SL>
__device__ __forceinline__ void down_group_rows(const MlpDec &a, const Part &pt, int q, const Lds<TT> &s,
                                                unsigned long long tag) {
    static_assert(kRW == kMlpGroup, "one pass of a wave covers one output group");
    const DownLane dl;
    const int tn = min(TT, a.gu.T - a.gu.t0);
    if (dl.q != 0) return;
    const int o = q * kMlpGroup + dl.ro;
    const u32x4 wd = load_down_piece(a, pt, o);
    const u32x4 u = a.rd > 0 ? load_u_piece<SL>(a, dl.c, o) : u32x4{0u, 0u, 0u, 0u};
    const float so = a.sd ? ldg(a.sd + min(o, a.D - 1)) : 1.f;
    DownIn<TT, SL> d;
    load_down_in<TT, SL>(a, s, d);
    float p[TT];
    down_row<TT, SL>(pt, wd, u, so, d, p);
    if (dl.c == 0 && o < a.D)
        for (int t = 0; t < tn; ++t)
            __hip_atomic_store(part_word(a, q, pt.j, t, TT, o % kMlpGroup), tag | __float_as_uint(p[t]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- the gate/up V^T x from this launch's producers ----

// Read ahead: thread per (child, token, k) item loads that item's tagged slice
// words (at most kEarlyWords slices, when there are at most kThreads items);
// early_check then adds them in the association of gather_tagged_full (one
// group of 16 slices, padded with +0) if every word carries the tag.
struct EarlyVtx {
    unsigned long long w[kEarlyWords];
};
template <int TT>
__device__ __forceinline__ void early_issue(const GemvF &g, int n_items, EarlyVtx &e) {
    const int item = min((int)threadIdx.x, max(n_items - 1, 0));
    int c, t, k;
    vtx_item(g, TT, item, c, t, k);
    const int r = ch_r(g, c);
    const unsigned long long *base = tagged_base(g, c) + t * r + k;
#pragma unroll
    for (int u = 0; u < kEarlyWords; ++u) e.w[u] = ld_word(base + (size_t)min(u, g.S - 1) * (TT * r));
}
template <int TT>
__device__ __forceinline__ bool early_check(const GemvF &g, int n_items, uint32_t tag, const EarlyVtx &e,
                                            Lds<TT> &s) {
    const int item = threadIdx.x;
    if (item >= n_items) return true;
    int c, t, k;
    vtx_item(g, TT, item, c, t, k);
    const bool need = g.t0 + t < g.T;
    bool ok = true;
    float gs = 0.f;
#pragma unroll
    for (int u = 0; u < kEarlyWords; ++u) {
        ok = ok && (u >= g.S || !need || word_is(e.w[u], tag));
        gs += u < g.S ? word_value(e.w[u]) : 0.f;
    }
    float sum = 0.f;
    sum += gs;
    if (ok) s.vs[c][t][k] = sum;
    return ok;
}

// Gate/up V^T x into s.vs: from the words read ahead when they all carried the
// tag, else by reading them again (bounded), else computed here. Ends with a
// barrier.
template <int TT>
__device__ __forceinline__ void finish_gateup_vtx(const MlpDec &a, Lds<TT> &s, bool early, const EarlyVtx &e) {
    const GemvF &g = a.gu;
    const int n_items = vtx_items(g, TT);
    if (n_items == 0) return;
    const bool ready = early && early_check<TT>(g, n_items, s.tag, e, s);
    if (!__syncthreads_or(!ready)) return;
    const int retries = g.spin_limit - 1;
    const bool got = g.spin_limit > 0 && gather_tagged_full<TT>(g, n_items, s.tag, retries, s.vs);
    if (__syncthreads_or(!got)) {
        if (threadIdx.x == 0)
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
template <int TT>
__device__ __forceinline__ bool reduce_poll(const MlpDec &a, int q, int t, uint32_t tag, int retries, float &sum) {
    const int tid = threadIdx.x, oo = tid % kMlpGroup, js = tid / kMlpGroup;
    const bool real = q * kMlpGroup + oo < a.D;
    constexpr int M = kMlpMaxSlices / 32;
    unsigned long long w[M];
    bool ok = false;
    for (int spin = 0;; ++spin) {
        bool ready = true;
#pragma unroll
        for (int m = 0; m < M; ++m) w[m] = ld_word(part_word(a, q, min(js + 32 * m, a.NS - 1), t, TT, oo));
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

// The whole slice j's h in LDS, computed here part by part (a reducer whose
// wait for slice j's words ran out): U rows, s, gate/up rows and h of every
// part, then the slice's V rows.
template <int TT>
__device__ void slice_h_here(const MlpDec &a, int j, Lds<TT> &s) {
    for (int p = 0; p < a.P; ++p) {
        const Part pt = make_part(a, j, p);
        __syncthreads();
        const float sv = stage_part<TT>(a, pt, s);
        wait_vm<0>();
        put_scale<TT>(sv, s);
        __syncthreads();
        gateup_rows<TT, false>(a, pt, s, []() {}, []() {});
        __syncthreads();
        form_h<TT>(a, pt, s);
    }
    stage_vd<TT>(a, make_part(a, j, 0), s);
    wait_vm<0>();
    __syncthreads();
}

template <int TT, bool ONE, int SL>
__global__ __launch_bounds__(kThreads) void mlp_dec_kernel(MlpDec a) {
    __shared__ Lds<TT> s;
    const GemvF &g = a.gu;
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < g.n_prod) {
        vtx_produce<TT>(g, s.vred, s.xstage, &s.tag, s.gsum, s.vs);
        return;
    }
    const int wg = blockIdx.x - g.n_prod;          // this workgroup among the slices' workgroups
    const Part pt = make_part(a, wg / a.P, wg % a.P);
    const int tn = min(TT, g.T - g.t0);
    const int o0 = pt.p * a.Dp, o1 = min(a.D, o0 + a.Dp);   // the part's down rows
    const int n_items = vtx_items(g, TT);
    const bool early = n_items <= kThreads && g.S <= kEarlyWords && g.spin_limit > 0;

    // Issue order per wave (measured best of the orders tried): the first
    // gate/up batch, then down's W0 pieces of the part (registers), so that
    // the whole workgroup's bytes are in flight together; behind the last
    // batch, the slice's small operands (direct-to-LDS), the read-ahead of the
    // gate/up V^T x words and the ticket of thread 0 (last: the compiler may
    // wait for the atomic's result at once, and a wait for any load also
    // waits for every load issued before it).
    unsigned long long ticket;   // thread 0 only; left undefined elsewhere, so that no copy
                                 // of the atomic's result (and no wait for it) is needed here
    DownRows dr;
    EarlyVtx ev;
    float sv = 0.f;
    gateup_rows<TT, ONE>(
        a, pt, s,
        [&]() {
            if (blockIdx.x == 0) advance_empty_copies(g);
            if constexpr (TT > 1) load_down_w0(a, pt, o0, dr);
        },
        [&]() {
            sv = stage_part<TT>(a, pt, s);
            stage_vd<TT>(a, pt, s);
            early_issue<TT>(g, n_items, ev);   // safe addresses whether or not it is used
            // Last: the compiler may wait for the atomic's result at once, and
            // such a wait also waits for everything issued before it.
            if (tid == 0) ticket = take_ticket(g);
        });
    // One token per pass: the whole part's gate/up rows are one batch, and
    // down's W0 follows once they have arrived (measured faster there).
    if constexpr (TT == 1) load_down_w0(a, pt, o0, dr);
    if (tid == 0) s.tag = ticket_tag(ticket);
    __syncthreads();
    finish_gateup_vtx<TT>(a, s, early, ev);
    wait_vm<0>();   // the slice's small operands (direct-to-LDS), issued with the last batch
    load_down_us<SL>(a, o0, dr);   // L2 reads, in flight while h is formed and exchanged
    put_scale<TT>(sv, s);
    __syncthreads();
    form_h<TT>(a, pt, s);
    const uint32_t tag32 = s.tag;
    const unsigned long long tag = (unsigned long long)tag32 << 32;

    // The other parts' h rows of the slice.
    if (a.P > 1) {
        publish_h<TT>(a, pt, s, tag);
        const bool got = g.spin_limit > 0 && fetch_h<TT>(a, pt, s, tag32, g.spin_limit - 1);
        if (__syncthreads_or(!got)) {
            // Compute every other part's h rows here, with the same arithmetic.
            for (int p = 0; p < a.P; ++p) {
                if (p == pt.p) continue;
                const Part op = make_part(a, pt.j, p);
                __syncthreads();
                const float svp = stage_part<TT>(a, op, s);
                wait_vm<0>();
                put_scale<TT>(svp, s);
                __syncthreads();
                gateup_rows<TT, false>(a, op, s, []() {}, []() {});
                __syncthreads();
                form_h<TT>(a, op, s);
            }
        }
        __syncthreads();
    }
    if (a.rd > 0) form_vj<TT>(a, pt, s);
    DownIn<TT, SL> din;
    load_down_in<TT, SL>(a, s, din);
    down_part_rows<TT, SL>(a, pt, o0, o1, dr, din, tag);

    // ---- sums over slices for this workgroup's output groups ----
    const int retries = g.spin_limit - 1;
    const int oo = tid % kMlpGroup, js = tid / kMlpGroup;
    for (int q = wg; q < a.NG; q += a.NS * a.P) {
        for (int t = 0; t < tn; ++t) {
            float sum = 0.f;
            const bool ok = g.spin_limit > 0 && reduce_poll<TT>(a, q, t, tag32, retries, sum);
            if (tid == 0) s.miss = 0;
            __syncthreads();
            if (!ok) atomicOr(&s.miss, 1);
            __syncthreads();
            if (s.miss) {
                // Compute the words of this group that are not there (every
                // slice's when the waits are switched off), one slice at a time
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
                    slice_h_here<TT>(a, jj, s);
                    if (a.rd > 0) form_vj<TT>(a, make_part(a, jj, 0), s);
                    down_group_rows<TT, SL>(a, make_part(a, jj, 0), q, s, tag);
                    __syncthreads();
                }
                reduce_poll<TT>(a, q, t, tag32, kSpinLimit, sum);
            }
            s.red[oo][js] = sum;
            __syncthreads();
            if (tid < kMlpGroup) {
                const int o = q * kMlpGroup + tid;
                // All 32 values read first (vector reads), then added in order.
                f32x4 rv[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) rv[m] = lds_ld(reinterpret_cast<const f32x4 *>(&s.red[tid][4 * m]));
                float y = 0.f;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    y += rv[m].x;
                    y += rv[m].y;
                    y += rv[m].z;
                    y += rv[m].w;
                }
                if (o < a.D) a.y[(size_t)(g.t0 + t) * a.D + o] = f_bf16(y);
            }
            __syncthreads();
        }
    }
    if (blockIdx.x == 0 && tid == 0) sweep_tagged(g.sync, ticket, tag32);
}

}  // namespace

// Workgroups per slice P: the fewest of 1, 2, 4, 8 that keep a part's down
// rows in registers (kMlpDownPasses passes of 32 rows), within 256 slice
// workgroups (one per compute unit). The down rank must fit one 16-byte piece
// per lane (a multiple of 8 up to 64, or below 8); the gate/up V^T x read-ahead
// holds up to 16 slices (d_model up to 2048).
MlpPlan mlp_dec_plan(int d_model, int F, int d_out, int r_gate, int r_up, int r_down, int T) {
    MlpPlan p;
    const int tt = gemv_tokens_per_pass(d_model, T);
    if (tt == 0 || tt > kInLaunchMaxTok) return p;
    if (r_down % 8 != 0 && r_down >= 8) return p;
    const int NS = (F + kW - 1) / kW;
    if (NS > kMlpMaxSlices) return p;
    // A part's down rows start on a boundary of the output groups of 8.
    auto part_rows = [&](int c) { return ((d_out + c - 1) / c + kMlpGroup - 1) / kMlpGroup * kMlpGroup; };
    int P = 0;
    for (int c = 1; c <= 8 && P == 0; c *= 2)
        if (part_rows(c) <= kMlpDownPasses * kWaves * kRW && NS * c <= 256) P = c;
    if (P == 0) return p;
    const int NG = (d_out + kMlpGroup - 1) / kMlpGroup;
    if ((size_t)NG * NS * tt * kMlpGroup > kSyncPartWords) return p;
    if ((size_t)NS * (kW / 2) * tt > kSyncHxWords) return p;
    p.tt = tt;
    p.NS = NS;
    p.P = P;
    p.Dp = part_rows(P);
    p.NG = NG;
    p.slice_len = gemv_slice_len(d_model);
    const int n_v = (r_gate > 0) + (r_up > 0);
    p.S = n_v > 0 ? (d_model + p.slice_len - 1) / p.slice_len : 0;
    p.n_prod = p.S * n_v;
    return p;
}

namespace {
template <int SL>
void launch_tt(const MlpDec &b, int tt, bool one, int grid, hipStream_t stream) {
    switch (tt * 2 + one) {
        case 8: hipLaunchKernelGGL((mlp_dec_kernel<4, false, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
        case 9: hipLaunchKernelGGL((mlp_dec_kernel<4, true, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
        case 4: hipLaunchKernelGGL((mlp_dec_kernel<2, false, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
        case 5: hipLaunchKernelGGL((mlp_dec_kernel<2, true, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
        case 3: hipLaunchKernelGGL((mlp_dec_kernel<1, true, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
        default: hipLaunchKernelGGL((mlp_dec_kernel<1, false, SL>), dim3(grid), dim3(kThreads), 0, stream, b); break;
    }
}
}  // namespace

hipError_t launch_mlp_dec(const MlpDec &a, const MlpPlan &p, hipStream_t stream) {
    MlpDec b = a;
    b.gu.S = p.S;
    b.gu.slice_len = p.slice_len;
    b.gu.n_prod = p.n_prod;
    b.gu.vmode = p.n_prod > 0 ? kVtxInLaunch : kVtxNone;
    b.gu.two_level = 0;
    b.NS = p.NS;
    b.P = p.P;
    b.WR = kW / p.P;
    b.Dp = p.Dp;
    b.NG = p.NG;
    const int grid = p.n_prod + p.NS * p.P;
    const bool one = (kW / p.P) / 8 <= (p.tt == 1 ? kSB<1> : kSB<2>);   // one batch of gate/up row steps per part
    if (rank_slots(a.rd) == 4)
        launch_tt<4>(b, p.tt, one, grid, stream);
    else
        launch_tt<8>(b, p.tt, one, grid, stream);
    return hipGetLastError();
}

}  // namespace wl
