// In-launch hand-off of V^T x between the workgroups of one decode launch:
// producer workgroups compute V^T x slices and store them as generation-tagged
// 64-bit words; consumer workgroups read the words, and compute every slice
// themselves when a bounded wait runs out. Shared by the decode projection
// kernel (k_gemv.hip) and the one-dispatch MLP kernel (k_mlp.hip), so that both
// form V^T x with the same sums in the same association.
//
// The quantity handed over is the inner sum over i of V[i,k] x[t,i] in the
// per-element expansion of the reconstruction formula ("In-kernel
// reconstruction", introduction), computed once per call and shared by every
// workgroup that needs it ("In-kernel reconstruction", the custom-op path:
// V^T x formed cooperatively once, then reused for the rank-r epilogue).
#pragma once

#include "wl_device.h"
#include "wl_kernels.h"
#include "wl_vtx_slice.h"

namespace wl {
namespace {

constexpr int kHThreads = 256;               // threads of every workgroup that uses these helpers
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
    for (int u = 0; u < kGroup; ++u) v[u] = ldg(base + (size_t)min(s0 + u, s1 - 1) * stride);
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
    for (int item = threadIdx.x; item < n_items; item += kHThreads) {
        int c, t, k;
        vtx_item(g, TT, item, c, t, k);
        const int r = ch_r(g, c);
        const float *base = g.partial + (size_t)c * kGemvPartialPerChild + t * r + k;
        float sum = 0.f;
        for (int s0 = 0; s0 < g.S; s0 += kGroup) sum += group_sum(base, TT * r, s0, min(g.S, s0 + kGroup));
        vs[c][t][k] = sum;
    }
}

// ---- in-launch hand-off ----

// This workgroup's ticket (thread 0 only): one fetch-add on counter copy
// blockIdx % kSyncCopies. Every copy gains exactly kSyncStride per launch: the
// copy's last workgroup adds what its others leave, and workgroup 0 also
// advances the copies no workgroup maps to. So every ticket of one launch lies
// in [gen * kSyncStride, (gen + 1) * kSyncStride), whatever the order of the adds.
__device__ __forceinline__ unsigned long long take_ticket(const GemvF &g) {
    const int grid = gridDim.x, b = blockIdx.x, c = b % kSyncCopies;
    const int n_c = (grid - c + kSyncCopies - 1) / kSyncCopies;
    const unsigned long long add = b + kSyncCopies >= grid ? kSyncStride - (unsigned long long)(n_c - 1) : 1ull;
    // The address is uniform; hiding that keeps the compiler from rewriting the
    // add as a wave-combined one whose result it would wait for right here,
    // before the loads that follow are issued.
    auto *ctr = (__attribute__((address_space(1))) unsigned long long *)(g.sync + c);
    asm volatile("" : "+v"(ctr));
    return __hip_atomic_fetch_add(ctr, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void advance_empty_copies(const GemvF &g) {
    const int e = threadIdx.x;
    if (blockIdx.x == 0 && e >= (int)gridDim.x && e < kSyncCopies)
        __hip_atomic_fetch_add(g.sync + e, kSyncStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The launch's tag from thread 0's ticket: the generation mapped into
// [1, 2^32 - 1] (never 0, the tag of a word no launch has written).
__device__ __forceinline__ uint32_t ticket_tag(unsigned long long ticket) {
    // Opaque to the compiler, so the division is not moved up to the atomic
    // (where its wait would hold back the loads issued after it).
    asm volatile("" : "+v"(ticket));
    return (uint32_t)((ticket / kSyncStride) % 0xFFFFFFFFull) + 1u;
}


// A tag is 32 bits, so a word whose last write is exactly 2^32 - 1 generations
// old would carry the current tag again. Every launch that hands words over
// clears one word of the tagged areas that does not carry its own tag (by
// compare-and-swap, so a word stored in the meantime is left alone), walking
// through all kSweepWords words in turn: each word is cleared or rewritten at
// least once every kSweepWords launches, far fewer than 2^32 - 1.
__device__ __forceinline__ void sweep_tagged(unsigned long long *sync, unsigned long long ticket, uint32_t tag) {
    asm volatile("" : "+v"(ticket));
    const unsigned long long gen = ticket / kSyncStride;
    unsigned long long *p = sync + kSyncTaggedOffset / 8 + (size_t)(gen % kSweepWords);
    unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (w != 0ull && (uint32_t)(w >> 32) != tag)
        __hip_atomic_compare_exchange_strong(p, &w, 0ull, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
}

// Child index of the j-th child with r > 0 (j < number of such children).
__device__ __forceinline__ int vtx_child(const GemvF &g, int j) {
    const int a0 = g.ch[0].r > 0, a1 = g.n_ch > 1 && g.ch[1].r > 0;
    if (j == 0) return a0 ? 0 : a1 ? 1 : 2;
    if (j == 1) return a0 && a1 ? 1 : 2;
    return 2;
}

// Tagged slice partials: word [c][slice][t][k] of the partial area, 64 bits,
// the launch's tag in the high half and the fp32 partial in the low half,
// written and read with single device-scope atomic accesses. A reader that
// sees the tag of its own launch therefore sees that launch's value: nothing
// depends on the order in which different words become visible.
__device__ __forceinline__ unsigned long long *tagged_base(const GemvF &g, int c) {
    return g.tagged + (size_t)c * kGemvTaggedPerChild;
}
__device__ __forceinline__ unsigned long long ld_word(const unsigned long long *p) {
    return __hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float word_value(unsigned long long w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool word_is(unsigned long long w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Tagged gathers, in the association of the plain ones. Only words of tokens
// present in the pass (t < tn) are waited for; a group of words with one still
// lacking this launch's tag is read again, at most `retries` more times. False
// when some wait ran out.

// Split mapping: thread (item, group) reads its group's words.
template <int TT>
__device__ __forceinline__ bool gather_tagged_split(const GemvF &g, int n_items, int n_groups, uint32_t tag,
                                                    int retries, float (&v)[kGroup], int &n) {
    int item = threadIdx.x / n_groups;
    const int grp = threadIdx.x - item * n_groups;
    const bool in = item < n_items;
    item = in ? item : 0;
    int c, t, k;
    vtx_item(g, TT, item, c, t, k);
    const int r = ch_r(g, c);
    const unsigned long long *base = tagged_base(g, c) + t * r + k;
    const int s0 = grp * kGroup, s1 = min(g.S, s0 + kGroup);
    const bool need = in && g.t0 + t < g.T;
    unsigned long long w[kGroup];
    bool ok = false;
    for (int spin = 0;; ++spin) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) w[u] = ld_word(base + (size_t)min(s0 + u, s1 - 1) * (TT * r));
        bool ready = true;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) ready = ready && (!need || word_is(w[u], tag));
        if (ready) {
            ok = true;
            break;
        }
        if (spin >= retries) break;
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) v[u] = word_value(w[u]);
    n = in ? s1 - s0 : 0;
    return ok;
}

// Full mapping: thread per item, groups in order, into vs.
template <int TT>
__device__ bool gather_tagged_full(const GemvF &g, int n_items, uint32_t tag, int retries,
                                   float (*vs)[TT][kMaxRank]) {
    bool ok = true;
    for (int item = threadIdx.x; item < n_items && ok; item += kHThreads) {
        int c, t, k;
        vtx_item(g, TT, item, c, t, k);
        const int r = ch_r(g, c);
        const unsigned long long *base = tagged_base(g, c) + t * r + k;
        const bool need = g.t0 + t < g.T;
        float sum = 0.f;
        for (int s0 = 0; s0 < g.S && ok; s0 += kGroup) {
            const int s1 = min(g.S, s0 + kGroup);
            unsigned long long w[kGroup];
            for (int spin = 0;; ++spin) {
#pragma unroll
                for (int u = 0; u < kGroup; ++u) w[u] = ld_word(base + (size_t)min(s0 + u, s1 - 1) * (TT * r));
                bool ready = true;
#pragma unroll
                for (int u = 0; u < kGroup; ++u) ready = ready && (!need || word_is(w[u], tag));
                if (ready) break;
                if (spin >= retries) {
                    ok = false;
                    break;
                }
            }
            float gs = 0.f;
#pragma unroll
            for (int u = 0; u < kGroup; ++u) gs += s0 + u < s1 ? word_value(w[u]) : 0.f;
            sum += gs;
        }
        vs[c][t][k] = sum;
    }
    return ok;
}

__device__ __forceinline__ unsigned long long *final_words(const GemvF &g) { return g.fin; }

// One slice's x for the producers and the fallback. Up to 2 tokens: read
// straight from global memory with the V loads. More: staged in LDS first
// (xs: TT x kXStageMax bf16, absent tokens zero), as the V^T x launch does, so
// that the x values held in registers stay few. The values, and so the bits of
// the sums, are the same either way.
constexpr int kXStageMax = 512;   // >= every slice length of the decode kernel (d_in <= 32768, <= 64 slices)
template <int TT>
__device__ __forceinline__ void stage_x(const GemvF &g, int i0, int len, int tn, u32x4 *xs) {
    if constexpr (TT > 2) {
        const int nchunk = len >> 3, row_chunks = g.d_in >> 3;
        const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
        for (int idx = threadIdx.x; idx < TT * nchunk; idx += kHThreads) {
            const int t = idx / nchunk, j = idx - t * nchunk;
            xs[t * (kXStageMax / 8) + j] =
                t < tn ? xg[(size_t)(g.t0 + t) * row_chunks + (i0 >> 3) + j] : u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
    }
}
template <int TT, class Hook = NoHook>
__device__ __forceinline__ void slice_sums(const GemvF &g, const uint16_t *V, int r, int i0, int len, int tn,
                                           const u32x4 *xs, float (*red)[TT + 1], Hook hook = Hook()) {
    if constexpr (TT > 2) {
        const uint16_t *x16 = reinterpret_cast<const uint16_t *>(xs);
        vtx_slice_sums<TT>(V, r, i0, len, [&](int ic, int t) { return bf16_f(x16[t * kXStageMax + ic]); }, red,
                           hook);
    } else {
        const VtxXGlobal<TT> xg{g.x + (size_t)g.t0 * g.d_in, g.d_in, i0, tn};
        vtx_slice_sums<TT>(V, r, i0, len, xg, red, hook);
    }
}

// Producer workgroup p: slice p % S of child vtx_child(p / S), for the pass's
// tokens, as the V^T x launch computes it, stored as tagged words. With
// two_level, the last producer (dispatched last, so usually the last to finish
// and the one whose first read finds every word) then gathers every slice as a
// projection workgroup would (same association, same bits) and stores the
// complete V^T x as one tagged word per item.
template <int TT>
__device__ void vtx_produce(const GemvF &g, float (*red)[TT + 1], u32x4 *xs, uint32_t *tag_lds, float *gsum,
                            float (*vs)[TT][kMaxRank]) {
    const int tid = threadIdx.x, p = blockIdx.x;
    unsigned long long ticket;
    const int slice = p % g.S, c = vtx_child(g, p / g.S);
    const int r = ch_r(g, c);
    const uint16_t *V = reinterpret_cast<const uint16_t *>(
        blend3(c, (uint64_t)g.ch[0].V, (uint64_t)g.ch[1].V, (uint64_t)g.ch[2].V));
    const int i0 = slice * g.slice_len, len = max(0, min(g.d_in - i0, g.slice_len));
    const int tn = min(TT, g.T - g.t0);
    stage_x<TT>(g, i0, len, tn, xs);
    // The ticket is taken once the V (and x) loads are issued, so its round trip
    // overlaps theirs.
    slice_sums<TT>(g, V, r, i0, len, tn, xs, red, [&]() {
        if (tid == 0) ticket = take_ticket(g);
    });
    advance_empty_copies(g);
    if (tid == 0) *tag_lds = ticket_tag(ticket);
    __syncthreads();
    const uint32_t tag32 = *tag_lds;
    const unsigned long long tag = (unsigned long long)tag32 << 32;
    unsigned long long *part = tagged_base(g, c) + (size_t)slice * TT * r;
    for (int idx = tid; idx < r * tn; idx += kHThreads) {
        const int t = idx / r, kk = idx - t * r;
        const unsigned long long w = tag | __float_as_uint(vtx_slice_total<TT>(red, r, t, kk));
        __hip_atomic_store(part + t * r + kk, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (p == 0 && tid == 0) sweep_tagged(g.sync, ticket, tag32);
    if (!g.two_level || p != g.n_prod - 1 || g.spin_limit == 0) return;
    const int retries = g.spin_limit - 1;

    const int n_items = vtx_items(g, TT);
    const int n_groups = (g.S + kGroup - 1) / kGroup;
    const bool split = n_items * n_groups <= kHThreads;
    float gv[kGroup];
    int gn = 0;
    const bool got = split ? gather_tagged_split<TT>(g, n_items, n_groups, tag32, retries, gv, gn)
                           : gather_tagged_full<TT>(g, n_items, tag32, retries, vs);
    if (__syncthreads_or(!got)) return;   // the projection workgroups will compute V^T x themselves
    if (split) {
        gsum[tid] = gather_finish(gv, gn);
        __syncthreads();
    }
    unsigned long long *fin = final_words(g);
    for (int item = tid; item < n_items; item += kHThreads) {
        int cc, t, k;
        vtx_item(g, TT, item, cc, t, k);
        float v;
        if (split) {
            v = 0.f;
            for (int j = 0; j < n_groups; ++j) v += gsum[item * n_groups + j];
        } else {
            v = vs[cc][t][k];
        }
        __hip_atomic_store(fin + item, tag | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Two-level: thread per item reads the complete word (again while it lacks the
// tag, at most `retries` more times) into vs.
template <int TT>
__device__ bool gather_final(const GemvF &g, int n_items, uint32_t tag, int retries, float (*vs)[TT][kMaxRank]) {
    bool ok = true;
    const unsigned long long *fin = final_words(g);
    for (int item = threadIdx.x; item < n_items && ok; item += kHThreads) {
        int c, t, k;
        vtx_item(g, TT, item, c, t, k);
        const bool need = g.t0 + t < g.T;
        unsigned long long w;
        for (int spin = 0;; ++spin) {
            w = ld_word(fin + item);
            if (!need || word_is(w, tag)) break;
            if (spin >= retries) {
                ok = false;
                break;
            }
        }
        vs[c][t][k] = word_value(w);
    }
    return ok;
}

// Fallback of a workgroup whose wait ran out: every slice of every child with
// r > 0, computed as the producers do, added in the gathers' association
// (groups of kGroup slices, each group's sum from 0 and padded with +0 as the
// gathers pad a short group, group sums in order from 0). gs: LDS, n_items floats.
template <int TT>
__device__ void vtx_fallback(const GemvF &g, int n_items, float (*vs)[TT][kMaxRank], float (*red)[TT + 1],
                             u32x4 *xs, float *gs) {
    const int tid = threadIdx.x;
    for (int item = tid; item < n_items; item += kHThreads) {
        int c, t, k;
        vtx_item(g, TT, item, c, t, k);
        vs[c][t][k] = 0.f;
        gs[item] = 0.f;
    }
    const int n_v = g.n_prod / g.S;
    const int tn = min(TT, g.T - g.t0);
    for (int s = 0; s < g.S; ++s) {
        const int i0 = s * g.slice_len, len = max(0, min(g.d_in - i0, g.slice_len));
        stage_x<TT>(g, i0, len, tn, xs);   // the previous slice's reads ended before its sums' barriers
        for (int j = 0; j < n_v; ++j) {
            const int c = vtx_child(g, j);
            const int r = ch_r(g, c);
            const uint16_t *V = reinterpret_cast<const uint16_t *>(
                blend3(c, (uint64_t)g.ch[0].V, (uint64_t)g.ch[1].V, (uint64_t)g.ch[2].V));
            slice_sums<TT>(g, V, r, i0, len, tn, xs, red);   // begins and ends with a barrier
            for (int item = tid; item < n_items; item += kHThreads) {
                int cc, t, k;
                vtx_item(g, TT, item, cc, t, k);
                if (cc == c) gs[item] += vtx_slice_total<TT>(red, r, t, k);
            }
        }
        const bool group_end = (s % kGroup) == kGroup - 1 || s == g.S - 1;
        if (group_end)
            for (int item = tid; item < n_items; item += kHThreads) {
                int c, t, k;
                vtx_item(g, TT, item, c, t, k);
                float v = gs[item];
                if ((s % kGroup) != kGroup - 1) v += 0.f;   // a short last group
                vs[c][t][k] += v;
                gs[item] = 0.f;
            }
    }
}


}  // namespace
}  // namespace wl
