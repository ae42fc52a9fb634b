// Host side of the C ABI declared in include/wl.h: argument checks, workspace
// layout, regime choice (wave-per-row GEMV for a few tokens, matrix-core GEMM
// above that) and kernel launches. Nothing here computes any part of the
// projection; every arithmetic step runs in the HIP kernels.
#include "wl.h"
#include "wl_testing.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "wl_kernels.h"

namespace {

thread_local std::string g_error;
std::atomic<int> g_spin_limit{wl::kSpinLimit};   // polls before a decode workgroup computes V^T x itself
// 0 auto, 1 GEMV, 2 matrix-core GEMM, 3 GEMV always after a V^T x launch, 4 skinny,
// 5 GEMV with the MLP as two launches (gate/up, then down)
std::atomic<int> g_regime{0};

// WL_LOG is read once per process.
bool log_on() {
    static const bool on = getenv("WL_LOG") != nullptr;
    return on;
}

constexpr size_t kAlign = 256;

wl_status fail(wl_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    if (log_on()) fprintf(stderr, "wl: %s\n", buf);
    return st;
}

wl_status ok() {
    g_error.clear();
    return WL_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Range {
    const void *p;
    size_t bytes;
};

bool overlaps(Range a, Range b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

const int64_t kMaxElems = (int64_t)1 << 31;

wl_status check_theta(const wl_theta *th, const char *name) {
    if (!th) return fail(WL_ERR_INVALID_ARG, "%s: theta is NULL", name);
    if (th->dtype != WL_DTYPE_BF16 && th->dtype != WL_DTYPE_F32)
        return fail(WL_ERR_UNSUPPORTED, "%s: dtype=%d is neither WL_DTYPE_BF16 nor WL_DTYPE_F32", name, th->dtype);
    if (th->d_in < 1 || th->d_out < 1)
        return fail(WL_ERR_INVALID_ARG, "%s: d_in=%d d_out=%d must be >= 1", name, th->d_in, th->d_out);
    if (th->d_in % 8)
        return fail(WL_ERR_INVALID_ARG, "%s: d_in=%d is not a multiple of 8", name, th->d_in);
    if (th->r < 0) return fail(WL_ERR_INVALID_ARG, "%s: r=%d is negative", name, th->r);
    if (th->r > wl::kMaxRank)
        return fail(WL_ERR_UNSUPPORTED, "%s: r=%d exceeds the supported maximum %d", name, th->r, wl::kMaxRank);
    if ((int64_t)th->d_in * th->d_out >= kMaxElems)
        return fail(WL_ERR_INVALID_ARG, "%s: W0 has 2^31 or more elements", name);
    if (!th->W0) return fail(WL_ERR_INVALID_ARG, "%s: W0 is NULL", name);
    if (!aligned(th->W0, 16)) return fail(WL_ERR_INVALID_ARG, "%s: W0 is not 16-byte aligned", name);
    if (th->s && !aligned(th->s, 4)) return fail(WL_ERR_INVALID_ARG, "%s: s is not 4-byte aligned", name);
    if (th->r > 0) {
        if (!th->U || !th->V) return fail(WL_ERR_INVALID_ARG, "%s: r=%d but U or V is NULL", name, th->r);
        if (!aligned(th->U, 16) || !aligned(th->V, 16))
            return fail(WL_ERR_INVALID_ARG, "%s: U or V is not 16-byte aligned", name);
    }
    return WL_OK;
}

// Bytes per element of W0, U, V and of the call's x, y (and h, W_eff).
size_t elem_bytes(const wl_theta *th) { return th->dtype == WL_DTYPE_F32 ? 4 : 2; }

void theta_ranges(const wl_theta *th, Range *out /* 4 */) {
    const size_t es = elem_bytes(th);
    out[0] = {th->W0, (size_t)th->d_out * th->d_in * es};
    out[1] = {th->s, th->s ? (size_t)th->d_out * 4 : 0};
    out[2] = {th->r > 0 ? th->U : nullptr, (size_t)th->d_out * th->r * es};
    out[3] = {th->r > 0 ? th->V : nullptr, (size_t)th->d_in * th->r * es};
}

// The thetas of one fused call must share their element type.
wl_status check_same_dtype(const wl_theta *const *ths, int n, const char *op) {
    for (int c = 1; c < n; ++c)
        if (ths[c]->dtype != ths[0]->dtype)
            return fail(WL_ERR_INVALID_ARG, "%s: the thetas' dtypes differ (%d and %d)", op, ths[0]->dtype, ths[c]->dtype);
    return WL_OK;
}

// ---------------------------------------------------------------------------
// Kernel regime of one projection: decode GEMV (T up to kGemvMaxTok), the
// two-launch skinny path (a few tens of tokens), or the matrix-core GEMM.
enum Kind { kKindGemv, kKindSkinny, kKindGemm };

bool skinny_ok(int T, int d_in, int sum_r) {
    (void)sum_r;
    return T >= 1 && T <= wl::kSkMaxTok && d_in <= wl::kSkMaxDin;
}

Kind choose(int T, int d_in, int sum_r) {
    const int regime = g_regime.load(std::memory_order_relaxed);
    const int tt = wl::gemv_tokens_per_pass(d_in, T);
    const bool sk = skinny_ok(T, d_in, sum_r);
    switch (regime) {
        case 1:
        case 3:
        case 5: return tt ? kKindGemv : kKindGemm;
        case 2:
        case 6: return kKindGemm;
        case 4: return sk ? kKindSkinny : kKindGemm;
        default: break;
    }
    if (T <= wl::kGemvMaxTok && tt) return kKindGemv;
    return sk ? kKindSkinny : kKindGemm;
}

// Workspace layout. One layout function serves both wl_workspace_bytes and the
// calls, so the two always agree. Every region any regime could use at this T
// is reserved, so the size does not depend on the regime switch.
//
//   [0, kSyncBytes)   sync area of the decode kernel's in-launch V^T x hand-off:
//                     ticket counters, a fallback count and the tagged V^T x
//                     words (64-bit); zero before the workspace's first use,
//                     then kept consistent by the kernels
//   gemv_partial      fp32 3 x [kGemvMaxSlices][kGemvMaxTok][kMaxRank] V^T x slices
//                     (decode regime, V^T x in a launch of its own)
//   skinny part       fp32 [S][P][T][rows] split partials (T <= kSkMaxTok), the
//                     largest of the call's projections
//   skinny vpart      fp32 [n_vsl][n_ch][T][kMaxRank] V^T x slice partials
//   mm_vtx            fp32 [S][T][r_c] per child: V^T x split partials of the
//                     matrix-core regime (the largest of the call's projections)
//   mm_part           fp32 [ksplit][T][d_out]: input-axis split partials of the
//                     matrix-core regime (the largest of the call's projections)
//   h                 bf16 [T][d_ff] (MLP only)

constexpr size_t kReservedBytes = wl::kSyncBytes;
static_assert(WL_SYNC_BYTES == wl::kSyncBytes, "sync area size");

struct Layout {
    size_t gemv_partial = 0;
    size_t sk_part = 0, sk_vpart = 0;
    size_t mm_vtx = 0;
    size_t mm_part = 0;
    size_t f32_part = 0, f32_vtx = 0;   // fp32 variant only
    size_t h = 0;
    size_t total = 0;
};

struct ProjShape {
    int rows, d_in, P, n_ch, sum_r, n_vtx_ch;
};

// The projections a call runs, in order.
int proj_shapes(int op, const wl_theta *const *th, ProjShape *out) {
    auto nv = [](const wl_theta *const *t, int n) {
        int c = 0;
        for (int j = 0; j < n; ++j) c += t[j]->r > 0;
        return c;
    };
    if (op == WL_OP_LINEAR) {
        out[0] = {th[0]->d_out, th[0]->d_in, 1, 1, th[0]->r, nv(th, 1)};
        return 1;
    }
    if (op == WL_OP_QKV) {
        out[0] = {th[0]->d_out + th[1]->d_out + th[2]->d_out, th[0]->d_in, 1, 3, th[0]->r + th[1]->r + th[2]->r,
                  nv(th, 3)};
        return 1;
    }
    out[0] = {th[0]->d_out, th[0]->d_in, 2, 2, th[0]->r + th[1]->r, nv(th, 2)};
    out[1] = {th[2]->d_out, th[2]->d_in, 1, 1, th[2]->r, nv(th + 2, 1)};
    return 2;
}

// fp32 variant: V^T x slice partials [n_slices][T][r_c] and complete V^T x
// [T][r_c] per child (the largest of the call's projections), MLP h fp32 [T][d_ff].
Layout layout_f32(int op, const wl_theta *const *th, int T) {
    Layout L;
    size_t off = kReservedBytes;
    ProjShape ps[2];
    const int n = proj_shapes(op, th, ps);
    size_t part = 0, vtx = 0;
    int first = 0;
    for (int j = 0; j < n; ++j) {
        const int n_th = ps[j].P == 2 ? 2 : ps[j].n_ch;
        size_t a = 0, b = 0;
        for (int c = 0; c < n_th; ++c) {
            const int r = th[first + c]->r;
            if (r == 0) continue;
            a += round_up((size_t)wl::f32_vtx_slices(ps[j].d_in) * T * r * 4, kAlign);
            b += round_up((size_t)T * r * 4, kAlign);
        }
        part = a > part ? a : part;
        vtx = b > vtx ? b : vtx;
        first += n_th;
    }
    L.f32_part = off;
    off = round_up(off + part, kAlign);
    L.f32_vtx = off;
    off = round_up(off + vtx, kAlign);
    if (op == WL_OP_MLP) {
        L.h = off;
        off = round_up(off + (size_t)T * th[0]->d_out * 4, kAlign);
    }
    L.total = off;
    return L;
}

Layout layout(int op, const wl_theta *const *th, int T) {
    if (th[0]->dtype == WL_DTYPE_F32) return layout_f32(op, th, T);
    Layout L;
    size_t off = kReservedBytes;
    L.gemv_partial = off;
    off = round_up(off + wl::kMaxChildren * wl::kGemvPartialPerChild * 4, kAlign);
    ProjShape ps[2];
    const int n = proj_shapes(op, th, ps);
    size_t part = 0, vpart = 0;
    for (int j = 0; j < n; ++j) {
        if (!skinny_ok(T, ps[j].d_in, ps[j].sum_r)) continue;
        const wl::SkinnyPlan p = wl::skinny_plan(ps[j].rows, ps[j].d_in, T, ps[j].P, ps[j].n_vtx_ch);
        const size_t a = (size_t)p.S * ps[j].P * T * ps[j].rows * 4;
        const size_t b = (size_t)p.n_vsl * ps[j].n_ch * T * wl::kMaxRank * 4;
        part = a > part ? a : part;
        vpart = b > vpart ? b : vpart;
    }
    L.sk_part = off;
    off = round_up(off + part, kAlign);
    L.sk_vpart = off;
    off = round_up(off + vpart, kAlign);
    size_t mm = 0;
    for (int j = 0; j < n; ++j) {
        const size_t b = (size_t)wl::vtxmm_splits(ps[j].d_in, wl::kMaxRank) * T * ps[j].sum_r * 4 + wl::kMaxChildren * kAlign;
        mm = ps[j].sum_r > 0 && b > mm ? b : mm;
    }
    L.mm_vtx = off;
    off = round_up(off + mm, kAlign);
    size_t mp = 0;
    for (int j = 0; j < n; ++j) {
        const wl::GemmSplit sp = wl::gemm_split_plan(T, ps[j].d_in, ps[j].rows, ps[j].n_ch, ps[j].P == 2);
        const size_t b = sp.ksplit > 1 ? (size_t)sp.ksplit * T * ps[j].rows * 4 : 0;
        mp = b > mp ? b : mp;
    }
    L.mm_part = off;
    off = round_up(off + mp, kAlign);
    if (op == WL_OP_MLP) {
        L.h = off;
        off = round_up(off + (size_t)T * th[0]->d_out * 2, kAlign);
    }
    L.total = off;
    return L;
}

wl::Child make_child(const wl_theta *th, int col0) {
    wl::Child c;
    c.W0 = static_cast<const uint16_t *>(th->W0);
    c.s = th->s;
    c.U = static_cast<const uint16_t *>(th->U);
    c.V = static_cast<const uint16_t *>(th->V);
    c.vtx = nullptr;
    c.vtx_splits = 0;
    c.r = th->r;
    c.d_out = th->d_out;
    c.col0 = col0;
    return c;
}

// V^T x slice partials for the children with r > 0 (all sharing input x of
// width d_in): tokens [t0, t0 + T) of x, partial of child c at partial_c(c),
// laid out [n_slices][ld_T][r_c].
template <class PartialOf>
wl_status run_vtx(const wl::Child *ch, int n, PartialOf partial_c, const void *x, int d_in, int t0, int T, int ld_T,
                  int slice_len, hipStream_t stream) {
    wl::VtxJob job{};
    job.x = static_cast<const uint16_t *>(x) + (size_t)t0 * d_in;
    job.d_in = d_in;
    job.T = T;
    job.ld_T = ld_T;
    for (int c = 0; c < n; ++c) {
        if (ch[c].r == 0) continue;
        job.V[job.n_ch] = ch[c].V;
        job.partial[job.n_ch] = partial_c(c);
        job.r[job.n_ch] = ch[c].r;
        ++job.n_ch;
    }
    if (job.n_ch == 0) return WL_OK;
    job.slice_len = slice_len;
    job.n_slices = (d_in + slice_len - 1) / slice_len;
    const hipError_t e = wl::launch_vtx(job, stream);
    if (e != hipSuccess) return fail(WL_ERR_HIP, "V^T x launch failed: %s", hipGetErrorString(e));
    return WL_OK;
}

// One projection over shared input x: children side by side in y (ldy = total
// width), or the gate/up pair (pair = true, y = h).
wl_status run_proj(const wl::Child *ch, int n_ch, bool pair, int d_in, int T, const void *x, void *y, int ldy,
                   char *ws, const Layout &L, hipStream_t stream) {
    hipError_t e = hipSuccess;
    int sum_r = 0, rows = 0;
    for (int c = 0; c < n_ch; ++c) {
        sum_r += ch[c].r;
        rows += ch[c].d_out;
    }
    if (pair) rows = ch[0].d_out;
    const Kind kind = choose(T, d_in, sum_r);
    const int tt = kind == kKindGemv ? wl::gemv_tokens_per_pass(d_in, T) : 0;
    if (log_on())
        fprintf(stderr, "wl: proj n_ch=%d pair=%d d_in=%d T=%d -> %s (tt=%d)\n", n_ch, (int)pair, d_in, T,
                kind == kKindGemv ? "gemv" : kind == kKindSkinny ? "skinny" : "mfma", tt);
    if (kind == kKindSkinny) {
        wl::Skinny g{};
        int nv = 0;
        for (int c = 0; c < n_ch; ++c) {
            g.ch[c] = ch[c];
            if (ch[c].r > 0) g.vtx_ch[nv++] = c;
        }
        g.n_ch = n_ch;
        g.pair = pair;
        g.d_in = d_in;
        g.rows = rows;
        g.ldy = ldy;
        g.T = T;
        g.x = static_cast<const uint16_t *>(x);
        g.y = static_cast<uint16_t *>(y);
        g.part = reinterpret_cast<float *>(ws + L.sk_part);
        g.vpart = reinterpret_cast<float *>(ws + L.sk_vpart);
        const wl::SkinnyPlan p = wl::skinny_plan(rows, d_in, T, pair ? 2 : 1, nv);
        g.S = p.S;
        g.n_rowblk = p.n_rowblk;
        g.kb_per_split = p.kb_per_split;
        g.n_vsl = p.n_vsl;
        // Ranks 32 and 64 split their V^T x work over two workgroups per slice.
        g.vsplit = nv > 0 ? 2 : 1;
        for (int c = 0; c < n_ch; ++c)
            if (ch[c].r > 0 && ch[c].r != 32 && ch[c].r != 64) g.vsplit = 1;
        g.n_vtx_wg = p.n_vtx_wg * g.vsplit;
        e = wl::launch_skinny(g, stream);
    } else if (kind == kKindGemv) {
        wl::GemvF g{};
        for (int c = 0; c < n_ch; ++c) g.ch[c] = ch[c];
        g.n_ch = n_ch;
        g.pair = pair;
        g.d_in = d_in;
        g.rows = rows;
        g.ldy = ldy;
        g.T = T;
        g.x = static_cast<const uint16_t *>(x);
        g.y = static_cast<uint16_t *>(y);
        g.partial = reinterpret_cast<float *>(ws + L.gemv_partial);
        g.tagged = reinterpret_cast<unsigned long long *>(ws + wl::kSyncTaggedOffset);
        g.sync = reinterpret_cast<unsigned long long *>(ws);   // the sync area at offset 0
        g.fin = reinterpret_cast<unsigned long long *>(ws + wl::kSyncFinalOffset);
        g.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
        const bool separate = g_regime.load(std::memory_order_relaxed) == 3;
        const wl::GemvPlan plan = wl::gemv_plan(g, tt, !separate);
        auto part = [&](int c) { return g.partial + (size_t)c * wl::kGemvPartialPerChild; };
        for (int t0 = 0; t0 < T && e == hipSuccess; t0 += tt) {
            g.t0 = t0;
            if (plan.vmode == wl::kVtxPartials) {
                const int n_tok = T - t0 < tt ? T - t0 : tt;
                wl_status st = run_vtx(ch, n_ch, part, x, d_in, t0, n_tok, tt, plan.slice_len, stream);
                if (st != WL_OK) return st;
            }
            e = wl::launch_gemv(g, plan, tt, stream);
        }
    } else {
        wl::Gemm g{};
        for (int c = 0; c < n_ch; ++c) g.ch[c] = ch[c];
        const wl::GemmSplit sp = wl::gemm_split_plan(T, d_in, rows, n_ch, pair);
        // A split input axis (one child, r <= 32, at most 4 splits) adds the rank term in its
        // reduction: V^T x (one split) then comes from extra workgroups of the
        // GEMM launch itself, whose tiles do not read it. Regime 6 keeps the
        // launch of its own.
        const bool in_reduce = sp.ksplit > 1 && sp.ksplit <= wl::kRedMaxSplits && sum_r > 0 && sum_r <= 32 &&
                               g_regime.load(std::memory_order_relaxed) != 6;
        if (sum_r > 0) {
            // V^T x split partials on the matrix cores, added in order by their consumer.
            wl::VtxMM mm{};
            mm.x = static_cast<const uint16_t *>(x);
            mm.d_in = d_in;
            mm.T = T;
            int max_r = 0;
            for (int c = 0; c < n_ch; ++c) max_r = ch[c].r > max_r ? ch[c].r : max_r;
            const int nkb = (d_in + 63) / 64;
            mm.S = in_reduce ? 1 : wl::vtxmm_splits(d_in, max_r);
            mm.kb_per_split = (nkb + mm.S - 1) / mm.S;
            mm.S = (nkb + mm.kb_per_split - 1) / mm.kb_per_split;
            size_t moff = L.mm_vtx;
            for (int c = 0; c < n_ch; ++c) {
                if (ch[c].r == 0) continue;
                float *part = reinterpret_cast<float *>(ws + moff);
                moff += round_up((size_t)mm.S * T * ch[c].r * 4, kAlign);
                g.ch[c].vtx = part;
                g.ch[c].vtx_splits = mm.S;
                mm.V[mm.n] = ch[c].V;
                mm.part[mm.n] = part;
                mm.r[mm.n] = ch[c].r;
                ++mm.n;
            }
            if (in_reduce) {
                g.job = mm;
                g.n_prod = (T + 31) / 32 * mm.S * mm.n;
            } else {
                e = wl::launch_vtxmm(mm, stream);
                if (e != hipSuccess) return fail(WL_ERR_HIP, "V^T x launch failed: %s", hipGetErrorString(e));
            }
        }
        g.n_ch = n_ch;
        g.pair = pair;
        g.d_in = d_in;
        g.ldy = ldy;
        g.T = T;
        g.x = static_cast<const uint16_t *>(x);
        g.y = static_cast<uint16_t *>(y);
        g.ksplit = sp.ksplit;
        g.kb_per_split = sp.kb_per_split;
        g.part = reinterpret_cast<float *>(ws + L.mm_part);
        e = wl::launch_gemm(g, stream);
    }
    if (e != hipSuccess) return fail(WL_ERR_HIP, "projection launch failed: %s", hipGetErrorString(e));
    return WL_OK;
}

// One fp32 projection over shared x (children side by side in y, or the
// gate/up pair into h): V^T x slices and their ordered sum, then the GEMV
// (a few tokens) or the matrix-core GEMM.
wl_status run_proj_f32(const wl_theta *const *ths, int n_ch, bool pair, int d_in, int T, const void *x, void *y,
                       int ldy, char *ws, const Layout &L, hipStream_t stream) {
    wl::F32Proj g{};
    wl::F32Vtx vj{};
    vj.x = static_cast<const float *>(x);
    vj.d_in = d_in;
    vj.T = T;
    vj.n_slices = wl::f32_vtx_slices(d_in);
    size_t poff = L.f32_part, voff = L.f32_vtx;
    int col0 = 0;
    for (int c = 0; c < n_ch; ++c) {
        const wl_theta *t = ths[c];
        wl::F32Child &C = g.ch[c];
        C.W0 = static_cast<const float *>(t->W0);
        C.s = t->s;
        C.U = static_cast<const float *>(t->U);
        C.vtx = nullptr;
        C.r = t->r;
        C.d_out = t->d_out;
        C.col0 = pair ? 0 : col0;
        if (!pair) col0 += t->d_out;
        if (t->r == 0) continue;
        float *part = reinterpret_cast<float *>(ws + poff);
        poff += round_up((size_t)vj.n_slices * T * t->r * 4, kAlign);
        float *vtx = reinterpret_cast<float *>(ws + voff);
        voff += round_up((size_t)T * t->r * 4, kAlign);
        C.vtx = vtx;
        vj.V[vj.n_ch] = static_cast<const float *>(t->V);
        vj.part[vj.n_ch] = part;
        vj.vtx[vj.n_ch] = vtx;
        vj.r[vj.n_ch] = t->r;
        ++vj.n_ch;
    }
    hipError_t e = wl::launch_f32_vtx(vj, stream);
    if (e != hipSuccess) return fail(WL_ERR_HIP, "fp32 V^T x launch failed: %s", hipGetErrorString(e));
    g.n_ch = n_ch;
    g.pair = pair;
    g.d_in = d_in;
    g.T = T;
    g.ldy = ldy;
    g.x = static_cast<const float *>(x);
    g.y = static_cast<float *>(y);
    const int regime = g_regime.load(std::memory_order_relaxed);
    const bool gemv = T <= wl::kF32GemvMaxTok && regime != 2 && regime != 4;
    if (log_on())
        fprintf(stderr, "wl: fp32 proj n_ch=%d pair=%d d_in=%d T=%d -> %s\n", n_ch, (int)pair, d_in, T,
                gemv ? "gemv" : "mfma");
    e = gemv ? wl::launch_f32_gemv(g, stream) : wl::launch_f32_gemm(g, stream);
    if (e != hipSuccess) return fail(WL_ERR_HIP, "fp32 projection launch failed: %s", hipGetErrorString(e));
    return WL_OK;
}

wl_status check_io(const void *x, const void *y, int T, int d_in, int ldy) {
    if (T < 0) return fail(WL_ERR_INVALID_ARG, "T=%d is negative", T);
    if (T == 0) return WL_OK;
    if (!x || !y) return fail(WL_ERR_INVALID_ARG, "x or y is NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(WL_ERR_INVALID_ARG, "x or y is not 16-byte aligned");
    if ((int64_t)T * d_in >= kMaxElems || (int64_t)T * ldy >= kMaxElems)
        return fail(WL_ERR_INVALID_ARG, "x or y has 2^31 or more elements");
    return WL_OK;
}

wl_status check_ws(size_t need, const void *ws, size_t ws_bytes) {
    if (ws_bytes < need)
        return fail(WL_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu", ws_bytes, need);
    if (need > 0 && !ws) return fail(WL_ERR_INVALID_ARG, "workspace is NULL");
    if (ws && !aligned(ws, kAlign)) return fail(WL_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    return WL_OK;
}

// y must not overlap x, the workspace or any theta tensor.
wl_status check_overlap(Range y, const Range *in, int n) {
    for (int j = 0; j < n; ++j)
        if (overlaps(y, in[j])) return fail(WL_ERR_INVALID_ARG, "output overlaps an input or the workspace");
    return WL_OK;
}

}  // namespace

extern "C" {

int32_t wl_abi_version(void) { return WL_ABI_VERSION; }

size_t wl_sync_bytes(void) { return wl::kSyncBytes; }

wl_status wl_workspace_init(void *ws, size_t ws_bytes, void *hip_stream) {
    if (!ws) return fail(WL_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(ws, kAlign)) return fail(WL_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < wl::kSyncBytes)
        return fail(WL_ERR_WORKSPACE, "workspace of %zu bytes is below the sync area's %zu", ws_bytes,
                    (size_t)wl::kSyncBytes);
    const hipError_t e = wl::launch_sync_clear(static_cast<unsigned long long *>(ws), wl::kSyncBytes / 8,
                                               static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(WL_ERR_HIP, "workspace init launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char *wl_status_str(wl_status st) {
    switch (st) {
        case WL_OK: return "ok";
        case WL_ERR_INVALID_ARG: return "invalid argument";
        case WL_ERR_UNSUPPORTED: return "unsupported";
        case WL_ERR_HIP: return "HIP error";
        case WL_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char *wl_last_error(void) { return g_error.c_str(); }

int32_t wl_set_regime(int32_t regime) {
    if (regime < 0 || regime > 6) return -1;
    return g_regime.exchange(regime);
}

int32_t wl_set_spin_limit(int32_t polls) {
    if (polls < 0) return -1;
    return g_spin_limit.exchange(polls);
}

size_t wl_workspace_bytes(int32_t op, const wl_theta *const *th, int32_t n_th, int32_t T) {
    if (!th || T < 0) return 0;
    if (op == WL_OP_LINEAR) {
        if (n_th != 1 || check_theta(th[0], "theta") != WL_OK) return 0;
    } else if (op == WL_OP_QKV || op == WL_OP_MLP) {
        if (n_th != 3) return 0;
        for (int c = 0; c < 3; ++c)
            if (check_theta(th[c], "theta") != WL_OK) return 0;
    } else {
        return 0;
    }
    return layout(op, th, T).total;
}

wl_status wl_linear(const wl_theta *th, const void *x, void *y, int32_t T, void *ws, size_t ws_bytes,
                    void *hip_stream) {
    wl_status st = check_theta(th, "theta");
    if (st != WL_OK) return st;
    if ((st = check_io(x, y, T, th->d_in, th->d_out)) != WL_OK) return st;
    if (T == 0) return ok();
    const wl_theta *ths[1] = {th};
    const Layout L = layout(WL_OP_LINEAR, ths, T);
    if ((st = check_ws(L.total, ws, ws_bytes)) != WL_OK) return st;
    const size_t es = elem_bytes(th);
    Range in[6];
    theta_ranges(th, in);
    in[4] = {x, (size_t)T * th->d_in * es};
    in[5] = {ws, ws_bytes};
    if ((st = check_overlap({y, (size_t)T * th->d_out * es}, in, 6)) != WL_OK) return st;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char *w = static_cast<char *>(ws);
    if (th->dtype == WL_DTYPE_F32) {
        if ((st = run_proj_f32(ths, 1, false, th->d_in, T, x, y, th->d_out, w, L, stream)) != WL_OK) return st;
        return ok();
    }
    const wl::Child ch = make_child(th, 0);
    if ((st = run_proj(&ch, 1, false, th->d_in, T, x, y, th->d_out, w, L, stream)) != WL_OK) return st;
    return ok();
}

static_assert(WL_STATIC_SCRATCH_BYTES == wl::kStaticScratchBytes, "static scratch size");
static_assert(WL_STATIC_SCRATCH_BYTES >= wl::kSyncBytes, "the static scratch holds the sync area");

wl_status wl_linear_static(const wl_theta *th, const void *x, void *y, int32_t T, void *hip_stream) {
    wl_status st = check_theta(th, "theta");
    if (st != WL_OK) return st;
    if ((st = check_io(x, y, T, th->d_in, th->d_out)) != WL_OK) return st;
    if (T == 0) return ok();
    const wl_theta *ths[1] = {th};
    const size_t need = layout(WL_OP_LINEAR, ths, T).total;
    if (need > wl::kStaticScratchBytes)
        return fail(WL_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the static scratch holds %zu", need,
                    (size_t)wl::kStaticScratchBytes);
    void *ws = nullptr;
    const hipError_t e = wl::static_scratch(static_cast<hipStream_t>(hip_stream), &ws);
    if (e != hipSuccess) return fail(WL_ERR_HIP, "static scratch set-up failed: %s", hipGetErrorString(e));
    return wl_linear(th, x, y, T, ws, wl::kStaticScratchBytes, hip_stream);
}

wl_status wl_qkv_fused(const wl_theta *q, const wl_theta *k, const wl_theta *v, const void *x, void *y_qkv,
                       int32_t T, void *ws, size_t ws_bytes, void *hip_stream) {
    const wl_theta *ths[3] = {q, k, v};
    const char *names[3] = {"q", "k", "v"};
    wl_status st;
    for (int c = 0; c < 3; ++c)
        if ((st = check_theta(ths[c], names[c])) != WL_OK) return st;
    if ((st = check_same_dtype(ths, 3, "qkv")) != WL_OK) return st;
    if (k->d_in != q->d_in || v->d_in != q->d_in)
        return fail(WL_ERR_INVALID_ARG, "q, k, v must share d_in (%d, %d, %d)", q->d_in, k->d_in, v->d_in);
    const int64_t width = (int64_t)q->d_out + k->d_out + v->d_out;
    if (width >= kMaxElems) return fail(WL_ERR_INVALID_ARG, "q, k, v outputs are too wide");
    if ((st = check_io(x, y_qkv, T, q->d_in, (int)width)) != WL_OK) return st;
    if (T == 0) return ok();
    const Layout L = layout(WL_OP_QKV, ths, T);
    if ((st = check_ws(L.total, ws, ws_bytes)) != WL_OK) return st;
    const size_t es = elem_bytes(q);
    Range in[14];
    for (int c = 0; c < 3; ++c) theta_ranges(ths[c], in + 4 * c);
    in[12] = {x, (size_t)T * q->d_in * es};
    in[13] = {ws, ws_bytes};
    if ((st = check_overlap({y_qkv, (size_t)T * width * es}, in, 14)) != WL_OK) return st;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char *w = static_cast<char *>(ws);
    if (q->dtype == WL_DTYPE_F32) {
        if ((st = run_proj_f32(ths, 3, false, q->d_in, T, x, y_qkv, (int)width, w, L, stream)) != WL_OK) return st;
        return ok();
    }
    wl::Child ch[3];
    int col0 = 0;
    for (int c = 0; c < 3; ++c) {
        ch[c] = make_child(ths[c], col0);
        col0 += ths[c]->d_out;
    }
    if ((st = run_proj(ch, 3, false, q->d_in, T, x, y_qkv, (int)width, w, L, stream)) != WL_OK) return st;
    return ok();
}

wl_status wl_mlp_fused(const wl_theta *gate, const wl_theta *up, const wl_theta *down, const void *x, void *y,
                       int32_t T, void *ws, size_t ws_bytes, void *hip_stream) {
    const wl_theta *ths[3] = {gate, up, down};
    const char *names[3] = {"gate", "up", "down"};
    wl_status st;
    for (int c = 0; c < 3; ++c)
        if ((st = check_theta(ths[c], names[c])) != WL_OK) return st;
    if ((st = check_same_dtype(ths, 3, "mlp")) != WL_OK) return st;
    if (up->d_in != gate->d_in || up->d_out != gate->d_out || down->d_in != gate->d_out)
        return fail(WL_ERR_INVALID_ARG,
                    "MLP shapes disagree: gate %dx%d, up %dx%d, down %dx%d (need gate == up, down.d_in == d_ff)",
                    gate->d_out, gate->d_in, up->d_out, up->d_in, down->d_out, down->d_in);
    if ((st = check_io(x, y, T, gate->d_in, down->d_out)) != WL_OK) return st;
    if ((int64_t)T * gate->d_out >= kMaxElems) return fail(WL_ERR_INVALID_ARG, "h has 2^31 or more elements");
    if (T == 0) return ok();
    const Layout L = layout(WL_OP_MLP, ths, T);
    if ((st = check_ws(L.total, ws, ws_bytes)) != WL_OK) return st;
    const size_t es = elem_bytes(gate);
    Range in[14];
    for (int c = 0; c < 3; ++c) theta_ranges(ths[c], in + 4 * c);
    in[12] = {x, (size_t)T * gate->d_in * es};
    in[13] = {ws, ws_bytes};
    if ((st = check_overlap({y, (size_t)T * down->d_out * es}, in, 14)) != WL_OK) return st;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char *w = static_cast<char *>(ws);
    void *h = w + L.h;
    const int d_ff = gate->d_out;
    if (gate->dtype == WL_DTYPE_F32) {
        // gate/up -> h = gelu_tanh(g) * u (fp32), then down over h
        if ((st = run_proj_f32(ths, 2, true, gate->d_in, T, x, h, d_ff, w, L, stream)) != WL_OK) return st;
        if ((st = run_proj_f32(ths + 2, 1, false, d_ff, T, h, y, down->d_out, w, L, stream)) != WL_OK) return st;
        return ok();
    }
    const wl::Child gu[2] = {make_child(gate, 0), make_child(up, 0)};
    const int regime = g_regime.load(std::memory_order_relaxed);
    if (regime == 0 || regime == 1) {
        const wl::MlpPlan plan =
            wl::mlp_dec_plan(gate->d_in, d_ff, down->d_out, gate->r, up->r, down->r, T);
        // Passes of four tokens run faster as two launches (the one-launch
        // kernel holds too many registers there); regime 1 still forces it.
        if (plan.tt > 0 && (regime == 1 || plan.tt <= wl::kMlpAutoMaxTok)) {
            // One launch per pass: gate/up, GELU-tanh and down together.
            if (log_on())
                fprintf(stderr, "wl: mlp d_model=%d d_ff=%d d_out=%d T=%d -> one launch (tt=%d, slices=%d x %d)\n",
                        gate->d_in, d_ff, down->d_out, T, plan.tt, plan.NS, plan.P);
            wl::MlpDec a{};
            wl::GemvF &g = a.gu;
            g.ch[0] = gu[0];
            g.ch[1] = gu[1];
            g.n_ch = 2;
            g.pair = 1;
            g.d_in = gate->d_in;
            g.rows = d_ff;
            g.ldy = d_ff;
            g.T = T;
            g.x = static_cast<const uint16_t *>(x);
            g.tagged = reinterpret_cast<unsigned long long *>(w + wl::kSyncTaggedOffset);
            g.sync = reinterpret_cast<unsigned long long *>(w);
            g.fin = reinterpret_cast<unsigned long long *>(w + wl::kSyncFinalOffset);
            g.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
            a.W0d = static_cast<const uint16_t *>(down->W0);
            a.Ud = static_cast<const uint16_t *>(down->U);
            a.Vd = static_cast<const uint16_t *>(down->V);
            a.sd = down->s;
            a.rd = down->r;
            a.D = down->d_out;
            a.F = d_ff;
            a.y = static_cast<uint16_t *>(y);
            a.hx = reinterpret_cast<unsigned long long *>(w + wl::kSyncHxOffset);
            a.part = reinterpret_cast<unsigned long long *>(w + wl::kSyncPartOffset);
            for (int t0 = 0; t0 < T; t0 += plan.tt) {
                g.t0 = t0;
                const hipError_t e = wl::launch_mlp_dec(a, plan, stream);
                if (e != hipSuccess) return fail(WL_ERR_HIP, "MLP launch failed: %s", hipGetErrorString(e));
            }
            return ok();
        }
    }
    // gate/up -> h = bf16(gelu_tanh(g) * u), then down over h
    if ((st = run_proj(gu, 2, true, gate->d_in, T, x, h, d_ff, w, L, stream)) != WL_OK) return st;
    const wl::Child dc = make_child(down, 0);
    if ((st = run_proj(&dc, 1, false, d_ff, T, h, y, down->d_out, w, L, stream)) != WL_OK) return st;
    return ok();
}

wl_status wl_materialize_weff(const wl_theta *th, void *W_eff, void *hip_stream) {
    wl_status st = check_theta(th, "theta");
    if (st != WL_OK) return st;
    if (!W_eff) return fail(WL_ERR_INVALID_ARG, "W_eff is NULL");
    if (!aligned(W_eff, 16)) return fail(WL_ERR_INVALID_ARG, "W_eff is not 16-byte aligned");
    Range in[4];
    theta_ranges(th, in);
    if ((st = check_overlap({W_eff, (size_t)th->d_out * th->d_in * elem_bytes(th)}, in, 4)) != WL_OK) return st;
    if (th->dtype == WL_DTYPE_F32) {
        wl::WeffF32 w{};
        w.W0 = static_cast<const float *>(th->W0);
        w.s = th->s;
        w.U = static_cast<const float *>(th->U);
        w.V = static_cast<const float *>(th->V);
        w.W_eff = static_cast<float *>(W_eff);
        w.d_in = th->d_in;
        w.d_out = th->d_out;
        w.r = th->r;
        const hipError_t e = wl::launch_weff_f32(w, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return fail(WL_ERR_HIP, "materialize launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    wl::Weff w{};
    w.W0 = static_cast<const uint16_t *>(th->W0);
    w.s = th->s;
    w.U = static_cast<const uint16_t *>(th->U);
    w.V = static_cast<const uint16_t *>(th->V);
    w.W_eff = static_cast<uint16_t *>(W_eff);
    w.d_in = th->d_in;
    w.d_out = th->d_out;
    w.r = th->r;
    const hipError_t e = wl::launch_weff(w, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(WL_ERR_HIP, "materialize launch failed: %s", hipGetErrorString(e));
    return ok();
}

wl_status wl_materialize_weff_batch(const wl_theta *const *th, void *const *W_eff, int32_t n, void *hip_stream) {
    if (n < 0) return fail(WL_ERR_INVALID_ARG, "n=%d is negative", n);
    if (n == 0) return ok();
    if (!th || !W_eff) return fail(WL_ERR_INVALID_ARG, "th or W_eff is NULL");
    // Every argument is checked before anything is launched.
    for (int32_t j = 0; j < n; ++j) {
        char name[32];
        snprintf(name, sizeof name, "theta %d", j);
        wl_status st = check_theta(th[j], name);
        if (st != WL_OK) return st;
        if (th[j]->dtype != th[0]->dtype)
            return fail(WL_ERR_INVALID_ARG, "thetas 0 and %d differ in dtype", j);
        if (!W_eff[j]) return fail(WL_ERR_INVALID_ARG, "W_eff %d is NULL", j);
        if (!aligned(W_eff[j], 16)) return fail(WL_ERR_INVALID_ARG, "W_eff %d is not 16-byte aligned", j);
    }
    for (int32_t j = 0; j < n; ++j) {
        const Range out{W_eff[j], (size_t)th[j]->d_out * th[j]->d_in * elem_bytes(th[j])};
        for (int32_t i = 0; i < n; ++i) {
            Range in[4];
            theta_ranges(th[i], in);
            for (int q = 0; q < 4; ++q)
                if (overlaps(out, in[q])) return fail(WL_ERR_INVALID_ARG, "W_eff %d overlaps an input of theta %d", j, i);
            if (i != j && overlaps(out, {W_eff[i], (size_t)th[i]->d_out * th[i]->d_in * elem_bytes(th[i])}))
                return fail(WL_ERR_INVALID_ARG, "W_eff %d and %d overlap", j, i);
        }
    }
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (th[0]->dtype == WL_DTYPE_F32) {
        // The fp32 variant has no batched kernel: one launch per projection.
        for (int32_t j = 0; j < n; ++j) {
            const wl_status st = wl_materialize_weff(th[j], W_eff[j], hip_stream);
            if (st != WL_OK) return st;
        }
        return ok();
    }
    for (int32_t j0 = 0; j0 < n; j0 += wl::kWeffBatchMax) {
        wl::WeffBatch bt{};
        int tiles = 0;
        for (int32_t j = j0; j < n && j < j0 + wl::kWeffBatchMax; ++j) {
            wl::Weff &w = bt.w[bt.n];
            w.W0 = static_cast<const uint16_t *>(th[j]->W0);
            w.s = th[j]->s;
            w.U = static_cast<const uint16_t *>(th[j]->U);
            w.V = static_cast<const uint16_t *>(th[j]->V);
            w.W_eff = static_cast<uint16_t *>(W_eff[j]);
            w.d_in = th[j]->d_in;
            w.d_out = th[j]->d_out;
            w.r = th[j]->r;
            tiles += wl::weff_tiles(w.d_in, w.d_out);
            bt.tiles_end[bt.n++] = tiles;
        }
        const hipError_t e = wl::launch_weff_batch(bt, stream);
        if (e != hipSuccess) return fail(WL_ERR_HIP, "materialize launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

wl_status wl_bundle_size(const wl_theta *const *th, int32_t n_th, size_t *bundle_bytes, size_t *dense_bytes) {
    if (!th || n_th < 1) return fail(WL_ERR_INVALID_ARG, "no thetas");
    if (!bundle_bytes || !dense_bytes) return fail(WL_ERR_INVALID_ARG, "bundle_bytes or dense_bytes is NULL");
    size_t bundle = 0, dense = 0;
    for (int32_t j = 0; j < n_th; ++j) {
        const wl_theta *t = th[j];
        char name[32];
        snprintf(name, sizeof name, "theta %d", j);
        const wl_status st = check_theta(t, name);
        if (st != WL_OK) return st;
        bool seen = false;
        for (int32_t i = 0; i < j; ++i)
            if (th[i]->W0 == t->W0) {
                if (th[i]->d_in != t->d_in || th[i]->d_out != t->d_out || th[i]->dtype != t->dtype)
                    return fail(WL_ERR_INVALID_ARG, "thetas %d and %d share W0 but not its shape or dtype", i, j);
                seen = true;
                break;
            }
        const size_t es = elem_bytes(t);
        const size_t w0 = es * t->d_out * t->d_in;
        if (!seen) bundle += w0;
        bundle += (t->s ? (size_t)4 * t->d_out : 0) + es * t->r * ((size_t)t->d_out + t->d_in);
        dense += w0;
    }
    *bundle_bytes = bundle;
    *dense_bytes = dense;
    return ok();
}

size_t wl_rel_frob_workspace_bytes(int64_t n) {
    if (n < 1) return 0;
    return round_up((size_t)wl::frob_workgroups(n) * 2 * sizeof(double), kAlign);
}

wl_status wl_relative_frobenius_error(const void *W, const void *R, int64_t n, double *result, void *ws,
                                      size_t ws_bytes, void *hip_stream) {
    if (n < 1 || n >= ((int64_t)1 << 40)) return fail(WL_ERR_INVALID_ARG, "n=%lld is out of range", (long long)n);
    if (!W || !R || !result || !ws) return fail(WL_ERR_INVALID_ARG, "W, R, result or ws is NULL");
    if (!aligned(W, 16) || !aligned(R, 16)) return fail(WL_ERR_INVALID_ARG, "W or R is not 16-byte aligned");
    if (!aligned(result, 8)) return fail(WL_ERR_INVALID_ARG, "result is not 8-byte aligned");
    if (!aligned(ws, kAlign)) return fail(WL_ERR_INVALID_ARG, "the workspace is not 256-byte aligned");
    const size_t need = wl_rel_frob_workspace_bytes(n);
    if (ws_bytes < need) return fail(WL_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    const size_t mb = (size_t)n * 2;
    const Range wr{W, mb}, rr{R, mb};
    if (overlaps({result, sizeof(double)}, wr) || overlaps({result, sizeof(double)}, rr) ||
        overlaps({ws, need}, wr) || overlaps({ws, need}, rr) || overlaps({ws, need}, {result, sizeof(double)}))
        return fail(WL_ERR_INVALID_ARG, "result or workspace overlaps an input");
    wl::FrobJob job{};
    job.W = static_cast<const uint16_t *>(W);
    job.R = static_cast<const uint16_t *>(R);
    job.n = n;
    job.part = static_cast<double *>(ws);
    job.n_wg = wl::frob_workgroups(n);
    job.out = result;
    const hipError_t e = wl::launch_frob(job, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(WL_ERR_HIP, "relative Frobenius error launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode steps: a fixed list of projection calls recorded once into a HIP graph
// ("Throughput" page, "Versus vanilla MAX": at batch 1 the extra dispatches,
// not the arithmetic, dominate), launched with one call.

struct wl_step_s {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

constexpr int kMaxStepCalls = 1 << 16;

int step_thetas(int32_t op) { return op == WL_OP_LINEAR ? 1 : 3; }

// x and y of a call whose thetas passed check_theta.
void call_ranges(const wl_call &c, Range &x, Range &y) {
    const size_t es = elem_bytes(c.th[0]);
    size_t width = 0;
    if (c.op == WL_OP_QKV)
        width = (size_t)c.th[0]->d_out + c.th[1]->d_out + c.th[2]->d_out;
    else if (c.op == WL_OP_MLP)
        width = (size_t)c.th[2]->d_out;
    else
        width = (size_t)c.th[0]->d_out;
    x = {c.x, (size_t)(c.T > 0 ? c.T : 0) * c.th[0]->d_in * es};
    y = {c.y, (size_t)(c.T > 0 ? c.T : 0) * width * es};
}

wl_status run_call(const wl_call &c, void *ws, size_t ws_bytes, hipStream_t s) {
    switch (c.op) {
        case WL_OP_LINEAR: return wl_linear(c.th[0], c.x, c.y, c.T, ws, ws_bytes, s);
        case WL_OP_QKV: return wl_qkv_fused(c.th[0], c.th[1], c.th[2], c.x, c.y, c.T, ws, ws_bytes, s);
        default: return wl_mlp_fused(c.th[0], c.th[1], c.th[2], c.x, c.y, c.T, ws, ws_bytes, s);
    }
}

// The calls' own checks that need no launch: op, thetas, a workspace size.
wl_status check_calls(const wl_call *calls, int32_t n_calls) {
    if (!calls) return fail(WL_ERR_INVALID_ARG, "calls is NULL");
    if (n_calls <= 0 || n_calls > kMaxStepCalls)
        return fail(WL_ERR_INVALID_ARG, "n_calls=%d is outside [1, %d]", n_calls, kMaxStepCalls);
    for (int i = 0; i < n_calls; ++i) {
        const wl_call &c = calls[i];
        if (c.op != WL_OP_LINEAR && c.op != WL_OP_QKV && c.op != WL_OP_MLP)
            return fail(WL_ERR_INVALID_ARG, "call %d: op=%d is not WL_OP_LINEAR, WL_OP_QKV or WL_OP_MLP", i, c.op);
        for (int j = 0; j < step_thetas(c.op); ++j) {
            char name[32];
            snprintf(name, sizeof name, "call %d theta %d", i, j);
            const wl_status st = check_theta(c.th[j], name);
            if (st != WL_OK) return st;
        }
        if (c.T < 0) return fail(WL_ERR_INVALID_ARG, "call %d: T=%d is negative", i, c.T);
        if (wl_workspace_bytes(c.op, c.th, step_thetas(c.op), c.T) == 0)
            return fail(WL_ERR_INVALID_ARG, "call %d: invalid thetas for the op", i);
    }
    return WL_OK;
}

}  // namespace

size_t wl_step_workspace_bytes(const wl_call *calls, int32_t n_calls) {
    if (!calls || n_calls <= 0 || n_calls > kMaxStepCalls) return 0;
    size_t need = 0;
    for (int i = 0; i < n_calls; ++i) {
        const wl_call &c = calls[i];
        if (c.op != WL_OP_LINEAR && c.op != WL_OP_QKV && c.op != WL_OP_MLP) return 0;
        const size_t b = wl_workspace_bytes(c.op, c.th, step_thetas(c.op), c.T);
        if (b == 0) return 0;
        need = b > need ? b : need;
    }
    return need;
}

wl_status wl_step_create(const wl_call *calls, int32_t n_calls, int32_t flags, void *ws, size_t ws_bytes,
                         wl_step *step) {
    if (!step) return fail(WL_ERR_INVALID_ARG, "step is NULL");
    *step = nullptr;
    wl_status st = check_calls(calls, n_calls);
    if (st != WL_OK) return st;
    if (flags & ~WL_STEP_GROUP_SHARED_W0) return fail(WL_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    if ((st = check_ws(wl_step_workspace_bytes(calls, n_calls), ws, ws_bytes)) != WL_OK) return st;

    // Launch order: as given, or (WL_STEP_GROUP_SHARED_W0) the calls that share
    // their first theta's W0 back to back, groups in order of first appearance,
    // calls in their given order within a group. Reordering needs calls that do
    // not read or overwrite one another's outputs.
    std::vector<int> order(n_calls);
    for (int i = 0; i < n_calls; ++i) order[i] = i;
    if (flags & WL_STEP_GROUP_SHARED_W0) {
        for (int i = 0; i < n_calls; ++i) {
            Range xi, yi;
            call_ranges(calls[i], xi, yi);
            for (int j = 0; j < n_calls; ++j) {
                Range xj, yj;
                call_ranges(calls[j], xj, yj);
                if (overlaps(yi, xj))
                    return fail(WL_ERR_INVALID_ARG, "call %d reads the output of call %d: the calls cannot be "
                                "regrouped (WL_STEP_GROUP_SHARED_W0)", j, i);
                if (j != i && overlaps(yi, yj))
                    return fail(WL_ERR_INVALID_ARG, "calls %d and %d write overlapping outputs: the calls cannot be "
                                "regrouped (WL_STEP_GROUP_SHARED_W0)", i, j);
            }
        }
        std::vector<int> grouped;
        std::vector<bool> taken(n_calls, false);
        for (int i = 0; i < n_calls; ++i) {
            if (taken[i]) continue;
            for (int j = i; j < n_calls; ++j)
                if (!taken[j] && calls[j].th[0]->W0 == calls[i].th[0]->W0) {
                    grouped.push_back(j);
                    taken[j] = true;
                }
        }
        order = grouped;
    }

    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(WL_ERR_HIP, "capture stream: %s", hipGetErrorString(e));
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return fail(WL_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
    }
    for (int k : order) {
        st = run_call(calls[k], ws, ws_bytes, cs);
        if (st != WL_OK) {
            const std::string msg = "call " + std::to_string(k) + ": " + g_error;
            hipGraph_t g = nullptr;
            (void)hipStreamEndCapture(cs, &g);
            if (g) (void)hipGraphDestroy(g);
            (void)hipStreamDestroy(cs);
            return fail(st, "%s", msg.c_str());
        }
    }
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    (void)hipStreamDestroy(cs);
    if (e != hipSuccess || !graph) return fail(WL_ERR_HIP, "end capture: %s", hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return fail(WL_ERR_HIP, "graph instantiation: %s", hipGetErrorString(e));
    }
    *step = new wl_step_s{graph, exec};
    return ok();
}

wl_status wl_step_launch(wl_step step, void *hip_stream) {
    if (!step) return fail(WL_ERR_INVALID_ARG, "step is NULL");
    const hipError_t e = hipGraphLaunch(step->exec, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(WL_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
    return ok();
}

wl_status wl_step_destroy(wl_step step) {
    if (!step) return ok();
    if (step->exec) (void)hipGraphExecDestroy(step->exec);
    if (step->graph) (void)hipGraphDestroy(step->graph);
    delete step;
    return ok();
}
