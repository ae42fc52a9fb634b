// Matrix-core path for larger token counts (prefill-sized calls), one launch.
//
//   m[t,o]   = sum_i x[t,i] W0[o,i]                 bf16 x bf16 -> fp32 on MFMA
//   vtx[t,k] = sum_i x[t,i] V[i,k]                  computed before, split partials
//   y[t,o]   = bf16( s[o] * m[t,o] + sum_k vtx[t,k] U[o,k] )
//
// ("In-kernel reconstruction", introduction: the reconstruction formula and its
// per-element expansion; s scales the W0 product, the rank-r term is added
// unscaled.)
//
// Operands. x[T][d_in] and W0[d_out][d_in] are contiguous along the input axis,
// so their tiles go to LDS as 16-byte pieces without any transpose. A
// workgroup of WM x WN waves owns a BM x BN output tile (tokens x outputs);
// each wave owns TM x TN 32x32 blocks, each the accumulator of one
// v_mfma_f32_32x32x16_bf16 chain. The input axis is walked BK at a time through
// a ring of D LDS stages filled by direct-to-LDS loads (global_load_lds, 16
// bytes per lane, no registers), D-1 stages in flight while one is multiplied,
// one barrier per step.
// LDS rows of BK bf16 keep their 16-byte pieces XOR-swizzled by the row index
// so that the fragment reads are free of bank conflicts.
//
// V^T x is not computed here: a small matrix-core launch before this one writes
// it as S split partials over the input axis (fp32 [S][T][r] per child), and
// the epilogue adds them in split order, so vtx never depends on scheduling.
// Keeping it out of the main loop leaves every K step to the W0 product.

// Workgroups are numbered so that each of the 8 XCDs (which take workgroups
// round-robin) works through its own contiguous band of output tiles, keeping
// the W0 rows it reads in its own L2.
//
// Epilogue: the accumulators are scaled by s[o] (one output column per lane in
// the 32x32 layout); vtx (its partials summed) is read straight into the
// A-operand layout (8 ranks of one token row per lane), split into a bf16 head and a bf16
// remainder (vtx = hi + lo to about 2^-16 relative) and both are run against U
// on the matrix cores as extra K steps, so the rank term keeps close to fp32
// accuracy. Results are rounded once to bf16. Pair mode (the MLP's gate/up)
// keeps two accumulator sets over the same x tile and writes
// bf16(gelu_tanh(g) * u).
#include "wl_vtxmm.h"

namespace wl {

namespace {

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f_bf16(a) | ((uint32_t)f_bf16(b) << 16);
}
__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
    u32x4 r;
    r.x = pack2(v[0], v[1]);
    r.y = pack2(v[2], v[3]);
    r.z = pack2(v[4], v[5]);
    r.w = pack2(v[6], v[7]);
    return r;
}

template <int WM, int WN, int TM, int TN, int BK, int P, int D, int NV>
struct Cfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    static constexpr int KP = BK / 8;                          // 16-byte pieces per LDS row
    static constexpr int A_PIECES = BM * KP, B_PIECES = BN * KP;
    static constexpr int A_PER = A_PIECES / kThreads, B_PER = B_PIECES / kThreads;
    static constexpr int STAGE_PIECES = A_PIECES + P * B_PIECES;
    static constexpr int PER_STAGE = A_PER + P * B_PER;        // direct-to-LDS loads per thread
    static constexpr int TILE_PIECES = D * STAGE_PIECES;
    static constexpr int LDS_PIECES = TILE_PIECES;
    static_assert(A_PIECES % kThreads == 0 && B_PIECES % kThreads == 0, "tile pieces must split evenly");
    static_assert(D >= 2 && D <= 4 && (D - 1) * PER_STAGE <= 63, "stages in flight must fit vmcnt");
    static_assert(D - 2 <= 2, "wait counts cover at most two stages ahead");
};

// A 16-byte piece of zeros: the source of every out-of-range piece of a
// direct-to-LDS tile load (the load always writes its LDS slot).
__device__ __attribute__((aligned(16))) const uint32_t kZeroPiece[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// PV > 0: the launch also carries g.n_prod V^T x units (32-wide rank blocks
// PV), workgroups after the tiles, which the tiles do not read (the split
// reduction adds the rank term after this launch).
template <int WM, int WN, int TM, int TN, int BK, int P, int D, int NV, int PV = 0>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(Gemm g) {
    using C = Cfg<WM, WN, TM, TN, BK, P, D, NV>;
    constexpr int BM = C::BM, BN = C::BN, KP = C::KP, NT = C::kThreads;
    constexpr int kVtxPieces = PV > 0 ? vtx_unit_lds_bytes<WM * WN, PV>() / 16 : 0;
    __shared__ u32x4 lds[C::LDS_PIECES > kVtxPieces ? C::LDS_PIECES : kVtxPieces];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    // Tile numbering: XCD x (blockIdx % 8) takes a contiguous band of logical tiles.
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + BN - 1) / BN;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + BN - 1) / BN;
    const int n_mt = (g.T + BM - 1) / BM;
    const int tiles = n_nt * n_mt, total = tiles * g.ksplit;
    if constexpr (PV > 0) {
        if ((int)blockIdx.x >= total) {
            const int q = blockIdx.x - total, n_tb = (g.T + 31) / 32;
            vtxmm_unit<WM * WN, PV, 0>(g.job, q % n_tb, (q / n_tb) % g.job.S, q / (n_tb * g.job.S),
                                       reinterpret_cast<unsigned char *>(lds));
            return;
        }
    }
    int tile;
    {
        const int per = (total + 7) / 8, x = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int full = total - 8 * (per - 1);   // XCDs 0..full-1 hold `per` tiles, the rest per-1
        tile = x < full ? x * per + slot : full * per + (x - full) * (per - 1) + slot;
    }
    // Split of the input axis (split slowest, so that an XCD's band mostly shares one).
    const int split = tile / tiles;
    tile -= split * tiles;
    // Within the band: token tiles fastest (consecutive tiles share W0 rows), or
    // output tiles fastest (they share x rows) when x is the larger operand, so
    // that each XCD re-reads the smaller one.
    const int mt = g.col_fast ? tile / n_nt : tile % n_mt;
    const int ntile = g.col_fast ? tile % n_nt : tile / n_mt;
    int cidx = 0, n0 = ntile * BN;
    if (!g.pair) {
        int left = ntile;
        for (; cidx < g.n_ch - 1; ++cidx) {
            const int nt = (g.ch[cidx].d_out + BN - 1) / BN;
            if (left < nt) break;
            left -= nt;
        }
        n0 = left * BN;
    }
    const Child &C0 = g.ch[cidx];
    const int d_out = C0.d_out;
    const int m0 = mt * BM;
    const int d_in = g.d_in, nch = d_in >> 3;
    const int nk_all = (d_in + BK - 1) / BK;
    // This split's steps [kt0, nk) (the split plan counts 64-wide steps; the split tile has BK = 64).
    const int kt0 = g.ksplit > 1 ? split * g.kb_per_split : 0;
    const int nk = g.ksplit > 1 ? min(nk_all, kt0 + g.kb_per_split) : nk_all;

    const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
    const Child *ch[P];
#pragma unroll
    for (int p = 0; p < P; ++p) ch[p] = &g.ch[P == 2 ? p : cidx];

    f32x16 acc[P][TM][TN];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[p][i][j][e] = 0.f;

    // Full steps (the whole 64-wide K block inside d_in) take precomputed per-lane
    // piece offsets: tile rows past T or d_out read the last valid row instead (their
    // outputs are never stored), so no step but a partial last one needs a check.
    int a_off[C::A_PER];
#pragma unroll
    for (int h = 0; h < C::A_PER; ++h) {
        const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row);
        a_off[h] = min(m0 + row, g.T - 1) * nch + kc;
    }
    int b_off[P][C::B_PER];
    const u32x4 *wg[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        wg[p] = reinterpret_cast<const u32x4 *>(ch[p]->W0);
        const int dout_p = ch[p]->d_out;
#pragma unroll
        for (int h = 0; h < C::B_PER; ++h) {
            const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row);
            b_off[p][h] = min(n0 + row, dout_p - 1) * nch + kc;
        }
    }
    // The ring: the 64 lanes of one load write 64 consecutive 16-byte LDS slots,
    // so each lane fetches the global piece that belongs in its (swizzled) slot.
    // This is the checked form for a partial last step; it reads only values
    // already in registers (a kernel-argument load inside the loop would make
    // every LDS wait a full drain).
    const u32x4 *zero = reinterpret_cast<const u32x4 *>(kZeroPiece);
    int dout_of[P];
#pragma unroll
    for (int p = 0; p < P; ++p) dout_of[p] = ch[p]->d_out;
    auto issue = [&](int kt, int sl) {
        u32x4 *st = lds + sl * C::STAGE_PIECES;
#pragma unroll
        for (int h = 0; h < C::A_PER; ++h) {
            const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row), gk = kt * KP + kc;
            const u32x4 *src = (gk < nch && m0 + row < g.T) ? xg + (size_t)(m0 + row) * nch + gk : zero;
            lds_dma16(src, st + h * NT + wave * kWave);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            u32x4 *bst = st + C::A_PIECES + p * C::B_PIECES;
#pragma unroll
            for (int h = 0; h < C::B_PER; ++h) {
                const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row), gk = kt * KP + kc;
                const u32x4 *src = (gk < nch && n0 + row < dout_of[p]) ? wg[p] + (size_t)(n0 + row) * nch + gk : zero;
                lds_dma16(src, bst + h * NT + wave * kWave);
            }
        }
    };
    auto issue_full = [&](int kt, int sl) {
        u32x4 *st = lds + sl * C::STAGE_PIECES;
        const u32x4 *xk = xg + kt * KP;
#pragma unroll
        for (int h = 0; h < C::A_PER; ++h) lds_dma16(xk + a_off[h], st + h * NT + wave * kWave);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            u32x4 *bst = st + C::A_PIECES + p * C::B_PIECES;
            const u32x4 *wk = wg[p] + kt * KP;
#pragma unroll
            for (int h = 0; h < C::B_PER; ++h) lds_dma16(wk + b_off[p][h], bst + h * NT + wave * kWave);
        }
    };
    auto issue_any = [&](int kt, int sl) {
        if ((kt + 1) * BK <= d_in)
            issue_full(kt, sl);
        else
            issue(kt, sl);
    };


    const int fr = lane & 31, fk = lane >> 5;   // fragment row / column, K half of a 16-step
    // Fragments of 16-wide step s of a stage; the next step's fragments are read
    // while the current step's products run (two register sets).
    auto load_frags = [&](const u32x4 *st, int s, u32x4 (&a)[TM], u32x4 (&b)[P][TN]) {
        const int kc = 2 * s + fk;
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = st[swz<KP>(wm * TM * 32 + i * 32 + fr, kc)];
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[p][j] = st[C::A_PIECES + p * C::B_PIECES + swz<KP>(wn * TN * 32 + j * 32 + fr, kc)];
    };
    auto step_mfma = [&](const u32x4 *st, int s, const u32x4 (&a)[TM], const u32x4 (&b)[P][TN]) {
        // Diagonal order: every fragment is used early and late in the step, so all
        // of them stay in registers of their own (and the next step's reads can be
        // issued before this step's products) instead of sharing one register set.
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int d = 0; d < TN; ++d)
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int j = (i + d) % TN;
                    acc[p][i][j] = mfma(a[i], b[p][j], acc[p][i][j]);
                }
    };
    static_assert((BK / 16) % 2 == 0, "steps are taken in pairs");
    auto compute = [&](const u32x4 *st) {
        u32x4 a0[TM], b0[P][TN], a1[TM], b1[P][TN];
        load_frags(st, 0, a0, b0);
#pragma unroll
        for (int s = 0; s < BK / 16; s += 2) {
            load_frags(st, s + 1, a1, b1);
            step_mfma(st, s, a0, b0);
            if (s + 2 < BK / 16) load_frags(st, s + 2, a0, b0);
            step_mfma(st, s + 1, a1, b1);
        }
    };

    // One barrier per step: after it, stage kt has landed for every wave and every
    // wave has finished step kt - 1, so that step's slot takes stage kt + D - 1.
    // Ring slots count from the split's first step.
    for (int s0 = 0; s0 < D - 1 && kt0 + s0 < nk; ++s0) issue_any(kt0 + s0, s0);
    for (int kt = kt0; kt < nk; ++kt) {
        // This wave's loads of stage kt are done; up to D - 2 later stages stay in flight.
        const int ahead = min(D - 2, nk - 1 - kt);
        if (ahead >= 2) wait_vm<2 * C::PER_STAGE>();
        else if (ahead == 1) wait_vm<C::PER_STAGE>();
        else wait_vm<0>();
        barrier();
        if (kt + D - 1 < nk) issue_any(kt + D - 1, (kt - kt0 + D - 1) % D);
        compute(lds + ((kt - kt0) % D) * C::STAGE_PIECES);
    }

    // ---- epilogue ----
    // Lane (fr, fk) of block (i, j) holds output column o = n0 + (wn*TN + j)*32 + fr
    // and token rows m0 + (wm*TM + i)*32 + 8*(e/4) + 4*fk + (e%4), e = 0..15.
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const Child &Cp = *ch[p];
        // The loads of this child's epilogue are issued before their first use
        // (s of the lane's outputs, then per batch of two 16-wide rank steps
        // the V^T x rows of its tokens and the U pieces of its outputs), as
        // straight-line code with clamped addresses and masks applied
        // afterwards, so the epilogue waits once per batch instead of once per
        // load.
        float sv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int o = n0 + (wn * TN + j) * 32 + fr;
            const float *sp = Cp.s ? Cp.s + min(o, d_out - 1) : reinterpret_cast<const float *>(Cp.W0);
            const float v = ldg(sp);
            sv[j] = Cp.s ? v : 1.0f;
        }
        const int r = Cp.r;
        // The rank term is added once: by split 0 when the input axis is split.
        auto scale = [&]() {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[p][i][j] *= sv[j];
        };
        if constexpr (NV > 0) {
            if (split == 0 && r > 0) {
                const int S = Cp.vtx_splits;
                const size_t ss = (size_t)g.T * r;        // split stride of the partials
                // Batches of two 16-wide rank steps (one batch holds r <= 32, NV = 1).
#pragma unroll
                for (int b = 0; b < NV; ++b) {
                    if (b > 0 && 32 * b >= r) break;
                    f32x4 va[2][TM][2];   // vtx[t][kb .. kb + 8) per step and token block, masked
                    u32x4 ub[2][TN];      // U[o][kb .. kb + 8) per step and output block, masked
                    if ((r & 3) == 0) {
                        // Split 0 of every step's V^T x rows, and the U pieces: every
                        // address clamped into the tensors, the masks applied after
                        // the other splits are added in split order.
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq) {
                            const int kb = 32 * b + 16 * kq + 8 * fk;
#pragma unroll
                            for (int i = 0; i < TM; ++i) {
                                const int t = m0 + (wm * TM + i) * 32 + fr;
                                const float *src = Cp.vtx + (size_t)min(t, g.T - 1) * r;
                                va[kq][i][0] = ldg(reinterpret_cast<const f32x4 *>(src + min(kb, r - 4)));
                                va[kq][i][1] = ldg(reinterpret_cast<const f32x4 *>(src + min(kb + 4, r - 4)));
                            }
#pragma unroll
                            for (int j = 0; j < TN; ++j) {
                                const int o = n0 + (wn * TN + j) * 32 + fr;
                                const uint16_t *urow = Cp.U + (size_t)min(o, d_out - 1) * r;
                                if ((r & 7) == 0) {
                                    ub[kq][j] = ldg(reinterpret_cast<const u32x4 *>(urow + min(kb, r - 8)));
                                } else {
                                    // rows 8-byte aligned only: four words of two entries each
                                    const uint32_t *uw = reinterpret_cast<const uint32_t *>(urow);
                                    const int w0 = kb / 2, wl = r / 2 - 1;
                                    ub[kq][j] = u32x4{ldg(uw + min(w0, wl)), ldg(uw + min(w0 + 1, wl)),
                                                      ldg(uw + min(w0 + 2, wl)), ldg(uw + min(w0 + 3, wl))};
                                }
                            }
                        }
                        for (int q = 1; q < S; ++q) {
#pragma unroll
                            for (int kq = 0; kq < 2; ++kq) {
                                const int kb = 32 * b + 16 * kq + 8 * fk;
#pragma unroll
                                for (int i = 0; i < TM; ++i) {
                                    const int t = m0 + (wm * TM + i) * 32 + fr;
                                    const float *src = Cp.vtx + q * ss + (size_t)min(t, g.T - 1) * r;
                                    va[kq][i][0] += ldg(reinterpret_cast<const f32x4 *>(src + min(kb, r - 4)));
                                    va[kq][i][1] += ldg(reinterpret_cast<const f32x4 *>(src + min(kb + 4, r - 4)));
                                }
                            }
                        }
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq) {
                            const int kb = 32 * b + 16 * kq + 8 * fk;
                            const f32x4 z{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int i = 0; i < TM; ++i) {
                                va[kq][i][0] = kb < r ? va[kq][i][0] : z;
                                va[kq][i][1] = kb + 4 < r ? va[kq][i][1] : z;
                            }
#pragma unroll
                            for (int j = 0; j < TN; ++j) {
                                // entries past d_out or r are zero (r even: a word holds
                                // two entries that are both present or both absent)
                                const bool ok = n0 + (wn * TN + j) * 32 + fr < d_out;
                                const u32x4 u = ub[kq][j];
                                ub[kq][j] = u32x4{ok && kb < r ? u.x : 0u, ok && kb + 2 < r ? u.y : 0u,
                                                  ok && kb + 4 < r ? u.z : 0u, ok && kb + 6 < r ? u.w : 0u};
                            }
                        }
                    } else {
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq) {
                            const int kb = 32 * b + 16 * kq + 8 * fk;
#pragma unroll
                            for (int i = 0; i < TM; ++i) {
                                // vtx[t][kb .. kb+8) for this lane's token row, its split
                                // partials added in split order; values past T or r masked to
                                // zero.
                                const int t = m0 + (wm * TM + i) * 32 + fr;
                                const float *src = Cp.vtx + (size_t)min(t, g.T - 1) * r;
                                float v[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const int kk = min(kb + e, r - 1);
                                    float a = ldg(src + kk);
                                    for (int q = 1; q < S; ++q) a += ldg(src + q * ss + kk);
                                    v[e] = kb + e < r ? a : 0.f;
                                }
                                va[kq][i][0] = f32x4{v[0], v[1], v[2], v[3]};
                                va[kq][i][1] = f32x4{v[4], v[5], v[6], v[7]};
                            }
#pragma unroll
                            for (int j = 0; j < TN; ++j) {
                                const int o = n0 + (wn * TN + j) * 32 + fr;
                                const uint16_t *urow = Cp.U + (size_t)min(o, d_out - 1) * r;
                                uint32_t h[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint32_t bb = ldg(urow + min(kb + e, r - 1));
                                    h[e] = (o < d_out && kb + e < r) ? bb : 0u;
                                }
                                ub[kq][j] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                                  h[6] | (h[7] << 16)};
                            }
                        }
                    }
                    if (b == 0) scale();
                    // vtx = head + remainder, both bf16, run against U on the matrix cores.
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq) {
                        if (32 * b + 16 * kq >= r) break;
                        u32x4 ahi[TM], alo[TM];
#pragma unroll
                        for (int i = 0; i < TM; ++i) {
                            const float v[8] = {va[kq][i][0].x, va[kq][i][0].y, va[kq][i][0].z, va[kq][i][0].w,
                                                va[kq][i][1].x, va[kq][i][1].y, va[kq][i][1].z, va[kq][i][1].w};
                            float hi[8], lo[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                hi[e] = bf16_f(f_bf16(v[e]));
                                lo[e] = v[e] - hi[e];
                            }
                            ahi[i] = pack8(hi);
                            alo[i] = pack8(lo);
                        }
#pragma unroll
                        for (int i = 0; i < TM; ++i)
#pragma unroll
                            for (int j = 0; j < TN; ++j) {
                                acc[p][i][j] = mfma(ahi[i], ub[kq][j], acc[p][i][j]);
                                acc[p][i][j] = mfma(alo[i], ub[kq][j], acc[p][i][j]);
                            }
                    }
                }
            } else {
                scale();
            }
        } else {
            scale();
        }
    }

    if (g.ksplit > 1) {
        // Split partials, fp32 [split][T][d_out] (single child, no pair); the
        // reduction launch adds them in split order and rounds once.
        float *part = g.part + (size_t)split * g.T * d_out;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int o = n0 + (wn * TN + j) * 32 + fr;
            if (o >= d_out) continue;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = m0 + (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
                    if (t < g.T) part[(size_t)t * d_out + o] = acc[0][i][j][e];
                }
        }
        return;
    }
    const int col0 = g.pair ? 0 : C0.col0;
    const size_t ldy = g.ldy;
    auto out_value = [&](int i, int j, int e) {
        return P == 2 ? gelu_tanh_bf16out(acc[0][i][j][e]) * acc[P - 1][i][j][e] : acc[0][i][j][e];
    };
    // Element e of block (i, j) sits 8 (e / 4) + e % 4 rows below the lane's first
    // row of the block: one row pointer per block, row offsets common to all lanes.
    if (m0 + BM <= g.T) {
        // Every token row of the tile is present: no per-element checks.
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int o = n0 + (wn * TN + j) * 32 + fr;
            if (o >= d_out) continue;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                uint16_t *yr = g.y + (size_t)(m0 + (wm * TM + i) * 32 + 4 * fk) * ldy + col0 + o;
#pragma unroll
                for (int e = 0; e < 16; ++e) yr[(8 * (e >> 2) + (e & 3)) * ldy] = f_bf16(out_value(i, j, e));
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int o = n0 + (wn * TN + j) * 32 + fr;
        if (o >= d_out) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int tr = m0 + (wm * TM + i) * 32 + 4 * fk;
            uint16_t *yr = g.y + (size_t)tr * ldy + col0 + o;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int dr = 8 * (e >> 2) + (e & 3);
                if (tr + dr < g.T) yr[dr * ldy] = f_bf16(out_value(i, j, e));
            }
        }
    }
}

template <int WM, int WN, int TM, int TN, int BK, int D, int P, int NV, int PV = 0>
hipError_t launch_cfg(const Gemm &g, hipStream_t stream) {
    using C = Cfg<WM, WN, TM, TN, BK, P, D, NV>;
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + C::BN - 1) / C::BN;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + C::BN - 1) / C::BN;
    const int total = n_nt * ((g.T + C::BM - 1) / C::BM) * g.ksplit + (PV > 0 ? g.n_prod : 0);
    hipLaunchKernelGGL((gemm_kernel<WM, WN, TM, TN, BK, P, D, NV, PV>), dim3(total), dim3(C::kThreads), 0, stream,
                       g);
    return hipGetLastError();
}

// y[t][col0 + o] = bf16( sum over splits q, in order, of part[q][t][o] ); four
// consecutive outputs per thread (8-byte stores when the row offsets allow).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *part, int S, int T, int d_out, uint16_t *y,
                                                           int ldy, int col0) {
    const int nq = (d_out + 3) >> 2;
    const int64_t n = (int64_t)T * nq;
    const size_t ss = (size_t)T * d_out;
    const bool vec = ((d_out | ldy | col0) & 3) == 0;
    for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < n; it += (int64_t)gridDim.x * 256) {
        const int t = (int)(it / nq), o = (int)(it - (int64_t)t * nq) * 4;
        const float *src = part + (size_t)t * d_out + o;
        uint16_t *dst = y + (size_t)t * ldy + col0 + o;
        if (vec) {
            f32x4 a = ldg(reinterpret_cast<const f32x4 *>(src));
            for (int q = 1; q < S; ++q) a += ldg(reinterpret_cast<const f32x4 *>(src + q * ss));
            *reinterpret_cast<u32x2 *>(dst) = u32x2{(uint32_t)f_bf16(a.x) | ((uint32_t)f_bf16(a.y) << 16),
                                                    (uint32_t)f_bf16(a.z) | ((uint32_t)f_bf16(a.w) << 16)};
        } else {
            for (int e = 0; e < 4 && o + e < d_out; ++e) {
                float a = src[e];
                for (int q = 1; q < S; ++q) a += src[q * ss + e];
                dst[e] = f_bf16(a);
            }
        }
    }
}

// The same with the rank term (0 < r <= 32) formed here, from the complete V^T x:
//   y[t][col0 + o] = bf16( sum over splits q, in order, of part[q][t][o]
//                          + sum over k, in increasing order, of U[o][k] vtx[t][k] )
// in fp32, S (2 to kRedMaxSplit) splits. Thread per output o (its U row held in
// registers), kRedTok tokens per workgroup: the workgroup's V^T x rows go to
// LDS once, every load is issued before any is used (addresses clamped into
// the tensors, masks applied afterwards, so no branch stands between them), and
// partials and outputs are read and written in runs across the lanes.
constexpr int kRedTok = 16;
constexpr int kRedMaxSplit = kRedMaxSplits;
static_assert(kRedTok * 32 % 256 == 0, "the V^T x rows of a workgroup fill whole passes of its 256 threads");
template <int S>
__global__ __launch_bounds__(256) void split_reduce_rank_kernel(const float *part, int T, int d_out, uint16_t *y,
                                                                int ldy, int col0, const uint16_t *U,
                                                                const float *vtx, int r) {
    __shared__ __attribute__((aligned(16))) float vl[kRedTok][32];
    const int tid = threadIdx.x;
    const int o = blockIdx.x * 256 + tid;
    const int t0 = blockIdx.y * kRedTok;
    const int oc = min(o, d_out - 1);
    const size_t ss = (size_t)T * d_out;
    float pv[kRedTok][S];
#pragma unroll
    for (int j = 0; j < kRedTok; ++j) {
        const float *src = part + (size_t)min(t0 + j, T - 1) * d_out + oc;
#pragma unroll
        for (int q = 0; q < S; ++q) pv[j][q] = ldg(src + (size_t)q * ss);
    }
    float u[32];
    const uint16_t *ur = U + (size_t)oc * r;
    if ((r & 7) == 0) {
#pragma unroll
        for (int k0 = 0; k0 < 32; k0 += 8) {
            const u32x4 w = ldg(reinterpret_cast<const u32x4 *>(ur + min(k0, r - 8)));
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[k0 + 2 * e] = k0 < r ? bf16_f(ww[e] & 0xFFFFu) : 0.f;
                u[k0 + 2 * e + 1] = k0 < r ? bf16_f(ww[e] >> 16) : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const float v = bf16_f(ldg(ur + min(k, r - 1)));
            u[k] = k < r ? v : 0.f;
        }
    }
    // V^T x rows of the workgroup's tokens (zero past T or r).
#pragma unroll
    for (int m = 0; m < kRedTok * 32 / 256; ++m) {
        const int e = tid + 256 * m, j = e / 32, k = e % 32;
        const float v = ldg(vtx + (size_t)min(t0 + j, T - 1) * r + min(k, r - 1));
        vl[j][k] = (t0 + j < T && k < r) ? v : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRedTok; ++j) {
        float a = pv[j][0];
#pragma unroll
        for (int q = 1; q < S; ++q) a += pv[j][q];
        float rank = 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k) rank = __builtin_fmaf(u[k], vl[j][k], rank);
        if (o < d_out && t0 + j < T) y[(size_t)(t0 + j) * ldy + col0 + o] = f_bf16(a + rank);
    }
}

template <int WM, int WN, int TM, int TN, int BK, int D, int P>
hipError_t launch_nv(const Gemm &g, hipStream_t stream) {
    int max_r = 0;
    for (int c = 0; c < (g.pair ? 2 : g.n_ch); ++c) max_r = g.ch[c].r > max_r ? g.ch[c].r : max_r;
    if (max_r == 0) return launch_cfg<WM, WN, TM, TN, BK, D, P, 0>(g, stream);
    if (max_r <= 32) return launch_cfg<WM, WN, TM, TN, BK, D, P, 1>(g, stream);
    return launch_cfg<WM, WN, TM, TN, BK, D, P, 2>(g, stream);
}

}  // namespace

// Tile configurations (waves M x N, 32x32 blocks per wave M x N, K depth, LDS
// stages), chosen by measurement on the layer shapes; overridable at build time.
// The largest tile whose grid still gives most compute units a workgroup is used.
#ifndef WL_GEMM_TILE_BIG
#define WL_GEMM_TILE_BIG 4, 2, 2, 4, 64, 2
#endif
#ifndef WL_GEMM_TILE_BIG_PAIR
#define WL_GEMM_TILE_BIG_PAIR 4, 2, 2, 2, 64, 2
#endif
#ifndef WL_GEMM_TILE
#define WL_GEMM_TILE 2, 2, 2, 2, 64, 2
#endif
#ifndef WL_GEMM_TILE_PAIR
#define WL_GEMM_TILE_PAIR 2, 2, 2, 2, 64, 2
#endif
#ifndef WL_GEMM_TILE_SMALL
#define WL_GEMM_TILE_SMALL 2, 2, 2, 1, 64, 3
#endif
#ifndef WL_GEMM_TILE_SMALL_PAIR
#define WL_GEMM_TILE_SMALL_PAIR 2, 2, 2, 1, 64, 2
#endif
// Tile of the split-input-axis GEMM (long inputs, few output tiles).
#ifndef WL_GEMM_TILE_SPLIT
#define WL_GEMM_TILE_SPLIT 4, 2, 2, 2, 64, 3
#endif

namespace {

#ifndef WL_GEMM_FILL
#define WL_GEMM_FILL 200
#endif
constexpr int kFillTiles = WL_GEMM_FILL;   // workgroups that count as filling the 256 compute units

template <int WM, int WN, int TM, int TN, int BK, int D>
int tiles_of(const Gemm &g) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + BN - 1) / BN;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + BN - 1) / BN;
    return n_nt * ((g.T + BM - 1) / BM);
}

constexpr int kSplitMinSteps = 24;   // 64-wide input steps per split, at least
constexpr int kComputeUnits = 256;

template <int WM, int WN, int TM, int TN, int BK, int D>
constexpr int tile_bk() { return BK; }
static_assert(tile_bk<WL_GEMM_TILE_SPLIT>() == 64, "the split plan counts 64-wide steps");

}  // namespace

GemmSplit gemm_split_plan(int T, int d_in, int rows, int n_ch, int pair) {
    const int nk = (d_in + 63) / 64;
    GemmSplit p{1, nk};
    if (pair || n_ch != 1 || T <= 0 || rows <= 0) return p;
    Gemm g{};
    g.n_ch = 1;
    g.T = T;
    g.ch[0].d_out = rows;
    // Split only where every unsplit tile choice leaves compute units without work.
    if (tiles_of<WL_GEMM_TILE_BIG>(g) >= kFillTiles || tiles_of<WL_GEMM_TILE>(g) >= kFillTiles) return p;
    const int tiles = tiles_of<WL_GEMM_TILE_SPLIT>(g);
    int S = kComputeUnits / tiles;
    if (S > nk / kSplitMinSteps) S = nk / kSplitMinSteps;
    if (S < 2) return p;
    p.kb_per_split = (nk + S - 1) / S;
    p.ksplit = (nk + p.kb_per_split - 1) / p.kb_per_split;
    return p;
}

hipError_t launch_gemm(const Gemm &g_in, hipStream_t stream) {
    Gemm g = g_in;
    int rows = 0;
    for (int c = 0; c < (g.pair ? 1 : g.n_ch); ++c) rows += g.ch[c].d_out;
    g.col_fast = g.T > rows * (g.pair ? 2 : 1);   // x ([T][d_in]) larger than the W0 rows it meets
    if (g.ksplit > 1) {
        // With g.n_prod > 0 the tiles leave out the rank term: the launch's extra
        // workgroups compute V^T x (one split), and the reduction adds U V^T x.
        // (ranks up to 32: with a second rank block the units' code would cost the
        // tiles registers).
        const bool in_reduce = g.n_prod > 0 && g.ch[0].r > 0 && g.ch[0].r <= 32 && g.ksplit <= kRedMaxSplit;
        const hipError_t e = in_reduce ? launch_cfg<WL_GEMM_TILE_SPLIT, 1, 0, 1>(g, stream)
                                       : launch_nv<WL_GEMM_TILE_SPLIT, 1>(g, stream);
        if (e != hipSuccess) return e;
        if (in_reduce) {
            const dim3 grid((g.ch[0].d_out + 255) / 256, (g.T + kRedTok - 1) / kRedTok);
            const Child &c = g.ch[0];
            if (g.ksplit == 2)
                hipLaunchKernelGGL(split_reduce_rank_kernel<2>, grid, dim3(256), 0, stream, g.part, g.T, c.d_out,
                                   g.y, g.ldy, c.col0, c.U, c.vtx, c.r);
            else if (g.ksplit == 3)
                hipLaunchKernelGGL(split_reduce_rank_kernel<3>, grid, dim3(256), 0, stream, g.part, g.T, c.d_out,
                                   g.y, g.ldy, c.col0, c.U, c.vtx, c.r);
            else
                hipLaunchKernelGGL(split_reduce_rank_kernel<4>, grid, dim3(256), 0, stream, g.part, g.T, c.d_out,
                                   g.y, g.ldy, c.col0, c.U, c.vtx, c.r);
            return hipGetLastError();
        }
        const int64_t n = (int64_t)g.T * ((g.ch[0].d_out + 3) / 4);
        const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
        hipLaunchKernelGGL(split_reduce_kernel, dim3(blocks), dim3(256), 0, stream, g.part, g.ksplit, g.T,
                           g.ch[0].d_out, g.y, g.ldy, g.ch[0].col0);
        return hipGetLastError();
    }
    g.ksplit = 1;
    if (g.pair) {
        if (tiles_of<WL_GEMM_TILE_BIG_PAIR>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE_BIG_PAIR, 2>(g, stream);
        if (tiles_of<WL_GEMM_TILE_PAIR>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE_PAIR, 2>(g, stream);
        return launch_nv<WL_GEMM_TILE_SMALL_PAIR, 2>(g, stream);
    }
    if (tiles_of<WL_GEMM_TILE_BIG>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE_BIG, 1>(g, stream);
    if (tiles_of<WL_GEMM_TILE>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE, 1>(g, stream);
    return launch_nv<WL_GEMM_TILE_SMALL, 1>(g, stream);
}

}  // namespace wl
