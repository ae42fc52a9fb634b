// Matrix-core path for larger token counts (prefill-sized calls), one launch.
//
//   m[t,o]   = sum_i x[t,i] W0[o,i]                 bf16 x bf16 -> fp32 on MFMA
//   vtx[t,k] = sum_i x[t,i] V[i,k]                  same x tiles, same MFMA
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
// V^T x rides along: each stage also carries the matching BK rows of V (its
// natural layout, rank-contiguous), and the waves multiply the x fragments
// they already hold by V fragments gathered from LDS, splitting the K steps
// among the WN waves of a workgroup row; the WN partial results are added in
// wave order in the epilogue, so vtx never depends on scheduling. This costs
// about 1/WN of one extra MFMA per K step per 32 ranks and needs no separate
// launch and no workspace.
//
// Workgroups are numbered so that each of the 8 XCDs (which take workgroups
// round-robin) works through its own contiguous band of output tiles, keeping
// the W0 rows it reads in its own L2.
//
// Epilogue: the accumulators are scaled by s[o] (one output column per lane in
// the 32x32 layout); vtx is staged in LDS, split into a bf16 head and a bf16
// remainder (vtx = hi + lo to about 2^-16 relative) and both are run against U
// on the matrix cores as extra K steps, so the rank term keeps close to fp32
// accuracy. Results are rounded once to bf16. Pair mode (the MLP's gate/up)
// keeps two accumulator sets over the same x tile and writes
// bf16(gelu_tanh(g) * u).
#include "wl_device.h"
#include "wl_kernels.h"

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
    static constexpr int V_PIECES = BK * NV * 32 * 2 / 16;      // BK rows of V, up to NV*32 ranks
    static constexpr int A_PER = A_PIECES / kThreads, B_PER = B_PIECES / kThreads;
    static constexpr int V_PER = (V_PIECES + kThreads - 1) / kThreads;
    static constexpr int V_SLOTS = V_PER * kThreads;           // every lane's load writes a slot
    static constexpr int STAGE_PIECES = A_PIECES + P * (B_PIECES + V_SLOTS);
    static constexpr int PER_STAGE = A_PER + P * (B_PER + V_PER);   // direct-to-LDS loads per thread
    static constexpr int TILE_PIECES = D * STAGE_PIECES;
    static constexpr int VT_LD = kMaxRank + 4;                 // fp32 row stride of the epilogue vtx
    static constexpr int VT_PIECES = NV > 0 ? P * BM * VT_LD * 4 / 16 : 0;
    static constexpr int LDS_PIECES = TILE_PIECES > VT_PIECES ? TILE_PIECES : VT_PIECES;
    static_assert(A_PIECES % kThreads == 0 && B_PIECES % kThreads == 0, "tile pieces must split evenly");
    static_assert(D >= 2 && D <= 4 && (D - 1) * PER_STAGE <= 63, "stages in flight must fit vmcnt");
    static_assert(D - 2 <= 2, "wait counts cover at most two stages ahead");
    static_assert((BK / 16) % WN == 0, "V^T x K steps must split evenly over the WN waves");
};

// Swizzled position of piece kc of LDS row `row` (rows of KP pieces). The XOR
// pattern varies over 16 consecutive rows, so the 16 lanes that one LDS pass
// serves (32 rows x one piece per fragment read) land on distinct 4-bank
// groups of the 64 banks.
template <int KP>
__device__ __forceinline__ int swz_key(int row) {
    constexpr int sh = KP == 8 ? 0 : KP == 4 ? 1 : 2;
    return ((row >> sh) ^ (row >> 3)) & (KP - 1);
}
template <int KP>
__device__ __forceinline__ int swz(int row, int kc) {
    return row * KP + (kc ^ swz_key<KP>(row));
}

// A 16-byte piece of zeros: the source of every out-of-range piece of a
// direct-to-LDS tile load (the load always writes its LDS slot).
__device__ __attribute__((aligned(16))) const uint32_t kZeroPiece[4] = {0u, 0u, 0u, 0u};

// One direct-to-LDS load: the wave's 64 lanes each fetch 16 bytes from their
// own global address into 64 consecutive 16-byte LDS slots starting at dst.
__device__ __forceinline__ void lds_dma16(const u32x4 *src, u32x4 *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int WM, int WN, int TM, int TN, int BK, int P, int D, int NV>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(Gemm g) {
    using C = Cfg<WM, WN, TM, TN, BK, P, D, NV>;
    constexpr int BM = C::BM, BN = C::BN, KP = C::KP, NT = C::kThreads;
    constexpr int NVA = NV > 0 ? NV : 1;
    __shared__ u32x4 lds[C::LDS_PIECES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    // Tile numbering: XCD x (blockIdx % 8) takes a contiguous band of logical tiles.
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + BN - 1) / BN;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + BN - 1) / BN;
    const int n_mt = (g.T + BM - 1) / BM;
    const int total = n_nt * n_mt;
    int tile;
    {
        const int per = (total + 7) / 8, x = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int full = total - 8 * (per - 1);   // XCDs 0..full-1 hold `per` tiles, the rest per-1
        tile = x < full ? x * per + slot : full * per + (x - full) * (per - 1) + slot;
    }
    // Within the band: token tiles fastest, so consecutive tiles share W0 rows.
    const int mt = tile % n_mt, ntile = tile / n_mt;
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
    const int nk = (d_in + BK - 1) / BK;

    const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
    const Child *ch[P];
#pragma unroll
    for (int p = 0; p < P; ++p) ch[p] = &g.ch[P == 2 ? p : cidx];

    f32x16 acc[P][TM][TN];
    f32x16 accv[P][TM][NVA];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[p][i][j][e] = 0.f;
#pragma unroll
            for (int v = 0; v < NVA; ++v)
#pragma unroll
                for (int e = 0; e < 16; ++e) accv[p][i][v][e] = 0.f;
        }

    // The ring: the 64 lanes of one load write 64 consecutive 16-byte LDS slots,
    // so each lane fetches the global piece that belongs in its (swizzled) slot.
    const u32x4 *zero = reinterpret_cast<const u32x4 *>(kZeroPiece);
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
            const u32x4 *wgp = reinterpret_cast<const u32x4 *>(ch[p]->W0);
            u32x4 *bst = st + C::A_PIECES + p * (C::B_PIECES + C::V_SLOTS);
#pragma unroll
            for (int h = 0; h < C::B_PER; ++h) {
                const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row), gk = kt * KP + kc;
                const u32x4 *src = (gk < nch && n0 + row < d_out) ? wgp + (size_t)(n0 + row) * nch + gk : zero;
                lds_dma16(src, bst + h * NT + wave * kWave);
            }
            if constexpr (NV > 0) {
                // V rows [kt*BK, kt*BK + BK): BK*r bf16, contiguous, copied as they are.
                const int r = ch[p]->r;
                const u32x4 *vgp = reinterpret_cast<const u32x4 *>(ch[p]->V);
                const int q_end = BK * r / 8, q_all = d_in * r / 8, q0 = kt * BK * r / 8;
#pragma unroll
                for (int h = 0; h < C::V_PER; ++h) {
                    const int q = h * NT + tid;
                    const u32x4 *src = (q < q_end && q0 + q < q_all) ? vgp + q0 + q : zero;
                    lds_dma16(src, bst + C::B_PIECES + h * NT + wave * kWave);
                }
            }
        }
    };


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
    const u32x4 *vg[P];
    int vstep[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        wg[p] = reinterpret_cast<const u32x4 *>(ch[p]->W0);
        vg[p] = reinterpret_cast<const u32x4 *>(ch[p]->V);
        vstep[p] = BK * ch[p]->r / 8;
        const int dout_p = ch[p]->d_out;
#pragma unroll
        for (int h = 0; h < C::B_PER; ++h) {
            const int q = h * NT + tid, row = q / KP, kc = (q % KP) ^ swz_key<KP>(row);
            b_off[p][h] = min(n0 + row, dout_p - 1) * nch + kc;
        }
    }
    auto issue_full = [&](int kt, int sl) {
        u32x4 *st = lds + sl * C::STAGE_PIECES;
        const u32x4 *xk = xg + kt * KP;
#pragma unroll
        for (int h = 0; h < C::A_PER; ++h) lds_dma16(xk + a_off[h], st + h * NT + wave * kWave);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            u32x4 *bst = st + C::A_PIECES + p * (C::B_PIECES + C::V_SLOTS);
            const u32x4 *wk = wg[p] + kt * KP;
#pragma unroll
            for (int h = 0; h < C::B_PER; ++h) lds_dma16(wk + b_off[p][h], bst + h * NT + wave * kWave);
            if constexpr (NV > 0) {
                // Slots past the stage's BK * r / 8 pieces are never read: they repeat the
                // last piece. A child without a rank term (r = 0, V absent) reads the zero piece.
                const u32x4 *vk = vg[p] + kt * vstep[p];
#pragma unroll
                for (int h = 0; h < C::V_PER; ++h)
                    lds_dma16(vstep[p] > 0 ? vk + min(h * NT + tid, vstep[p] - 1) : zero,
                              bst + C::B_PIECES + h * NT + wave * kWave);
            }
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
                b[p][j] = st[C::A_PIECES + p * (C::B_PIECES + C::V_SLOTS) + swz<KP>(wn * TN * 32 + j * 32 + fr, kc)];
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
        if constexpr (NV > 0) {
            if (s % WN == wn) {
                // V fragment: lane (fr, fk) needs V[i][k] for the 8 stage rows
                // i = 16s + 8fk + e and rank k = 32v + fr.
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int r = ch[p]->r;
                    const uint16_t *vl = reinterpret_cast<const uint16_t *>(
                        st + C::A_PIECES + p * (C::B_PIECES + C::V_SLOTS) + C::B_PIECES);
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const int k = 32 * v + fr;
                        u32x4 vf = {0u, 0u, 0u, 0u};
                        if (k < r) {
                            const uint16_t *col = vl + (16 * s + 8 * fk) * r + k;
                            vf.x = (uint32_t)col[0] | ((uint32_t)col[r] << 16);
                            vf.y = (uint32_t)col[2 * r] | ((uint32_t)col[3 * r] << 16);
                            vf.z = (uint32_t)col[4 * r] | ((uint32_t)col[5 * r] << 16);
                            vf.w = (uint32_t)col[6 * r] | ((uint32_t)col[7 * r] << 16);
                        }
#pragma unroll
                        for (int i = 0; i < TM; ++i) accv[p][i][v] = mfma(a[i], vf, accv[p][i][v]);
                    }
                }
            }
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
    for (int s0 = 0; s0 < D - 1 && s0 < nk; ++s0) issue_any(s0, s0);
    for (int kt = 0; kt < nk; ++kt) {
        // This wave's loads of stage kt are done; up to D - 2 later stages stay in flight.
        const int ahead = min(D - 2, nk - 1 - kt);
        if (ahead >= 2) wait_vm<2 * C::PER_STAGE>();
        else if (ahead == 1) wait_vm<C::PER_STAGE>();
        else wait_vm<0>();
        barrier();
        if (kt + D - 1 < nk) issue_any(kt + D - 1, (kt + D - 1) % D);
        compute(lds + (kt % D) * C::STAGE_PIECES);
    }
    barrier();                                        // the ring is free for the epilogue

    // ---- epilogue ----
    // Lane (fr, fk) of block (i, j) holds output column o = n0 + (wn*TN + j)*32 + fr
    // and token rows m0 + (wm*TM + i)*32 + 8*(e/4) + 4*fk + (e%4), e = 0..15.
    if constexpr (NV > 0) {
        // vtx of child p: fp32 [BM][VT_LD] at vt + p*BM*VT_LD, the WN partials added in wave
        // order. The padded row stride puts the 16 rows one LDS pass reads on distinct banks.
        float *vt = reinterpret_cast<float *>(lds);
        for (int w = 0; w < WN; ++w) {
            if (wn == w) {
#pragma unroll
                for (int p = 0; p < P; ++p)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int v = 0; v < NV; ++v)
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                                const int row = (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
                                float *dst = vt + (p * BM + row) * C::VT_LD + 32 * v + fr;
                                *dst = w == 0 ? accv[p][i][v][e] : *dst + accv[p][i][v][e];
                            }
            }
            barrier();
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const Child &Cp = *ch[p];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int o = n0 + (wn * TN + j) * 32 + fr;
            const float sv = (Cp.s && o < d_out) ? Cp.s[o] : 1.0f;
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[p][i][j] *= sv;
        }
        if constexpr (NV > 0) {
            const int r = Cp.r;
            const float *vt = reinterpret_cast<const float *>(lds) + p * BM * C::VT_LD;
            for (int k0 = 0; k0 < r; k0 += 16) {
                const int kb = k0 + 8 * fk;
                u32x4 ahi[TM], alo[TM], bu[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    // Columns up to kb + 7 < 64 are inside the row; those at or past r
                    // (never written) are replaced by zeros.
                    const f32x4 *row = reinterpret_cast<const f32x4 *>(vt + ((wm * TM + i) * 32 + fr) * C::VT_LD + kb);
                    const f32x4 r0 = row[0], r1 = row[1];
                    const float raw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                    float hi[8], lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = kb + e < r ? raw[e] : 0.f;
                        hi[e] = bf16_f(f_bf16(v));
                        lo[e] = v - hi[e];
                    }
                    ahi[i] = pack8(hi);
                    alo[i] = pack8(lo);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int o = n0 + (wn * TN + j) * 32 + fr;
                    float u[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        u[e] = (o < d_out && kb + e < r) ? bf16_f(Cp.U[(size_t)o * r + kb + e]) : 0.f;
                    bu[j] = pack8(u);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc[p][i][j] = mfma(ahi[i], bu[j], acc[p][i][j]);
                        acc[p][i][j] = mfma(alo[i], bu[j], acc[p][i][j]);
                    }
            }
        }
    }

    const int col0 = g.pair ? 0 : C0.col0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int o = n0 + (wn * TN + j) * 32 + fr;
        if (o >= d_out) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = m0 + (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
                if (t < g.T) {
                    const float v = P == 2 ? gelu_tanh(acc[0][i][j][e]) * acc[P - 1][i][j][e] : acc[0][i][j][e];
                    g.y[(size_t)t * g.ldy + col0 + o] = f_bf16(v);
                }
            }
    }
}

template <int WM, int WN, int TM, int TN, int BK, int D, int P, int NV>
hipError_t launch_cfg(const Gemm &g, hipStream_t stream) {
    using C = Cfg<WM, WN, TM, TN, BK, P, D, NV>;
    int n_nt = 0;
    if (g.pair)
        n_nt = (g.ch[0].d_out + C::BN - 1) / C::BN;
    else
        for (int c = 0; c < g.n_ch; ++c) n_nt += (g.ch[c].d_out + C::BN - 1) / C::BN;
    const int total = n_nt * ((g.T + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((gemm_kernel<WM, WN, TM, TN, BK, P, D, NV>), dim3(total), dim3(C::kThreads), 0, stream, g);
    return hipGetLastError();
}

template <int WM, int WN, int TM, int TN, int BK, int D, int P, int NV_MAX = 2>
hipError_t launch_nv(const Gemm &g, hipStream_t stream) {
    int max_r = 0;
    for (int c = 0; c < (g.pair ? 2 : g.n_ch); ++c) max_r = g.ch[c].r > max_r ? g.ch[c].r : max_r;
    if (max_r == 0 || NV_MAX == 0) return launch_cfg<WM, WN, TM, TN, BK, D, P, 0>(g, stream);
    if (max_r <= 32 || NV_MAX == 1) return launch_cfg<WM, WN, TM, TN, BK, D, P, (NV_MAX < 1 ? NV_MAX : 1)>(g, stream);
    return launch_cfg<WM, WN, TM, TN, BK, D, P, NV_MAX>(g, stream);
}

}  // namespace

// Tile configurations (waves M x N, 32x32 blocks per wave M x N, K depth, LDS
// stages), chosen by measurement on the layer shapes; overridable at build time.
// The largest tile whose grid still gives most compute units a workgroup is used
// (the largest only without a rank term, whose extra registers it has no room for).
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
#define WL_GEMM_TILE_SMALL 2, 2, 2, 1, 64, 2
#endif
#ifndef WL_GEMM_TILE_SMALL_PAIR
#define WL_GEMM_TILE_SMALL_PAIR 2, 2, 2, 1, 64, 2
#endif

namespace {

constexpr int kFillTiles = 232;   // workgroups that count as filling the 256 compute units

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

}  // namespace

hipError_t launch_gemm(const Gemm &g, hipStream_t stream) {
    int max_r = 0;
    for (int c = 0; c < (g.pair ? 2 : g.n_ch); ++c) max_r = g.ch[c].r > max_r ? g.ch[c].r : max_r;
    if (g.pair) {
        if (max_r == 0 && tiles_of<WL_GEMM_TILE_BIG_PAIR>(g) >= kFillTiles)
            return launch_nv<WL_GEMM_TILE_BIG_PAIR, 2, 0>(g, stream);
        if (tiles_of<WL_GEMM_TILE_PAIR>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE_PAIR, 2>(g, stream);
        return launch_nv<WL_GEMM_TILE_SMALL_PAIR, 2>(g, stream);
    }
    if (max_r == 0 && tiles_of<WL_GEMM_TILE_BIG>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE_BIG, 1, 0>(g, stream);
    if (tiles_of<WL_GEMM_TILE>(g) >= kFillTiles) return launch_nv<WL_GEMM_TILE, 1>(g, stream);
    return launch_nv<WL_GEMM_TILE_SMALL, 1>(g, stream);
}

}  // namespace wl
