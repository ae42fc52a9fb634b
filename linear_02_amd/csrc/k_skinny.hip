// Projections at a few tens of tokens (batched decode, 8 < T <= 64): two launches.
//
//   m[t,o]   = sum_i W0[o,i] x[t,i]       matrix cores, split over the input axis
//   vtx[t,k] = sum_i V[i,k] x[t,i]        vector ALUs, in the same launch
//   y[t,o]   = bf16( s[o] * m[t,o] + sum_k U[o,k] vtx[t,k] )      second launch
//
// ("In-kernel reconstruction", introduction: the reconstruction formula and its
// per-element expansion.)
//
// At these sizes W0 is still nearly all of the memory traffic, but every W0
// element is used T times, more than the vector ALUs can feed from LDS; so the
// products run on v_mfma_f32_32x32x16_bf16 with x as the A operand (32 token
// rows) and W0 as the B operand (32 output rows). Each W0 element is used by
// exactly one wave, so both operands go straight from global memory into
// registers, with no LDS staging: within a 64-wide block of the input axis,
// lanes 0..31 take inputs [0, 32) and lanes 32..63 inputs [32, 64) of their
// row, 64 contiguous bytes per lane, and the MFMA steps pair them up. (Any
// assignment of the input index to steps gives the same sum; this one makes
// the loads contiguous.) Two blocks are in flight per wave.
//
// Launch 1 (main): workgroup (row block of 32 outputs, split of the input axis);
// its four waves take interleaved 64-wide blocks of the split and add their
// accumulators in wave order through LDS, then store fp32 partial sums
// part[split][p][t][o]. Extra workgroups, dispatched first, compute V^T x on the
// vector ALUs, one (child, 8 tokens, 512 inputs) each, into vpart[slice][c][t][k].
// Launch 2 (epilogue): one thread per (output, token) adds the splits in order,
// scales by s, adds U . vtx (vtx summed over slices in order, staged in LDS) and
// rounds once to bf16; pair mode (gate/up of the MLP) writes
// bf16(gelu_tanh(g) * u). No atomics: the result does not depend on scheduling.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int kKB = 64;                 // inputs per block (4 MFMA steps)

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Per-lane child fields as a sum of masked differences (see the decode kernel:
// a per-lane index into the kernel-argument array, or a select chain, costs
// dependent loads or a scratch table).
template <class T>
__device__ __forceinline__ T blend3(int ci, T a, T b, T c) {
    return a + (ci > 0 ? b - a : T(0)) + (ci > 1 ? c - b : T(0));
}
__device__ __forceinline__ int child_of(const Skinny &g, int row) {
    return (g.n_ch > 2 && row >= g.ch[2].col0) ? 2 : (g.n_ch > 1 && row >= g.ch[1].col0) ? 1 : 0;
}
__device__ __forceinline__ uint64_t ptr_of(const void *p) { return reinterpret_cast<uint64_t>(p); }

// ---- launch 1, main workgroups ----------------------------------------------------------

template <int MT, int P>
__device__ void main_wg(const Skinny &g, int wgi) {
    __shared__ float red[P][MT][16][kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = wgi % g.n_rowblk, sp = wgi / g.n_rowblk;
    const int n = lane & 31, h = lane >> 5;
    const int nch = g.d_in >> 3;
    const int row = rb * 32 + n, rowc = min(row, g.rows - 1);

    // This lane's W0 rows (pair: gate row and up row).
    const u32x4 *wrow[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        if (P == 2) {
            wrow[p] = reinterpret_cast<const u32x4 *>(g.ch[p].W0) + (size_t)rowc * nch;
        } else {
            const int ci = child_of(g, rowc);
            const uint64_t base = blend3(ci, ptr_of(g.ch[0].W0), ptr_of(g.ch[1].W0), ptr_of(g.ch[2].W0));
            const int col0 = blend3(ci, 0, g.ch[1].col0, g.ch[2].col0);
            wrow[p] = reinterpret_cast<const u32x4 *>(base) + (size_t)(rowc - col0) * nch;
        }
    }
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
    const u32x4 *xrow[MT];
    bool tok_ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = mt * 32 + n;
        tok_ok[mt] = t < g.T;
        xrow[mt] = xg + (size_t)min(t, g.T - 1) * nch;
    }

    const int nkb = (g.d_in + kKB - 1) / kKB;
    const int kb0 = sp * g.kb_per_split, kb1 = min(nkb, kb0 + g.kb_per_split);
    const int nb = kb1 > kb0 + wave ? (kb1 - kb0 - wave + 3) / 4 : 0;   // blocks of this wave

    f32x16 acc[P][MT];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[p][mt][e] = 0.f;

    // Block loads: every address valid (block index and pieces clamped), values
    // past the input axis replaced by zeros.
    auto load = [&](u32x4 (&wb)[P][4], u32x4 (&xa)[MT][4], int i) {
        const int kb = min(kb0 + wave + 4 * i, kb1 - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = kb * 8 + 4 * h + j;
            const bool in = pc < nch;
            const int pcc = in ? pc : nch - 1;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const u32x4 v = ldg(wrow[p] + pcc);
                wb[p][j] = in ? v : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4 v = xrow[mt][pcc];
                xa[mt][j] = (in && tok_ok[mt]) ? v : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute = [&](const u32x4 (&wb)[P][4], const u32x4 (&xa)[MT][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[p][mt] = mfma(xa[mt][j], wb[p][j], acc[p][mt]);
    };

    if (kb1 > kb0) {
        u32x4 wA[P][4], xA[MT][4], wB[P][4], xB[MT][4];
        load(wA, xA, 0);
        for (int i = 0; i < nb; i += 2) {
            load(wB, xB, i + 1);
            compute(wA, xA);
            if (i + 1 >= nb) break;
            load(wA, xA, i + 2);
            compute(wB, xB);
        }
    }

    // Wave sums added in wave order through LDS, then fp32 partials of this split.
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float &dst = red[p][mt][e][lane];
                        dst = w == 0 ? acc[p][mt][e] : dst + acc[p][mt][e];
                    }
        }
        __syncthreads();
    }
    constexpr int kItems = P * MT * 16 * kWave;
    const float *r0 = &red[0][0][0][0];
    for (int it = tid; it < kItems; it += kThreads) {
        const int l = it % kWave, e = (it / kWave) % 16, mt = (it / (kWave * 16)) % MT, p = it / (kWave * 16 * MT);
        const int t = mt * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        const int o = rb * 32 + (l & 31);
        if (t < g.T && o < g.rows) g.part[(((size_t)sp * P + p) * g.T + t) * g.rows + o] = r0[it];
    }
}

// ---- launch 1, V^T x workgroups -----------------------------------------------------------

// Workgroup (child, block of kSkVtxTok tokens, slice of kSkVtxSlice inputs):
// vpart[slice][c][t][k] = sum over the slice's inputs i of V_c[i][k] x[t][i].
__device__ void vtx_wg(const Skinny &g, int wgi) {
    __shared__ u32x4 xs[kSkVtxSlice];           // xs[i] = the 8 tokens' x[t][i0 + i], bf16
    __shared__ float vred[kThreads][kSkVtxTok + 1];
    const int tid = threadIdx.x;
    const int n_tb = (g.T + kSkVtxTok - 1) / kSkVtxTok;
    const int sl = wgi % g.n_vsl, tb = (wgi / g.n_vsl) % n_tb, cj = wgi / (g.n_vsl * n_tb);
    const int c = cj == 0 ? g.vtx_ch[0] : cj == 1 ? g.vtx_ch[1] : g.vtx_ch[2];   // uniform
    const Child &C = g.ch[c];
    const int r = C.r;
    const int t0 = tb * kSkVtxTok, tn = min(kSkVtxTok, g.T - t0);
    const int i0 = sl * kSkVtxSlice, len = min(kSkVtxSlice, g.d_in - i0);

    // Stage x[t0 .. t0 + 8)[i0 .. i0 + len) transposed, 8 tokens per input
    // (absent tokens and inputs as zeros).
    {
        constexpr int kPer = kSkVtxSlice / 8;                 // 16-byte pieces per token
        constexpr int kN = kSkVtxTok * kPer / kThreads;
        static_assert(kSkVtxTok * kPer % kThreads == 0, "x staging split");
        const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.x);
        const int nch = g.d_in >> 3;
        u32x4 v[kN];
#pragma unroll
        for (int m = 0; m < kN; ++m) {
            const int q = tid + m * kThreads, t = q / kPer, j = q - t * kPer;
            v[m] = ldg(xg + (size_t)(t0 + min(t, tn - 1)) * nch + (i0 >> 3) + min(j, (len >> 3) - 1));
        }
        uint16_t *xd = reinterpret_cast<uint16_t *>(xs);
#pragma unroll
        for (int m = 0; m < kN; ++m) {
            const int q = tid + m * kThreads, t = q / kPer, j = q - t * kPer;
            const bool ok = t < tn && 8 * j < len;
            const uint32_t w[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xd[(8 * j + e) * kSkVtxTok + t] = ok ? (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu) : 0;
        }
    }
    __syncthreads();

    int rp = 1;
    while (rp < r) rp <<= 1;
    const int k = tid & (rp - 1), grp = tid / rp, G = kThreads / rp;
    float acc[kSkVtxTok];
#pragma unroll
    for (int t = 0; t < kSkVtxTok; ++t) acc[t] = 0.f;
    if (k < r) {
        const uint16_t *V = C.V + (size_t)i0 * r + k;
        for (int ib = grp; ib < len; ib += 32 * G) {
            float v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int i = ib + u * G;
                const float vv = bf16_f(ldg(V + (size_t)min(i, len - 1) * r));
                v[u] = i < len ? vv : 0.f;
            }
#pragma unroll 4
            for (int u = 0; u < 32; ++u) {
                const u32x4 xv = xs[min(ib + u * G, kSkVtxSlice - 1)];
                const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int t = 0; t < kSkVtxTok; ++t)
                    acc[t] += v[u] * bf16_f(t & 1 ? w[t >> 1] >> 16 : w[t >> 1] & 0xFFFFu);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSkVtxTok; ++t) vred[tid][t] = acc[t];
    __syncthreads();
    for (int it = tid; it < r * tn; it += kThreads) {
        const int t = it / r, kk = it - t * r;
        float sum = 0.f;
        for (int gg = 0; gg < G; ++gg) sum += vred[gg * rp + kk][t];
        g.vpart[(((size_t)sl * g.n_ch + c) * g.T + t0 + t) * kMaxRank + kk] = sum;
    }
}

template <int MT, int P>
__global__ __launch_bounds__(kThreads) void skinny_main(Skinny g) {
    const int b = blockIdx.x;
    if (b < g.n_vtx_wg)
        vtx_wg(g, b);
    else
        main_wg<MT, P>(g, b - g.n_vtx_wg);
}

// ---- launch 2: epilogue -------------------------------------------------------------------

// Workgroup: 4 waves, each one 32-output block x all tokens (MT blocks of 32).
// The accumulators start as the split partials added in split order (in the
// MFMA output layout), are scaled by s, and take the rank term on the matrix
// cores: A = vtx (tokens x ranks, split into a bf16 head and a bf16 remainder,
// so that the product keeps close to fp32 accuracy), B = U (ranks x outputs).
// Rows of a block that belong to different children take one pass per child,
// with the U of the other children's rows zeroed.
constexpr int kEpiRowsWG = 4 * 32;

template <int MT, int P, int SMAX>
__global__ __launch_bounds__(kThreads) void skinny_epilogue(Skinny g) {
    __shared__ float vs[kMaxChildren][kSkMaxTok][kMaxRank];
    __shared__ f32x4 lv[kSkEpiMaxLoads / 4];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int rb = blockIdx.x * 4 + wave;                     // this wave's 32-output block
    const int row = rb * 32 + n, rowc = min(row, g.rows - 1);
    const int r0 = g.ch[0].r, r1 = g.n_ch > 1 ? g.ch[1].r : 0, r2 = g.n_ch > 2 ? g.ch[2].r : 0;
    const int q0 = (r0 + 3) / 4, q1 = (r1 + 3) / 4, q2 = (r2 + 3) / 4, qsum = q0 + q1 + q2;

    // Split partials of this lane's outputs, issued before anything else.
    f32x16 acc[P][MT];
    {
        float pm[P][MT][SMAX][16];
        const size_t pstride = (size_t)P * g.T * g.rows;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int sp = 0; sp < SMAX; ++sp)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = min(mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3), g.T - 1);
                        pm[p][mt][sp][e] = ldg(g.part + (size_t)min(sp, g.S - 1) * pstride +
                                               ((size_t)p * g.T + t) * g.rows + rowc);
                    }
        // Per-output s.
        float sv[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int ci = P == 2 ? p : child_of(g, rowc);
            const int col0 = P == 2 ? 0 : blend3(ci, 0, g.ch[1].col0, g.ch[2].col0);
            const uint64_t sb = P == 2 ? ptr_of(g.ch[p].s)
                                       : blend3(ci, ptr_of(g.ch[0].s), ptr_of(g.ch[1].s), ptr_of(g.ch[2].s));
            const float *sp = reinterpret_cast<const float *>(sb);
            const float s_raw = ldg(sp ? sp + (rowc - col0) : reinterpret_cast<const float *>(g.x));
            sv[p] = sp ? s_raw : 1.f;
        }
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float m = pm[p][mt][0][e];
#pragma unroll
                    for (int sp = 1; sp < SMAX; ++sp) m += sp < g.S ? pm[p][mt][sp][e] : 0.f;
                    acc[p][mt][e] = sv[p] * m;
                }
    }

    // vtx[c][t][k]: the slice partials added in slice order. Items are (child,
    // token, 4 ranks), in child order; a chunk's 16-byte loads are issued
    // together into LDS, then each item adds its slices. Chunks of tokens keep a
    // chunk within lv. Rank slots past r hold unwritten values and are never used.
    if (qsum > 0) {
        const int tc = max(1, (kSkEpiMaxLoads / 4) / (qsum * g.n_vsl));
        for (int tb = 0; tb < g.T; tb += tc) {
            const int nt = min(tc, g.T - tb);
            const int n_items = nt * qsum, n_loads = n_items * g.n_vsl;
            auto item_of = [&](int item, int &c, int &t, int &k) {
                const int a0 = nt * q0, a1 = nt * q1;
                c = item >= a0 ? (item >= a0 + a1 ? 2 : 1) : 0;
                const int rel = item - (c > 0 ? a0 : 0) - (c > 1 ? a1 : 0);
                const int qc = max(1, c == 0 ? q0 : c == 1 ? q1 : q2);
                const int tt = rel / qc;
                t = tb + tt;
                k = 4 * (rel - tt * qc);
            };
            for (int f0 = 0; f0 < n_loads; f0 += 16 * kThreads) {
                f32x4 v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int f = min(f0 + u * kThreads + tid, n_loads - 1);
                    const int item = f / g.n_vsl, sl = f - item * g.n_vsl;
                    int c, t, k;
                    item_of(item, c, t, k);
                    v[u] = ldg(reinterpret_cast<const f32x4 *>(
                        g.vpart + (((size_t)sl * g.n_ch + c) * g.T + t) * kMaxRank + k));
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int f = f0 + u * kThreads + tid;
                    if (f < n_loads) lv[f] = v[u];
                }
            }
            __syncthreads();
            for (int item = tid; item < n_items; item += kThreads) {
                int c, t, k;
                item_of(item, c, t, k);
                f32x4 sum = lv[item * g.n_vsl];
                for (int sl = 1; sl < g.n_vsl; ++sl) sum += lv[item * g.n_vsl + sl];
                *reinterpret_cast<f32x4 *>(&vs[c][t][k]) = sum;
            }
            __syncthreads();
        }
    }

    // Rank term, one pass per child present in this block (uniform loop).
    if (qsum > 0) {
        const int c_lo = P == 2 ? 0 : child_of(g, min(rb * 32, g.rows - 1));
        const int c_hi = P == 2 ? 1 : child_of(g, min(rb * 32 + 31, g.rows - 1));
        for (int c = c_lo; c <= c_hi; ++c) {
            const int rc = c == 0 ? r0 : c == 1 ? r1 : r2;
            if (rc == 0) continue;
            const int col0 = c == 0 ? 0 : c == 1 ? g.ch[1].col0 : g.ch[2].col0;
            const int p = P == 2 ? c : 0;
            const uint16_t *U = c == 0 ? g.ch[0].U : c == 1 ? g.ch[1].U : g.ch[2].U;
            const bool mine = P == 2 || child_of(g, rowc) == c;
            const bool rok = row < g.rows && mine;
            const uint16_t *Urow = U + (size_t)(rok ? row - col0 : 0) * rc;
            for (int k0 = 0; k0 < rc; k0 += 16) {
                const int kb = k0 + 8 * h;
                // B: U[row][kb .. kb + 8), zero past r and for rows of other children.
                float uf[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = bf16_f(ldg(Urow + min(kb + e, rc - 1)));
                    uf[e] = (rok && kb + e < rc) ? v : 0.f;
                }
                u32x4 bu;
                bu.x = (uint32_t)f_bf16(uf[0]) | ((uint32_t)f_bf16(uf[1]) << 16);
                bu.y = (uint32_t)f_bf16(uf[2]) | ((uint32_t)f_bf16(uf[3]) << 16);
                bu.z = (uint32_t)f_bf16(uf[4]) | ((uint32_t)f_bf16(uf[5]) << 16);
                bu.w = (uint32_t)f_bf16(uf[6]) | ((uint32_t)f_bf16(uf[7]) << 16);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // A: vtx[c][t][kb .. kb + 8) for token t = mt*32 + n, as head + remainder.
                    const int t = min(mt * 32 + n, g.T - 1);
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&vs[c][t][min(kb, kMaxRank - 8)]);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&vs[c][t][min(kb, kMaxRank - 8) + 4]);
                    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    float hi[8], lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = kb + e < rc ? av[e] : 0.f;
                        hi[e] = bf16_f(f_bf16(v));
                        lo[e] = v - hi[e];
                    }
                    u32x4 ah, al;
                    ah.x = (uint32_t)f_bf16(hi[0]) | ((uint32_t)f_bf16(hi[1]) << 16);
                    ah.y = (uint32_t)f_bf16(hi[2]) | ((uint32_t)f_bf16(hi[3]) << 16);
                    ah.z = (uint32_t)f_bf16(hi[4]) | ((uint32_t)f_bf16(hi[5]) << 16);
                    ah.w = (uint32_t)f_bf16(hi[6]) | ((uint32_t)f_bf16(hi[7]) << 16);
                    al.x = (uint32_t)f_bf16(lo[0]) | ((uint32_t)f_bf16(lo[1]) << 16);
                    al.y = (uint32_t)f_bf16(lo[2]) | ((uint32_t)f_bf16(lo[3]) << 16);
                    al.z = (uint32_t)f_bf16(lo[4]) | ((uint32_t)f_bf16(lo[5]) << 16);
                    al.w = (uint32_t)f_bf16(lo[6]) | ((uint32_t)f_bf16(lo[7]) << 16);
                    acc[p][mt] = mfma(ah, bu, acc[p][mt]);
                    acc[p][mt] = mfma(al, bu, acc[p][mt]);
                }
            }
        }
    }

    if (row >= g.rows) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (t < g.T) {
                const float v = P == 2 ? gelu_tanh(acc[0][mt][e]) * acc[P - 1][mt][e] : acc[0][mt][e];
                g.y[(size_t)t * g.ldy + row] = f_bf16(v);
            }
        }
}

template <int MT, int P>
hipError_t launch_mp(const Skinny &g, hipStream_t stream) {
    const int n_main = g.n_rowblk * g.S;
    hipLaunchKernelGGL((skinny_main<MT, P>), dim3(g.n_vtx_wg + n_main), dim3(kThreads), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kSMax = kSkMaxPartials / (P * MT);
    const dim3 grid((g.rows + kEpiRowsWG - 1) / kEpiRowsWG);
    if (g.S <= 2)
        hipLaunchKernelGGL((skinny_epilogue<MT, P, 2>), grid, dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL((skinny_epilogue<MT, P, kSMax>), grid, dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

}  // namespace

// Splits of the input axis: enough workgroups to keep the memory system busy
// (about 384), at least four 64-wide blocks per split (one per wave) where the
// input axis allows it, and S * P * (token blocks) at most kSkMaxPartials.
SkinnyPlan skinny_plan(int rows, int d_in, int T, int P, int n_vtx_ch) {
    SkinnyPlan p;
    p.n_rowblk = (rows + 31) / 32;
    const int nkb = (d_in + kKB - 1) / kKB;
    const int MT = T > 32 ? 2 : 1;
    const int s_max = kSkMaxPartials / (P * MT);   // partials the epilogue holds per output
    int S = (384 + p.n_rowblk - 1) / p.n_rowblk;
    S = S < (nkb + 3) / 4 ? S : (nkb + 3) / 4;
    S = S < s_max ? S : s_max;
    S = S > 1 ? S : 1;
    p.kb_per_split = (nkb + S - 1) / S;
    p.S = (nkb + p.kb_per_split - 1) / p.kb_per_split;   // no empty split
    p.n_vsl = (d_in + kSkVtxSlice - 1) / kSkVtxSlice;
    p.n_vtx_wg = n_vtx_ch * ((T + kSkVtxTok - 1) / kSkVtxTok) * p.n_vsl;
    return p;
}

hipError_t launch_skinny(const Skinny &g, hipStream_t stream) {
    const bool two = g.T > 32;
    if (g.pair) return two ? launch_mp<2, 2>(g, stream) : launch_mp<1, 2>(g, stream);
    return two ? launch_mp<2, 1>(g, stream) : launch_mp<1, 1>(g, stream);
}

}  // namespace wl
