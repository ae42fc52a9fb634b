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
// the loads contiguous.)
//
// Launch 1 (main): workgroup (row block of 32 outputs, split of the input axis);
// its four waves take interleaved 64-wide blocks of the split, each wave loading
// all of its blocks at once (one memory round trip), and add their accumulators
// in wave order through LDS, then store fp32 partial sums part[split][p][t][o]. Extra workgroups, dispatched first, compute V^T x on the
// vector ALUs, one (child, 8 tokens, 512 inputs) each, into vpart[slice][c][t][k].
// Launch 2 (epilogue): one thread per (output, a few tokens) adds the splits in
// order, scales by s, adds U . vtx in fp32 (vtx summed over slices in order,
// staged in LDS) and rounds once to bf16; pair mode (gate/up of the MLP) writes
// bf16(gelu_tanh(g) * u). No atomics: the result does not depend on scheduling.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kThreads = 256;
constexpr int kKB = 64;                 // inputs per block (4 MFMA steps)
constexpr int kVtxRedLd = 33;           // padded row of the V^T x per-thread sums

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

// Blocks of the input axis a wave loads at once (all of them in flight): its
// LDS region holds NB * P W0 tiles of 4 KB.
template <int MT, int P>
constexpr int blocks_at_once() { return P * MT == 1 ? 4 : 2; }
template <int MT, int P>
constexpr int main_lds_floats() { return 4 * blocks_at_once<MT, P>() * P * 32 * 8 * 4; }

// W0 tiles (32 rows x 64 inputs = 32 x 8 pieces) come in by direct-to-LDS loads
// in 128-byte runs of a row (8 lanes per row, 8 rows per load), which the memory
// system serves far better than the MFMA operand layout (32 rows per load, 16
// bytes each); the slots are XOR-swizzled by row so that the fragment reads
// (32 rows, one piece) are free of bank conflicts. x, read from L2, goes straight
// into registers in the operand layout.
template <int MT, int P>
__device__ void main_wg(const Skinny &g, float *smem, int wgi) {
    constexpr int NB = blocks_at_once<MT, P>();
    constexpr int KP = 8;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = wgi % g.n_rowblk, sp = wgi / g.n_rowblk;
    const int n = lane & 31, h = lane >> 5;
    const int nch = g.d_in >> 3;
    u32x4 *tiles = reinterpret_cast<u32x4 *>(smem) + wave * (NB * P * 32 * KP);   // this wave's region

    // Rows this lane fetches into the tiles: row 8j + lane/8 of the block for load
    // j, slot lane%8, which holds piece (lane%8) ^ key(row) of that row.
    const int lrow = lane >> 3, lslot = lane & 7;
    const u32x4 *wsrc[P][4];
    int wpiece[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rl = 8 * j + lrow;
        const int rowc = min(rb * 32 + rl, g.rows - 1);   // rows past the end re-read the last (never stored)
        wpiece[j] = lslot ^ swz_key<KP>(rl);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (P == 2) {
                wsrc[p][j] = reinterpret_cast<const u32x4 *>(g.ch[p].W0) + (size_t)rowc * nch;
            } else {
                const int ci = child_of(g, rowc);
                const uint64_t base = blend3(ci, ptr_of(g.ch[0].W0), ptr_of(g.ch[1].W0), ptr_of(g.ch[2].W0));
                const int col0 = blend3(ci, 0, g.ch[1].col0, g.ch[2].col0);
                wsrc[p][j] = reinterpret_cast<const u32x4 *>(base) + (size_t)(rowc - col0) * nch;
            }
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

    // Rounds of NB blocks, every load of a round issued before any product. Every
    // address is valid (block index and pieces clamped); x values past the input
    // axis are zeros, so the clamped W0 pieces there add nothing, and blocks past
    // this wave's share are loaded but not used.
    for (int b0 = 0; b0 < nb; b0 += NB) {
        u32x4 xa[NB][MT][4];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int kb = min(kb0 + wave + 4 * (b0 + b), kb1 - 1);
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lds_dma16(wsrc[p][j] + min(kb * KP + wpiece[j], nch - 1), tiles + ((b * P + p) * 4 + j) * kWave);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pc = kb * 8 + 4 * h + j;
                const bool in = pc < nch;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 v = ldg(xrow[mt] + min(pc, nch - 1));
                    xa[b][mt][j] = (in && tok_ok[mt]) ? v : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        wait_vm<0>();   // this wave's tiles have landed (the region is its own: no barrier)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b0 + b >= nb) break;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    // Lane (n, h): row n, logical piece 4h + j (the same inputs as its x piece).
                    const u32x4 w = tiles[(b * P + p) * 32 * KP + swz<KP>(n, 4 * h + j)];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[p][mt] = mfma(xa[b][mt][j], w, acc[p][mt]);
                }
        }
        if (b0 + NB < nb) __builtin_amdgcn_wave_barrier();   // reads of this round before the next round's loads
    }

    // Wave sums through LDS (one slot per wave, after every wave is done with its
    // tiles), added in wave order, then the fp32 partials of this split.
    constexpr int kItems = P * MT * 16 * kWave;
    float *red = smem;                               // [4][kItems]
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[wave * kItems + ((p * MT + mt) * 16 + e) * kWave + lane] = acc[p][mt][e];
    __syncthreads();
    for (int it = tid; it < kItems; it += kThreads) {
        const float v = ((red[it] + red[kItems + it]) + red[2 * kItems + it]) + red[3 * kItems + it];
        const int l = it % kWave, e = (it / kWave) % 16, mt = (it / (kWave * 16)) % MT, p = it / (kWave * 16 * MT);
        const int t = mt * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        const int o = rb * 32 + (l & 31);
        if (t < g.T && o < g.rows) g.part[(((size_t)sp * P + p) * g.T + t) * g.rows + o] = v;
    }
}

// ---- launch 1, V^T x workgroups -----------------------------------------------------------

// Workgroup (child, block of kSkVtxTok tokens, slice of kSkVtxSlice inputs):
// vpart[slice][c][t][k] = sum over the slice's inputs i of V_c[i][k] x[t][i].
// Ranks 4, 8, 16, 32 and 64 take 8-byte pieces of V and runs of x straight from
// memory (vtx_quads); other ranks stage x in LDS and take one rank per thread
// (vtx_any).

__device__ __forceinline__ void stage_x(const Skinny &g, u32x4 *xs, int t0, int tn, int i0, int len) {
    constexpr int kPer = kSkVtxSlice / 8;                 // 16-byte pieces per token
    constexpr int kN = kSkVtxTok * kPer / kThreads;
    static_assert(kSkVtxTok * kPer % kThreads == 0, "x staging split");
    const int tid = threadIdx.x;
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

// Sum over each 16-lane row of the wave (every lane of the row gets it).
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);             // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);             // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);            // row_half_mirror
    v += dpp<0x140>(v);            // row_mirror
    return v;
}

// x[t0 + t][i .. i + n) for n in {2, 4, 8, 16} inputs, as n / 2 packed words.
template <int N>
__device__ __forceinline__ void load_x_run(const uint16_t *p, uint32_t (&w)[N / 2]) {
    if constexpr (N >= 8) {
#pragma unroll
        for (int q = 0; q < N / 8; ++q) {
            const u32x4 v = ldg(reinterpret_cast<const u32x4 *>(p) + q);
            w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
        }
    } else if constexpr (N == 4) {
        const u32x2 v = ldg(reinterpret_cast<const u32x2 *>(p));
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = ldg(reinterpret_cast<const uint32_t *>(p));
    }
}

// Ranks [k_off, k_off + 4 NQ) of a child of rank rs (NQ a power of two up to
// 16; the whole rank, or one half of rank 32 or 64 when the V^T x work of a
// slice is split over two workgroups). Thread (rank quad kc, group grp) takes
// the M = 2 NQ consecutive inputs [grp M, grp M + M) of the slice: it loads
// V[i][k_off + 4kc .. + 4) of each as an 8-byte piece and the 8 tokens' x values
// of the run as whole vectors, all in flight together (in chunks of at most 16
// inputs), with no LDS staging. The G = 256 / NQ group sums of each (rank,
// token) are added in a fixed order: 16-lane row sums (DPP), then the rows of a
// rank quad in row order through LDS.
template <int NQ>
__device__ void vtx_quads(const Skinny &g, float *smem, int c, int t0, int tn, int i0, int len, int sl, int k_off,
                          int rs) {
    constexpr int r = 4 * NQ, G = kThreads / NQ, M = kSkVtxSlice / G, MC = M < 16 ? M : 16;
    constexpr int RPQ = G / 16;                                           // 16-lane rows per rank quad
    const int tid = threadIdx.x, kc = tid / G, grp = tid % G;
    const uint16_t *V = g.ch[c].V + (size_t)i0 * rs + k_off + 4 * kc;
    float acc[4][kSkVtxTok];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < kSkVtxTok; ++t) acc[e][t] = 0.f;
#pragma unroll 1
    for (int m0 = 0; m0 < M; m0 += MC) {
        const int ib = grp * M + m0;                                      // first input of the run
        // Runs start at multiples of MC inside the slice; a run past the end of
        // the input axis re-reads the last one (its rows are zeroed below).
        const int ibc = min(ib, ((len - 1) / MC) * MC);
        u32x2 vq[MC];
#pragma unroll
        for (int u = 0; u < MC; ++u) vq[u] = ldg(reinterpret_cast<const u32x2 *>(V + (size_t)min(ib + u, len - 1) * rs));
        uint32_t xw[kSkVtxTok][MC / 2];
#pragma unroll
        for (int t = 0; t < kSkVtxTok; ++t)
            load_x_run<MC>(g.x + (size_t)(t0 + min(t, tn - 1)) * g.d_in + i0 + ibc, xw[t]);
        // Inputs come in pairs (len is a multiple of 8): products on packed bf16
        // pairs, v_dot2 (each product exact in fp32, added to the fp32 sum).
        const bool run_ok = ib == ibc;
#pragma unroll
        for (int u = 0; u < MC; u += 2) {
            const bool in = run_ok && ib + u < len;
            // V[u][4kc + e] and V[u+1][4kc + e] packed, for e = 0..3.
            const uint32_t a = vq[u].x, b = vq[u + 1].x, c2 = vq[u].y, d = vq[u + 1].y;
            const uint32_t vp[4] = {(a & 0xFFFFu) | (b << 16), (a >> 16) | (b & 0xFFFF0000u),
                                    (c2 & 0xFFFFu) | (d << 16), (c2 >> 16) | (d & 0xFFFF0000u)};
#pragma unroll
            for (int t = 0; t < kSkVtxTok; ++t) {
                const uint32_t xp = (in && t < tn) ? xw[t][u >> 1] : 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e][t] = dot2(vp[e], xp, acc[e][t]);
            }
        }
    }
    // Row sums (all 32 first, so that their DPP chains interleave); lane 0 of
    // each 16-lane row stores its row's 32 values.
    float *red = smem;                                                    // [16 rows][kVtxRedLd]
    const int row16 = tid >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < kSkVtxTok; ++t) acc[e][t] = row_sum16(acc[e][t]);
    if ((tid & 15) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int t = 0; t < kSkVtxTok; ++t) red[row16 * kVtxRedLd + e * kSkVtxTok + t] = acc[e][t];
    }
    __syncthreads();
    for (int it = tid; it < r * tn; it += kThreads) {
        const int t = it / r, k = it - t * r, q = k >> 2, e = k & 3;
        float sum = red[(q * RPQ) * kVtxRedLd + e * kSkVtxTok + t];
#pragma unroll
        for (int sub = 1; sub < RPQ; ++sub) sum += red[(q * RPQ + sub) * kVtxRedLd + e * kSkVtxTok + t];
        g.vpart[(((size_t)sl * g.n_ch + c) * g.T + t0 + t) * kMaxRank + k_off + k] = sum;
    }
}

// Any rank: thread (group, rank k) sums rows grp, grp + G, ... one element at a time.
__device__ void vtx_any(const Skinny &g, float *smem, int c, int r, int t0, int tn, int i0, int len, int sl) {
    u32x4 *xs = reinterpret_cast<u32x4 *>(smem);
    float *vred = smem + kSkVtxSlice * 4;                                  // [kThreads][kSkVtxTok + 1]
    const int tid = threadIdx.x;
    stage_x(g, xs, t0, tn, i0, len);
    __syncthreads();
    int rp = 1;
    while (rp < r) rp <<= 1;
    const int k = tid & (rp - 1), grp = tid / rp, G = kThreads / rp;
    float acc[kSkVtxTok];
#pragma unroll
    for (int t = 0; t < kSkVtxTok; ++t) acc[t] = 0.f;
    if (k < r) {
        const uint16_t *V = g.ch[c].V + (size_t)i0 * r + k;
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
    for (int t = 0; t < kSkVtxTok; ++t) vred[tid * (kSkVtxTok + 1) + t] = acc[t];
    __syncthreads();
    for (int it = tid; it < r * tn; it += kThreads) {
        const int t = it / r, kk = it - t * r;
        float sum = 0.f;
        for (int gg = 0; gg < G; ++gg) sum += vred[(gg * rp + kk) * (kSkVtxTok + 1) + t];
        g.vpart[(((size_t)sl * g.n_ch + c) * g.T + t0 + t) * kMaxRank + kk] = sum;
    }
}

// Workgroup (child, token block, slice[, rank half]): with vsplit == 2 (every
// child with V^T x has rank 32 or 64) two workgroups share a slice, each taking
// half of the rank quads, so that each has half the vector-ALU work.
__device__ void vtx_wg(const Skinny &g, float *smem, int wgi) {
    const int n_tb = (g.T + kSkVtxTok - 1) / kSkVtxTok;
    const int hs = wgi % g.vsplit;
    wgi /= g.vsplit;
    const int sl = wgi % g.n_vsl, tb = (wgi / g.n_vsl) % n_tb, cj = wgi / (g.n_vsl * n_tb);
    const int c = cj == 0 ? g.vtx_ch[0] : cj == 1 ? g.vtx_ch[1] : g.vtx_ch[2];   // uniform
    const int r = g.ch[c].r;
    const int t0 = tb * kSkVtxTok, tn = min(kSkVtxTok, g.T - t0);
    const int i0 = sl * kSkVtxSlice, len = min(kSkVtxSlice, g.d_in - i0);
    switch (r) {
        case 4: vtx_quads<1>(g, smem, c, t0, tn, i0, len, sl, 0, 4); break;
        case 8: vtx_quads<2>(g, smem, c, t0, tn, i0, len, sl, 0, 8); break;
        case 16: vtx_quads<4>(g, smem, c, t0, tn, i0, len, sl, 0, 16); break;
        case 32:
            if (g.vsplit == 2)
                vtx_quads<4>(g, smem, c, t0, tn, i0, len, sl, 16 * hs, 32);
            else
                vtx_quads<8>(g, smem, c, t0, tn, i0, len, sl, 0, 32);
            break;
        case 64:
            if (g.vsplit == 2)
                vtx_quads<8>(g, smem, c, t0, tn, i0, len, sl, 32 * hs, 64);
            else
                vtx_quads<16>(g, smem, c, t0, tn, i0, len, sl, 0, 64);
            break;
        default: vtx_any(g, smem, c, r, t0, tn, i0, len, sl); break;
    }
}

// LDS: the V^T x workgroups' staged x slice and per-thread sums, or the main
// workgroups' four wave slots.
constexpr int kVtxSmemFloats = kSkVtxSlice * 4 + kThreads * kVtxRedLd;
template <int MT, int P>
constexpr int smem_floats() {
    constexpr int a = kVtxSmemFloats > 4 * P * MT * 16 * kWave ? kVtxSmemFloats : 4 * P * MT * 16 * kWave;
    return a > main_lds_floats<MT, P>() ? a : main_lds_floats<MT, P>();
}

template <int MT, int P>
__global__ __launch_bounds__(kThreads) void skinny_main(Skinny g) {
    __shared__ __attribute__((aligned(16))) float smem[smem_floats<MT, P>()];
    const int b = blockIdx.x;
    if (b < g.n_vtx_wg)
        vtx_wg(g, smem, b);
    else
        main_wg<MT, P>(g, smem, b - g.n_vtx_wg);
}

// ---- launch 2: epilogue -------------------------------------------------------------------

// Workgroup: kEpiRows consecutive outputs x all tokens; thread (output o, token
// group tg) handles tokens tg, tg + 8, ... Every load is issued first: the split
// partials of its outputs, s, its U row, and the V^T x slice partials the
// workgroup needs (summed in slice order into LDS). After one barrier each
// thread forms, on the vector ALUs in fp32,
//   y[t,o] = bf16( s[o] * sum_sp part[sp][t][o] + sum_k U[o,k] vtx[t,k] )
// (splits in split order, ranks in ascending order); pair mode writes
// bf16(gelu_tanh(g) * u).
constexpr int kEpiRows = 32;
constexpr int kEpiGroups = kThreads / kEpiRows;     // 8 token groups

// NVS: a bucket (4 or kSkMaxDin / kSkVtxSlice) holding the call's V^T x slices;
// the slice loads past n_vsl re-read the last slice and are not added.
template <int P, int J, int SMAX, int RB, int NVS>
__global__ __launch_bounds__(kThreads) void skinny_epilogue(Skinny g) {
    __shared__ float vs[kMaxChildren][kSkMaxTok][kMaxRank];
    const int tid = threadIdx.x;
    const int ol = tid % kEpiRows, tg = tid / kEpiRows;
    const int o0 = blockIdx.x * kEpiRows;
    const int row = o0 + ol, rowc = min(row, g.rows - 1);

    // ---- loads ----
    // Split partials: pm[p][j][sp] for token tg + 8 j.
    float pm[P][J][SMAX];
    const size_t pstride = (size_t)P * g.T * g.rows;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = min(tg + kEpiGroups * j, g.T - 1);
#pragma unroll
            for (int sp = 0; sp < SMAX; ++sp)
                pm[p][j][sp] = ldg(g.part + (size_t)min(sp, g.S - 1) * pstride + ((size_t)p * g.T + t) * g.rows + rowc);
        }
    // s and the U row (packed bf16 pairs) of each of the thread's outputs.
    int cidx[P], rk[P];
    float sv[P];
    uint32_t uw[P][RB / 2];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int ci = P == 2 ? p : child_of(g, rowc);
        const int col0 = P == 2 ? 0 : blend3(ci, 0, g.ch[1].col0, g.ch[2].col0);
        const int r = blend3(ci, g.ch[0].r, g.n_ch > 1 ? g.ch[1].r : 0, g.n_ch > 2 ? g.ch[2].r : 0);
        cidx[p] = ci;
        rk[p] = r;
        const uint64_t sb = P == 2 ? ptr_of(g.ch[p].s) : blend3(ci, ptr_of(g.ch[0].s), ptr_of(g.ch[1].s), ptr_of(g.ch[2].s));
        const float *sp = reinterpret_cast<const float *>(sb);
        const float s_raw = ldg(sp ? sp + (rowc - col0) : reinterpret_cast<const float *>(g.x));
        sv[p] = sp ? s_raw : 1.f;
        const uint64_t ub = P == 2 ? ptr_of(g.ch[p].U) : blend3(ci, ptr_of(g.ch[0].U), ptr_of(g.ch[1].U), ptr_of(g.ch[2].U));
        const uint16_t *Urow = reinterpret_cast<const uint16_t *>(ub ? ub : ptr_of(g.x)) + (size_t)(rowc - col0) * r;
        if ((r & 7) == 0) {
            // 16-byte pieces of the row; pieces past r re-read the last one (never used).
#pragma unroll
            for (int q = 0; q < RB / 8; ++q) {
                const u32x4 v = ldg(reinterpret_cast<const u32x4 *>(Urow) + min(q, max(r / 8 - 1, 0)));
                uw[p][4 * q] = v.x; uw[p][4 * q + 1] = v.y; uw[p][4 * q + 2] = v.z; uw[p][4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < RB / 2; ++q) {
                const uint32_t lo = ldg(Urow + min(2 * q, r - 1)), hi = ldg(Urow + min(2 * q + 1, r - 1));
                uw[p][q] = lo | (hi << 16);
            }
        }
    }

    // vtx of the children these outputs belong to: items (child, token, 4 ranks),
    // each the sum of its slice partials in slice order, into vs.
    const int c_lo = P == 2 ? 0 : child_of(g, min(o0, g.rows - 1));
    const int c_hi = P == 2 ? 1 : child_of(g, min(o0 + kEpiRows - 1, g.rows - 1));
    for (int c = c_lo; c <= c_hi; ++c) {
        const int rc = c == 0 ? g.ch[0].r : c == 1 ? g.ch[1].r : g.ch[2].r;
        const int q4 = (rc + 3) / 4, n_items = g.T * q4;
        for (int item = tid; item < n_items; item += kThreads) {
            const int t = item / q4, k = 4 * (item - t * q4);
            const float *src = g.vpart + ((size_t)c * g.T + t) * kMaxRank + k;
            const size_t sl_stride = (size_t)g.n_ch * g.T * kMaxRank;
            f32x4 v[NVS];
#pragma unroll
            for (int sl = 0; sl < NVS; ++sl)
                v[sl] = ldg(reinterpret_cast<const f32x4 *>(src + (size_t)min(sl, g.n_vsl - 1) * sl_stride));
            f32x4 sum = v[0];
#pragma unroll
            for (int sl = 1; sl < NVS; ++sl)
                if (sl < g.n_vsl) sum += v[sl];
            *reinterpret_cast<f32x4 *>(&vs[c][t][k]) = sum;
        }
    }
    __syncthreads();

    // ---- outputs ----
    if (row >= g.rows) return;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int t = tg + kEpiGroups * j;
        if (t >= g.T) break;
        float val[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float m = pm[p][j][0];
#pragma unroll
            for (int sp = 1; sp < SMAX; ++sp) m += sp < g.S ? pm[p][j][sp] : 0.f;
            // Ranks in ascending order; every slot below the rank bucket RB >= r is
            // visited (the U array is indexed by constants only), those past r add
            // nothing.
            float d = 0.f;
            const float *vt = &vs[P == 2 ? p : cidx[p]][t][0];
#pragma unroll
            for (int q = 0; q < RB / 2; ++q) {
                const float2 v = *reinterpret_cast<const float2 *>(vt + 2 * q);
                const float u0 = 2 * q < rk[p] ? bf16_f(uw[p][q] & 0xFFFFu) : 0.f;
                const float u1 = 2 * q + 1 < rk[p] ? bf16_f(uw[p][q] >> 16) : 0.f;
                d += u0 * (2 * q < rk[p] ? v.x : 0.f);
                d += u1 * (2 * q + 1 < rk[p] ? v.y : 0.f);
            }
            val[p] = sv[p] * m + d;
        }
        const float out = P == 2 ? gelu_tanh_bf16out(val[0]) * val[P - 1] : val[0];
        g.y[(size_t)t * g.ldy + row] = f_bf16(out);
    }
}

template <int P, int J, int SMAX, int NVS>
void launch_epi_r(const Skinny &g, int max_r, hipStream_t stream) {
    const dim3 grid((g.rows + kEpiRows - 1) / kEpiRows);
    if (max_r <= 8)
        hipLaunchKernelGGL((skinny_epilogue<P, J, SMAX, 8, NVS>), grid, dim3(kThreads), 0, stream, g);
    else if (max_r <= 16)
        hipLaunchKernelGGL((skinny_epilogue<P, J, SMAX, 16, NVS>), grid, dim3(kThreads), 0, stream, g);
    else if (max_r <= 32)
        hipLaunchKernelGGL((skinny_epilogue<P, J, SMAX, 32, NVS>), grid, dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL((skinny_epilogue<P, J, SMAX, 64, NVS>), grid, dim3(kThreads), 0, stream, g);
}
template <int P, int J, int SMAX>
void launch_epi(const Skinny &g, int max_r, hipStream_t stream) {
    if (g.n_vsl <= 4)
        launch_epi_r<P, J, SMAX, 4>(g, max_r, stream);
    else
        launch_epi_r<P, J, SMAX, kSkMaxDin / kSkVtxSlice>(g, max_r, stream);
}

template <int MT, int P>
hipError_t launch_mp(const Skinny &g, hipStream_t stream) {
    const int n_main = g.n_rowblk * g.S;
    hipLaunchKernelGGL((skinny_main<MT, P>), dim3(g.n_vtx_wg + n_main), dim3(kThreads), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kSMax = kSkMaxPartials / (P * MT);
    constexpr int J = MT * 32 / kEpiGroups;
    int max_r = 0;
    for (int c = 0; c < g.n_ch; ++c) max_r = g.ch[c].r > max_r ? g.ch[c].r : max_r;
    if (g.S <= 2)
        launch_epi<P, J, 2>(g, max_r, stream);
    else
        launch_epi<P, J, kSMax>(g, max_r, stream);
    return hipGetLastError();
}

}  // namespace

// Splits of the input axis: each wave takes at most the blocks it loads at once
// (four waves per split), unless that needs more partials than the epilogue adds
// (S * P * token blocks <= kSkMaxPartials); then the waves take several rounds.
SkinnyPlan skinny_plan(int rows, int d_in, int T, int P, int n_vtx_ch) {
    SkinnyPlan p;
    p.n_rowblk = (rows + 31) / 32;
    const int nkb = (d_in + kKB - 1) / kKB;
    const int MT = T > 32 ? 2 : 1;
    const int nb = MT == 1 ? (P == 1 ? blocks_at_once<1, 1>() : blocks_at_once<1, 2>())
                           : (P == 1 ? blocks_at_once<2, 1>() : blocks_at_once<2, 2>());
    const int s_max = kSkMaxPartials / (P * MT);   // partials the epilogue holds per output
    int S = (nkb + 4 * nb - 1) / (4 * nb);
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
