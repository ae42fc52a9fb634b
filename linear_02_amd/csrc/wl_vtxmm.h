// V^T x on the matrix cores for the prefill-sized path, as one unit of work
// (32 tokens, one split of the input axis, one child):
//   part[c][split][t][k] = sum over the split's inputs i of x[t][i] V_c[i][k]
// (the first factor of the low-rank correction, "In-kernel reconstruction",
// introduction; formed once per call and shared by every output tile, as in
// the custom-op path). Its consumer, in a later launch, adds the splits in
// split order.
//
// The unit runs on W = 4 or 8 waves: in a launch of its own (k_vtxmm.hip), or
// as extra workgroups of a GEMM launch whose tiles do not need it (k_gemm.hip).
// The split's 64-wide input blocks are dealt to 8 virtual waves in turn
// (block b to virtual wave b % 8, each adding its blocks in increasing order),
// and the 8 sums are added in virtual-wave order, so the bits of every partial
// are the same whatever W is. Per block a wave loads
//   * the x tile (32 tokens x 64 inputs) as 128-byte runs of a token row, 8 rows
//     per load (the memory system serves these far better than the MFMA operand
//     layout), stores it to its own LDS stage with the pieces XOR-swizzled by
//     row, and reads it back as A fragments: lane (n, h) takes token n and
//     inputs [32h + 8j, 32h + 8j + 8) of the block in MFMA step j;
//   * V rows [i0, i0 + 64), one contiguous chunk of 128 r bytes in the [d_in][r]
//     layout, copied into LDS as 16-byte pieces and read back transposed as B
//     fragments (8 inputs of one rank column per lane and step), so no
//     transposed copy of V is ever written to memory.
// The next block's loads are in flight while one is multiplied.
#pragma once
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

constexpr int kVtxKB = 64;                     // inputs per block
constexpr int kVtxVW = 8;                      // virtual waves
constexpr int kVtxXTile = 32 * 8;              // 16-byte pieces of an x tile

// Bytes of one wave's V chunk in LDS: 64 rows of r <= 32 NV ranks, with a
// 64-byte gap before row 32 so that the two half-waves (rows 32 apart) read
// different banks.
template <int NV>
constexpr int vtx_chunk_bytes() { return 64 * 32 * NV * 2 + 64; }
template <int NV>
constexpr int vtx_wave_lds_bytes() { return kVtxXTile * 16 + vtx_chunk_bytes<NV>(); }
// LDS of a unit on W waves: each wave's x tile and V chunk, or (afterwards)
// the 8 virtual waves' sums of one 32-wide rank block.
template <int W, int NV>
constexpr int vtx_unit_lds_bytes() {
    constexpr int a = W * vtx_wave_lds_bytes<NV>(), b = kVtxVW * 16 * kWave * 4;
    return a > b ? a : b;
}

// One unit: token block tb, split sp, child c of job. All W * 64 threads of the
// workgroup call it (it holds workgroup barriers); lds holds at least
// vtx_unit_lds_bytes<W, NV>() bytes. RS: the rank when every child's rank is
// exactly 32 NV (constant offsets for every transposed read), else 0 (the
// rank, at run time); the sums do not depend on it.
template <int W, int NV, int RS>
__device__ __forceinline__ void vtxmm_unit(const VtxMM &job, int tb, int sp, int c, unsigned char *lds) {
    static_assert(kVtxVW % W == 0, "the virtual waves split evenly over the waves");
    constexpr int VPW = kVtxVW / W;
    constexpr int kPieces = 32 * NV * 64 * 2 / 16 / kWave;   // 16-byte V pieces per lane, at most
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = RS ? RS : c == 0 ? job.r[0] : c == 1 ? job.r[1] : job.r[2];
    const u32x4 *vg = reinterpret_cast<const u32x4 *>(c == 0 ? job.V[0] : c == 1 ? job.V[1] : job.V[2]);
    float *out = c == 0 ? job.part[0] : c == 1 ? job.part[1] : job.part[2];
    const int v_total = (job.d_in * r) >> 3;         // 16-byte pieces of all of V
    const int v_pieces = 8 * r, half = 4 * r;        // pieces of one 64-row chunk, of rows 0..31
    const int n = lane & 31, h = lane >> 5;
    const int nch = job.d_in >> 3;
    u32x4 *xt = reinterpret_cast<u32x4 *>(lds + wave * vtx_wave_lds_bytes<NV>());
    unsigned char *chunk = lds + wave * vtx_wave_lds_bytes<NV>() + kVtxXTile * 16;
    const int nkb = (job.d_in + kVtxKB - 1) / kVtxKB;
    const int kb0 = sp * job.kb_per_split, kb1 = min(nkb, kb0 + job.kb_per_split);

    // x: lane l loads token row 8j + l/8, piece l%8 of the block (load j = 0..3).
    const int xr = lane >> 3, xp = lane & 7;
    const u32x4 *xsrc[4];
    bool xok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = tb * 32 + 8 * j + xr;
        xok[j] = t < job.T;
        xsrc[j] = reinterpret_cast<const u32x4 *>(job.x) + (size_t)min(t, job.T - 1) * nch;
    }

    f32x16 acc[VPW][NV];
#pragma unroll
    for (int q = 0; q < VPW; ++q)
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[q][v][e] = 0.f;

    // Every address valid (pieces clamped); x values past d_in or T are zeros, so
    // the V rows past d_in (the next rows of V, or repeated pieces) add nothing.
    auto load = [&](u32x4 (&xa)[4], u32x4 (&vr)[kPieces], int kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = kb * 8 + xp;
            const u32x4 v = ldg(xsrc[j] + min(pc, nch - 1));
            xa[j] = (pc < nch && xok[j]) ? v : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int m = 0; m < kPieces; ++m) vr[m] = ldg(vg + min(kb * v_pieces + m * kWave + lane, v_total - 1));
    };
    auto compute = [&](f32x16 (&ac)[NV], const u32x4 (&xa)[4], const u32x4 (&vr)[kPieces]) {
        // x tile into LDS (swizzled) and back as A fragments.
#pragma unroll
        for (int j = 0; j < 4; ++j) xt[swz<8>(8 * j + xr, xp)] = xa[j];
        __builtin_amdgcn_wave_barrier();
        u32x4 af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = xt[swz<8>(n, 4 * h + j)];
        // V chunk into LDS (piece q at byte 16 q, plus the gap from row 32 on) and
        // back transposed.
#pragma unroll
        for (int m = 0; m < kPieces; ++m) {
            const int q = m * kWave + lane;
            if (q < v_pieces) *reinterpret_cast<u32x4 *>(chunk + 16 * q + (q >= half ? 64 : 0)) = vr[m];
        }
        __builtin_amdgcn_wave_barrier();
        const uint16_t *c16 = reinterpret_cast<const uint16_t *>(chunk);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int k = 32 * v + n;
            const bool k_ok = k < r;
            const int kc = min(k, r - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row0 = 32 * h + 8 * j;
                uint32_t wv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = c16[(row0 + 2 * e) * r + kc + 32 * h];
                    const uint32_t hi = c16[(row0 + 2 * e + 1) * r + kc + 32 * h];
                    wv[e] = k_ok ? (lo | (hi << 16)) : 0u;
                }
                ac[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[j]),
                                                                 __builtin_bit_cast(bf16x8, u32x4{wv[0], wv[1], wv[2], wv[3]}),
                                                                 ac[v], 0, 0, 0);
            }
        }
        __builtin_amdgcn_wave_barrier();   // this block's LDS reads are done before the next block's stores
    };
#pragma unroll
    for (int q = 0; q < VPW; ++q) {
        const int vw = wave + W * q;
        const int nb = kb1 > kb0 + vw ? (kb1 - kb0 - vw + kVtxVW - 1) / kVtxVW : 0;
        if (nb > 0) {
            u32x4 xA[4], vA[kPieces], xB[4], vB[kPieces];
            load(xA, vA, kb0 + vw);
            for (int i = 0; i < nb; i += 2) {
                load(xB, vB, kb0 + vw + kVtxVW * min(i + 1, nb - 1));   // a repeat past the end
                compute(acc[q], xA, vA);
                if (i + 1 >= nb) break;
                load(xA, vA, kb0 + vw + kVtxVW * min(i + 2, nb - 1));
                compute(acc[q], xB, vB);
            }
        }
    }

    // Virtual-wave order through LDS, one 32-wide rank block at a time, then this
    // split's partial. Lane holds rank column k = 32v + n and tokens
    // 8*(e/4) + 4h + (e%4) of the block.
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < VPW; ++q)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[((wave + W * q) * 16 + e) * kWave + lane] = acc[q][v][e];
        __syncthreads();
        for (int it = tid; it < 16 * kWave; it += W * kWave) {
            const int l = it % kWave, e = it / kWave;
            float sum = red[e * kWave + l];
            for (int w = 1; w < kVtxVW; ++w) sum += red[(w * 16 + e) * kWave + l];
            const int tt = tb * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3), k = 32 * v + (l & 31);
            if (tt < job.T && k < r) out[((size_t)sp * job.T + tt) * r + k] = sum;
        }
    }
}

}  // namespace wl
