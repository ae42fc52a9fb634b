// V^T x on the matrix cores for the prefill-sized path:
//   part[c][split][t][k] = sum over the split's inputs i of x[t][i] V_c[i][k]
// (the first factor of the low-rank correction, "In-kernel reconstruction",
// introduction). The GEMM epilogue adds the splits in split order.
//
// Workgroup (32 tokens, split of the input axis, child): W waves take
// interleaved 64-wide blocks of the split. Per block a wave loads
//   * the x tile (32 tokens x 64 inputs) as 128-byte runs of a token row, 8 rows
//     per load (the memory system serves these far better than the MFMA operand
//     layout), stores it to its own LDS stage with the pieces XOR-swizzled by
//     row, and reads it back as A fragments: lane (n, h) takes token n and
//     inputs [32h + 8j, 32h + 8j + 8) of the block in MFMA step j;
//   * V rows [i0, i0 + 64), one contiguous chunk of 128 r bytes
//     in the [d_in][r] layout, copied into LDS as 16-byte pieces and read back
//     transposed as B fragments (8 inputs of one rank column per lane and step),
//     so no transposed copy of V is ever written to memory.
// The next block's loads are in flight while one is multiplied. The W
// accumulators are added in wave order through LDS.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kKB = 64;
constexpr int kW = 8;                          // waves per workgroup
constexpr int kXTile = 32 * 8;                 // 16-byte pieces of an x tile

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Bytes of one wave's V chunk in LDS: 64 rows of r <= 32 NV ranks, with a
// 64-byte gap before row 32 so that the two half-waves (rows 32 apart) read
// different banks.
template <int NV>
constexpr int chunk_bytes() { return 64 * 32 * NV * 2 + 64; }
template <int NV>
constexpr int wave_lds_bytes() { return kXTile * 16 + chunk_bytes<NV>(); }

// RS: the LDS row stride in elements when every child's rank is exactly 32 NV
// (constant offsets for every transposed read), else 0 (the rank, at run time).
template <int NV, int RS>
__global__ __launch_bounds__(kW * 64) void vtxmm_kernel(VtxMM job) {
    constexpr int kRed = kW * NV * 16 * kWave * 4;
    constexpr int kLds = kW * wave_lds_bytes<NV>() > kRed ? kW * wave_lds_bytes<NV>() : kRed;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    constexpr int kPieces = 32 * NV * 64 * 2 / 16 / kWave;   // 16-byte V pieces per lane, at most

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tb = blockIdx.x, sp = blockIdx.y, c = blockIdx.z;
    const int r = RS ? RS : c == 0 ? job.r[0] : c == 1 ? job.r[1] : job.r[2];
    const u32x4 *vg = reinterpret_cast<const u32x4 *>(c == 0 ? job.V[0] : c == 1 ? job.V[1] : job.V[2]);
    float *out = c == 0 ? job.part[0] : c == 1 ? job.part[1] : job.part[2];
    const int v_total = (job.d_in * r) >> 3;         // 16-byte pieces of all of V
    const int v_pieces = 8 * r, half = 4 * r;        // pieces of one 64-row chunk, of rows 0..31
    const int n = lane & 31, h = lane >> 5;
    const int nch = job.d_in >> 3;
    u32x4 *xt = reinterpret_cast<u32x4 *>(lds + wave * wave_lds_bytes<NV>());
    unsigned char *chunk = lds + wave * wave_lds_bytes<NV>() + kXTile * 16;
    const int nkb = (job.d_in + kKB - 1) / kKB;
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

    f32x16 acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[v][e] = 0.f;

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
    auto compute = [&](const u32x4 (&xa)[4], const u32x4 (&vr)[kPieces]) {
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
                acc[v] = mfma(af[j], u32x4{wv[0], wv[1], wv[2], wv[3]}, acc[v]);
            }
        }
        __builtin_amdgcn_wave_barrier();   // this block's LDS reads are done before the next block's stores
    };
    const int nb = kb1 > kb0 + wave ? (kb1 - kb0 - wave + kW - 1) / kW : 0;
    if (nb > 0) {
        u32x4 xA[4], vA[kPieces], xB[4], vB[kPieces];
        load(xA, vA, kb0 + wave);
        for (int i = 0; i < nb; i += 2) {
            load(xB, vB, kb0 + wave + kW * min(i + 1, nb - 1));   // a repeat past the end
            compute(xA, vA);
            if (i + 1 >= nb) break;
            load(xA, vA, kb0 + wave + kW * min(i + 2, nb - 1));
            compute(xB, vB);
        }
    }

    // Wave order through LDS, then this split's partial. Lane holds rank column
    // k = 32v + n and tokens 8*(e/4) + 4h + (e%4) of the block.
    float *red = reinterpret_cast<float *>(lds);
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[((wave * NV + v) * 16 + e) * kWave + lane] = acc[v][e];
    __syncthreads();
    for (int it = tid; it < NV * 16 * kWave; it += kW * kWave) {
        const int l = it % kWave, e = (it / kWave) % 16, v = it / (kWave * 16);
        float sum = red[(v * 16 + e) * kWave + l];
        for (int w = 1; w < kW; ++w) sum += red[((w * NV + v) * 16 + e) * kWave + l];
        const int tt = tb * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3), k = 32 * v + (l & 31);
        if (tt < job.T && k < r) out[((size_t)sp * job.T + tt) * r + k] = sum;
    }
}

template <int NV, int RS>
void launch_one(const VtxMM &job, hipStream_t stream) {
    const dim3 grid((job.T + 31) / 32, job.S, job.n);
    hipLaunchKernelGGL((vtxmm_kernel<NV, RS>), grid, dim3(kW * kWave), 0, stream, job);
}

bool all_rank(const VtxMM &job, int r) {
    for (int c = 0; c < job.n; ++c)
        if (job.r[c] != r) return false;
    return true;
}

}  // namespace

int vtxmm_splits(int d_in, int max_r) {
    // About four blocks per wave.
    (void)max_r;
    const int nkb = (d_in + kKB - 1) / kKB;
    const int per = 4 * kW;
    const int S = (nkb + per - 1) / per;
    return S < 1 ? 1 : S < kVtxMaxSplits ? S : kVtxMaxSplits;
}

hipError_t launch_vtxmm(const VtxMM &job, hipStream_t stream) {
    int max_r = 0;
    for (int c = 0; c < job.n; ++c) max_r = job.r[c] > max_r ? job.r[c] : max_r;
    if (max_r <= 32) {
        if (all_rank(job, 32)) launch_one<1, 32>(job, stream);
        else launch_one<1, 0>(job, stream);
    } else {
        if (all_rank(job, 64)) launch_one<2, 64>(job, stream);
        else launch_one<2, 0>(job, stream);
    }
    return hipGetLastError();
}

}  // namespace wl
