// V^T x on the matrix cores for the prefill-sized path:
//   part[c][split][t][k] = sum over the split's inputs i of x[t][i] V_c[i][k]
// (the first factor of the low-rank correction, "In-kernel reconstruction",
// introduction). The GEMM epilogue adds the splits in split order.
//
// x is the A operand, loaded straight from memory into registers: lanes 0..31
// take inputs [0, 32) and lanes 32..63 inputs [32, 64) of a 64-wide block (64
// contiguous bytes per lane), and the MFMA steps pair them up (any assignment of
// the input index to steps gives the same sum). V is the B operand. Its rows
// [i0, i0 + 64) are one contiguous chunk of 128 r bytes in the [d_in][r] layout,
// which a wave copies into LDS as 16-byte pieces and reads back transposed (8
// inputs of one rank column per lane and step), so no transposed copy of V is
// ever written to memory.
//
// Workgroup (32 tokens, split of the input axis, child), W waves: wave w takes
// 64-wide blocks w, w + W, ... of the split; the W accumulators are added in
// wave order through LDS. The split count is chosen so that each wave has about
// four blocks; it stays at 1 or 2 for inputs up to 8192 wide.
#include "wl_device.h"
#include "wl_kernels.h"

namespace wl {

namespace {

constexpr int kKB = 64;

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Bytes of one wave's V chunk in LDS: 64 rows of r <= 32 NV ranks, with a
// 64-byte gap before row 32 so that the two half-waves (rows 32 apart) read
// different banks.
template <int NV>
constexpr int chunk_bytes() { return 64 * 32 * NV * 2 + 64; }

// RS: the LDS row stride in elements when every child's rank is exactly 32 NV
// (constant offsets for every transposed read), else 0 (the rank, at run time).
template <int NV, int W, int RS>
__global__ __launch_bounds__(W * 64) void vtxmm_kernel(VtxMM job) {
    constexpr int kChunk = chunk_bytes<NV>();
    constexpr int kRed = W * NV * 16 * kWave * 4;
    constexpr int kLds = W * kChunk > kRed ? W * kChunk : kRed;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    constexpr int kPieces = 32 * NV * 64 * 2 / 16 / kWave;   // 16-byte V pieces per lane, at most

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tb = blockIdx.x, sp = blockIdx.y, c = blockIdx.z;
    const int r = RS ? RS : c == 0 ? job.r[0] : c == 1 ? job.r[1] : job.r[2];
    const uint16_t *V = c == 0 ? job.V[0] : c == 1 ? job.V[1] : job.V[2];
    float *out = c == 0 ? job.part[0] : c == 1 ? job.part[1] : job.part[2];
    const int n = lane & 31, h = lane >> 5;
    const int nch = job.d_in >> 3;
    const int t = tb * 32 + n;
    const bool t_ok = t < job.T;
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(job.x) + (size_t)min(t, job.T - 1) * nch;
    const u32x4 *vg = reinterpret_cast<const u32x4 *>(V);
    const int v_pieces = 8 * r;                      // 16-byte pieces of one 64-row chunk
    const int v_total = (job.d_in * r) >> 3;         // 16-byte pieces of all of V
    unsigned char *chunk = lds + wave * kChunk;
    const int nkb = (job.d_in + kKB - 1) / kKB;
    const int kb0 = sp * job.kb_per_split, kb1 = min(nkb, kb0 + job.kb_per_split);

    f32x16 acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[v][e] = 0.f;

    // Every address valid (pieces clamped), values past d_in or T zeroed. V pieces
    // past the chunk are loaded from a valid place and never stored.
    auto load = [&](u32x4 (&xa)[4], u32x4 (&vr)[kPieces], int kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = kb * 8 + 4 * h + j;
            const bool in = pc < nch;
            const u32x4 xv = ldg(xrow + min(pc, nch - 1));
            xa[j] = (in && t_ok) ? xv : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int m = 0; m < kPieces; ++m) {
            const int q = kb * v_pieces + m * kWave + lane;
            vr[m] = ldg(vg + min(q, v_total - 1));
        }
    };
    auto compute = [&](const u32x4 (&xa)[4], const u32x4 (&vr)[kPieces], int kb) {
        // Chunk into LDS: piece q at byte 16 q, plus the gap from row 32 on.
        const int half = 4 * r;                       // pieces in rows 0..31
#pragma unroll
        for (int m = 0; m < kPieces; ++m) {
            const int q = m * kWave + lane;
            if (q < v_pieces)
                *reinterpret_cast<u32x4 *>(chunk + 16 * q + (q >= half ? 64 : 0)) = vr[m];
        }
        __builtin_amdgcn_wave_barrier();
        // Rows past d_in hold data of the next rows of V (or repeated pieces) but
        // meet zeros in x, so they add nothing.
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
                acc[v] = mfma(xa[j], u32x4{wv[0], wv[1], wv[2], wv[3]}, acc[v]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        (void)kb;
    };
    const int nb = kb1 > kb0 + wave ? (kb1 - kb0 - wave + W - 1) / W : 0;
    if (nb > 0) {
        u32x4 xA[4], vA[kPieces], xB[4], vB[kPieces];
        load(xA, vA, kb0 + wave);
        for (int i = 0; i < nb; i += 2) {
            load(xB, vB, kb0 + wave + W * min(i + 1, nb - 1));   // a repeat past the end
            compute(xA, vA, kb0 + wave + W * i);
            if (i + 1 >= nb) break;
            load(xA, vA, kb0 + wave + W * min(i + 2, nb - 1));
            compute(xB, vB, kb0 + wave + W * (i + 1));
        }
    }

    // Wave order through LDS, then this split's partial: lane holds rank column
    // k = 32v + n and tokens 8*(e/4) + 4h + (e%4) of the block.
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[((wave * NV + v) * 16 + e) * kWave + lane] = acc[v][e];
    __syncthreads();
    for (int it = tid; it < NV * 16 * kWave; it += W * kWave) {
        const int l = it % kWave, e = (it / kWave) % 16, v = it / (kWave * 16);
        float sum = red[(v * 16 + e) * kWave + l];
        for (int w = 1; w < W; ++w) sum += red[((w * NV + v) * 16 + e) * kWave + l];
        const int tt = tb * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3), k = 32 * v + (l & 31);
        if (tt < job.T && k < r) out[((size_t)sp * job.T + tt) * r + k] = sum;
    }
}

template <int NV, int RS>
constexpr int waves_of() { return NV == 1 && RS ? 16 : 8; }

template <int NV, int RS>
void launch_one(const VtxMM &job, hipStream_t stream) {
    constexpr int W = waves_of<NV, RS>();
    const dim3 grid((job.T + 31) / 32, job.S, job.n);
    hipLaunchKernelGGL((vtxmm_kernel<NV, W, RS>), grid, dim3(W * kWave), 0, stream, job);
}

bool all_rank(const VtxMM &job, int r) {
    for (int c = 0; c < job.n; ++c)
        if (job.r[c] != r) return false;
    return true;
}

}  // namespace

int vtxmm_splits(int d_in, int max_r) {
    // About four blocks per wave of the kernel for ranks of exactly 32 or 64.
    const int nkb = (d_in + kKB - 1) / kKB;
    const int per = 4 * (max_r <= 32 ? waves_of<1, 32>() : waves_of<2, 64>());
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
