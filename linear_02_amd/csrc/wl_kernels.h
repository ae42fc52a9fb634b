// Kernel argument blocks and launchers of the reconstruct-and-project linear.
// Shared by the host dispatcher (wl_abi.cpp) and the kernel translation units.
//
// Every launcher only enqueues work on `stream` and returns the launch status;
// the host dispatcher has already checked every shape, pointer and size the
// kernels rely on (the limits below).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wl {

constexpr int kMaxChildren = 3;   // Q, K, V
constexpr int kMaxRank = 64;

// One theta bundle placed at output columns [col0, col0 + d_out) of y.
struct Child {
    const uint16_t *W0;   // bf16 [d_out][d_in]
    const float *s;       // fp32 [d_out], or null: every s[o] is 1
    const uint16_t *U;    // bf16 [d_out][r]  (r > 0)
    const uint16_t *V;    // bf16 [d_in][r]   (r > 0)
    const float *vtx;     // fp32 [T][r]: V^T x of this child (workspace); r > 0
    int r, d_out, col0;
};

// ---------------------------------------------------------------------------
// V^T x for up to three children that share one input x.
//   vtx[c][t][k] = sum_i V_c[i][k] * x[t][i]         (fp32)
// The input axis is cut into n_slices slices; each workgroup reduces one slice
// for one child and a block of tokens, writes its partial sums, and the last
// workgroup of that (child, token block) to finish adds the partials in slice
// order (deterministic). counter[] must be zero on entry and is zero again when
// the kernel has finished.
struct VtxJob {
    const uint16_t *x;                 // bf16 [T][d_in]
    const uint16_t *V[kMaxChildren];   // bf16 [d_in][r_c]
    float *vtx[kMaxChildren];          // fp32 [T][r_c]
    int r[kMaxChildren];
    int n_ch, d_in, T;
    int n_slices, slice_len;           // slice_len: multiple of 8, n_slices*slice_len >= d_in
    float *partial;                    // fp32 [n_tb][n_ch][n_slices][kVtxTok][kMaxRank]
    uint32_t *counter;                 // [n_tb][n_ch]
};
constexpr int kVtxTok = 8;             // tokens per workgroup
constexpr int kVtxMaxSlice = 1024;     // input elements per slice (x slice staged in LDS)
hipError_t launch_vtx(const VtxJob &job, hipStream_t stream);

// ---------------------------------------------------------------------------
// Decode-sized GEMV over the concatenated rows of up to three children:
//   y[t][col0_c + o] = bf16( s_c[o] * sum_i W0_c[o][i] x[t][i] + sum_k U_c[o][k] vtx_c[t][k] )
// for tokens [t0, t0 + tt) of one pass (tt <= kGemvTok).
// Pair mode (the MLP's gate/up): ch[0] = gate, ch[1] = up with equal shapes, and
//   y[t][o] = bf16( gelu_tanh(gate value) * up value ).
struct Gemv {
    Child ch[kMaxChildren];
    int n_ch;
    int pair;             // 1: gate/up pair mode
    int d_in;
    int rows;             // total output rows (sum of d_out; d_ff in pair mode)
    int ldy;              // row stride of y (elements)
    int T;
    const uint16_t *x;    // bf16 [T][d_in]
    uint16_t *y;          // bf16 [T][ldy]
};
constexpr int kGemvTok = 4;                   // tokens per pass
constexpr int kGemvMaxStaged = 32768;         // tt * d_in elements staged in LDS (64 KiB)
hipError_t launch_gemv(const Gemv &g, int n_cu, hipStream_t stream);

// ---------------------------------------------------------------------------
// Matrix-core GEMM for larger token counts, same result as Gemv (including pair
// mode). Output tiles never span two children.
struct Gemm {
    Child ch[kMaxChildren];
    int n_ch;
    int pair;
    int d_in;
    int ldy;
    int T;
    const uint16_t *x;    // bf16 [T][d_in]
    uint16_t *y;          // bf16 [T][ldy]
};
hipError_t launch_gemm(const Gemm &g, hipStream_t stream);

// ---------------------------------------------------------------------------
// Effective weight: W_eff[o][i] = bf16( s[o] * W0[o][i] + sum_k U[o][k] V[i][k] ).
struct Weff {
    const uint16_t *W0;
    const float *s;
    const uint16_t *U, *V;
    uint16_t *W_eff;
    int d_in, d_out, r;
};
hipError_t launch_weff(const Weff &w, hipStream_t stream);

}  // namespace wl
