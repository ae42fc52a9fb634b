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
    const float *vtx;     // matrix-core regime: V^T x split partials, fp32 [vtx_splits][T][r]
    int vtx_splits;
    int r, d_out, col0;
};

// V^T x of up to three children on the matrix cores (matrix-core regime):
//   part[c][split][t][k] = sum over the split's inputs i of x[t][i] V[c][i][k],
// splits of kb_per_split 64-wide blocks of the input axis, added in order by the GEMM.
// vtxmm_splits gives the split count for an input width and the largest rank.
constexpr int kVtxMaxSplits = 8;
struct VtxMM {
    const uint16_t *x;                 // bf16 [T][d_in]
    const uint16_t *V[kMaxChildren];   // bf16 [d_in][r_c], 1 <= r_c <= kMaxRank
    float *part[kMaxChildren];         // fp32 [S][T][r_c]
    int r[kMaxChildren];
    int n, d_in, T, S, kb_per_split;
};
int vtxmm_splits(int d_in, int max_r);
hipError_t launch_vtxmm(const VtxMM &job, hipStream_t stream);

// ---------------------------------------------------------------------------
// V^T x slice partials for up to three children that share one input x
// (decode regime, when the slices are computed by a launch of their own):
//   partial[c][slice][t][k] = sum over the slice's inputs i of V_c[i][k] * x[t][i]
// Plain stores; the consumer, launched after on the same stream, adds the
// slices in order.
struct VtxJob {
    const uint16_t *x;                 // bf16 [T][d_in]
    const uint16_t *V[kMaxChildren];   // bf16 [d_in][r_c]
    float *partial[kMaxChildren];      // fp32 [n_slices][ld_T][r_c]
    int r[kMaxChildren];
    int n_ch, d_in, T;
    int ld_T;                          // tokens per slice block of partial (>= T)
    int n_slices, slice_len;           // slice_len: multiple of 8, <= kVtxMaxSlice
};
constexpr int kVtxMaxSlice = 1024;     // input elements per slice (x slice staged in LDS)
hipError_t launch_vtx(const VtxJob &job, hipStream_t stream);

// ---------------------------------------------------------------------------
// Decode-sized projection, one launch per pass of tt <= 8 tokens [t0, t0 + tt):
//   y[t][col0_c + o] = bf16( s_c[o] * sum_i W0_c[o][i] x[t][i] + sum_k U_c[o][k] vtx_c[t][k] )
// over the concatenated rows of up to three children. Pair mode (the MLP's
// gate/up): ch[0] = gate, ch[1] = up with equal shapes, and
//   y[t][o] = bf16( gelu_tanh(gate value) * up value ).
// vtx comes from slice partials written by a V^T x launch just before
// (kVtxPartials) or by the first workgroups of the same launch (kVtxInLaunch).
// kVtxInLaunch: the slice partials are computed by the first n_prod workgroups of
// the projection's own launch and stored as tagged 64-bit words (the launch's
// tag beside the value); the other workgroups stream W0, then read the words
// until each carries their launch's tag (bounded). The tag comes from ticket
// counters in the workspace's sync area (see kSyncBytes), which also holds the
// words, so no word is ever reset. A workgroup whose wait runs out computes V^T x itself.
enum { kVtxNone = 0, kVtxPartials = 2, kVtxInLaunch = 3 };
// The sync area, the first kSyncBytes of every workspace, 64-bit words:
//   [0, kSyncCopies)          ticket counters, each advanced by exactly
//                             kSyncStride per launch that hands words over
//                             in-launch, so that ticket / kSyncStride is the
//                             launch's generation in every workgroup
//   kSyncFallbackWord         count of workgroups that computed V^T x themselves
//   from kSyncTaggedOffset    the tagged V^T x slice words, kGemvTaggedPerChild
//                             per child slot (kSyncTaggedChildren slots)
//   from kSyncFinalOffset     the tagged complete V^T x words, one per (child,
//                             token, k) item (two-level hand-off),
//                             kSyncFinalPerChild per child slot
//   from kSyncHxOffset        the one-launch MLP's h, exchanged between the
//                             workgroups of a slice (kSyncHxWords)
//   from kSyncPartOffset      the tagged partial outputs of the one-launch MLP
//                             (kSyncPartWords)
// Zero before first use (wl_workspace_init); never reset afterwards. Each
// launch clears one word of the tagged areas that is not its own (walking
// through the kSweepWords words in turn), so that no word keeps a tag for the
// 2^32 - 1 generations after which tags repeat.
constexpr int kSyncCopies = 64;
constexpr unsigned long long kSyncStride = 1ull << 24;
constexpr int kSyncFallbackWord = 511;
constexpr size_t kSyncTaggedOffset = 4096;
constexpr int kSpinLimit = 1 << 12;   // reads of a group of tagged words before a workgroup computes V^T x itself
constexpr int kGemvMaxTok = 8;                // tokens per pass
constexpr int kGemvMaxDin = 32768;            // widest input of the decode kernel
constexpr int kGemvMaxSlices = 64;
constexpr size_t kGemvPartialPerChild = (size_t)kGemvMaxSlices * kGemvMaxTok * kMaxRank;
// The in-launch hand-off serves passes of up to kInLaunchMaxTok tokens (measured:
// at 8 tokens the producer code's registers cost the MLP kernels more than the
// separate V^T x launch it saves).
constexpr int kInLaunchMaxTok = 4;
constexpr size_t kGemvTaggedPerChild = (size_t)kGemvMaxSlices * kInLaunchMaxTok * kMaxRank;
constexpr int kSyncTaggedChildren = 8;
constexpr size_t kSyncFinalOffset = kSyncTaggedOffset + kSyncTaggedChildren * kGemvTaggedPerChild * 8;
constexpr size_t kSyncFinalPerChild = (size_t)kInLaunchMaxTok * kMaxRank;
constexpr size_t kSyncHxOffset = kSyncFinalOffset + kSyncTaggedChildren * kSyncFinalPerChild * 8;
constexpr size_t kSyncHxWords = (size_t)1 << 15;
constexpr size_t kSyncPartOffset = (kSyncHxOffset + kSyncHxWords * 8 + 65535) / 65536 * 65536;
constexpr size_t kSyncPartWords = (size_t)1 << 20;
constexpr size_t kSyncBytes = kSyncPartOffset + kSyncPartWords * 8;
constexpr size_t kSweepWords = (kSyncBytes - kSyncTaggedOffset) / 8;

// Clears the sync area (n_words 64-bit words at sync) with a fill kernel.
hipError_t launch_sync_clear(unsigned long long *sync, size_t n_words, hipStream_t stream);

// The static workspace of wl_linear_static: its size per device, and its
// address on the current device. The first request on a device looks the
// address up and enqueues, on `stream`, a fill kernel that clears the sync area.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(hipStream_t stream, void **out);

struct GemvF {
    Child ch[kMaxChildren];
    int n_ch;
    int pair;             // 1: gate/up pair mode
    int d_in;
    int rows;             // output rows (sum of d_out; d_ff in pair mode)
    int ldy;              // row stride of y (elements)
    int T, t0;            // all tokens, first token of this pass
    const uint16_t *x;    // bf16 [T][d_in]
    uint16_t *y;          // bf16 [T][ldy]
    float *partial;       // slice partials, child c at c * kGemvPartialPerChild: fp32 [S][tt][r_c]
    unsigned long long *tagged;   // in-launch tagged words, child c at c * kGemvTaggedPerChild: [S][tt][r_c]
    // set from the plan
    int nseg;             // segments per row (1, 2 or 4)
    int S;                // slices of the partials
    int vmode;            // kVtxNone / kVtxPartials / kVtxInLaunch
    // kVtxInLaunch: workgroup p < n_prod of the grid is a producer, slice p % S of
    // the (p / S)-th child with r > 0 (slice_len inputs per slice, all tt tokens
    // of the pass) into tagged; the other workgroups are the projection's. sync = the workspace's sync area; spin_limit bounds each
    // workgroup's wait. n_prod = 0 in the other modes.
    // two_level: the last producer also adds the slices up (in the gathers' order) and
    // publishes complete V^T x words, so that projection workgroups read one
    // word per item instead of one per (item, slice).
    int n_prod, slice_len, spin_limit, two_level;
    unsigned long long *sync;   // the workspace's sync area (ticket counters)
    unsigned long long *fin;    // two-level: this launch's complete V^T x words (kSyncFinalPerChild per child)
};
struct GemvPlan {
    int nseg = 1, R = 1, n_wg = 1, S = 0, slice_len = 0, vmode = kVtxNone, n_prod = 0, two_level = 0;
};
int gemv_tokens_per_pass(int d_in, int T);
int gemv_slice_len(int d_in);
// allow_inlaunch: the in-launch hand-off may replace a separate V^T x launch
// (at most kInLaunchMaxTok tokens per pass).
GemvPlan gemv_plan(const GemvF &g, int tt, bool allow_inlaunch);
hipError_t launch_gemv(const GemvF &g, const GemvPlan &plan, int tt, hipStream_t stream);

// ---------------------------------------------------------------------------
// The MLP at decode sizes (1 to kInLaunchMaxTok tokens per pass) in one launch.
// The first n_prod workgroups produce the gate/up pair's V^T x slices (the
// in-launch hand-off of GemvF). The intermediate axis is cut into slices of
// kMlpSlice rows, each taken by P workgroups: part p forms, for the pass's
// tokens, h[t][i] = bf16( gelu_tanh(gate[t][i]) * up[t][i] ) for its kMlpSlice /
// P rows of the slice, and the slice's workgroups exchange their h rows through
// tagged words. Part p then forms the slice's share of down for its d_out / P
// output rows o,
//   p_j[t][o] = s_d[o] * sum_{i in j} W0_d[o][i] h[t][i]
//               + sum_k U_d[o][k] * sum_{i in j} V_d[i][k] h[t][i]
// (down split along its input axis, 128-byte pieces of each row), stored as
// tagged words; groups of kMlpGroup outputs are added over the slices in slice
// order and rounded once: y[t][o] = bf16( sum_j p_j[t][o] ). A wait that runs
// out computes what it waited for itself, with the same arithmetic.
constexpr int kMlpSlice = 64;        // intermediate rows per slice (down inputs, 128 bytes)
constexpr int kMlpGroup = 8;         // outputs per reduction group
constexpr int kMlpMaxSlices = 256;   // slices
constexpr int kMlpDownPasses = 18;   // down rows per workgroup <= kMlpDownPasses x 32 (held in registers)
constexpr int kMlpAutoMaxTok = 2;    // widest pass the automatic regime gives the one-launch MLP
struct MlpDec {
    GemvF gu;                        // gate (ch[0]) / up (ch[1]) pair: x, tokens, producers, hand-off
    const uint16_t *W0d, *Ud, *Vd;   // down: bf16 [D][F], [D][rd], [F][rd]
    const float *sd;                 // fp32 [D], or null: every s is 1
    int rd, D, F;
    int NS, P, WR, Dp, NG;           // slices, workgroups per slice, their rows, down rows per part, groups
    uint16_t *y;                     // bf16 [T][D]
    unsigned long long *hx;          // tagged h words [NS][kMlpSlice / 2][tt]
    unsigned long long *part;        // tagged partial words [NG][NS][tt][kMlpGroup]
};
struct MlpPlan {
    int tt = 0, NS = 0, P = 0, Dp = 0, NG = 0, S = 0, slice_len = 0, n_prod = 0;
};
// tt = 0 when the one-launch MLP does not serve this shape.
MlpPlan mlp_dec_plan(int d_model, int F, int d_out, int r_gate, int r_up, int r_down, int T);
hipError_t launch_mlp_dec(const MlpDec &a, const MlpPlan &p, hipStream_t stream);

// ---------------------------------------------------------------------------
// A few tens of tokens (8 < T <= kSkMaxTok), same result as Gemv (including pair
// mode), in two launches: split-K matrix-core products into fp32 partials (and
// V^T x slice partials from extra workgroups of the same launch), then an
// epilogue launch that adds both in order.
constexpr int kSkMaxTok = 64;
constexpr int kSkMaxDin = 8192;
constexpr int kSkMaxPartials = 8;     // split partials x pair x token blocks per output
constexpr int kSkVtxTok = 8;          // tokens per V^T x workgroup
constexpr int kSkVtxSlice = 512;      // inputs per V^T x workgroup
struct Skinny {
    Child ch[kMaxChildren];
    int n_ch;
    int pair;
    int d_in;
    int rows;             // output rows (sum of d_out; d_ff in pair mode)
    int ldy;
    int T;
    const uint16_t *x;    // bf16 [T][d_in]
    uint16_t *y;          // bf16 [T][ldy]
    float *part;          // fp32 [S][P][T][rows]
    float *vpart;         // fp32 [n_vsl][n_ch][T][kMaxRank]
    // plan
    int S, n_rowblk, kb_per_split, n_vsl, n_vtx_wg;
    int vsplit;                 // V^T x workgroups per (child, token block, slice): 1, or 2
                                // when every child with r > 0 has r = 32 or 64
    int vtx_ch[kMaxChildren];   // children with r > 0, in order
};
struct SkinnyPlan {
    int S = 1, n_rowblk = 0, kb_per_split = 0, n_vsl = 0, n_vtx_wg = 0;
};
SkinnyPlan skinny_plan(int rows, int d_in, int T, int P, int n_vtx_ch);
hipError_t launch_skinny(const Skinny &g, hipStream_t stream);

// ---------------------------------------------------------------------------
// Matrix-core GEMM for larger token counts, same result as Gemv (including pair
// mode); V^T x comes from the split partials of a VtxMM launch just before.
// Output tiles never span two children.
struct Gemm {
    Child ch[kMaxChildren];
    int n_ch;
    int pair;
    int d_in;
    int ldy;
    int T;
    const uint16_t *x;    // bf16 [T][d_in]
    uint16_t *y;          // bf16 [T][ldy]
    int col_fast;         // tile order within an XCD's band (set by launch_gemm)
    // Split of the input axis (single child, no pair): ksplit workgroups per
    // output tile, each over kb_per_split 64-wide steps, writing fp32 partials
    // part[ksplit][T][d_out]; a second launch adds them in order into y.
    // ksplit = 1: no split (part unused).
    int ksplit;
    int kb_per_split;
    float *part;
    // Split path only (1 < ksplit <= kRedMaxSplits, one child with 0 < r <= 32): n_prod > 0 moves the
    // rank term out of the tiles into the reduction; the launch then also runs
    // n_prod V^T x units of job (one split: job.S = 1, token block fastest),
    // workgroups after the tiles, writing the child's vtx.
    VtxMM job;
    int n_prod;
};
constexpr int kRedMaxSplits = 4;   // splits of the input axis the rank-term reduction takes
struct GemmSplit {
    int ksplit, kb_per_split;
};
// The split used for a GEMM-regime projection of `rows` outputs (n_ch children,
// pair or not) at T tokens; the same plan sizes the workspace.
GemmSplit gemm_split_plan(int T, int d_in, int rows, int n_ch, int pair);
hipError_t launch_gemm(const Gemm &g, hipStream_t stream);

// ---------------------------------------------------------------------------
// The fp32 variant (W0, U, V, x, y in binary32; s fp32).
struct F32Child {
    const float *W0;      // [d_out][d_in]
    const float *s;       // [d_out], or null: every s[o] is 1
    const float *U;       // [d_out][r]  (r > 0)
    const float *vtx;     // [T][r]: V^T x, complete (r > 0)
    int r, d_out, col0;
};
// One projection over shared x: children side by side in y (ldy = total width),
// or the gate/up pair (pair = 1, y = h = gelu_tanh(gate) * up).
struct F32Proj {
    F32Child ch[kMaxChildren];
    int n_ch, pair, d_in, T, ldy;
    const float *x;       // [T][d_in]
    float *y;             // [T][ldy]
};
constexpr int kF32GemvMaxTok = 8;   // T above this runs on the matrix cores
hipError_t launch_f32_gemv(const F32Proj &g, hipStream_t stream);
hipError_t launch_f32_gemm(const F32Proj &g, hipStream_t stream);
// V^T x of up to three children: slice partials part[c] ([n_slices][T][r_c])
// then vtx[c] ([T][r_c]) with the slices added in order (two launches).
constexpr int kF32VtxSlice = 256;   // inputs per slice
struct F32Vtx {
    const float *x;                 // [T][d_in]
    const float *V[kMaxChildren];   // [d_in][r_c]
    float *part[kMaxChildren];
    float *vtx[kMaxChildren];
    int r[kMaxChildren];            // 1 <= r_c <= kMaxRank
    int n_ch, d_in, T, n_slices;    // n_slices = f32_vtx_slices(d_in)
};
int f32_vtx_slices(int d_in);
hipError_t launch_f32_vtx(const F32Vtx &job, hipStream_t stream);
struct WeffF32 {
    const float *W0, *s, *U, *V;
    float *W_eff;
    int d_in, d_out, r;
};
hipError_t launch_weff_f32(const WeffF32 &w, hipStream_t stream);

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
// Up to kWeffBatchMax projections in one launch; tiles_end[p] = tiles of
// entries 0..p (weff_tiles of each), n >= 1 entries.
constexpr int kWeffBatchMax = 8;
struct WeffBatch {
    Weff w[kWeffBatchMax];
    int tiles_end[kWeffBatchMax];
    int n;
};
int weff_tiles(int d_in, int d_out);
hipError_t launch_weff_batch(const WeffBatch &bt, hipStream_t stream);

// ---------------------------------------------------------------------------
// Relative Frobenius error of bf16 R against bf16 W (n elements each): fp64
// partial sums per workgroup into part[2 * n_wg], then one workgroup writes
// out[0] = ||W - R|| / ||W||.
constexpr int kFrobMaxWorkgroups = 1024;
struct FrobJob {
    const uint16_t *W, *R;
    int64_t n;
    double *part;
    int n_wg;
    double *out;
};
int frob_workgroups(int64_t n);
hipError_t launch_frob(const FrobJob &job, hipStream_t stream);

}  // namespace wl
