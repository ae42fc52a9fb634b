/*
 * wl.h: C ABI of the fused reconstruct-and-project linear for AMD MI355X (gfx950).
 *
 * The operation ("In-kernel reconstruction" page, introduction: the
 * reconstruction formula and its per-element expansion):
 *
 *     y[t,o] = s[o] * sum_i W0[o,i] * x[t,i]  +  sum_k U[o,k] * sum_i V[i,k] * x[t,i]
 *
 * i.e. y = s (.) (W0 x) + U (V^T x), computed without ever forming the dense
 * weight diag(s) W0 + U V^T in memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.    Every tensor pointer is a DEVICE pointer on the current HIP device.
 *            The caller allocates and owns every buffer, including the
 *            workspace; the library never allocates or frees memory. What
 *            carries from call to call lives in the caller's workspace (its
 *            sync area, below); the library's own global state is two
 *            process-wide switches for tests and measurements (wl_testing.h).
 * Layout.    All tensors are row-major and contiguous:
 *              W0 [d_out][d_in]   s fp32 [d_out]
 *              U  [d_out][r]      V [d_in][r]
 *              x  [T][d_in]       y [T][d_out]
 *            (the index roles of the per-element expansion; the GEMM form on
 *            the same page, "The GEMM path", multiplies x by W0 transposed, by
 *            V, and the result by U transposed).
 * Dtypes.    A theta's `dtype` sets the element type of its W0, U, V and of
 *            the call's x, y (and of the MLP's h and of W_eff): WL_DTYPE_BF16
 *            or WL_DTYPE_F32 (the custom op "also supports float32", "In-kernel
 *            reconstruction", the custom-op path). s is fp32 in both. The
 *            thetas of one fused call share one dtype. A zero-filled theta is
 *            bf16.
 * Alignment. W0, U, V, x, y and W_eff must be 16-byte aligned, s 4-byte
 *            aligned, the workspace 256-byte aligned. d_in must be a multiple
 *            of 8 (rows are read in 16-byte pieces).
 * Limits.    0 <= r <= 64; d_in, d_out >= 1; T >= 0 (T == 0 is a no-op that
 *            returns WL_OK, and x, y may then be NULL). Sizes are int32 and
 *            every tensor must hold fewer than 2^31 elements.
 * Numerics.  Products accumulate in fp32; the epilogue s[o]*m + U[o,:].vtx is
 *            fp32; a bf16 y is rounded once, round-to-nearest-even ("In-kernel
 *            reconstruction", "The custom-op path": every implementation
 *            accumulates in float32 and casts back to the output dtype); an
 *            fp32 y is the fp32 result. The bf16 matrix-core regime feeds
 *            vtx = V^T x to the matrix cores as a bf16 head plus a bf16
 *            remainder. Results are deterministic from run to
 *            run (no floating-point atomics) but not bit-exact against other
 *            summation orders ("Serve and generate with weightless", "Set the
 *            fast path on NVIDIA": parity is logit parity, not bit equality).
 * Streams.   Every call only enqueues work on `hip_stream` (a hipStream_t;
 *            NULL = the default stream) and returns; errors that happen on the
 *            device surface at the caller's next synchronization.
 * Workspace. Operations that take `ws` need at least wl_workspace_bytes(...)
 *            bytes of device memory. For wl_linear, wl_qkv_fused and
 *            wl_mlp_fused its first WL_SYNC_BYTES bytes are a sync area:
 *            ticket counters and generation-tagged 64-bit words by which the
 *            workgroups of one decode launch hand each other V^T x and partial
 *            outputs ("In-kernel reconstruction", the custom-op path: V^T x
 *            formed once and shared). Before a workspace's first use, and after
 *            anything other than these calls has written its first
 *            WL_SYNC_BYTES, the caller runs wl_workspace_init on it (a kernel,
 *            so it may be captured in a graph); the calls keep the area
 *            consistent from then on. Bytes 4088 to 4095 of the area count
 *            (int64) the decode workgroups that stopped waiting and computed
 *            V^T x themselves (a diagnostic; the result is the same). The rest
 *            of the workspace is scratch whose contents on entry do not matter.
 *            Calls that can run at the same time (different streams) must not
 *            share a workspace.
 * Errors.    Every argument is checked on the host before anything is
 *            enqueued; a fused operation checks all of its thetas first, so an
 *            invalid argument never leaves a partial launch.
 *              WL_ERR_INVALID_ARG  null or misaligned pointer, bad size or
 *                                  shape mismatch, output overlapping an input
 *                                  or the workspace
 *              WL_ERR_UNSUPPORTED  r > 64, or a dtype other than the two
 *              WL_ERR_WORKSPACE    ws_bytes below the required size
 *              WL_ERR_HIP          a kernel launch failed
 *            No call aborts, throws or prints (set the environment variable
 *            WL_LOG to log the regime chosen and every failure to stderr).
 *            wl_last_error() describes the last failure on the calling thread.
 * Devices.   One device per call; nothing here shards across GPUs ("Serve and
 *            generate with weightless", "Supported encodings and devices": the
 *            pages' implementation runs on a single device as well).
 */
#ifndef WL_H
#define WL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WL_ABI_VERSION 6

/* Bytes at the start of a projection workspace that hold the sync area. */
#define WL_SYNC_BYTES 9764864
/* Bytes of the static workspace of wl_linear_static, per device. */
#define WL_STATIC_SCRATCH_BYTES 33554432

typedef enum {
    WL_OK = 0,
    WL_ERR_INVALID_ARG = 1,
    WL_ERR_UNSUPPORTED = 2,
    WL_ERR_HIP = 3,
    WL_ERR_WORKSPACE = 4
} wl_status;

/* One projection's theta bundle ("Serve and generate with weightless",
 * introduction: a shared block W0 per band of layers, a per-row scale s and a
 * low-rank delta U, V of rank r). Several thetas may point at the same W0
 * (band sharing). The library only reads through these pointers. */
/* Element types of W0, U, V, x, y. */
enum { WL_DTYPE_BF16 = 0, WL_DTYPE_F32 = 1 };

typedef struct {
    const void  *W0;   /* dtype [d_out][d_in]                                  */
    const float *s;    /* fp32 [d_out]; NULL means every s[o] is 1              */
    const void  *U;    /* dtype [d_out][r]; ignored (may be NULL) when r == 0   */
    const void  *V;    /* dtype [d_in][r];  ignored (may be NULL) when r == 0   */
    int32_t d_in, d_out, r;
    int32_t dtype;     /* WL_DTYPE_BF16 (0) or WL_DTYPE_F32 (1)                 */
} wl_theta;

/* Operation codes for wl_workspace_bytes. */
enum { WL_OP_LINEAR = 0, WL_OP_QKV = 1, WL_OP_MLP = 2 };

/* Bytes of workspace `op` needs for these thetas at T tokens:
 *   WL_OP_LINEAR: th[0]                      (n_th == 1)
 *   WL_OP_QKV:    th[0..2] = Q, K, V         (n_th == 3)
 *   WL_OP_MLP:    th[0..2] = gate, up, down  (n_th == 3)
 * Returns 0 for invalid arguments (the matching call then fails with the
 * specific status). The value is a multiple of 256 and grows with T. */
size_t wl_workspace_bytes(int32_t op, const wl_theta *const *th, int32_t n_th, int32_t T);

/* The reconstruct-and-project linear ("In-kernel reconstruction",
 * introduction: reconstruction formula and per-element expansion).
 *   th    one theta bundle
 *   x     dtype [T][th->d_in]
 *   y     dtype [T][th->d_out] (written; must not overlap any input)
 *   T     tokens (rows of x)
 *   ws    workspace, ws_bytes >= wl_workspace_bytes(WL_OP_LINEAR, &th, 1, T)
 * With th->r == 0 and th->s == NULL this is the dense product y = x W0^T: the
 * comparator of the precompute-outside path ("Serve and generate with
 * weightless", "Set the fast path on NVIDIA") when W0 is a materialized W_eff. */
wl_status wl_linear(const wl_theta *th, const void *x, void *y, int32_t T,
                    void *ws, size_t ws_bytes, void *hip_stream);

/* wl_linear without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Arguments, result and errors as wl_linear; the
 * workspace is a static device array of WL_STATIC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends. The call
 * allocates nothing. Its first call on a device looks the array up and
 * enqueues on hip_stream a fill kernel that clears the array's sync area,
 * ahead of its own kernels. Every call on a device shares that device's array
 * and the array keeps the last call's contents, so calls that overlap on one
 * device (other streams, other host threads) race and must be serialized by
 * the caller; wl_linear with workspaces of its own does not share it. A call
 * whose workspace would exceed WL_STATIC_SCRATCH_BYTES (the decode and
 * few-token kernels of the Gemma-3 shapes fit; long prefill passes may not)
 * fails with WL_ERR_WORKSPACE before launching anything. */
wl_status wl_linear_static(const wl_theta *th, const void *x, void *y, int32_t T, void *hip_stream);

/* Q/K/V fusion ("In-kernel reconstruction", "Q/K/V fusion"): the three
 * attention projections that read the same x, computed in one pass over the
 * concatenated W0 rows, each child with its own V^T x (a block-diagonal U).
 *   q, k, v   thetas with equal d_in and dtype; ranks, scales and d_out may differ
 *   x         dtype [T][d_in]
 *   y_qkv     dtype [T][q->d_out + k->d_out + v->d_out], columns Q | K | V
 *   ws        ws_bytes >= wl_workspace_bytes(WL_OP_QKV, {q, k, v}, 3, T)
 * Each child's columns equal wl_linear of that child to within rounding. */
wl_status wl_qkv_fused(const wl_theta *q, const wl_theta *k, const wl_theta *v,
                       const void *x, void *y_qkv, int32_t T,
                       void *ws, size_t ws_bytes, void *hip_stream);

/* Fused MLP ("In-kernel reconstruction", "The custom-op path": the fused MLP
 * op runs gate, up, the activation and down as one operation):
 *   g = linear(gate, x), u = linear(up, x)       (fp32, not rounded)
 *   h = round(gelu_tanh(g) * u)                  (rounded once to the dtype:
 *                                                 bf16 RNE, or the fp32 value)
 *   y = linear(down, h)
 * with gelu_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 * Shapes: gate.d_in == up.d_in (= d_model), gate.d_out == up.d_out ==
 * down.d_in (= d_ff), one dtype; x dtype [T][d_model], y dtype [T][down.d_out].
 * h lives in the workspace:
 *   ws_bytes >= wl_workspace_bytes(WL_OP_MLP, {gate, up, down}, 3, T). */
wl_status wl_mlp_fused(const wl_theta *gate, const wl_theta *up, const wl_theta *down,
                       const void *x, void *y, int32_t T,
                       void *ws, size_t ws_bytes, void *hip_stream);

/* The effective weight of the precompute-outside path ("Serve and generate
 * with weightless", "Set the fast path on NVIDIA"):
 *   W_eff[o,i] = round( s[o] * W0[o,i] + sum_k U[o,k] * V[i,k] )
 * W_eff: th->dtype [th->d_out][th->d_in] (bf16: rounded once, RNE; fp32: the
 * fp32 result), written; must not overlap any input.
 * Needs no workspace. */
wl_status wl_materialize_weff(const wl_theta *th, void *W_eff, void *hip_stream);

/* The effective weight of the precompute-outside path ("Serve and generate
 * with weightless", "Set the fast path on NVIDIA") for n projections (a
 * layer's seven, say): wl_materialize_weff for each, in one launch per eight
 * of them instead of one each; the same values, bit for bit.
 * th[j], W_eff[j] for j < n as in wl_materialize_weff, all thetas of one
 * dtype (fp32: one launch per projection); no W_eff may overlap another or
 * any theta's tensors. Every argument is checked before anything is
 * launched. n = 0: nothing to do. Needs no workspace. */
wl_status wl_materialize_weff_batch(const wl_theta *const *th, void *const *W_eff, int32_t n, void *hip_stream);

/* Decode steps ("Throughput" page, "Versus vanilla MAX": at batch 1 a step's
 * dispatches, not its arithmetic, dominate; "Serve and generate with
 * weightless", "Current limits": shared-W0 (G = 1) configurations). A step is a
 * fixed list of wl_linear / wl_qkv_fused / wl_mlp_fused calls that the library
 * records once into a HIP graph and launches with one call.
 *   op   WL_OP_LINEAR (th[0]), WL_OP_QKV (th = Q, K, V) or WL_OP_MLP (th =
 *        gate, up, down); unused th entries are ignored
 *   x, y, T   as in the op's own call (QKV: y is [T][dq + dk + dv]) */
typedef struct {
    int32_t op;
    const wl_theta *th[3];
    const void *x;
    void *y;
    int32_t T;
} wl_call;

/* wl_step_create flag: launch the calls that share their first theta's W0 back
 * to back (groups in order of first appearance, given order within a group),
 * so that a W0 shared by several layers (G = 1) is read while it is still in
 * the caches. Allowed only when no call reads or overwrites another call's
 * output (else WL_ERR_INVALID_ARG); results are the same as in given order. */
enum { WL_STEP_GROUP_SHARED_W0 = 1 };

typedef struct wl_step_s *wl_step;

/* Workspace bytes of a step: the largest of its calls' wl_workspace_bytes
 * (the calls run one after another on one workspace). 0 for invalid calls. */
size_t wl_step_workspace_bytes(const wl_call *calls, int32_t n_calls);

/* Records the calls (1 <= n_calls <= 65536) into a HIP graph, in the given
 * order or as WL_STEP_GROUP_SHARED_W0 regroups them, each exactly as its own
 * entry point would launch it (the regime switch is read now), and
 * instantiates it. Every call is checked as by its own entry point, before
 * anything runs; on an error no step is made and the message names the call.
 * The theta structs and the call array are read only here; the device buffers
 * they and x, y, ws point at must stay allocated while the step exists, and
 * their contents are read or written at each launch (new x values between
 * launches are used). ws: ws_bytes >= wl_step_workspace_bytes, 256-byte
 * aligned, prepared by wl_workspace_init; it may be shared with other calls
 * and steps that never overlap this step's launches. Creating a step makes
 * host-side objects (a capture stream, the graph); launching allocates
 * nothing. A call may read an earlier call's output (given order only). */
wl_status wl_step_create(const wl_call *calls, int32_t n_calls, int32_t flags, void *ws, size_t ws_bytes,
                         wl_step *step);

/* One launch of the step's graph on hip_stream (every call, in order). Two
 * launches of one step, or of steps sharing a workspace, must not overlap:
 * they share the workspace. */
wl_status wl_step_launch(wl_step step, void *hip_stream);

/* Frees the step's graph. NULL is accepted. The caller makes sure no launch
 * of the step is still running (for example by synchronizing its stream). */
wl_status wl_step_destroy(wl_step step);

/* Size of a set of theta bundles against the dense weights they replace
 * ("What weightless inference costs", "Compression": the ratio of the theta
 * bundle, W0 + s + U + V across every layer and family, to the original
 * projection weights). For th[0 .. n_th):
 *   *bundle_bytes = e d_out d_in once per distinct W0 pointer
 *                   + per theta: 4 d_out (when s is not NULL) + e r (d_out + d_in)
 *   *dense_bytes  = per theta: e d_out d_in (the weight it stands for)
 * with e = 2 for bf16 thetas and 4 for fp32 ones.
 * Thetas that share a W0 pointer must share its shape and dtype (else
 * WL_ERR_INVALID_ARG). Host only: reads the structs, never the tensors. */
wl_status wl_bundle_size(const wl_theta *const *th, int32_t n_th,
                         size_t *bundle_bytes, size_t *dense_bytes);

/* Reconstruction fidelity ("What weightless inference costs", "Reconstruction
 * fidelity"): result[0] = ||W - R||_F / ||W||_F, accumulated in fp64 (the
 * differences and squares of bf16 values are exact there), in a fixed order
 * that depends on n only.
 *   W, R    bf16 [n] device tensors, 16-byte aligned: e.g. an original weight
 *           and the W_eff of wl_materialize_weff
 *   n       elements, 1 <= n < 2^40
 *   result  device pointer to one double, 8-byte aligned, written
 *   ws      workspace, ws_bytes >= wl_rel_frob_workspace_bytes(n)
 * When ||W||_F is 0 the result is 0 if R equals W and +inf otherwise. */
size_t wl_rel_frob_workspace_bytes(int64_t n);
wl_status wl_relative_frobenius_error(const void *W, const void *R, int64_t n, double *result,
                                      void *ws, size_t ws_bytes, void *hip_stream);

/* Prepares a projection workspace: clears its sync area (the first
 * WL_SYNC_BYTES) with a kernel enqueued on hip_stream. Needed once before the
 * workspace's first use by wl_linear, wl_qkv_fused or wl_mlp_fused, and again
 * after anything else has written that area (the calls write it with
 * generation-tagged words that are never reset; a tag left by foreign data
 * could make a later call take a stale value). ws must be 256-byte aligned and
 * ws_bytes >= WL_SYNC_BYTES (else WL_ERR_INVALID_ARG / WL_ERR_WORKSPACE). */
wl_status wl_workspace_init(void *ws, size_t ws_bytes, void *hip_stream);

/* WL_SYNC_BYTES of the built library. */
size_t wl_sync_bytes(void);

/* Static description of a status code. */
const char *wl_status_str(wl_status status);

/* Message describing the last non-WL_OK return on the calling thread ("" after
 * a success). The pointer stays valid until the thread's next library call. */
const char *wl_last_error(void);

/* WL_ABI_VERSION of the built library. */
int32_t wl_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WL_H */
