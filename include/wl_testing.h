/*
 * wl_testing.h: process-wide switches of libwl for tests and measurements.
 * They are not part of the product interface (include/wl.h): results agree
 * within rounding whatever they are set to, and a program that never calls
 * them gets the default choices. Both are exported by libwl.so.
 */
#ifndef WL_TESTING_H
#define WL_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel regime for the projection calls:
 *   0  chooses by token count (the default; the MLP in one launch at one or
 *      two tokens per pass where its shape allows);
 *   1  forces the decode kernels wherever they apply (V^T x computed by the
 *      first workgroups of the same launch at 1 to 4 tokens per pass, else by
 *      a separate launch before it; the MLP in one launch where its shape
 *      allows);
 *   2  forces the matrix-core GEMM;
 *   3  forces the decode GEMV with V^T x always computed by a separate launch
 *      (the MLP as a gate/up launch and a down launch);
 *   4  forces the few-token path (split matrix-core products and an epilogue
 *      launch) wherever it applies (T <= 64, d_in <= 8192);
 *   5  as 1, but the MLP as a gate/up launch and a down launch;
 *   6  as 2, with V^T x always computed by a launch of its own before the GEMM
 *      and the rank term in the GEMM's epilogue (by default a GEMM whose input
 *      axis is split computes V^T x in its own launch and adds the rank term in
 *      its reduction).
 * Where a forced regime does not apply the matrix-core GEMM runs. Returns the
 * previous value, or -1 (and changes nothing) for any other argument. */
int32_t wl_set_regime(int32_t regime);

/* Bound on the waits of a decode workgroup for words that other workgroups of
 * its launch write (V^T x slices, and the one-launch MLP's partial outputs):
 * the number of times it reads each group of words, default 4096. A workgroup
 * whose wait runs out computes what it waited for itself, with the same
 * arithmetic, so the result does not change; 0 makes every workgroup do so.
 * Returns the previous value, or -1 (and changes nothing) for a negative
 * argument. */
int32_t wl_set_spin_limit(int32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* WL_TESTING_H */
