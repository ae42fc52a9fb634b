/*
 * CPU oracle for the fused reconstruct-and-project linear.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The product
 * path never does: it has no CPU fallback.
 *
 * Plain, slow, obviously correct: fp64 arithmetic on the exact values of the
 * bf16 / fp32 inputs, sequential loops in the index order of the definitions,
 * no blocking, no fusion, no reordering. Independent results (output elements,
 * V^T x entries, h entries, W_eff entries) are shared out over OpenMP threads;
 * each is still one thread's sequential loop, so the values do not depend on
 * the number of threads. Nothing here is shared with the HIP
 * library (no header, helper, table or constant), and this file includes none
 * of its files.
 *
 * What it computes (sources are the weightless documentation pages; each
 * function names the passage it follows):
 *
 *   "In-kernel reconstruction" page, reconstruction equation and its
 *   per-element expansion:
 *       y[t,o] = s[o] * sum_i W0[o,i] * x[t,i]  +  sum_k U[o,k] * sum_i V[i,k] * x[t,i]
 *
 * Layouts (row-major, contiguous): W0 [d_out][d_in], s [d_out], U [d_out][r],
 * V [d_in][r], x [T][d_in], y [T][d_out]. W0, U, V and x share one element
 * type per call: bf16 (passed as 16-bit patterns) or IEEE binary32 (the
 * "also supports float32" remark of the custom-op description on the
 * "In-kernel reconstruction" page); s is always binary32.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One projection's theta bundle ("Serve and generate with weightless",
 * introduction: a shared block W0 per band, a per-row scale s and a low-rank
 * delta U, V of rank r). s may be NULL, meaning every s[o] is 1. U and V may be
 * NULL only when r == 0. */
enum { ORC_BF16 = 0, ORC_F32 = 1 };

typedef struct {
    const void *W0;
    const float *s;
    const void *U;
    const void *V;
    int64_t d_in, d_out, r;
    int64_t dtype;          /* ORC_BF16 or ORC_F32: W0, U, V and the call's x (and y's rounding) */
} orc_theta;

/* The exact value of a bf16 bit pattern: bf16 is the upper half of an IEEE
 * binary32, so the pattern shifted up 16 bits is that float, and a float
 * converts to double exactly. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even (IEEE 754
 * roundTiesToEven applied to the bfloat16 format: 1 sign bit, 8 exponent bits,
 * 7 fraction bits, subnormals below 2^-126 with quantum 2^-133).
 * Returns the bit pattern. */
uint16_t orc_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isinf(v))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    /* quantum (spacing of bf16 values) in the binade holding a */
    int e;
    frexp(a, &e);           /* a = m * 2^e with m in [0.5, 1) -> binade [2^(e-1), 2^e) */
    int q = (e - 1) - 7;    /* 7 fraction bits below the leading bit */
    if (q < -133)
        q = -133;           /* subnormal range: fixed quantum 2^-133 */
    double n = nearbyint(ldexp(a, -q));   /* exact scaling; default mode rounds ties to even */
    double r = ldexp(n, q);
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;             /* rounds past the largest finite bf16 */
    float f = (float)r;                   /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

double orc_bf16_value(uint16_t bits) { return bf16_value(bits); }

/* Element j of a tensor of the given element type, exactly, as a double. */
static double elem(const void *p, int64_t dtype, int64_t j)
{
    if (dtype == ORC_F32)
        return (double)((const float *)p)[j];
    return bf16_value(((const uint16_t *)p)[j]);
}

/* Threads used by the loops below: n > 0 sets it, n <= 0 leaves it; returns
 * the count now in force (by default every core the process may run on). */
int orc_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
}

/* tanh-approximated GELU (Hendrycks & Gimpel, 2016):
 *   gelu(z) = 0.5 * z * (1 + tanh(sqrt(2/pi) * (z + 0.044715 * z^3)))
 * The pages name an activation between gate/up and down ("In-kernel
 * reconstruction", the custom-op path, fused MLP paragraph) but not which one;
 * the tanh form is the one Gemma uses. */
double orc_gelu_tanh(double z)
{
    double a = sqrt(2.0 / M_PI) * (z + 0.044715 * z * z * z);
    return 0.5 * z * (1.0 + tanh(a));
}

/* "In-kernel reconstruction", per-element expansion of the reconstruction
 * equation. For every token t and output row o:
 *   vtx[k]   = sum_i V[i,k] * x[t,i]
 *   m        = sum_i W0[o,i] * x[t,i]
 *   y[t,o]   = s[o] * m + sum_k U[o,k] * vtx[k]
 * Also the magnitude bound used by the acceptance test:
 *   bound[t,o] = |s[o]| * sum_i |W0[o,i] * x[t,i]| + sum_k |U[o,k] * vtx[k]|
 * y and bound are [T][d_out], fp64, unrounded. bound may be NULL.
 * Returns 0, or -1 if scratch memory cannot be had. */
int orc_linear(const orc_theta *th, int64_t T, const void *x, double *y, double *bound)
{
    const int64_t d_in = th->d_in, d_out = th->d_out, r = th->r, dt = th->dtype;
    /* token t's vtx[k] at vtx_all[t * r + k], every token first */
    double *vtx_all = (double *)malloc(sizeof(double) * (size_t)(T * r > 0 ? T * r : 1));
    if (!vtx_all)
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < r; ++k) {
            const int64_t x0 = t * d_in;   /* token t's row of x */
            double *vtx = vtx_all + t * r;
            double acc = 0.0;
            for (int64_t i = 0; i < d_in; ++i)
                acc += elem(th->V, dt, i * r + k) * elem(x, dt, x0 + i);
            vtx[k] = acc;
        }
    /* output rows outer, tokens inner: a W0 row is read once per thread pass
     * while x stays in cache (the order of independent elements only) */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t o = 0; o < d_out; ++o)
        for (int64_t t = 0; t < T; ++t) {
            const int64_t x0 = t * d_in;
            const double *vtx = vtx_all + t * r;
            double m = 0.0, m_abs = 0.0;
            for (int64_t i = 0; i < d_in; ++i) {
                double p = elem(th->W0, dt, o * d_in + i) * elem(x, dt, x0 + i);
                m += p;
                m_abs += fabs(p);
            }
            double delta = 0.0, delta_abs = 0.0;
            for (int64_t k = 0; k < r; ++k) {
                double p = elem(th->U, dt, o * r + k) * vtx[k];
                delta += p;
                delta_abs += fabs(p);
            }
            double so = th->s ? (double)th->s[o] : 1.0;
            y[t * d_out + o] = so * m + delta;
            if (bound)
                bound[t * d_out + o] = fabs(so) * m_abs + delta_abs;
        }
    free(vtx_all);
    return 0;
}

/* "In-kernel reconstruction", Q/K/V fusion: the three attention projections
 * share one input x; the fused result is the three projections' outputs side
 * by side, columns Q | K | V. y and bound are [T][dq + dk + dv]. The three
 * thetas must share one element type (else -1). */
int orc_qkv(const orc_theta *q, const orc_theta *k, const orc_theta *v, int64_t T,
            const void *x, double *y, double *bound)
{
    const orc_theta *child[3] = {q, k, v};
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return -1;
    int64_t width = q->d_out + k->d_out + v->d_out;
    int64_t col0 = 0;
    for (int c = 0; c < 3; ++c) {
        int64_t n = child[c]->d_out;
        double *yc = (double *)malloc(sizeof(double) * (size_t)(T * n > 0 ? T * n : 1));
        double *bc = (double *)malloc(sizeof(double) * (size_t)(T * n > 0 ? T * n : 1));
        if (!yc || !bc || orc_linear(child[c], T, x, yc, bc) != 0) {
            free(yc);
            free(bc);
            return -1;
        }
        for (int64_t t = 0; t < T; ++t)
            for (int64_t o = 0; o < n; ++o) {
                y[t * width + col0 + o] = yc[t * n + o];
                if (bound)
                    bound[t * width + col0 + o] = bc[t * n + o];
            }
        free(yc);
        free(bc);
        col0 += n;
    }
    return 0;
}

/* "In-kernel reconstruction", the custom-op path, fused MLP paragraph: gate,
 * up, activation and down in one operation:
 *   g = linear(gate, x),  u = linear(up, x)
 *   h = gelu_tanh(g) * u
 *   y = linear(down, round(h))
 * The intermediate h is rounded once to the call's element type (bf16 or
 * binary32, round-to-nearest-even) before the down projection: down is a
 * projection like every other, and the pages' three-call fallback casts each
 * call's result to the activation dtype ("In-kernel reconstruction", the
 * custom-op path: accumulate in float32, cast back to the output dtype). bound
 * is that of the down projection with x := round(h). h_out (optional,
 * [T][d_ff]) receives the rounded h: bf16 patterns or binary32 values. The
 * three thetas must share one element type (else -1). */
int orc_mlp(const orc_theta *gate, const orc_theta *up, const orc_theta *down, int64_t T,
            const void *x, double *y, double *bound, void *h_out)
{
    int64_t d_ff = gate->d_out, dt = gate->dtype;
    if (up->dtype != dt || down->dtype != dt)
        return -1;
    size_t n = (size_t)(T * d_ff > 0 ? T * d_ff : 1);
    size_t esz = dt == ORC_F32 ? sizeof(float) : sizeof(uint16_t);
    double *g = (double *)malloc(sizeof(double) * n);
    double *u = (double *)malloc(sizeof(double) * n);
    void *hr = malloc(esz * n);
    int rc = -1;
    if (!g || !u || !hr)
        goto done;
    if (orc_linear(gate, T, x, g, NULL) != 0 || orc_linear(up, T, x, u, NULL) != 0)
        goto done;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < T * d_ff; ++j) {
        double h = orc_gelu_tanh(g[j]) * u[j];
        if (dt == ORC_F32)
            ((float *)hr)[j] = (float)h;   /* C conversion: round to nearest, ties to even */
        else
            ((uint16_t *)hr)[j] = orc_bf16_rne(h);
    }
    if (orc_linear(down, T, hr, y, bound) != 0)
        goto done;
    if (h_out)
        memcpy(h_out, hr, esz * (size_t)(T * d_ff));
    rc = 0;
done:
    free(g);
    free(u);
    free(hr);
    return rc;
}

/* "Serve and generate with weightless", fast path on NVIDIA: the effective
 * weight materialized once,
 *   W_eff[o,i] = s[o] * W0[o,i] + sum_k U[o,k] * V[i,k]
 * (the "What weightless inference costs" page writes the same matrix as
 * diag(s)*W0 + U*V^T under "Reconstruction fidelity"). W_eff and bound are
 * [d_out][d_in], fp64, unrounded; bound[o,i] = |s[o]*W0[o,i]| +
 * sum_k |U[o,k]*V[i,k]|. bound may be NULL. */
int orc_weff(const orc_theta *th, double *W_eff, double *bound)
{
    const int64_t d_in = th->d_in, d_out = th->d_out, r = th->r, dt = th->dtype;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < d_out; ++o) {
        double so = th->s ? (double)th->s[o] : 1.0;
        for (int64_t i = 0; i < d_in; ++i) {
            double base = so * elem(th->W0, dt, o * d_in + i);
            double delta = 0.0, delta_abs = 0.0;
            for (int64_t k = 0; k < r; ++k) {
                double p = elem(th->U, dt, o * r + k) * elem(th->V, dt, i * r + k);
                delta += p;
                delta_abs += fabs(p);
            }
            W_eff[o * d_in + i] = base + delta;
            if (bound)
                bound[o * d_in + i] = fabs(base) + delta_abs;
        }
    }
    return 0;
}

/* "What weightless inference costs", Reconstruction fidelity: the relative
 * Frobenius error ||W - R||_F / ||W||_F of a reconstruction R of W, both n
 * values. When ||W||_F is 0 the ratio is 0 if R equals W and +inf otherwise. */
double orc_rel_frob(int64_t n, const double *W, const double *R)
{
    double num = 0.0, den = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double d = W[j] - R[j];
        num += d * d;
        den += W[j] * W[j];
    }
    if (den == 0.0)
        return num == 0.0 ? 0.0 : INFINITY;
    return sqrt(num) / sqrt(den);
}
