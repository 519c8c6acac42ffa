/*
 * mn_oracle.c -- plain fp64 CPU oracle for the row-wise normalization
 * training pair (RMSNorm, LayerNorm, fused residual-add + RMSNorm; forward and
 * backward).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it. It shares no code, header, table or constant with
 * the HIP implementation.
 *
 * Every result is the plain definition written out, row by row, in double
 * precision, with sums taken in ascending column (and row) order and no
 * blocking or reordering. The sources are two pages:
 *   [meTile] "Kernel coverage and training scope", section "Exact native
 *            normalization contract" (formulas, bounds, backward semantics);
 *   [tensorcore] "Training kernels", sections "RMSnorm -- Llama-style" (Math)
 *            and "LayerNorm -- standard" (buffers and saved statistics).
 *
 * Inputs are IEEE binary16 bit patterns (uint16_t), widened exactly to double.
 * Outputs are doubles; rounding to binary16 for comparison is a separate step
 * (mno_f64_to_f16, round to nearest, ties to even, straight from double).
 *
 * Backward functions recompute their statistics in fp64 from X and take no
 * saved statistics: what they define is the exact derivative of the forward
 * formula with respect to its inputs and parameters (the [meTile] contract
 * ignores the rounding of casts and gives no epsilon gradient).
 *
 * Pins (tests/test_oracle_pins.py): torch fp64 layer_norm / rms_norm and
 * autograd on random inputs, central finite differences, closed forms for
 * constant and zero rows, the LayerNorm worked example of the [meTile]
 * contract, row invariants, and the binary16 codec against numpy over every
 * bit pattern. No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MNO_OK 0
#define MNO_ERR_ARG 1
#define MNO_ERR_MEM 2

/* ---------------------------------------------------------------------------
 * binary16 codec, from the IEEE 754 binary16 layout: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 encodes zero and subnormals
 * (fraction * 2^-24), exponent 31 encodes infinities and NaNs.
 * ------------------------------------------------------------------------- */

double mno_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* Round a non-negative double q to an integer, ties to even. q < 2^52. */
static double round_half_even(double q)
{
    double fl = floor(q);
    double diff = q - fl; /* exact (Sterbenz: fl <= q <= 2 fl when fl >= 1) */
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t mno_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7e00);
    if (isinf(v)) return (uint16_t)(sign | 0x7c00);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: value = q * 2^-24 with q an integer in [0, 1024];
         * q = 1024 is the smallest normal, whose encoding is also 1024 */
        double q = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    double m = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7c00); /* overflow rounds to inf */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

void mno_decode_f16(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mno_f16_to_f64(h[i]);
}

void mno_encode_f16(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mno_f64_to_f16(v[i]);
}

static int bad_shape(int64_t N, int64_t D) { return N < 0 || D < 1; }

/* ---------------------------------------------------------------------------
 * Row statistics.
 * ------------------------------------------------------------------------- */

/* [tensorcore] RMSnorm Math: rms(x) = sqrt(mean(x^2) + eps); the saved value
 * is its reciprocal. [meTile] contract: inverse = 1 / sqrt(mean(x*x) + eps). */
static double rms_rstd(const double* x, int64_t D, double eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < D; ++j) ss += x[j] * x[j];
    return 1.0 / sqrt(ss / (double)D + eps);
}

/* [meTile] contract: LayerNorm centres the row by its mean, then takes the
 * population variance of the centred values (divisor D); epsilon is added to
 * that variance inside the square root, as for RMSNorm. */
static void ln_stats(const double* x, int64_t D, double eps, double* mean, double* rstd)
{
    double s = 0.0;
    for (int64_t j = 0; j < D; ++j) s += x[j];
    double mu = s / (double)D;
    double v = 0.0;
    for (int64_t j = 0; j < D; ++j) v += (x[j] - mu) * (x[j] - mu);
    *mean = mu;
    *rstd = 1.0 / sqrt(v / (double)D + eps);
}

/* Widening table: entry h is mno_f16_to_f64(h), filled on first use so the
 * per-element decode in the row loops is a lookup. */
static double f16_table[65536];
static int f16_table_ready = 0;

static double widen(uint16_t h)
{
    if (!f16_table_ready) {
        for (int k = 0; k < 65536; ++k) f16_table[k] = mno_f16_to_f64((uint16_t)k);
        f16_table_ready = 1;
    }
    return f16_table[h];
}

/* An input operand: either binary16 bits or doubles (exactly one of h, d is
 * set), or absent (both NULL). The fp64 entry points let the finite-difference
 * pins perturb inputs by amounts binary16 cannot represent. */
typedef struct {
    const uint16_t* h;
    const double* d;
} operand;

static operand op16(const uint16_t* p) { operand o = {p, NULL}; return o; }
static operand op64(const double* p) { operand o = {NULL, p}; return o; }
static int present(operand a) { return a.h != NULL || a.d != NULL; }

/* Row i of an [N, D] operand (or the [D] vector when i = 0), widened. */
static void get_row(operand a, int64_t i, int64_t D, double* dst)
{
    if (a.h) {
        for (int64_t j = 0; j < D; ++j) dst[j] = widen(a.h[i * D + j]);
    } else {
        for (int64_t j = 0; j < D; ++j) dst[j] = a.d[i * D + j];
    }
}

/* Scratch rows for one call. */
typedef struct {
    double *x, *r, *g, *b, *dy, *dh, *xh, *dx;
} rows;

static int rows_alloc(rows* w, int64_t D)
{
    size_t n = sizeof(double) * (size_t)D;
    w->x = malloc(n); w->r = malloc(n); w->g = malloc(n); w->b = malloc(n);
    w->dy = malloc(n); w->dh = malloc(n); w->xh = malloc(n); w->dx = malloc(n);
    return w->x && w->r && w->g && w->b && w->dy && w->dh && w->xh && w->dx;
}

static void rows_free(rows* w)
{
    free(w->x); free(w->r); free(w->g); free(w->b);
    free(w->dy); free(w->dh); free(w->xh); free(w->dx);
}

/* The row being normalised: x, or for the fused add the unrounded sum
 * x + residual (exact in double for binary16 operands: both are multiples of
 * 2^-24 below 2^16 in magnitude, so the sum has at most 41 significant bits). */
static void source_row(operand X, operand R, int64_t i, int64_t D, rows* w)
{
    get_row(X, i, D, w->x);
    if (present(R)) {
        get_row(R, i, D, w->r);
        for (int64_t j = 0; j < D; ++j) w->x[j] = w->x[j] + w->r[j];
    }
}

/* ---------------------------------------------------------------------------
 * Forward.
 * ------------------------------------------------------------------------- */

/* RMSNorm forward on x (or on x + residual when R is present).
 * [meTile] contract, rms_norm_forward: y = x * inverse * weight.
 * [tensorcore] RMSnorm: y = (x / rms) * gamma, with rstd saved per row.
 * [meTile] contract, add_rms_norm_forward: the sum is formed without rounding
 * to the storage type and normalised; S (if not NULL) receives that sum. */
static int rms_forward(operand X, operand R, operand G, int64_t N, int64_t D, double eps,
                       double* S, double* Y, double* rstd)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    for (int64_t i = 0; i < N; ++i) {
        source_row(X, R, i, D, &w);
        double r = rms_rstd(w.x, D, eps);
        rstd[i] = r;
        for (int64_t j = 0; j < D; ++j) {
            if (S) S[i * D + j] = w.x[j];
            Y[i * D + j] = w.x[j] * r * w.g[j];
        }
    }
    rows_free(&w);
    return MNO_OK;
}

/* [meTile] contract, layer_norm_forward: centre, population variance, then
 * weight and bias: y = (x - mean) * rstd * gamma + beta.
 * [tensorcore] LayerNorm: mean and rstd saved per row. */
static int ln_forward(operand X, operand G, operand B, int64_t N, int64_t D, double eps,
                      double* Y, double* mean, double* rstd)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    get_row(B, 0, D, w.b);
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        double mu, r;
        ln_stats(w.x, D, eps, &mu, &r);
        mean[i] = mu;
        rstd[i] = r;
        for (int64_t j = 0; j < D; ++j) Y[i * D + j] = (w.x[j] - mu) * r * w.g[j] + w.b[j];
    }
    rows_free(&w);
    return MNO_OK;
}

/* ---------------------------------------------------------------------------
 * Backward. With g = dY * gamma and xhat the normalised row, differentiating
 * y = xhat * gamma (+ beta) through the row statistics gives
 *   RMSNorm:   dX = rstd * (g - xhat * mean(g * xhat))
 *   LayerNorm: dX = rstd * (g - mean(g) - xhat * mean(g * xhat))
 * and the parameter gradients dgamma = sum over rows of dY * xhat,
 * dbeta = sum over rows of dY. The finite-difference and autograd pins in the
 * test suite check these closed forms against the forward functions above.
 * dX may be NULL (only the parameter gradients are produced); parameter
 * gradients are overwritten, never accumulated into ([meTile] contract:
 * independent calls do not accumulate into existing parameter buffers).
 * ------------------------------------------------------------------------- */

/* RMSNorm backward at x (or at the unrounded sum x + residual when R is
 * present: the [meTile] contract takes the derivative of the exact formula,
 * not of the rounded H). For the fused add the residual-output cotangent dH (zero when
 * absent) is added, and the result is both the source and the residual
 * gradient ([meTile] contract: its contribution goes to both). */
static int rms_backward(operand X, operand R, operand G, operand DY, operand DH,
                        int64_t N, int64_t D, double eps, double* dX, double* dgamma)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    for (int64_t j = 0; j < D; ++j) dgamma[j] = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        source_row(X, R, i, D, &w);
        get_row(DY, i, D, w.dy);
        double r = rms_rstd(w.x, D, eps);
        double c1 = 0.0;
        for (int64_t j = 0; j < D; ++j) {
            w.xh[j] = w.x[j] * r;
            c1 += w.dy[j] * w.g[j] * w.xh[j];
        }
        c1 /= (double)D;
        if (dX) {
            if (present(DH)) get_row(DH, i, D, w.dh);
            for (int64_t j = 0; j < D; ++j) {
                double d = r * (w.dy[j] * w.g[j] - w.xh[j] * c1);
                dX[i * D + j] = present(DH) ? w.dh[j] + d : d;
            }
        }
        for (int64_t j = 0; j < D; ++j) dgamma[j] += w.dy[j] * w.xh[j];
    }
    rows_free(&w);
    return MNO_OK;
}

/* [meTile] contract, norm_backward for layer_norm_forward: source, weight and
 * bias gradients (the contract's worked example returns all three). */
static int ln_backward(operand X, operand G, operand DY, int64_t N, int64_t D, double eps,
                       double* dX, double* dgamma, double* dbeta)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    for (int64_t j = 0; j < D; ++j) { dgamma[j] = 0.0; dbeta[j] = 0.0; }
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        get_row(DY, i, D, w.dy);
        double mu, r;
        ln_stats(w.x, D, eps, &mu, &r);
        double c1 = 0.0, c2 = 0.0;
        for (int64_t j = 0; j < D; ++j) {
            w.xh[j] = (w.x[j] - mu) * r;
            c1 += w.dy[j] * w.g[j] * w.xh[j];
            c2 += w.dy[j] * w.g[j];
        }
        c1 /= (double)D;
        c2 /= (double)D;
        if (dX)
            for (int64_t j = 0; j < D; ++j)
                dX[i * D + j] = r * (w.dy[j] * w.g[j] - c2 - w.xh[j] * c1);
        for (int64_t j = 0; j < D; ++j) {
            dgamma[j] += w.dy[j] * w.xh[j];
            dbeta[j] += w.dy[j];
        }
    }
    rows_free(&w);
    return MNO_OK;
}

/* ---------------------------------------------------------------------------
 * Entry points on binary16 inputs (the storage type of the path) and on
 * double inputs (for the finite-difference pins). Shapes: X, R, dY, dH, Y, S,
 * dX are [N, D] row-major; gamma, beta, dgamma, dbeta are [D]; rstd, mean [N].
 * ------------------------------------------------------------------------- */

int mno_rmsnorm_forward(const uint16_t* X, const uint16_t* gamma, int64_t N, int64_t D,
                        double eps, double* Y, double* rstd)
{
    return rms_forward(op16(X), op16(NULL), op16(gamma), N, D, eps, NULL, Y, rstd);
}

int mno_layernorm_forward(const uint16_t* X, const uint16_t* gamma, const uint16_t* beta,
                          int64_t N, int64_t D, double eps, double* Y, double* mean,
                          double* rstd)
{
    return ln_forward(op16(X), op16(gamma), op16(beta), N, D, eps, Y, mean, rstd);
}

int mno_add_rmsnorm_forward(const uint16_t* X, const uint16_t* R, const uint16_t* gamma,
                            int64_t N, int64_t D, double eps, double* S, double* Y,
                            double* rstd)
{
    if (!R) return MNO_ERR_ARG;
    return rms_forward(op16(X), op16(R), op16(gamma), N, D, eps, S, Y, rstd);
}

int mno_rmsnorm_backward(const uint16_t* X, const uint16_t* gamma, const uint16_t* dY,
                         int64_t N, int64_t D, double eps, double* dX, double* dgamma)
{
    return rms_backward(op16(X), op16(NULL), op16(gamma), op16(dY), op16(NULL), N, D, eps,
                        dX, dgamma);
}

int mno_layernorm_backward(const uint16_t* X, const uint16_t* gamma, const uint16_t* dY,
                           int64_t N, int64_t D, double eps, double* dX, double* dgamma,
                           double* dbeta)
{
    return ln_backward(op16(X), op16(gamma), op16(dY), N, D, eps, dX, dgamma, dbeta);
}

int mno_add_rmsnorm_backward(const uint16_t* X, const uint16_t* R, const uint16_t* gamma,
                             const uint16_t* dY, const uint16_t* dH, int64_t N, int64_t D,
                             double eps, double* dX, double* dgamma)
{
    if (!R) return MNO_ERR_ARG;
    return rms_backward(op16(X), op16(R), op16(gamma), op16(dY), op16(dH), N, D, eps, dX,
                        dgamma);
}

int mno_rmsnorm_forward_f64(const double* X, const double* gamma, int64_t N, int64_t D,
                            double eps, double* Y, double* rstd)
{
    return rms_forward(op64(X), op64(NULL), op64(gamma), N, D, eps, NULL, Y, rstd);
}

int mno_layernorm_forward_f64(const double* X, const double* gamma, const double* beta,
                              int64_t N, int64_t D, double eps, double* Y, double* mean,
                              double* rstd)
{
    return ln_forward(op64(X), op64(gamma), op64(beta), N, D, eps, Y, mean, rstd);
}

int mno_add_rmsnorm_forward_f64(const double* X, const double* R, const double* gamma,
                                int64_t N, int64_t D, double eps, double* S, double* Y,
                                double* rstd)
{
    if (!R) return MNO_ERR_ARG;
    return rms_forward(op64(X), op64(R), op64(gamma), N, D, eps, S, Y, rstd);
}

int mno_rmsnorm_backward_f64(const double* X, const double* gamma, const double* dY,
                             int64_t N, int64_t D, double eps, double* dX, double* dgamma)
{
    return rms_backward(op64(X), op64(NULL), op64(gamma), op64(dY), op64(NULL), N, D, eps,
                        dX, dgamma);
}

int mno_layernorm_backward_f64(const double* X, const double* gamma, const double* dY,
                               int64_t N, int64_t D, double eps, double* dX, double* dgamma,
                               double* dbeta)
{
    return ln_backward(op64(X), op64(gamma), op64(dY), N, D, eps, dX, dgamma, dbeta);
}

int mno_add_rmsnorm_backward_f64(const double* X, const double* R, const double* gamma,
                                 const double* dY, const double* dH, int64_t N, int64_t D,
                                 double eps, double* dX, double* dgamma)
{
    if (!R) return MNO_ERR_ARG;
    return rms_backward(op64(X), op64(R), op64(gamma), op64(dY), op64(dH), N, D, eps, dX,
                        dgamma);
}
