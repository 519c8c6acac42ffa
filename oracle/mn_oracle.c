/*
 * mn_oracle.c -- plain fp64 CPU oracle for the row-wise normalization
 * training pair (RMSNorm, LayerNorm, fused residual-add + RMSNorm; forward and
 * backward), for the other row-wise norms the [meTile] coverage inventory
 * lists (Dynamic Tanh, PolyNorm, Modulated RMSNorm, GroupNorm), and for the
 * inference-only fused normalization + GEMV of [tensorcore].
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
 * Inputs are IEEE binary16 or bfloat16 bit patterns (uint16_t), binary32 or
 * binary64 values, widened exactly to double. Outputs are doubles; rounding
 * to a storage type for comparison is a separate step (mno_f64_to_f16,
 * mno_f64_to_bf16: round to nearest, ties to even, straight from double).
 *
 * Backward functions recompute their statistics in fp64 from X and take no
 * saved statistics: what they define is the exact derivative of the forward
 * formula with respect to its inputs and parameters (the [meTile] contract
 * ignores the rounding of casts and gives no epsilon gradient).
 *
 * Pins (tests/test_oracle_pins.py): torch fp64 layer_norm / rms_norm /
 * group_norm and autograd on random inputs, central finite differences,
 * closed forms for constant and zero rows, the LayerNorm worked example of
 * the [meTile] contract, row invariants, the binary16 codec against numpy
 * and the bfloat16 codec against torch over every bit pattern, agreement of
 * the typed entry points across storage types on values all types
 * represent; for Dynamic Tanh its exponential form, odd symmetry, alpha = 0
 * and saturation; for PolyNorm each power against torch rms_norm and
 * linearity in its weights. No function here is "parity unpinned".
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

/* Round a double to a binary format with `mbits` stored fraction bits and
 * exponents emin..emax (normal range), to nearest with ties to even, and
 * return its bit pattern (1 sign bit, then exponent with bias -emin + 1,
 * then fraction), as IEEE 754 defines binary16 and bfloat16 does binary32's
 * upper half. Subnormals below 2^emin are multiples of 2^(emin - mbits);
 * values that round beyond the largest finite number become infinity. */
static uint32_t encode_binary(double v, int mbits, int emin, int emax)
{
    const uint32_t inf_exp = (uint32_t)(emax - emin + 2); /* biased exponent of inf */
    int ewidth = 0;                                        /* exponent field width */
    while ((1u << ewidth) <= inf_exp) ++ewidth;
    const uint32_t sign = signbit(v) ? (1u << (mbits + ewidth)) : 0u;
    const uint32_t inf = inf_exp << mbits;
    double a = fabs(v);
    if (isnan(v)) return sign | inf | (1u << (mbits - 1));
    if (isinf(v)) return sign | inf;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    if (e < emin) {
        /* subnormal range: value = q * 2^(emin - mbits), q an integer in
         * [0, 2^mbits]; q = 2^mbits is the smallest normal, same encoding */
        double q = round_half_even(ldexp(a, mbits - emin));
        return sign | (uint32_t)q;
    }
    double m = round_half_even(ldexp(a, mbits - e)); /* in [2^mbits, 2^(mbits+1)] */
    if (m == ldexp(1.0, mbits + 1)) {
        m = ldexp(1.0, mbits);
        e += 1;
    }
    if (e > emax) return sign | inf;                  /* overflow rounds to inf */
    return sign | ((uint32_t)(e - emin + 1) << mbits) | (uint32_t)(m - ldexp(1.0, mbits));
}

uint16_t mno_f64_to_f16(double v) { return (uint16_t)encode_binary(v, 10, -14, 15); }

/* bfloat16: the upper half of an IEEE binary32 -- 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits; exponent 0 encodes zero and subnormals
 * (fraction * 2^-133), exponent 255 infinities and NaNs. */
double mno_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);
    } else if (e == 255) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(128 + f), e - 134);
    }
    return sign ? -v : v;
}

uint16_t mno_f64_to_bf16(double v) { return (uint16_t)encode_binary(v, 7, -126, 127); }

void mno_decode_bf16(const uint16_t* b, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mno_bf16_to_f64(b[i]);
}

void mno_encode_bf16(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mno_f64_to_bf16(v[i]);
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

/* Widening tables: entry h is mno_f16_to_f64(h) (resp. mno_bf16_to_f64(h)),
 * filled on first use so the per-element decode in the row loops is a
 * lookup. */
static double f16_table[65536];
static double bf16_table[65536];
static int tables_ready = 0;

static void fill_tables(void)
{
    if (tables_ready) return;
    for (int k = 0; k < 65536; ++k) {
        f16_table[k] = mno_f16_to_f64((uint16_t)k);
        bf16_table[k] = mno_bf16_to_f64((uint16_t)k);
    }
    tables_ready = 1;
}

/* Storage types of an input operand. */
#define MNO_F16 0
#define MNO_BF16 1
#define MNO_F32 2
#define MNO_F64 3

/* An input operand: a pointer and its storage type, or absent (p == NULL).
 * The fp64 type lets the finite-difference pins perturb inputs by amounts
 * no 16-bit type can represent. */
typedef struct {
    const void* p;
    int type;
} operand;

static operand opt(const void* p, int type) { operand o = {p, type}; return o; }
static operand op16(const uint16_t* p) { return opt(p, MNO_F16); }
static operand op64(const double* p) { return opt(p, MNO_F64); }
static int present(operand a) { return a.p != NULL; }
static int type_ok(int t) { return t == MNO_F16 || t == MNO_BF16 || t == MNO_F32 || t == MNO_F64; }

/* Row i of an [N, D] operand (or the [D] vector when i = 0), widened exactly
 * to double. */
static void get_row(operand a, int64_t i, int64_t D, double* dst)
{
    const int64_t o = i * D;
    switch (a.type) {
    case MNO_F16: {
        const uint16_t* h = (const uint16_t*)a.p + o;
        for (int64_t j = 0; j < D; ++j) dst[j] = f16_table[h[j]];
        break;
    }
    case MNO_BF16: {
        const uint16_t* b = (const uint16_t*)a.p + o;
        for (int64_t j = 0; j < D; ++j) dst[j] = bf16_table[b[j]];
        break;
    }
    case MNO_F32: {
        const float* f = (const float*)a.p + o;
        for (int64_t j = 0; j < D; ++j) dst[j] = (double)f[j];
        break;
    }
    default: {
        const double* d = (const double*)a.p + o;
        for (int64_t j = 0; j < D; ++j) dst[j] = d[j];
        break;
    }
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
 * x + residual. For binary16 operands the double sum is exact (both are
 * multiples of 2^-24 below 2^16 in magnitude, so the sum has at most 41
 * significant bits). For bfloat16 and binary32 operands it is exact unless
 * the exponents differ by more than 45 (resp. 29) binades; then the smaller
 * operand is below 2^-45 (2^-29) of the larger's unit in the last place, far
 * from any rounding boundary of the storage type, so rounding the double sum
 * to the storage type still gives the correctly rounded exact sum. */
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
    fill_tables();
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
    fill_tables();
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
    fill_tables();
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
    fill_tables();
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

/* Entry points with a storage type per operand group (MNO_F16, MNO_BF16,
 * MNO_F32, MNO_F64): tx for the activations X (and R), tg for gamma (and
 * beta), ty for the cotangents dY (and dH). */
int mno_rmsnorm_forward_t(const void* X, int tx, const void* gamma, int tg, int64_t N, int64_t D,
                          double eps, double* Y, double* rstd)
{
    if (!type_ok(tx) || !type_ok(tg)) return MNO_ERR_ARG;
    return rms_forward(opt(X, tx), opt(NULL, tx), opt(gamma, tg), N, D, eps, NULL, Y, rstd);
}

int mno_layernorm_forward_t(const void* X, int tx, const void* gamma, const void* beta, int tg,
                            int64_t N, int64_t D, double eps, double* Y, double* mean,
                            double* rstd)
{
    if (!type_ok(tx) || !type_ok(tg)) return MNO_ERR_ARG;
    return ln_forward(opt(X, tx), opt(gamma, tg), opt(beta, tg), N, D, eps, Y, mean, rstd);
}

int mno_add_rmsnorm_forward_t(const void* X, const void* R, int tx, const void* gamma, int tg,
                              int64_t N, int64_t D, double eps, double* S, double* Y,
                              double* rstd)
{
    if (!type_ok(tx) || !type_ok(tg) || !R) return MNO_ERR_ARG;
    return rms_forward(opt(X, tx), opt(R, tx), opt(gamma, tg), N, D, eps, S, Y, rstd);
}

int mno_rmsnorm_backward_t(const void* X, int tx, const void* gamma, int tg, const void* dY,
                           int ty, int64_t N, int64_t D, double eps, double* dX, double* dgamma)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ty)) return MNO_ERR_ARG;
    return rms_backward(opt(X, tx), opt(NULL, tx), opt(gamma, tg), opt(dY, ty), opt(NULL, ty),
                        N, D, eps, dX, dgamma);
}

int mno_layernorm_backward_t(const void* X, int tx, const void* gamma, int tg, const void* dY,
                             int ty, int64_t N, int64_t D, double eps, double* dX,
                             double* dgamma, double* dbeta)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ty)) return MNO_ERR_ARG;
    return ln_backward(opt(X, tx), opt(gamma, tg), opt(dY, ty), N, D, eps, dX, dgamma, dbeta);
}

int mno_add_rmsnorm_backward_t(const void* X, const void* R, int tx, const void* gamma, int tg,
                               const void* dY, const void* dH, int ty, int64_t N, int64_t D,
                               double eps, double* dX, double* dgamma)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ty) || !R) return MNO_ERR_ARG;
    return rms_backward(opt(X, tx), opt(R, tx), opt(gamma, tg), opt(dY, ty), opt(dH, ty), N, D,
                        eps, dX, dgamma);
}

/* ===========================================================================
 * The other row-wise normalizations the [meTile] coverage inventory lists as
 * missing (section "Normalization", parity checklist): Dynamic Tanh,
 * PolyNorm, Modulated RMSNorm and GroupNorm. The page names each with the
 * gradients it must return but gives no formula; each function below states
 * the published definition it writes out. Sums are in ascending order, row
 * by row, as above; backward functions recompute their statistics in fp64.
 * ======================================================================== */

/* ---------------------------------------------------------------------------
 * Dynamic Tanh (Zhu, Chen, He, LeCun and Liu, "Transformers without
 * Normalization", 2025): an element-wise stand-in for a normalization layer,
 *   y[i,j] = gamma[j] * tanh(alpha * x[i,j]) + beta[j]
 * with a trainable scalar alpha. [meTile] lists its gradients as alpha,
 * gamma and beta (and the input). With t = tanh(alpha x) and
 * dt/dx = alpha (1 - t^2):
 *   dX = dY * gamma * alpha * (1 - t^2)
 *   dalpha = sum over all elements of dY * gamma * x * (1 - t^2)
 *   dgamma[j] = sum_i dY * t,   dbeta[j] = sum_i dY.
 * ------------------------------------------------------------------------- */

static int dyt_forward(operand X, double alpha, operand G, operand B, int64_t N, int64_t D,
                       double* Y)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    get_row(B, 0, D, w.b);
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        for (int64_t j = 0; j < D; ++j) Y[i * D + j] = w.g[j] * tanh(alpha * w.x[j]) + w.b[j];
    }
    rows_free(&w);
    return MNO_OK;
}

static int dyt_backward(operand X, double alpha, operand G, operand DY, int64_t N, int64_t D,
                        double* dX, double* dalpha, double* dgamma, double* dbeta)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, D, w.g);
    for (int64_t j = 0; j < D; ++j) { dgamma[j] = 0.0; dbeta[j] = 0.0; }
    double da = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        get_row(DY, i, D, w.dy);
        for (int64_t j = 0; j < D; ++j) {
            double t = tanh(alpha * w.x[j]);
            double s = 1.0 - t * t;
            if (dX) dX[i * D + j] = w.dy[j] * w.g[j] * alpha * s;
            da += w.dy[j] * w.g[j] * w.x[j] * s;
            dgamma[j] += w.dy[j] * t;
            dbeta[j] += w.dy[j];
        }
    }
    *dalpha = da;
    rows_free(&w);
    return MNO_OK;
}

/* ---------------------------------------------------------------------------
 * PolyNorm (Zhuo et al., "Polynomial Composition Activations", 2024): a sum
 * of the RMS-normalised first three powers of the row,
 *   y = w[0] * n1 + w[1] * n2 + w[2] * n3 + b,   n_p = x^p * r_p,
 *   r_p = 1 / sqrt(mean_j((x_j^p)^2) + eps),
 * with trainable scalars w[0..2] and b; w[p-1] weighs the p-th power, and
 * eps enters as in RMSNorm (inside the square root). [meTile] asks for the
 * input and parameter gradients. Each n_p is an RMSNorm of u = x^p with a
 * scalar weight, so with g = dY:
 *   dU_p = w[p-1] * r_p * (g - n_p * mean_j(g * n_p))
 *   dX = sum_p p * x^(p-1) * dU_p
 *   dw[p-1] = sum over all elements of g * n_p,   db = sum of g.
 * The forward also returns the three r_p of each row (rstd[3 i + p - 1]).
 * ------------------------------------------------------------------------- */

static int poly_forward(operand X, const double* wp, double bias, int64_t N, int64_t D,
                        double eps, double* Y, double* rstd)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        double r[3];
        for (int p = 1; p <= 3; ++p) {
            for (int64_t j = 0; j < D; ++j) w.xh[j] = pow(w.x[j], (double)p);
            r[p - 1] = rms_rstd(w.xh, D, eps);
            if (rstd) rstd[3 * i + p - 1] = r[p - 1];
        }
        for (int64_t j = 0; j < D; ++j) {
            double y = bias;
            for (int p = 1; p <= 3; ++p) y += wp[p - 1] * (pow(w.x[j], (double)p) * r[p - 1]);
            Y[i * D + j] = y;
        }
    }
    rows_free(&w);
    return MNO_OK;
}

static int poly_backward(operand X, const double* wp, operand DY, int64_t N, int64_t D,
                         double eps, double* dX, double* dw, double* db)
{
    if (bad_shape(N, D)) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    double sw[3] = {0.0, 0.0, 0.0}, sb = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        get_row(X, i, D, w.x);
        get_row(DY, i, D, w.dy);
        if (dX)
            for (int64_t j = 0; j < D; ++j) dX[i * D + j] = 0.0;
        for (int p = 1; p <= 3; ++p) {
            for (int64_t j = 0; j < D; ++j) w.xh[j] = pow(w.x[j], (double)p);
            double r = rms_rstd(w.xh, D, eps);
            double c = 0.0;
            for (int64_t j = 0; j < D; ++j) {
                w.xh[j] *= r;                       /* n_p */
                c += w.dy[j] * w.xh[j];
                sw[p - 1] += w.dy[j] * w.xh[j];
            }
            c /= (double)D;
            if (dX)
                for (int64_t j = 0; j < D; ++j) {
                    double du = wp[p - 1] * r * (w.dy[j] - w.xh[j] * c);
                    dX[i * D + j] += (double)p * pow(w.x[j], (double)(p - 1)) * du;
                }
        }
        for (int64_t j = 0; j < D; ++j) sb += w.dy[j];
    }
    for (int p = 0; p < 3; ++p) dw[p] = sw[p];
    *db = sb;
    rows_free(&w);
    return MNO_OK;
}

/* ---------------------------------------------------------------------------
 * Modulated RMSNorm: RMSNorm whose output is modulated per sample by a
 * broadcast scale and shift (the adaptive-norm modulation of conditioned
 * transformers), rows grouped into B samples of S = N / B consecutive rows:
 *   y[i,j] = gamma[j] * xhat[i,j] * (1 + scale[b,j]) + shift[b,j],
 *   xhat = x * rstd (RMSNorm),  b = i / S.
 * [meTile] asks for the input, weight and broadcast scale/shift gradients.
 * With m[i,j] = gamma[j] (1 + scale[b,j]) the row is an RMSNorm with weight
 * m, so with g = dY * m:
 *   dX = rstd * (g - xhat * mean_j(g * xhat))
 *   dgamma[j] = sum_i dY * xhat * (1 + scale[b,j])
 *   dscale[b,j] = sum_{i in b} dY * xhat * gamma[j]
 *   dshift[b,j] = sum_{i in b} dY.
 * ------------------------------------------------------------------------- */

static int modrms_forward(operand X, operand G, operand SC, operand SH, int64_t B, int64_t N,
                          int64_t D, double eps, double* Y, double* rstd)
{
    if (bad_shape(N, D) || B < 1 || N % B != 0) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    const int64_t S = N / B;
    get_row(G, 0, D, w.g);
    for (int64_t i = 0; i < N; ++i) {
        const int64_t b = i / S;
        get_row(X, i, D, w.x);
        get_row(SC, b, D, w.r);
        get_row(SH, b, D, w.b);
        double r = rms_rstd(w.x, D, eps);
        rstd[i] = r;
        for (int64_t j = 0; j < D; ++j)
            Y[i * D + j] = w.g[j] * (w.x[j] * r) * (1.0 + w.r[j]) + w.b[j];
    }
    rows_free(&w);
    return MNO_OK;
}

static int modrms_backward(operand X, operand G, operand SC, operand DY, int64_t B, int64_t N,
                           int64_t D, double eps, double* dX, double* dgamma, double* dscale,
                           double* dshift)
{
    if (bad_shape(N, D) || B < 1 || N % B != 0) return MNO_ERR_ARG;
    fill_tables();
    rows w;
    if (!rows_alloc(&w, D)) { rows_free(&w); return MNO_ERR_MEM; }
    const int64_t S = N / B;
    get_row(G, 0, D, w.g);
    for (int64_t j = 0; j < D; ++j) dgamma[j] = 0.0;
    for (int64_t k = 0; k < B * D; ++k) { dscale[k] = 0.0; dshift[k] = 0.0; }
    for (int64_t i = 0; i < N; ++i) {
        const int64_t b = i / S;
        get_row(X, i, D, w.x);
        get_row(SC, b, D, w.r);
        get_row(DY, i, D, w.dy);
        double r = rms_rstd(w.x, D, eps);
        double c1 = 0.0;
        for (int64_t j = 0; j < D; ++j) {
            w.xh[j] = w.x[j] * r;
            c1 += w.dy[j] * w.g[j] * (1.0 + w.r[j]) * w.xh[j];
        }
        c1 /= (double)D;
        if (dX)
            for (int64_t j = 0; j < D; ++j)
                dX[i * D + j] = r * (w.dy[j] * w.g[j] * (1.0 + w.r[j]) - w.xh[j] * c1);
        for (int64_t j = 0; j < D; ++j) {
            dgamma[j] += w.dy[j] * w.xh[j] * (1.0 + w.r[j]);
            dscale[b * D + j] += w.dy[j] * w.xh[j] * w.g[j];
            dshift[b * D + j] += w.dy[j];
        }
    }
    rows_free(&w);
    return MNO_OK;
}

/* ---------------------------------------------------------------------------
 * GroupNorm (Wu and He, "Group Normalization", 2018) on X of shape
 * [N, C, L] (L positions per channel, contiguous): the C channels form G
 * groups of C / G consecutive channels; each (sample, group) slice of
 * (C / G) * L contiguous values is centred by its mean and scaled by its
 * rstd (population variance, eps inside the square root, as LayerNorm), and
 * channel c then takes its own affine weight and bias:
 *   y[n,c,l] = (x[n,c,l] - mean[n,g]) * rstd[n,g] * gamma[c] + beta[c].
 * [meTile] asks for the group/channel layouts and the affine gradients. The
 * backward is the LayerNorm backward over each slice with a per-channel
 * weight (g = dY * gamma[c], M = (C / G) * L):
 *   dX = rstd * (g - mean_M(g) - xhat * mean_M(g * xhat))
 *   dgamma[c] = sum_{n,l} dY * xhat,   dbeta[c] = sum_{n,l} dY.
 * mean and rstd are [N, G].
 * ------------------------------------------------------------------------- */

static int gn_forward(operand X, operand G, operand B, int64_t N, int64_t C, int64_t L,
                      int64_t groups, double eps, double* Y, double* mean, double* rstd)
{
    if (N < 0 || C < 1 || L < 1 || groups < 1 || C % groups != 0) return MNO_ERR_ARG;
    fill_tables();
    const int64_t M = (C / groups) * L;
    rows w;
    if (!rows_alloc(&w, M > C ? M : C)) { rows_free(&w); return MNO_ERR_MEM; }
    double* gam = malloc(sizeof(double) * (size_t)C);
    double* bet = malloc(sizeof(double) * (size_t)C);
    if (!gam || !bet) { free(gam); free(bet); rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, C, gam);
    get_row(B, 0, C, bet);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < groups; ++g) {
            const int64_t slice = n * groups + g;     /* row `slice` of [N*G, M] */
            get_row(X, slice, M, w.x);
            double mu, r;
            ln_stats(w.x, M, eps, &mu, &r);
            mean[slice] = mu;
            rstd[slice] = r;
            for (int64_t k = 0; k < M; ++k) {
                const int64_t c = g * (C / groups) + k / L;
                Y[slice * M + k] = (w.x[k] - mu) * r * gam[c] + bet[c];
            }
        }
    free(gam); free(bet);
    rows_free(&w);
    return MNO_OK;
}

static int gn_backward(operand X, operand G, operand DY, int64_t N, int64_t C, int64_t L,
                       int64_t groups, double eps, double* dX, double* dgamma, double* dbeta)
{
    if (N < 0 || C < 1 || L < 1 || groups < 1 || C % groups != 0) return MNO_ERR_ARG;
    fill_tables();
    const int64_t M = (C / groups) * L;
    rows w;
    if (!rows_alloc(&w, M > C ? M : C)) { rows_free(&w); return MNO_ERR_MEM; }
    double* gam = malloc(sizeof(double) * (size_t)C);
    if (!gam) { rows_free(&w); return MNO_ERR_MEM; }
    get_row(G, 0, C, gam);
    for (int64_t c = 0; c < C; ++c) { dgamma[c] = 0.0; dbeta[c] = 0.0; }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < groups; ++g) {
            const int64_t slice = n * groups + g;
            get_row(X, slice, M, w.x);
            get_row(DY, slice, M, w.dy);
            double mu, r;
            ln_stats(w.x, M, eps, &mu, &r);
            double c1 = 0.0, c2 = 0.0;
            for (int64_t k = 0; k < M; ++k) {
                const int64_t c = g * (C / groups) + k / L;
                w.xh[k] = (w.x[k] - mu) * r;
                c1 += w.dy[k] * gam[c] * w.xh[k];
                c2 += w.dy[k] * gam[c];
            }
            c1 /= (double)M;
            c2 /= (double)M;
            for (int64_t k = 0; k < M; ++k) {
                const int64_t c = g * (C / groups) + k / L;
                if (dX) dX[slice * M + k] = r * (w.dy[k] * gam[c] - c2 - w.xh[k] * c1);
                dgamma[c] += w.dy[k] * w.xh[k];
                dbeta[c] += w.dy[k];
            }
        }
    free(gam);
    rows_free(&w);
    return MNO_OK;
}

/* Typed entry points of the four (types as for the entry points above: tx
 * for X, tg for gamma/beta, ts for scale/shift, ty for dY). */
int mno_dyt_forward_t(const void* X, int tx, double alpha, const void* gamma, const void* beta,
                      int tg, int64_t N, int64_t D, double* Y)
{
    if (!type_ok(tx) || !type_ok(tg)) return MNO_ERR_ARG;
    return dyt_forward(opt(X, tx), alpha, opt(gamma, tg), opt(beta, tg), N, D, Y);
}

int mno_dyt_backward_t(const void* X, int tx, double alpha, const void* gamma, int tg,
                       const void* dY, int ty, int64_t N, int64_t D, double* dX, double* dalpha,
                       double* dgamma, double* dbeta)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ty)) return MNO_ERR_ARG;
    return dyt_backward(opt(X, tx), alpha, opt(gamma, tg), opt(dY, ty), N, D, dX, dalpha,
                        dgamma, dbeta);
}

int mno_polynorm_forward_t(const void* X, int tx, const double* w, double b, int64_t N,
                           int64_t D, double eps, double* Y, double* rstd)
{
    if (!type_ok(tx)) return MNO_ERR_ARG;
    return poly_forward(opt(X, tx), w, b, N, D, eps, Y, rstd);
}

int mno_polynorm_backward_t(const void* X, int tx, const double* w, const void* dY, int ty,
                            int64_t N, int64_t D, double eps, double* dX, double* dw, double* db)
{
    if (!type_ok(tx) || !type_ok(ty)) return MNO_ERR_ARG;
    return poly_backward(opt(X, tx), w, opt(dY, ty), N, D, eps, dX, dw, db);
}

int mno_modrms_forward_t(const void* X, int tx, const void* gamma, int tg, const void* scale,
                         const void* shift, int ts, int64_t B, int64_t N, int64_t D, double eps,
                         double* Y, double* rstd)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ts)) return MNO_ERR_ARG;
    return modrms_forward(opt(X, tx), opt(gamma, tg), opt(scale, ts), opt(shift, ts), B, N, D,
                          eps, Y, rstd);
}

int mno_modrms_backward_t(const void* X, int tx, const void* gamma, int tg, const void* scale,
                          int ts, const void* dY, int ty, int64_t B, int64_t N, int64_t D,
                          double eps, double* dX, double* dgamma, double* dscale,
                          double* dshift)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ts) || !type_ok(ty)) return MNO_ERR_ARG;
    return modrms_backward(opt(X, tx), opt(gamma, tg), opt(scale, ts), opt(dY, ty), B, N, D,
                           eps, dX, dgamma, dscale, dshift);
}

int mno_groupnorm_forward_t(const void* X, int tx, const void* gamma, const void* beta, int tg,
                            int64_t N, int64_t C, int64_t L, int64_t G, double eps, double* Y,
                            double* mean, double* rstd)
{
    if (!type_ok(tx) || !type_ok(tg)) return MNO_ERR_ARG;
    return gn_forward(opt(X, tx), opt(gamma, tg), opt(beta, tg), N, C, L, G, eps, Y, mean,
                      rstd);
}

int mno_groupnorm_backward_t(const void* X, int tx, const void* gamma, int tg, const void* dY,
                             int ty, int64_t N, int64_t C, int64_t L, int64_t G, double eps,
                             double* dX, double* dgamma, double* dbeta)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(ty)) return MNO_ERR_ARG;
    return gn_backward(opt(X, tx), opt(gamma, tg), opt(dY, ty), N, C, L, G, eps, dX, dgamma,
                       dbeta);
}

/* ---------------------------------------------------------------------------
 * Fused normalization + GEMV ([tensorcore] "Fused Norm + GEMV"): for an
 * inference batch X [M, K] (M small), Y [M, N] = Norm(X) @ W with W [K, N]
 * row-major and Norm the RMSNorm (gamma) or LayerNorm (gamma, beta) of each
 * row over its K columns, exactly as the forward functions above; the
 * normalised rows are not rounded to a storage type before the product (the
 * fused kernel never stores them). No statistics are returned. Sums over k
 * are in ascending order.
 * ------------------------------------------------------------------------- */

static int norm_gemv(int ln, operand X, operand G, operand B, operand W, int64_t M, int64_t N,
                     int64_t K, double eps, double* Y)
{
    if (bad_shape(M, K) || N < 1) return MNO_ERR_ARG;
    fill_tables();
    double* xn = malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)K);
    double *mean = malloc(sizeof(double) * (size_t)(M > 0 ? M : 1)),
           *rstd = malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double* wrow = malloc(sizeof(double) * (size_t)N);
    if (!xn || !mean || !rstd || !wrow) {
        free(xn); free(mean); free(rstd); free(wrow);
        return MNO_ERR_MEM;
    }
    int rc = ln ? ln_forward(X, G, B, M, K, eps, xn, mean, rstd)
                : rms_forward(X, opt(NULL, X.type), G, M, K, eps, NULL, xn, rstd);
    if (rc == MNO_OK) {
        for (int64_t i = 0; i < M * N; ++i) Y[i] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            get_row(W, k, N, wrow);
            for (int64_t m = 0; m < M; ++m) {
                const double a = xn[m * K + k];
                for (int64_t n = 0; n < N; ++n) Y[m * N + n] += a * wrow[n];
            }
        }
    }
    free(xn); free(mean); free(rstd); free(wrow);
    return rc;
}

int mno_rmsnorm_gemv_t(const void* X, int tx, const void* gamma, int tg, const void* W, int tw,
                       int64_t M, int64_t N, int64_t K, double eps, double* Y)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(tw)) return MNO_ERR_ARG;
    return norm_gemv(0, opt(X, tx), opt(gamma, tg), opt(NULL, tg), opt(W, tw), M, N, K, eps, Y);
}

int mno_layernorm_gemv_t(const void* X, int tx, const void* gamma, const void* beta, int tg,
                         const void* W, int tw, int64_t M, int64_t N, int64_t K, double eps,
                         double* Y)
{
    if (!type_ok(tx) || !type_ok(tg) || !type_ok(tw)) return MNO_ERR_ARG;
    return norm_gemv(1, opt(X, tx), opt(gamma, tg), opt(beta, tg), opt(W, tw), M, N, K, eps, Y);
}
