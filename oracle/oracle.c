/*
 * oracle.c -- double-precision CPU oracle for the fused (bias +) residual +
 * LayerNorm / RMSNorm forward with FP8 amax, and for the LayerNorm / RMSNorm
 * backward (dx, dgamma, dbeta).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU product
 * path never calls it, shares no code with it, and must fail loudly when its
 * own HIP library is missing instead of falling back to anything here.
 *
 * What it computes is the plain textbook definition, evaluated in double:
 *
 *  forward  -- nvFuser issue #1660 ("performance optimization for moving
 *              distributive reduction operation across broadcast dimensions"),
 *              the layernorm + amax comment: out1 = (x + bias) + residual,
 *              viewed as rows of the hidden size; out2 = layer_norm(out1, w,
 *              ln_bias, eps); amax = max(abs(out2)) written with fill_.
 *              IREE issue #9139 ("Investigate a fusion opportunity on Layer
 *              Normalization"), opening comment: the three steps are mean
 *              (reduction), variance (reduction) and the element-wise
 *              normalisation; the mean feeds the variance.
 *  backward -- PyTorch PR #165370 (Inductor mix-order reduction), PR
 *              description: the dx reduction runs over the hidden dimension,
 *              the dw/db reduction over the B x T rows; step 3: dw/db may end
 *              with a down-cast to fp16/bf16.  The pages do not write the
 *              gradient formulas out; they are the exact derivatives of the
 *              forward definition (standard calculus), stated where used.
 *              The gradient of the forward's bias (the column sums of dx) is
 *              the backward of the fused add that the nvFuser comment's
 *              forward starts with.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - variance is the biased one (divide by N), as in the layer_norm the
 *    nvFuser comment calls;  rstd = 1 / sqrt(var + eps);
 *  - RMSNorm: rstd = 1 / sqrt(mean(u^2) + eps), y = u * rstd * gamma (+ beta);
 *  - the sum x + bias + residual is formed exactly and rounded once to the
 *    I/O dtype; that rounded tensor u (residual_out) is what is normalised;
 *  - every cast to bf16 rounds to nearest, ties to even;
 *  - amax is the maximum absolute value of y *after* rounding to the I/O
 *    dtype, reported in double (the caller narrows it to fp32);
 *  - gamma == NULL means gamma = 1, beta == NULL means beta = 0, absent bias
 *    or residual means 0.
 *
 * Element types: dtype 0 = IEEE fp32, dtype 1 = bf16 given as raw 16-bit
 * patterns (the upper half of an fp32 pattern).
 *
 * Threads: rows are independent, so row-wise work is split over threads by
 * contiguous row ranges; each column sum is computed by one thread, over all
 * rows in ascending order.  Every output value is therefore produced by the
 * same sequence of operations for any thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* ---------------------------------------------------------------- scalars */

static double elem(const void *p, int dtype, int64_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)p)[i];
    /* a bf16 pattern is the upper 16 bits of the fp32 pattern of its value */
    uint32_t w = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Optional per-column vector: absent means the neutral value `dflt`. */
static double elem_or(const void *p, int dtype, int64_t i, double dflt)
{
    return p ? elem(p, dtype, i) : dflt;
}

/* Round a double to the nearest bf16 value, ties to even.  bf16 keeps 8
 * significant bits and fp32's exponent range, so a value in [2^(e-1), 2^e)
 * has spacing 2^(e-8); the smallest (subnormal) spacing is 2^-133. */
static double round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    (void)frexp(fabs(v), &e); /* |v| = m * 2^e with m in [0.5, 1) */
    int q = e - 8;
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(fabs(v), -q)), q); /* nearbyint: ties to even */
    if (r >= 0x1p128)
        r = INFINITY;
    return copysign(r, v);
}

static double round_io(double v, int dtype)
{
    return dtype == OR_F32 ? (double)(float)v : round_bf16(v);
}

/* Store the (already representable) value v in the I/O dtype. */
static void store_io(void *p, int dtype, int64_t i, double v)
{
    float f = (float)v;
    if (dtype == OR_F32) {
        ((float *)p)[i] = f;
    } else {
        uint32_t w;
        memcpy(&w, &f, sizeof w);
        ((uint16_t *)p)[i] = (uint16_t)(w >> 16);
    }
}

/* ------------------------------------------------------------ threading */

typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);

typedef struct {
    range_fn fn;
    void *ctx;
    int64_t lo, hi;
} range_job;

static void *range_trampoline(void *arg)
{
    range_job *j = (range_job *)arg;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

/* Run fn over [0, n) split into `nthreads` contiguous ranges. */
static void parallel_ranges(int nthreads, int64_t n, range_fn fn, void *ctx)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > n)
        nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t tid[256];
    range_job job[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        job[t].fn = fn;
        job[t].ctx = ctx;
        job[t].lo = n * t / nthreads;
        job[t].hi = n * (t + 1) / nthreads;
        started[t] = pthread_create(&tid[t], NULL, range_trampoline, &job[t]) == 0;
        if (!started[t])
            range_trampoline(&job[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t])
            pthread_join(tid[t], NULL);
}

/* -------------------------------------------------------------- forward */

typedef struct {
    int is_rms, dtype;
    const void *x, *bias, *res, *gamma, *beta;
    double eps;
    int64_t N;
    void *u_out;
    double *y, *mean, *rstd;
    double *row_amax; /* per row: max |round_io(y)| */
    int zero_centered;
} fwd_ctx;

/* The scale the normalised value is multiplied by: gamma (1 when absent),
 * or with a zero-centred gamma w = 1 + gamma, formed in the I/O dtype as the
 * nvFuser issue's layernorm + amax comment forms it (`1 + ln_weight` on the
 * weight tensor) before it is handed to layer_norm. */
static double weight_of(const void *gamma, int dtype, int zero_centered, int64_t j)
{
    const double g = elem_or(gamma, dtype, j, zero_centered ? 0.0 : 1.0);
    return zero_centered ? round_io(1.0 + g, dtype) : g;
}

static void fwd_rows(void *vctx, int64_t r0, int64_t r1)
{
    fwd_ctx *c = (fwd_ctx *)vctx;
    const int64_t N = c->N;
    double *u = (double *)malloc((size_t)N * sizeof(double));
    if (!u)
        abort();
    for (int64_t i = r0; i < r1; ++i) {
        /* out1 = (x + bias) + residual, formed exactly, rounded once */
        for (int64_t j = 0; j < N; ++j) {
            double t = elem(c->x, c->dtype, i * N + j) + elem_or(c->bias, c->dtype, j, 0.0) +
                       elem_or(c->res, c->dtype, i * N + j, 0.0);
            u[j] = round_io(t, c->dtype);
            if (c->u_out)
                store_io(c->u_out, c->dtype, i * N + j, u[j]);
        }
        double mean = 0.0, rstd;
        if (!c->is_rms) {
            /* mean, then the (biased) variance about that mean */
            double s = 0.0;
            for (int64_t j = 0; j < N; ++j)
                s += u[j];
            mean = s / (double)N;
            double v = 0.0;
            for (int64_t j = 0; j < N; ++j)
                v += (u[j] - mean) * (u[j] - mean);
            v /= (double)N;
            rstd = 1.0 / sqrt(v + c->eps);
        } else {
            /* mean square */
            double s = 0.0;
            for (int64_t j = 0; j < N; ++j)
                s += u[j] * u[j];
            rstd = 1.0 / sqrt(s / (double)N + c->eps);
        }
        double amax = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double g = weight_of(c->gamma, c->dtype, c->zero_centered, j);
            double b = elem_or(c->beta, c->dtype, j, 0.0);
            double yv = (u[j] - mean) * rstd * g + b;
            if (c->y)
                c->y[i * N + j] = yv;
            double a = fabs(round_io(yv, c->dtype));
            if (a > amax)
                amax = a;
        }
        if (c->mean)
            c->mean[i] = mean;
        if (c->rstd)
            c->rstd[i] = rstd;
        if (c->row_amax)
            c->row_amax[i] = amax;
    }
    free(u);
}

/*
 * Fused (bias +) residual + LayerNorm (is_rms = 0) or RMSNorm (is_rms = 1)
 * forward over an M x N row-major matrix.
 *   inputs : x [M,N]; bias [N], residual [M,N], gamma [N], beta [N] optional.
 *   outputs (each optional): u_out [M,N] in the I/O dtype (residual_out),
 *            y [M,N] exact (double, before any output rounding),
 *            mean [M] (LayerNorm; 0 for RMSNorm), rstd [M], *amax.
 *   zero_centered: the weight is w = round_io(1 + gamma) (weight_of).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_norm_fwd(int is_rms, const void *x, const void *bias, const void *residual,
                    const void *gamma, const void *beta, double eps, int64_t M, int64_t N,
                    int dtype, int nthreads, void *u_out, double *y, double *mean, double *rstd,
                    double *amax, int zero_centered)
{
    if (!x || M < 0 || N <= 0 || (dtype != OR_F32 && dtype != OR_BF16) || !(eps >= 0.0))
        return -1;
    double *row_amax = NULL;
    if (amax && M > 0) {
        row_amax = (double *)malloc((size_t)M * sizeof(double));
        if (!row_amax)
            return -1;
    }
    fwd_ctx c = {is_rms, dtype, x, bias, residual, gamma, beta, eps, N,
                 u_out, y, mean, rstd, row_amax, zero_centered};
    parallel_ranges(nthreads, M, fwd_rows, &c);
    if (amax) {
        double m = 0.0; /* M = 0: nothing to take the max of */
        for (int64_t i = 0; i < M; ++i)
            if (row_amax[i] > m)
                m = row_amax[i];
        *amax = m;
    }
    free(row_amax);
    return 0;
}

/* ------------------------------------------------------------- backward */

typedef struct {
    int is_rms, dtype;
    const void *dy, *x, *gamma;
    const double *mean, *rstd_in;
    double eps;
    int64_t M, N;
    double *rstd; /* per-row rstd actually used (given or recomputed) */
    double *dx;
    double *dgamma, *dbeta, *dgamma_l2, *dbeta_l2;
    double *dbias, *dbias_l2;
    int zero_centered;
} bwd_ctx;

static double xhat_of(const bwd_ctx *c, int64_t i, int64_t j)
{
    double xv = elem(c->x, c->dtype, i * c->N + j);
    return c->is_rms ? xv * c->rstd[i] : (xv - c->mean[i]) * c->rstd[i];
}

/* RMSNorm without a saved rstd: recompute it from x with the call's eps. */
static void bwd_rstd_rows(void *vctx, int64_t r0, int64_t r1)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    for (int64_t i = r0; i < r1; ++i) {
        if (c->rstd_in) {
            c->rstd[i] = c->rstd_in[i];
            continue;
        }
        double s = 0.0;
        for (int64_t j = 0; j < c->N; ++j) {
            double xv = elem(c->x, c->dtype, i * c->N + j);
            s += xv * xv;
        }
        c->rstd[i] = 1.0 / sqrt(s / (double)c->N + c->eps);
    }
}

/*
 * dx of one row.  With xhat the normalised input and g = dy * gamma:
 *   LayerNorm: dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
 *   RMSNorm  : dx = rstd * (g - xhat * mean_j(g * xhat))
 * (derivative of y = xhat * gamma + beta through the row's mean and rstd).
 */
static void bwd_dx_rows(void *vctx, int64_t r0, int64_t r1)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    const int64_t N = c->N;
    for (int64_t i = r0; i < r1; ++i) {
        double s_gx = 0.0, s_g = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double g = elem(c->dy, c->dtype, i * N + j) *
                       weight_of(c->gamma, c->dtype, c->zero_centered, j);
            s_gx += g * xhat_of(c, i, j);
            s_g += g;
        }
        double c1 = s_gx / (double)N;
        double c2 = c->is_rms ? 0.0 : s_g / (double)N;
        for (int64_t j = 0; j < N; ++j) {
            double g = elem(c->dy, c->dtype, i * N + j) *
                       weight_of(c->gamma, c->dtype, c->zero_centered, j);
            c->dx[i * N + j] = c->rstd[i] * (g - c2 - xhat_of(c, i, j) * c1);
        }
    }
}

/* dgamma_j = sum_i dy_ij * xhat_ij,  dbeta_j = sum_i dy_ij, rows in order.
 * Also the 2-norm of the summed terms, the scale the column sums are compared
 * against. */
static void bwd_col_sums(void *vctx, int64_t j0, int64_t j1)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    for (int64_t j = j0; j < j1; ++j) {
        double sg = 0.0, sb = 0.0, qg = 0.0, qb = 0.0;
        for (int64_t i = 0; i < c->M; ++i) {
            double d = elem(c->dy, c->dtype, i * c->N + j);
            double tg = d * xhat_of(c, i, j);
            sg += tg;
            qg += tg * tg;
            sb += d;
            qb += d * d;
        }
        if (c->dgamma)
            c->dgamma[j] = sg;
        if (c->dbeta)
            c->dbeta[j] = sb;
        if (c->dgamma_l2)
            c->dgamma_l2[j] = sqrt(qg);
        if (c->dbeta_l2)
            c->dbeta_l2[j] = sqrt(qb);
    }
}

/* dbias_j = sum_i dx_ij, rows in order, and the 2-norm of its terms.  The
 * forward adds bias to every row before normalising (nvFuser issue #1660,
 * layernorm + amax comment: out1 = (x + bias) + residual), so the gradient
 * of the loss with respect to bias_j is the column sum of the gradient with
 * respect to out1, which is dx; x and residual each receive dx itself.  A
 * third reduction over the B x T rows, of the kind PyTorch PR #165370
 * (description) computes next to dw/db. */
static void bwd_dbias_cols(void *vctx, int64_t j0, int64_t j1)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    for (int64_t j = j0; j < j1; ++j) {
        double s = 0.0, q = 0.0;
        for (int64_t i = 0; i < c->M; ++i) {
            double t = c->dx[i * c->N + j];
            s += t;
            q += t * t;
        }
        if (c->dbias)
            c->dbias[j] = s;
        if (c->dbias_l2)
            c->dbias_l2[j] = sqrt(q);
    }
}

/*
 * LayerNorm (is_rms = 0) or RMSNorm (is_rms = 1) backward.
 *   inputs : dy [M,N], x [M,N] (the tensor that was normalised), gamma [N]
 *            (NULL = 1); LayerNorm needs mean [M] and rstd [M]; RMSNorm takes
 *            rstd [M] or NULL to recompute it from x with eps.
 *   outputs (each optional): dx [M,N], dgamma [N], dbeta [N] in double,
 *            unrounded; dgamma_l2 / dbeta_l2 [N] = 2-norm of the summed terms;
 *            rstd_out [M] = the rstd used (given or recomputed); dbias [N] =
 *            the gradient of the forward's bias (column sums of dx) and
 *            dbias_l2 [N] the 2-norm of its terms.
 *   zero_centered: the forward's weight was w = round_io(1 + gamma); dx uses
 *            w, and dgamma (dL/dgamma = dL/dw) keeps its form.
 *   dparam_mean: the "division for mean" epilogue of PyTorch PR #165370
 *            (description, step 3): dgamma, dbeta, dbias and their 2-norms
 *            are divided by M (the mean over the rows instead of the sum).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_norm_bwd(int is_rms, const void *dy, const void *x, const void *gamma,
                    const double *mean, const double *rstd, double eps, int64_t M, int64_t N,
                    int dtype, int nthreads, double *dx, double *dgamma, double *dbeta,
                    double *dgamma_l2, double *dbeta_l2, double *rstd_out, double *dbias,
                    double *dbias_l2, int zero_centered, int dparam_mean)
{
    if (!dy || !x || M < 0 || N <= 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    if (!is_rms && (!mean || !rstd))
        return -1;
    if (is_rms && !rstd && !(eps >= 0.0))
        return -1;
    double *rstd_used = (double *)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
    if (!rstd_used)
        return -1;
    /* dbias needs dx: a scratch copy when the caller does not want dx */
    const int want_db = dbias || dbias_l2;
    double *dx_buf = dx;
    if (want_db && !dx_buf) {
        dx_buf = (double *)malloc((size_t)(M > 0 ? M * N : 1) * sizeof(double));
        if (!dx_buf) {
            free(rstd_used);
            return -1;
        }
    }
    bwd_ctx c = {is_rms, dtype, dy, x, gamma, mean, rstd, eps, M, N,
                 rstd_used, dx_buf, dgamma, dbeta, dgamma_l2, dbeta_l2, dbias, dbias_l2,
                 zero_centered};
    parallel_ranges(nthreads, M, bwd_rstd_rows, &c);
    if (dx_buf)
        parallel_ranges(nthreads, M, bwd_dx_rows, &c);
    if (dgamma || dbeta || dgamma_l2 || dbeta_l2)
        parallel_ranges(nthreads, N, bwd_col_sums, &c);
    if (want_db)
        parallel_ranges(nthreads, N, bwd_dbias_cols, &c);
    if (dparam_mean && M > 0) {
        double *outs[6] = {dgamma, dbeta, dgamma_l2, dbeta_l2, dbias, dbias_l2};
        for (int k = 0; k < 6; ++k)
            if (outs[k])
                for (int64_t j = 0; j < N; ++j)
                    outs[k][j] /= (double)M;
    }
    if (rstd_out && M > 0)
        memcpy(rstd_out, rstd_used, (size_t)M * sizeof(double));
    if (dx_buf != dx)
        free(dx_buf);
    free(rstd_used);
    return 0;
}

/* Round n doubles to the I/O dtype (ties to even) and store them as that
 * dtype's patterns; used for the down-cast of dgamma / dbeta. */
int oracle_round_to_dtype(const double *v, int64_t n, int dtype, void *out)
{
    if ((!v && n > 0) || (!out && n > 0) || n < 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        store_io(out, dtype, i, round_io(v[i], dtype));
    return 0;
}

/* ---------------------------------------------------------- FP8 output */

/*
 * OCP FP8 E4M3 (the "e4m3fn" variant): 1 sign, 4 exponent (bias 7) and 3
 * mantissa bits; normal magnitudes 2^-6 .. 448 (= 1.75 * 2^8), subnormals
 * k * 2^-9, no infinity, S.1111.111 is NaN.  Rounds to nearest, ties to
 * even; magnitudes beyond 448 saturate to 448, since the format has no
 * infinity to round to.  This is the FP8 output that the nvFuser issue's
 * layernorm + amax comment computes the scaling amax for.
 */
static uint8_t encode_e4m3(double v)
{
    if (isnan(v))
        return 0x7F;
    const uint8_t s = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    if (a == 0.0)
        return s;
    int e;
    (void)frexp(a, &e); /* a in [2^(e-1), 2^e): spacing 2^(e-1-3) */
    int q = e - 4;
    if (q < -9)
        q = -9; /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(a, -q)), q); /* nearbyint: ties to even */
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return s;
    if (r < 0x1p-6) /* subnormal: exponent field 0, mantissa r / 2^-9 */
        return (uint8_t)(s | (uint8_t)(r / 0x1p-9));
    int er;
    const double m = frexp(r, &er); /* r = (2m) 2^(er-1), 2m in [1, 2) */
    const int exp_field = er - 1 + 7;
    const int mant = (int)((2.0 * m - 1.0) * 8.0);
    return (uint8_t)(s | (exp_field << 3) | mant);
}

/* out[i] = E4M3 code of the fp32 product v[i] * scale (the product rounded
 * to fp32 first, as a kernel computing in fp32 forms it). */
int oracle_quantize_e4m3(const float *v, int64_t n, float scale, uint8_t *out)
{
    if (n < 0 || (n > 0 && (!v || !out)))
        return -1;
    for (int64_t i = 0; i < n; ++i) {
        const float p = v[i] * scale;
        out[i] = encode_e4m3((double)p);
    }
    return 0;
}

/* ------------------------------------------------------------- softmax */

/*
 * Row softmax, the other normalisation IREE issue #9139 ("Investigate a
 * fusion opportunity on Layer Normalization") fuses into one dispatch in its
 * softmax walk-through: per row, the max, the sum of exp(x - max), and the
 * division:
 *   y_ij = exp(x_ij - max_k x_ik) / sum_k exp(x_ik - max_k x_ik)
 * Subtracting the row max leaves y unchanged and keeps exp in range.
 */
typedef struct {
    const void *x;
    int dtype;
    int64_t N;
    double *y;
} smx_ctx;

static void smx_rows(void *vctx, int64_t r0, int64_t r1)
{
    smx_ctx *c = (smx_ctx *)vctx;
    const int64_t N = c->N;
    for (int64_t i = r0; i < r1; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            double v = elem(c->x, c->dtype, i * N + j);
            if (v > m)
                m = v;
        }
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j)
            s += exp(elem(c->x, c->dtype, i * N + j) - m);
        for (int64_t j = 0; j < N; ++j)
            c->y[i * N + j] = exp(elem(c->x, c->dtype, i * N + j) - m) / s;
    }
}

/* y [M,N] (double, unrounded) = row softmax of x [M,N] (finite values). */
int oracle_softmax_fwd(const void *x, int64_t M, int64_t N, int dtype, int nthreads, double *y)
{
    if (!x || !y || M < 0 || N <= 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    smx_ctx c = {x, dtype, N, y};
    parallel_ranges(nthreads, M, smx_rows, &c);
    return 0;
}
