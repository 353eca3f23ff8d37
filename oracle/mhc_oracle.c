/*
 * mhc_oracle.c -- plain, slow CPU oracle for the mHC seam block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * Sources (cited by page title and section):
 *   [p1] vLLM PR "[ROCm][DSV4.1][Perf] Use AITER mHC for the delayed pre block"
 *        -- Summary, Purpose, Approach, Result, Notes / follow-ups.
 *   [p3] vLLM PR "[ROCm][DSv4.1] Fix TileLang mHC pre on 64-wide wavefronts
 *        and use the fused kernels on the AMD path" -- The bug, Measurements.
 *
 * The pages name the stages but not every formula; where they are silent the
 * plainest reading is taken and the choice is stated at the function.  With
 * n = 4 streams, hidden size C, K = n*C and 24 = 2n + n*n logits per token:
 *
 *   s   = sum_k x_k^2,  r = 1/sqrt(s/K + eps)            (RMS of the 4C row)
 *   P_j = sum_k x_k fn[k][j]                              (skinny projection)
 *   l_j = alpha_g(j) * (r * P_j) + bias_j                 (g = pre|post|comb)
 *   pre_i = sigmoid(l_i), post_i = 2 sigmoid(l_{4+i})
 *   comb  = Sinkhorn_iters( exp(l_{8+4i+j}) ), row step then column step
 *   y_c   = sum_i p_i x_{i,c}   (p = pre, or the carried pre in the delayed form)
 *   li_c  = bf16(y_c)  or  bf16((y_c * ry) * w_c), ry = 1/sqrt(sum y^2/C + eps)
 *   out_{i,c} = bf16(post_i y'_c + sum_j comb[i][j] x_{j,c})
 *
 * All floating point is IEEE double except orc_collapse32 and orc_post32, which
 * evaluate the collapse and the post stage in single precision in one fixed
 * order.  Build with
 * -O2 -fno-fast-math -ffp-contract=off so that no product is fused into an
 * addition and every rounding written here happens.
 *
 * Parity pins: every function is checked by tests that do not reuse it --
 * closed forms, invariants, a numpy matmul for the projection, a pure-Python
 * correctly-rounded brute force at T = 1, a high-precision 2x2 recurrence for
 * the Sinkhorn iteration count and order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define NLOG 24 /* 2n + n*n logits for n = 4 streams */
#define NS 4    /* hc_mult: residual streams */

/* bf16 bits -> exact double (bf16 is the top half of an IEEE single). */
static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_bf16_to_double(uint16_t b) { return bf16_val(b); }

/*
 * Round a real value (given as a double) to the nearest bfloat16, ties to
 * even, directly (no intermediate single-precision rounding, so no double
 * rounding).  bfloat16 keeps 8 significant bits and the single-precision
 * exponent range; below 2^-126 the spacing is fixed at 2^-133.
 */
uint16_t orc_bf16_rne(double v)
{
    if (isnan(v))
        return (uint16_t)0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1, so 2^(e-1) <= a < 2^e */
    int q = e - 8; /* spacing of 8-significant-bit numbers in this binade */
    if (e - 1 < -126)
        q = -133; /* subnormal range of the single-precision exponent */
    double quantum = ldexp(1.0, q);
    double k = nearbyint(a / quantum); /* default mode: nearest, ties to even */
    double r = k * quantum;
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything rounding past it is inf */
    if (r > ldexp(255.0, 120))
        return (uint16_t)(sign | 0x7F80);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

void orc_bf16_rne_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(v[i]);
}

/*
 * Logits of one seam (projection + RMS + affine), one row per token.
 *   x     : [T][K] bf16 bits; for the 4-stream residual x[T][4][C] this is the
 *           plain row-major flattening, k = i*C + c.  For the model-entry seam
 *           it is the single stream h[T][C] with K = C.
 *   fn    : [K][24] fp32, row-major ("projection against fn", p1 Approach).
 *   bias  : [24] fp32; alpha: [3] fp32 = scale of the pre, post, comb groups.
 *   logits: [T][24] out;  rinv: [T] out (r), may be NULL.
 * Reading: the RMS is taken over the whole flattened row (K elements, eps
 * inside the root) and applied after the projection, l = alpha*(r*P) + bias;
 * p1 Approach computes the projection and the row square-sums side by side.
 */
void orc_logits(const uint16_t *x, int64_t T, int64_t K, const float *fn,
                const float *bias, const float *alpha, double eps,
                double *logits, double *rinv)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *row = x + t * K;
        double s = 0.0;
        double P[NLOG];
        for (int j = 0; j < NLOG; ++j)
            P[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xv = bf16_val(row[k]);
            s += xv * xv;
            const float *f = fn + k * NLOG;
            for (int j = 0; j < NLOG; ++j)
                P[j] += xv * (double)f[j];
        }
        double r = 1.0 / sqrt(s / (double)K + eps);
        if (rinv)
            rinv[t] = r;
        for (int j = 0; j < NLOG; ++j) {
            int g = j < NS ? 0 : (j < 2 * NS ? 1 : 2);
            logits[t * NLOG + j] = (double)alpha[g] * (r * P[j]) + (double)bias[j];
        }
    }
}

/*
 * Sinkhorn normalisation of one positive 4x4 matrix (row-major), `iters`
 * rounds of: divide every row by its sum, then every column by its sum
 * (p1 Summary and Approach: 20 iterations per seam).  Reading: no epsilon in
 * either denominator, so the column sums are 1 after the last round.
 */
void orc_sinkhorn(const double *m_in, int iters, double *m_out)
{
    double M[NS][NS];
    for (int i = 0; i < NS; ++i)
        for (int j = 0; j < NS; ++j)
            M[i][j] = m_in[i * NS + j];
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < NS; ++i) {
            double s = 0.0;
            for (int j = 0; j < NS; ++j)
                s += M[i][j];
            for (int j = 0; j < NS; ++j)
                M[i][j] = M[i][j] / s;
        }
        for (int j = 0; j < NS; ++j) {
            double s = 0.0;
            for (int i = 0; i < NS; ++i)
                s += M[i][j];
            for (int i = 0; i < NS; ++i)
                M[i][j] = M[i][j] / s;
        }
    }
    for (int i = 0; i < NS; ++i)
        for (int j = 0; j < NS; ++j)
            m_out[i * NS + j] = M[i][j];
}

/*
 * Gates from logits: pre = sigmoid(l[0:4]), post = 2*sigmoid(l[4:8]) in (0,2),
 * comb = Sinkhorn(exp(l[8:24]) as a row-major 4x4).  Layout reading: pre-mix,
 * post, comb in that order, comb[i][j] = l[8 + 4i + j], row i = output stream.
 */
void orc_gates(const double *logits, int64_t T, int iters, double *pre,
               double *post, double *comb)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *l = logits + t * NLOG;
        for (int i = 0; i < NS; ++i) {
            pre[t * NS + i] = 1.0 / (1.0 + exp(-l[i]));
            post[t * NS + i] = 2.0 / (1.0 + exp(-l[NS + i]));
        }
        double M[NS * NS];
        for (int q = 0; q < NS * NS; ++q)
            M[q] = exp(l[2 * NS + q]);
        orc_sinkhorn(M, iters, comb + t * NS * NS);
    }
}

/*
 * Collapse of the four streams, exact value in double:
 *   y[t][c] = sum_i p[t][i] * x[t][i][c].
 * p is the seam's own pre-mix, or for the delayed form the previous seam's
 * (p1 Purpose: collapse with the previous pre-mix, return the current one).
 * mag[t][c] = sum_i |p_i x_{i,c}| (size of the terms, for error bounds), may be NULL.
 */
void orc_collapse64(const uint16_t *x, const double *p, int64_t T, int64_t C,
                    double *y, double *mag)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0, m = 0.0;
            for (int i = 0; i < NS; ++i) {
                double term = p[t * NS + i] * bf16_val(x[(t * NS + i) * C + c]);
                acc += term;
                m += fabs(term);
            }
            y[t * C + c] = acc;
            if (mag)
                mag[t * C + c] = m;
        }
    }
}

/*
 * Collapse in single precision, one fixed order: every product rounded to
 * single, then summed left to right over the streams,
 *   y = fl(fl(fl(fl(p0 x0) + fl(p1 x1)) + fl(p2 x2)) + fl(p3 x3)).
 * p1 Result: the collapse is the same single-precision multiply-and-sum in
 * both paths and therefore bit-exact.  Compiled without contraction.
 */
void orc_collapse32(const uint16_t *x, const float *p, int64_t T, int64_t C,
                    float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < C; ++c) {
            float acc = 0.0f;
            for (int i = 0; i < NS; ++i) {
                volatile float prod = p[t * NS + i] * (float)bf16_val(x[(t * NS + i) * C + c]);
                acc = (i == 0) ? prod : acc + prod;
            }
            y[t * C + c] = acc;
        }
    }
}

/*
 * Folded RMSNorm of the collapsed row (p3 Measurements: x * rsqrt * weight in
 * single precision and rounded once; here the exact value in double):
 *   ry = 1/sqrt(sum_c y_c^2 / C + eps),  out_c = (y_c * ry) * w_c.
 * w: [C] bf16 bits.  rinv_y: [T] out, may be NULL.
 */
void orc_norm(const double *y, const uint16_t *w, int64_t T, int64_t C,
              double eps, double *out, double *rinv_y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *yr = y + t * C;
        double s = 0.0;
        for (int64_t c = 0; c < C; ++c)
            s += yr[c] * yr[c];
        double ry = 1.0 / sqrt(s / (double)C + eps);
        if (rinv_y)
            rinv_y[t] = ry;
        for (int64_t c = 0; c < C; ++c)
            out[t * C + c] = (yr[c] * ry) * bf16_val(w[c]);
    }
}

/*
 * Post recombination, exact value in double:
 *   out[t][i][c] = post[t][i] * y[t][c] + sum_j comb[t][i][j] * x[t][j][c]
 * (the mhc_post call sites of p1 Result; row index i = output stream).
 * y: [T][C] bf16 (the sublayer output), x: [T][4][C] bf16, post: [T][4] fp32,
 * comb: [T][16] fp32.  mag: sum of |terms|, may be NULL.
 */
void orc_post(const uint16_t *y, const uint16_t *x, const float *post,
              const float *comb, int64_t T, int64_t C, double *out, double *mag)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int i = 0; i < NS; ++i) {
            double pi = (double)post[t * NS + i];
            for (int64_t c = 0; c < C; ++c) {
                double yv = bf16_val(y[t * C + c]);
                double acc = pi * yv;
                double m = fabs(pi * yv);
                for (int j = 0; j < NS; ++j) {
                    double term = (double)comb[(t * NS + i) * NS + j] *
                                  bf16_val(x[(t * NS + j) * C + c]);
                    acc += term;
                    m += fabs(term);
                }
                out[(t * NS + i) * C + c] = acc;
                if (mag)
                    mag[(t * NS + i) * C + c] = m;
            }
        }
    }
}

/*
 * Post stage in single precision, one fixed order, rounded once to bf16:
 *   a = fl(post_i * y_c);  a = fma(comb[i][j], x_{j,c}, a) for j = 0, 1, 2, 3;
 *   out[t][i][c] = bf16_rne(a).
 * The next residual is a bf16 quantisation decided in single precision (p1
 * Result: the post call sites produce the bf16 residual the next seam reads).
 * When the next seam consumes it directly (cross-seam fusion), both sides take
 * that rounding decision in the same precision and order, so the next seam's
 * input is the same bits; orc_post gives the exact value it must stay within
 * one bf16 ulp of.  fmaf is the correctly rounded C99 fused multiply-add.
 */
void orc_post32(const uint16_t *y, const uint16_t *x, const float *post,
                const float *comb, int64_t T, int64_t C, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int i = 0; i < NS; ++i) {
            const float pi = post[t * NS + i];
            for (int64_t c = 0; c < C; ++c) {
                volatile float a = pi * (float)bf16_val(y[t * C + c]);
                for (int j = 0; j < NS; ++j)
                    a = fmaf(comb[(t * NS + i) * NS + j], (float)bf16_val(x[(t * NS + j) * C + c]), a);
                out[(t * NS + i) * C + c] = orc_bf16_rne((double)a);
            }
        }
    }
}
