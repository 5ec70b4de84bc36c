/*
 * orc_fit.c -- target functions, the endpoint-constrained least-squares fit,
 * coefficient rounding, the two error metrics and the (Li, Lc) selection.
 *
 * Test infrastructure (see orc.h).  Follows "Fast Polynomial Transcendentals
 * for LLMs" (arXiv 2610.00049):
 *   - section 3.1, Eqs. 2-6: clamp Lc, t = |x|, centered-odd sigmoid/tanh,
 *     x/2 + even residual for SiLU and exact GELU;
 *   - section 3.3, Eqs. 9-11: even sigmoid/tanh derivatives, centered-odd
 *     SiLU/GELU derivatives (s'(x) + s'(-x) = 1);
 *   - section 3.2, Eqs. 7-8 and steps 1-7: FP64 least squares with both
 *     endpoints fixed, BF16 coefficient rounding, replay, max-error scoring
 *     on 8,000 points over [0, 12], the Lc <= Li + 1 rule and shape gates;
 *   - section 4.1 / Table 2: the real-arithmetic metric over 20,001 uniform
 *     points on [-Lc, Lc].
 */
#include "orc.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define N_NODES 2000      /* section 3.2: 2,000 Chebyshev nodes */
#define N_SEARCH 8000     /* section 3.2 step 6: 8,000 points on [0, 12] */
#define N_TABLE2 20001    /* section 4.1: 20,001 points on [-Lc, Lc] */

/* sigma(x) without cancellation on either side: e = exp(-|x|) <= 1 */
static double sigm(double x)
{
    const double e = exp(-fabs(x));
    return x >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}
static double Phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }
static double phi(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }

/* The function a program approximates, in FP64, on the whole real line. */
double orc_ref(int func, int deriv, double x)
{
    if (!deriv) {
        switch (func) {
        case ORC_SIGMOID: return sigm(x);
        case ORC_TANH:    return tanh(x);
        case ORC_SILU:    return x * sigm(x);
        case ORC_GELU:    return x * Phi(x);
        }
    } else {
        switch (func) {
        case ORC_SIGMOID: return sigm(x) * sigm(-x);           /* Eq. 10 */
        case ORC_TANH: { const double c = cosh(x); return 1.0 / (c * c); }
        case ORC_SILU:    return sigm(x) * (1.0 + x * sigm(-x));   /* Eq. 9 */
        case ORC_GELU:    return Phi(x) + x * phi(x);
        }
    }
    return NAN;
}

/* The half-domain residual that is fitted, t >= 0 (section 3.1 / 3.3).
 *   sigmoid, SiLU fwd : sigma(t) - 1/2   (SiLU reuses the sigmoid residual:
 *                        s(x) - x/2 = |x| (sigma(|x|) - 1/2), Eqs. 5-6)
 *   tanh fwd          : tanh t
 *   GELU fwd          : Phi(t) - 1/2
 *   sigmoid', tanh'   : the even derivative itself
 *   SiLU', GELU'      : derivative minus 1/2 (odd, Eq. 9)                */
double orc_residual(int func, int deriv, double t)
{
    if (!deriv) {
        switch (func) {
        case ORC_SIGMOID:
        case ORC_SILU: return 0.5 * tanh(0.5 * t);
        case ORC_TANH: return tanh(t);
        case ORC_GELU: return 0.5 * erf(t / sqrt(2.0));
        }
    } else {
        switch (func) {
        case ORC_SIGMOID:
        case ORC_TANH: return orc_ref(func, 1, t);
        case ORC_SILU:
        case ORC_GELU: return orc_ref(func, 1, t) - 0.5;
        }
    }
    return NAN;
}

/* Solve min ||A x - r||_2 for an N x m column-major A by Householder QR in
 * FP64.  A and r are overwritten.  Returns 0 on success. */
int orc_lsq(int N, int m, double *A, double *r, double *x)
{
    for (int k = 0; k < m; k++) {
        double *ak = A + (size_t)k * N;
        double nrm = 0.0;
        for (int i = k; i < N; i++) nrm += ak[i] * ak[i];
        nrm = sqrt(nrm);
        if (nrm == 0.0) return -1;
        const double alpha = ak[k] > 0 ? -nrm : nrm;
        /* v = a_k[k:] - alpha e_1, stored in place of a_k[k:] */
        ak[k] -= alpha;
        double vv = 0.0;
        for (int i = k; i < N; i++) vv += ak[i] * ak[i];
        for (int j = k + 1; j < m; j++) {
            double *aj = A + (size_t)j * N;
            double d = 0.0;
            for (int i = k; i < N; i++) d += ak[i] * aj[i];
            const double tau = 2.0 * d / vv;
            for (int i = k; i < N; i++) aj[i] -= tau * ak[i];
        }
        double d = 0.0;
        for (int i = k; i < N; i++) d += ak[i] * r[i];
        const double tau = 2.0 * d / vv;
        for (int i = k; i < N; i++) r[i] -= tau * ak[i];
        ak[k] = alpha;   /* R[k][k]; entries of R above the diagonal are in
                            rows < k of later columns, already updated */
    }
    for (int k = m - 1; k >= 0; k--) {
        double s = r[k];
        for (int j = k + 1; j < m; j++) s -= A[(size_t)j * N + k] * x[j];
        x[k] = s / A[(size_t)k * N + k];
    }
    return 0;
}

/* Eqs. 7-8: P(0) = f(0), P(Li) = f(Li); in u = t / Li the free terms are
 * b_j (u^j - u), j = 2..D, solved by least squares on the Chebyshev nodes of
 * the first kind t_k = (Li/2)(1 + cos((2k - 1) pi / (2N))), k = 1..N.
 * Writes the FP64 monomial coefficients c_0..c_D of P(t). */
int orc_fit(int func, int deriv, int degree, double Li, double *coef)
{
    if (degree < 1 || degree > 7 || !(Li > 0)) return -1;
    const double f0 = orc_residual(func, deriv, 0.0);
    const double fL = orc_residual(func, deriv, Li);
    const int m = degree - 1;
    double b[8] = {0};
    if (m > 0) {
        double *A = malloc(sizeof(double) * (size_t)N_NODES * m);
        double *r = malloc(sizeof(double) * N_NODES);
        if (!A || !r) { free(A); free(r); return -2; }
        for (int k = 1; k <= N_NODES; k++) {
            const double t = 0.5 * Li * (1.0 + cos((2.0 * k - 1.0) * M_PI /
                                                   (2.0 * N_NODES)));
            const double u = t / Li;
            double uj = u;
            for (int j = 2; j <= degree; j++) {
                uj *= u;
                A[(size_t)(j - 2) * N_NODES + (k - 1)] = uj - u;
            }
            r[k - 1] = orc_residual(func, deriv, t) - f0 - (fL - f0) * u;
        }
        const int rc = orc_lsq(N_NODES, m, A, r, b);
        free(A);
        free(r);
        if (rc) return -3;
    }
    double sb = 0.0;
    for (int j = 0; j < m; j++) sb += b[j];
    coef[0] = f0;
    coef[1] = (fL - f0 - sb) / Li;
    for (int j = 2; j <= degree; j++) coef[j] = b[j - 2] / pow(Li, j);
    return 0;
}

static int representable_f16(double v)
{
    return orc_f16_to_f64(orc_f64_to_f16(v)) == v;
}

/* Fit, then round every coefficient to BF16 (section 3.2 step 3). */
int orc_make_prog(int func, int deriv, int degree, double Li, double Lc,
                  orc_prog *out)
{
    double c[8];
    memset(out, 0, sizeof *out);
    if (func < ORC_SIGMOID || func > ORC_GELU || deriv < 0 || deriv > 1)
        return -1;
    const int rc = orc_fit(func, deriv, degree, Li, c);
    if (rc) return rc;
    out->func = func;
    out->deriv = deriv;
    out->degree = degree;
    out->Li = Li;
    out->Lc = Lc;
    for (int j = 0; j <= degree; j++) out->c[j] = orc_f64_to_bf16(c[j]);
    /* the clamp must be a value of both 16-bit formats */
    if (orc_bf16_to_f64(orc_f64_to_bf16(Lc)) != Lc || !representable_f16(Lc))
        return -4;
    return 0;
}

/* Does the program's reconstruction add 1/2 (centered-odd forms)? */
static int has_half_offset(const orc_prog *p)
{
    if (!p->deriv) return p->func == ORC_SIGMOID;
    return p->func == ORC_SILU || p->func == ORC_GELU;
}

/* Real-arithmetic value of the program with its rounded coefficients: the
 * reconstruction of section 3.1 around the clamped Horner value. */
double orc_prog_real(const orc_prog *p, double x)
{
    const double t = fabs(x);
    const double th = t < p->Lc ? t : p->Lc;
    double v = orc_bf16_to_f64(p->c[p->degree]);
    for (int j = p->degree - 1; j >= 0; j--)
        v = v * th + orc_bf16_to_f64(p->c[j]);
    const double sg = signbit(x) ? -1.0 : 1.0;
    if (!p->deriv) {
        switch (p->func) {
        case ORC_SIGMOID: return 0.5 + sg * v;
        case ORC_TANH: return sg * v;
        default: return 0.5 * x + t * v;     /* SiLU, GELU */
        }
    }
    return has_half_offset(p) ? 0.5 + sg * v : v;
}

/* Table 2's metric: max |P(x) - f(x)| in real arithmetic with the BF16
 * coefficients over 20,001 uniform points on [-Lc, Lc], extended by every
 * finite FP16 and every finite BF16 value in that interval. */
double orc_table2_metric(const orc_prog *p)
{
    double worst = 0.0;
    const double Lc = p->Lc;
    for (int k = 0; k < N_TABLE2; k++) {
        const double x = -Lc + 2.0 * Lc * k / (N_TABLE2 - 1);
        const double e = fabs(orc_prog_real(p, x) - orc_ref(p->func, p->deriv, x));
        if (e > worst) worst = e;
    }
    for (uint32_t b = 0; b < 65536; b++) {
        const double xs[2] = {orc_f16_to_f64((uint16_t)b),
                              orc_bf16_to_f64((uint16_t)b)};
        for (int i = 0; i < 2; i++) {
            const double x = xs[i];
            if (!isfinite(x) || fabs(x) > Lc) continue;
            const double e =
                fabs(orc_prog_real(p, x) - orc_ref(p->func, p->deriv, x));
            if (e > worst) worst = e;
        }
    }
    return worst;
}

/* Range of f used by the boundary gate (section 3.2 step 6). */
static void f_range(const orc_prog *p, double *lo, double *hi)
{
    *lo = -INFINITY;
    *hi = INFINITY;
    if (!p->deriv) {
        switch (p->func) {
        case ORC_SIGMOID: *lo = 0.0; *hi = 1.0; break;
        case ORC_TANH: *lo = -1.0; *hi = 1.0; break;
        case ORC_SILU: *lo = -0.27846454276107380; break;   /* min of x sigma(x) */
        case ORC_GELU: *lo = -0.16997120747990005; break;   /* min of x Phi(x) */
        }
    } else {
        switch (p->func) {
        case ORC_SIGMOID: *lo = 0.0; *hi = 0.25; break;
        case ORC_TANH: *lo = 0.0; *hi = 1.0; break;
        case ORC_SILU: *lo = -0.0998996; *hi = 1.0998996; break;
        case ORC_GELU: *lo = -0.1289; *hi = 1.1289; break;
        }
    }
}

/* Section 3.2 steps 4-6: replay the program at 8,000 points of [0, 12]
 * (inputs rounded to BF16) and score the maximum absolute error against the
 * FP64 function at the same input.  Gate ("boundary violation"): the replayed
 * output stays inside f's range.  Monotonicity is not gated: intermediate
 * BF16 rounding produces multi-ulp reversals in every candidate, including
 * the D4 sigmoid-derivative program that Table 2's value pins bit for bit. */
double orc_search_objective(const orc_prog *p, int order, int *gates_ok)
{
    double lo, hi;
    f_range(p, &lo, &hi);
    double worst = 0.0;
    int ok = 1;
    for (int k = 0; k < N_SEARCH; k++) {
        const uint16_t xb = orc_f64_to_bf16(12.0 * k / (N_SEARCH - 1));
        const double x = orc_bf16_to_f64(xb);
        const double y = orc_bf16_to_f64(orc_prog_eval(p, xb, order));
        const double e = fabs(y - orc_ref(p->func, p->deriv, x));
        if (!(e <= worst)) worst = e;        /* NaN propagates as failure */
        if (!(y >= lo && y <= hi)) ok = 0;
    }
    if (isnan(worst)) ok = 0;
    if (gates_ok) *gates_ok = ok;
    return worst;
}

/* The (Li, Lc) selection of section 3.2 for one function and degree.
 * Grid: Li, Lc in {0.25, 0.5, ..., 12}; Lc > Li + 1 rejected; when Lc_fixed
 * > 0 only Li is searched.  Among candidates passing the gates, minimise the
 * search objective, then the Table-2 metric, then Li, then Lc.  When
 * bound > 0 the candidates are first restricted to those whose Table-2 metric
 * is <= bound, provided any such candidate also keeps the search objective
 * within twice the unrestricted optimum; otherwise the bound is reported as
 * unmet and does not restrict.  Returns 0 on success. */
int orc_search(int func, int deriv, int degree, double Lc_fixed, double bound,
               int order, orc_prog *out, double *objective, double *metric)
{
    enum { G = 48 };
    typedef struct { orc_prog p; double obj, met; int ok; } cand;
    cand *cs = calloc((size_t)G * G, sizeof(cand));
    if (!cs) return -2;
    /* every (Li, Lc) pair of the grid; candidates are independent, so the
     * grid is scored in parallel and reduced serially in grid order */
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 1; i <= G; i++) {
        const double Li = 0.25 * i;
        orc_prog base;
        if (orc_make_prog(func, deriv, degree, Li, 1.0, &base)) continue;
        for (int jj = 1; jj <= G; jj++) {
            const double Lc = Lc_fixed > 0 ? Lc_fixed : 0.25 * jj;
            if (Lc_fixed > 0 && jj > 1) break;
            if (Lc > Li + 1.0) continue;
            cand *c = &cs[(i - 1) * G + (jj - 1)];
            c->p = base;
            c->p.Lc = Lc;
            c->obj = orc_search_objective(&c->p, order, &c->ok);
        }
    }
    double best_obj = INFINITY;
    for (int i = 0; i < G * G; i++)
        if (cs[i].ok && cs[i].obj < best_obj) best_obj = cs[i].obj;
    if (!(best_obj < INFINITY)) { free(cs); return -1; }
    /* the Table-2 metric only matters for the bound restriction (objective
     * within twice the optimum) and for ties at the optimum */
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < G * G; i++) {
        cs[i].met = INFINITY;
        if (cs[i].ok && (cs[i].obj == best_obj ||
                         (bound > 0 && cs[i].obj <= 2.0 * best_obj)))
            cs[i].met = orc_table2_metric(&cs[i].p);
    }
    int restrict_to_bound = 0;
    if (bound > 0)
        for (int i = 0; i < G * G; i++)
            if (cs[i].ok && cs[i].met <= bound && cs[i].obj <= 2.0 * best_obj)
                restrict_to_bound = 1;
    int bi = -1;
    for (int i = 0; i < G * G; i++) {
        if (!cs[i].ok) continue;
        if (restrict_to_bound && !(cs[i].met <= bound && cs[i].obj <= 2.0 * best_obj))
            continue;
        if (bi < 0) { bi = i; continue; }
        const cand *a = &cs[i], *b = &cs[bi];
        int better = 0;
        if (a->obj != b->obj) better = a->obj < b->obj;
        else if (a->met != b->met) better = a->met < b->met;
        else if (a->p.Li != b->p.Li) better = a->p.Li < b->p.Li;
        else better = a->p.Lc < b->p.Lc;
        if (better) bi = i;
    }
    *out = cs[bi].p;
    if (objective) *objective = cs[bi].obj;
    if (metric) *metric = orc_table2_metric(&cs[bi].p);
    free(cs);
    return 0;
}
