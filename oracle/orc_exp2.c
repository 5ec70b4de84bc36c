/*
 * orc_exp2.c -- the fractional cores of a software exp2 (test
 * infrastructure, see orc.h).
 *
 * "Fast Polynomial Transcendentals for LLMs", Appendix B.1 (Eq. 16): 2^x is
 * split as 2^n 2^f with n = floor(x), f = x - n in [0, 1), and only 2^f is
 * approximated.  Online softmax moves its reference by integers and
 * intervals meet at f = 1, so a core must keep p(0) = 1 and p(1) = 2 (then
 * 2^n p(f) is continuous and p(f) 2^(n+k) = 2^k (2^n p(f)) holds exactly).
 * The families (Eqs. 17-19):
 *   D1    p(f) = 1 + f
 *   PWL2  p(f) = 1 + a f + 2 (1 - a) max(f - 1/2, 0)
 *   D2    p(f) = 1 + a f + (1 - a) f^2
 *   D3    p(f) = 1 + c1 f + c2 f^2 + c3 f^3 (the pages' printed coefficients;
 *         p(1) != 2)
 * and the one-parameter fits of PWL2 and D2 on the 1,000,001-point grid
 * f_k = k / 10^6 by least squares of the error p(f) - 2^f or by the sampled
 * maximum of the relative error |p(f) / 2^f - 1| (Table 8).  Which error the
 * least-squares fit weighs is not stated; the unweighted (absolute) one is
 * the one that reproduces the printed parameters.
 */
#include "orc.h"

#include <math.h>

#define GRID 1000001

static const double D3C[4] = {1.0, 0.6951461434, 0.2275643945, 0.0771190897};

/* p(f) in real arithmetic */
double orc_exp2_core(int core, double a, double f)
{
    switch (core) {
    case ORC_EXP2_D1: return 1.0 + f;
    case ORC_EXP2_PWL2: return 1.0 + a * f + 2.0 * (1.0 - a) * fmax(f - 0.5, 0.0);
    case ORC_EXP2_D2: return 1.0 + a * f + (1.0 - a) * f * f;
    case ORC_EXP2_D3: return D3C[0] + f * (D3C[1] + f * (D3C[2] + f * D3C[3]));
    default: return exp2(f);
    }
}

/* Maximum and root-mean-square relative error of p over the grid. */
void orc_exp2_errors(int core, double a, double *max_rel, double *rms_rel)
{
    double mx = 0.0, ss = 0.0;
    for (int k = 0; k < GRID; k++) {
        const double f = (double)k / (GRID - 1);
        const double r = orc_exp2_core(core, a, f) / exp2(f) - 1.0;
        if (fabs(r) > mx) mx = fabs(r);
        ss += r * r;
    }
    *max_rel = mx;
    *rms_rel = sqrt(ss / GRID);
}

/* PWL2 / D2 are affine in a: p(f) = u(f) + a w(f).  rel = 1 gives the
 * relative error's parts, (u / 2^f - 1) + a (w / 2^f); rel = 0 the absolute
 * error's, (u - 2^f) + a w. */
static void affine_parts(int core, double f, int rel, double *u, double *w)
{
    const double e = exp2(f);
    if (core == ORC_EXP2_PWL2) {
        const double h = fmax(f - 0.5, 0.0);
        *u = 1.0 + 2.0 * h;
        *w = f - 2.0 * h;
    } else {
        *u = 1.0 + f * f;
        *w = f - f * f;
    }
    if (rel) {
        *u = *u / e - 1.0;
        *w = *w / e;
    } else {
        *u -= e;
    }
}

static double max_rel_affine(int core, double a)
{
    double mx = 0.0;
    for (int k = 0; k < GRID; k++) {
        double u, w;
        affine_parts(core, (double)k / (GRID - 1), 1, &u, &w);
        const double r = fabs(u + a * w);
        if (r > mx) mx = r;
    }
    return mx;
}

/* The parameter a of PWL2 or D2: objective 0 = least squares of p - 2^f
 * (closed form), 1 = sampled minimax of the relative error (its maximum over
 * the grid is convex in a: golden-section search on [0, 1] to 1e-12). */
double orc_exp2_fit(int core, int minimax)
{
    if (!minimax) {
        double uw = 0.0, ww = 0.0;
        for (int k = 0; k < GRID; k++) {
            double u, w;
            affine_parts(core, (double)k / (GRID - 1), 0, &u, &w);
            uw += u * w;
            ww += w * w;
        }
        return -uw / ww;
    }
    const double g = (sqrt(5.0) - 1.0) / 2.0;
    double lo = 0.0, hi = 1.0;
    double x1 = hi - g * (hi - lo), x2 = lo + g * (hi - lo);
    double f1 = max_rel_affine(core, x1), f2 = max_rel_affine(core, x2);
    while (hi - lo > 1e-12) {
        if (f1 <= f2) {
            hi = x2; x2 = x1; f2 = f1;
            x1 = hi - g * (hi - lo);
            f1 = max_rel_affine(core, x1);
        } else {
            lo = x1; x1 = x2; f1 = f2;
            x2 = lo + g * (hi - lo);
            f2 = max_rel_affine(core, x2);
        }
    }
    return 0.5 * (lo + hi);
}

/* ---- target-precision cores (the arithmetic a kernel performs) ------------
 * FP32: coefficients rounded to FP32 (b = 1 - a is then exact), Horner with
 *   one FP32 rounding per fused multiply-add:
 *     D1 p = f + 1;  D2 p = fma(fma(b, f, a), f, 1);
 *     D3 p = fma(fma(fma(c3, f, c2), f, c1), f, 1).
 * FP16 (PWL2, the pages' packed form): f rounded to FP16, coefficients the
 *   pages' FP16 values a = 0.7978515625, 2 (1 - a) = 0.40380859375;
 *     h = max(f - 1/2, 0), p = fma(a, f, 1), p = fma(2 (1 - a), h, p)
 *   each rounded once to FP16.  Returns p as a float. */
float orc_exp2_core_target(int core, float f)
{
    switch (core) {
    case ORC_EXP2_D1: return orc_add_f32(f, 1.0f);
    case ORC_EXP2_D2: {
        const float a = (float)0.6602339719, b = 1.0f - a;
        return orc_fma_f32(orc_fma_f32(b, f, a), f, 1.0f);
    }
    case ORC_EXP2_D3: {
        const float c1 = (float)D3C[1], c2 = (float)D3C[2], c3 = (float)D3C[3];
        return orc_fma_f32(orc_fma_f32(orc_fma_f32(c3, f, c2), f, c1), f, 1.0f);
    }
    case ORC_EXP2_PWL2: {
        const uint16_t fh = orc_f64_to_f16((double)f);
        const uint16_t a = orc_f64_to_f16(0.7978515625), b = orc_f64_to_f16(0.40380859375);
        const uint16_t one = 0x3C00, half = 0x3800;
        /* f - 1/2 as an FMA with 1 (exact product), then max with +0 */
        uint16_t h = orc_fma_f16(fh, one, half | 0x8000);
        if (orc_f16_to_f64(h) <= 0.0) h = 0;
        const uint16_t p = orc_fma_f16(b, h, orc_fma_f16(a, fh, one));
        return (float)orc_f16_to_f64(p);
    }
    default: return (float)exp2((double)f);
    }
}
