/*
 * orc_rope.c -- paired sine / cosine programs and rotary position embedding
 * (test infrastructure, see orc.h).
 *
 * "Fast Polynomial Transcendentals for LLMs", Appendix B.2: the angle of
 * frequency i at position p is kept as an unsigned Q0.32 fraction of a
 * turn, phase = (p * inc_i) mod 2^32 with inc_i = round(w_i 2^32 / (2 pi));
 * the phase is reduced to a signed Q15 half-turn coordinate v (angle
 * pi v / 2^15) and a D5 sine and a D6 cosine are evaluated in packed FP16
 * on the shared square of that coordinate.  The rotation then turns each
 * interleaved pair (x_{2i}, x_{2i+1}) by the angle of frequency i.
 *
 * Readings (the appendix leaves them open):
 *   - w_i = base^(-2i / D) (the usual rotary frequencies), base a parameter;
 *   - v is the top 16 bits of the phase read as a signed integer
 *     (truncation), u = RN16(v / 2^15) in [-1, 1);
 *   - the programs follow section 3.2: least squares on Chebyshev nodes of
 *     the first kind over [0, 1] in FP64 with the endpoint values of Eq. 8
 *     imposed (sine: odd, u (a1 + a3 u^2 + a5 u^4) with sin(pi) = 0, so
 *     a1 + a3 + a5 = 0; cosine: even, b0 + b2 u^2 + b4 u^4 + b6 u^6 with
 *     cos(0) = 1 and cos(pi) = -1), then every coefficient rounded to BF16;
 *   - evaluation: w = RN16(u u); sine q = a5, q = fma(q, w, a3),
 *     q = fma(q, w, a1), s = RN16(q u); cosine c = b6, c = fma(c, w, b4),
 *     c = fma(c, w, b2), c = fma(c, w, b0); every FMA one FP16 rounding;
 *   - rotation: y0 = RN16(x0 c - RN16(x1 s)), y1 = RN16(x1 c + RN16(x0 s))
 *     (one packed product, one packed FMA).
 */
#include "orc.h"

#include <math.h>
#include <stdlib.h>

#define ROPE_NODES 4096

int orc_rope_fit(double *sin_coef, double *cos_coef)
{
    double *A = malloc(sizeof(double) * 2 * ROPE_NODES), *r = malloc(sizeof(double) * ROPE_NODES);
    if (!A || !r) { free(A); free(r); return -2; }
    double x[2];
    /* sine: u (a1 + a3 u^2 + a5 u^4) with a1 = -(a3 + a5)
     *     = a3 (u^3 - u) + a5 (u^5 - u) */
    for (int k = 1; k <= ROPE_NODES; k++) {
        const double u = 0.5 * (1.0 + cos((2.0 * k - 1.0) * M_PI / (2.0 * ROPE_NODES)));
        A[k - 1] = u * u * u - u;
        A[ROPE_NODES + k - 1] = u * u * u * u * u - u;
        r[k - 1] = sin(M_PI * u);
    }
    int rc = orc_lsq(ROPE_NODES, 2, A, r, x);
    sin_coef[0] = -(x[0] + x[1]);
    sin_coef[1] = x[0];
    sin_coef[2] = x[1];
    /* cosine: 1 + b2 u^2 + b4 u^4 + b6 u^6 with b2 = -2 - b4 - b6
     *       = 1 - 2 u^2 + b4 (u^4 - u^2) + b6 (u^6 - u^2) */
    for (int k = 1; k <= ROPE_NODES; k++) {
        const double u = 0.5 * (1.0 + cos((2.0 * k - 1.0) * M_PI / (2.0 * ROPE_NODES)));
        const double u2 = u * u;
        A[k - 1] = u2 * u2 - u2;
        A[ROPE_NODES + k - 1] = u2 * u2 * u2 - u2;
        r[k - 1] = cos(M_PI * u) - 1.0 + 2.0 * u2;
    }
    rc |= orc_lsq(ROPE_NODES, 2, A, r, x);
    cos_coef[0] = 1.0;
    cos_coef[1] = -2.0 - x[0] - x[1];
    cos_coef[2] = x[0];
    cos_coef[3] = x[1];
    free(A);
    free(r);
    return rc ? -3 : 0;
}

int orc_rope_prog(orc_rope *out)
{
    double s[3], c[4];
    const int rc = orc_rope_fit(s, c);
    if (rc) return rc;
    for (int j = 0; j < 3; j++) out->sin_c[j] = orc_f64_to_bf16(s[j]);
    for (int j = 0; j < 4; j++) out->cos_c[j] = orc_f64_to_bf16(c[j]);
    return 0;
}

void orc_rope_inc(int D, double base, uint32_t *inc)
{
    for (int i = 0; i < D / 2; i++) {
        const double w = pow(base, -2.0 * i / (double)D);
        inc[i] = (uint32_t)llround(w * 4294967296.0 / (2.0 * M_PI));
    }
}

uint16_t orc_rope_coord(uint32_t phase)
{
    const int v = (int16_t)(uint16_t)(phase >> 16);
    return orc_f64_to_f16((double)v / 32768.0);
}

/* FP16 value of a BF16 coefficient (exact: asserted when the program is made
 * into FP16 words by the caller's tests) */
static uint16_t bf16_as_f16(uint16_t b)
{
    return orc_f64_to_f16(orc_bf16_to_f64(b));
}

void orc_rope_sincos(const orc_rope *rp, uint32_t phase, uint16_t *s_out, uint16_t *c_out)
{
    const uint16_t NEG0 = 0x8000u;
    const uint16_t u = orc_rope_coord(phase);
    const uint16_t w = orc_fma_f16(u, u, NEG0);
    uint16_t q = bf16_as_f16(rp->sin_c[2]);
    q = orc_fma_f16(q, w, bf16_as_f16(rp->sin_c[1]));
    q = orc_fma_f16(q, w, bf16_as_f16(rp->sin_c[0]));
    *s_out = orc_fma_f16(q, u, NEG0);
    uint16_t c = bf16_as_f16(rp->cos_c[3]);
    c = orc_fma_f16(c, w, bf16_as_f16(rp->cos_c[2]));
    c = orc_fma_f16(c, w, bf16_as_f16(rp->cos_c[1]));
    *c_out = orc_fma_f16(c, w, bf16_as_f16(rp->cos_c[0]));
}

void orc_rope_rotate(uint16_t x0, uint16_t x1, uint16_t s, uint16_t c, uint16_t *y0, uint16_t *y1)
{
    const uint16_t NEG0 = 0x8000u;
    const uint16_t t1 = orc_fma_f16(x1, s, NEG0);   /* RN16(x1 s) */
    const uint16_t t0 = orc_fma_f16(x0, s, NEG0);   /* RN16(x0 s) */
    *y0 = orc_fma_f16(x0, c, (uint16_t)(t1 ^ 0x8000u));
    *y1 = orc_fma_f16(x1, c, t0);
}

void orc_rope_rows(const orc_rope *rp, const uint32_t *inc, int D, const uint16_t *x,
                   const int64_t *pos, int64_t nrows, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; r++) {
        const uint16_t *xr = x + r * D;
        uint16_t *yr = y + r * D;
        for (int i = 0; i < D / 2; i++) {
            const uint32_t phase = (uint32_t)((uint64_t)pos[r] * (uint64_t)inc[i]);
            uint16_t s, c;
            orc_rope_sincos(rp, phase, &s, &c);
            orc_rope_rotate(xr[2 * i], xr[2 * i + 1], s, c, &yr[2 * i], &yr[2 * i + 1]);
        }
    }
}
