/*
 * orc_eval.c -- replay of the programs in deployed order, element by element,
 * plus the fused SwiGLU and the softcapped attention forward.
 *
 * Test infrastructure (see orc.h).  Sources, "Fast Polynomial
 * Transcendentals for LLMs" (arXiv 2610.00049):
 *   - Eq. 2 (clamp, t = |x|); Eq. 3 (1/2 + sign(x) p(t)); the odd tanh form;
 *     Eq. 6 (x/2 + t p(t)); section 3.3 (even derivatives, centered-odd
 *     SiLU/GELU derivatives); section 3.2 (one rounding per multiply-add in
 *     the target format, Horner order);
 *   - section 3.3 and Eq. 15 (SwiGLU: SiLU(g) = g p(g) from the recomputed
 *     D3 sigmoid p, derivative p + g p (1 - p), both input gradients);
 *   - Eq. 1 (softcap alpha tanh(x / alpha) on attention logits) and section
 *     5.2.2 (D4 tanh inside attention).
 *
 * Special values, which the paper leaves open:
 *   - NaN input -> the same NaN with its quiet bit set;
 *   - +-inf takes the clamp (sigmoid(+inf) = 1/2 + p(Lc), not 1);
 *   - SiLU/GELU: -inf -> -0 (the limit), +inf -> +inf;
 *   - derivative programs: NaN x or NaN upstream gradient -> that NaN, quieted.
 */
#include "orc.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- target-format arithmetic for one rounding order ------------------- */
typedef struct {
    int order;
    uint16_t sign, nan_exp, quiet, half, one, negzero;
} fmt_ops;

static fmt_ops ops_for(int order)
{
    fmt_ops f;
    f.order = order;
    f.sign = 0x8000;
    f.negzero = 0x8000;
    if (order == ORC_ORDER_F16_FMA) {
        f.nan_exp = 0x7C00; f.quiet = 0x0200; f.half = 0x3800; f.one = 0x3C00;
    } else {
        f.nan_exp = 0x7F80; f.quiet = 0x0040; f.half = 0x3F00; f.one = 0x3F80;
    }
    return f;
}

static int is_nan(const fmt_ops *f, uint16_t x)
{
    return (x & 0x7FFF) > f->nan_exp;
}

static double val(const fmt_ops *f, uint16_t x)
{
    return f->order == ORC_ORDER_F16_FMA ? orc_f16_to_f64(x) : orc_bf16_to_f64(x);
}

static uint16_t t_fma(const fmt_ops *f, uint16_t a, uint16_t b, uint16_t c)
{
    switch (f->order) {
    case ORC_ORDER_F16_FMA: return orc_fma_f16(a, b, c);
    case ORC_ORDER_BF16_FMA: return orc_fma_bf16(a, b, c);
    case ORC_ORDER_F32FMA_BF16: return orc_fma_f32_bf16(a, b, c);
    default:   /* BF16_SPLIT: multiply rounded, then add rounded */
        return orc_fma_bf16(orc_fma_bf16(a, b, 0x8000), 0x3F80, c);
    }
}

static uint16_t t_mul(const fmt_ops *f, uint16_t a, uint16_t b)
{
    return t_fma(f, a, b, f->negzero);     /* a*b + (-0) == RN(a*b) */
}

static uint16_t t_add(const fmt_ops *f, uint16_t a, uint16_t b)
{
    return t_fma(f, a, f->one, b);          /* a*1 is exact */
}

/* Coefficient c_j in the target format; the BF16 values chosen by the fit
 * must be exactly representable in FP16 when the program runs in FP16. */
static uint16_t coef(const fmt_ops *f, const orc_prog *p, int j)
{
    if (f->order != ORC_ORDER_F16_FMA) return p->c[j];
    const double v = orc_bf16_to_f64(p->c[j]);
    const uint16_t h = orc_f64_to_f16(v);
    if (orc_f16_to_f64(h) != v) abort();
    return h;
}

static uint16_t enc(const fmt_ops *f, double v)
{
    return f->order == ORC_ORDER_F16_FMA ? orc_f64_to_f16(v) : orc_f64_to_bf16(v);
}

/* Horner value v(t_hat) of the half-domain polynomial, deployed order:
 * v = c_D; v = fma(v, t, c_j) for j = D-1..1; last stage v*t when c_0 = 0,
 * else fma(v, t, c_0). */
static uint16_t horner(const fmt_ops *f, const orc_prog *p, uint16_t th)
{
    uint16_t v = coef(f, p, p->degree);
    for (int j = p->degree - 1; j >= 1; j--) v = t_fma(f, v, th, coef(f, p, j));
    if (val(f, coef(f, p, 0)) == 0.0) return t_mul(f, v, th);
    return t_fma(f, v, th, coef(f, p, 0));
}

/* Program output y(x) for a forward program; for a derivative program the
 * surrogate derivative value f'(x). */
static uint16_t eval_one(const fmt_ops *f, const orc_prog *p, uint16_t x)
{
    if (is_nan(f, x)) return x | f->quiet;
    const uint16_t s = x & f->sign;
    const uint16_t t = x & 0x7FFF;            /* |x|, possibly +inf */
    const uint16_t lc = enc(f, p->Lc);
    const uint16_t th = val(f, t) > p->Lc ? lc : t;   /* min(|x|, Lc) */
    const uint16_t v = horner(f, p, th);
    if (!p->deriv) {
        switch (p->func) {
        case ORC_SIGMOID: return t_add(f, f->half, v ^ s);
        case ORC_TANH: return v ^ s;
        default:                                /* SiLU, GELU: x/2 + t v */
            if (s && val(f, t) == INFINITY) return f->negzero;
            return t_fma(f, t, v, t_mul(f, x, f->half));
        }
    }
    if (p->func == ORC_SILU || p->func == ORC_GELU)
        return t_add(f, f->half, v ^ s);      /* centered-odd derivative */
    return v;                                 /* even derivative */
}

uint16_t orc_prog_eval(const orc_prog *p, uint16_t x, int order)
{
    const fmt_ops f = ops_for(order);
    return eval_one(&f, p, x);
}

uint16_t orc_prog_bwd(const orc_prog *p, uint16_t x, uint16_t g, int order)
{
    const fmt_ops f = ops_for(order);
    if (is_nan(&f, x)) return x | f.quiet;
    if (is_nan(&f, g)) return g | f.quiet;
    return t_mul(&f, g, eval_one(&f, p, x));
}

void orc_act_fwd(const orc_prog *p, int order, const uint16_t *x, uint16_t *y,
                 int64_t n)
{
    const fmt_ops f = ops_for(order);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) y[i] = eval_one(&f, p, x[i]);
}

void orc_act_bwd(const orc_prog *p, int order, const uint16_t *x,
                 const uint16_t *g, uint16_t *dx, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) dx[i] = orc_prog_bwd(p, x[i], g[i], order);
}

/* ---- fused SwiGLU (BF16 in/out, FP32 combine) ---------------------------
 * p = sigma~(g) is the D3 sigmoid program in BF16, replayed as FP32 FMA then
 * BF16 rounding per stage.  Forward h = RN16(RN32(g p) * u); g p is exact in
 * FP32 (8 x 8 significant bits) away from underflow.  Backward:
 *   ds = RN32(g p (1 - p) + p)     (1 - p exact in FP32)
 *   du = RN16(dh * RN32(g p))
 *   dg = RN16(RN32(RN32(dh u) * ds))                                       */
void orc_swiglu_fwd(const orc_prog *sig, const uint16_t *gate, const uint16_t *up,
                    uint16_t *h, int64_t row_begin, int64_t row_end, int64_t cols,
                    int64_t ld_gate, int64_t ld_up, int64_t ld_h)
{
    const fmt_ops f = ops_for(ORC_ORDER_F32FMA_BF16);
#pragma omp parallel for schedule(static)
    for (int64_t r = row_begin; r < row_end; r++) {
        for (int64_t c = 0; c < cols; c++) {
            const uint16_t g = gate[r * ld_gate + c];
            const float gf = orc_bf16_to_f32(g);
            const float pf = orc_bf16_to_f32(eval_one(&f, sig, g));
            const float gp = orc_mul_f32(gf, pf);
            const float uf = orc_bf16_to_f32(up[r * ld_up + c]);
            h[r * ld_h + c] = orc_f32_to_bf16(orc_mul_f32(gp, uf));
        }
    }
}

void orc_swiglu_bwd(const orc_prog *sig, const uint16_t *gate, const uint16_t *up,
                    const uint16_t *dh, uint16_t *dgate, uint16_t *dup,
                    int64_t row_begin, int64_t row_end, int64_t cols,
                    int64_t ld_gate, int64_t ld_up, int64_t ld_dh,
                    int64_t ld_dgate, int64_t ld_dup)
{
    const fmt_ops f = ops_for(ORC_ORDER_F32FMA_BF16);
#pragma omp parallel for schedule(static)
    for (int64_t r = row_begin; r < row_end; r++) {
        for (int64_t c = 0; c < cols; c++) {
            const uint16_t g = gate[r * ld_gate + c];
            const float gf = orc_bf16_to_f32(g);
            const float pf = orc_bf16_to_f32(eval_one(&f, sig, g));
            const float uf = orc_bf16_to_f32(up[r * ld_up + c]);
            const float dhf = orc_bf16_to_f32(dh[r * ld_dh + c]);
            const float gp = orc_mul_f32(gf, pf);
            const float omp = orc_add_f32(1.0f, -pf);
            const float ds = orc_fma_f32(gp, omp, pf);
            dup[r * ld_dup + c] = orc_f32_to_bf16(orc_mul_f32(dhf, gp));
            dgate[r * ld_dgate + c] =
                orc_f32_to_bf16(orc_mul_f32(orc_mul_f32(dhf, uf), ds));
        }
    }
}

/* ---- softcapped attention forward, selected query rows ------------------
 * Q, K, V: BF16 [B, H, S, D] contiguous.  For each requested flat row index
 * r = (b H + h) S + i, computes O[r, :] in FP64 and the per-column noise
 * scale sqrt(sum_j P_j^2 V_jd^2) (the size of the output change caused by
 * relative perturbations of the probabilities; used to state tolerances).
 * Scores: S_ij = q_i . k_j exactly in FP64.
 *   poly = 1: x = RN_f16(RN32(RN32(S_ij) * RN32(1/(cap sqrt(D))))), the D4 tanh
 *             program in FP16 arithmetic (one rounding per FMA), s = cap * t~;
 *   poly = 0: s = cap * tanh(S_ij / (cap sqrt(D))) in FP64.
 * Causal: key j <= query i.  Softmax and the P V product in FP64. */
void orc_softcap_attn_rows(const orc_prog *tp, int poly,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int32_t B, int32_t H, int32_t S, int32_t D, float cap,
                           int32_t causal, const int64_t *rows, int64_t n_rows,
                           double *out, double *noise)
{
    const fmt_ops f = ops_for(ORC_ORDER_F16_FMA);
    const float scale = (float)(1.0 / ((double)cap * sqrt((double)D)));
    (void)B;
#pragma omp parallel
    {
        double *s = malloc(sizeof(double) * (size_t)S);
        double *qd = malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < n_rows; ri++) {
            const int64_t r = rows[ri];
            const int64_t bh = r / S;
            const int64_t i = r % S;
            (void)H;
            const uint16_t *qr = q + r * D;
            const uint16_t *kb = k + bh * (int64_t)S * D;
            const uint16_t *vb = v + bh * (int64_t)S * D;
            for (int d = 0; d < D; d++) qd[d] = orc_bf16_to_f64(qr[d]);
            const int64_t nk = causal ? i + 1 : S;
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; j++) {
                double acc = 0.0;
                for (int d = 0; d < D; d++)
                    acc += qd[d] * orc_bf16_to_f64(kb[j * D + d]);
                double sc;
                if (poly) {
                    const float xs = orc_mul_f32((float)acc, scale);
                    const uint16_t xh = orc_f64_to_f16((double)xs);
                    sc = (double)cap * orc_f16_to_f64(eval_one(&f, tp, xh));
                } else {
                    sc = (double)cap * tanh(acc / ((double)cap * sqrt((double)D)));
                }
                s[j] = sc;
                if (sc > m) m = sc;
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; j++) { s[j] = exp(s[j] - m); l += s[j]; }
            for (int d = 0; d < D; d++) {
                double o = 0.0, n2 = 0.0;
                for (int64_t j = 0; j < nk; j++) {
                    const double pj = s[j] / l;
                    const double vj = orc_bf16_to_f64(vb[j * D + d]);
                    o += pj * vj;
                    n2 += pj * pj * vj * vj;
                }
                out[ri * D + d] = o;
                if (noise) noise[ri * D + d] = sqrt(n2);
            }
        }
        free(s);
        free(qd);
    }
}
