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

/* ---- attention with a transformed score ------------------------------------
 * Layout: Q, O, dO [B, H, S, D]; K, V [B, Hkv, S, D] (grouped-query attention:
 * query head h reads key/value head h / (H / Hkv)); BF16 bit patterns, except
 * O and the log-sum-exp, which are passed as FP64 values.  Raw score
 * S_ij = q_i . k_j (exact in FP64: BF16 products have 16 significant bits).
 * Causal: key j visible from query i when j <= i.
 *
 * Score transforms:
 *   SOFTCAP (Eq. 1): logit s = cap tanh(S / (cap sqrt D)), P = softmax_j(s).
 *     POLY  x = RN_fmt(RN32(RN32(S) * RN32(1 / (cap sqrt D)))), tanh by the D4
 *           program in the program's format: BF16 (each stage an FP32 FMA
 *           rounded to BF16; the pages run the integrations on the BF16 path,
 *           section 3.4) or FP16 (one FP16 rounding per stage).  Backward
 *           (section 3.3, section 5.2.2): the analytic derivative of that
 *           program, the D3 with coefficients (j + 1) c_{j+1} (exact in FP16,
 *           rounded to BF16 for the BF16 program) evaluated in the same format
 *           at |x|; beyond the clamp Lc the forward program is constant, so
 *           its derivative is 0 there.
 *     EXACT tanh of the scaled score; derivative 1 - tanh^2 (Eq. 12).
 *   SIGMOID (Eq. 14): P = sigma(s - ln n) with s = S / sqrt D and n = S, the
 *     sequence length; no normalisation.
 *     POLY  x = RN_bf16(RN32(RN32(S) * RN32(1 / sqrt D))); the two-region
 *           cubic of section 3.4 / Appendix C on the clamped x, floored at 0,
 *           with ln n and 1 / n folded into its coefficients (so it holds for
 *           one n only); backward surrogate P~ (a + b x) per region.
 *     EXACT sigma; dP/dS = P (1 - P) / sqrt D.
 *
 * Two arithmetic models around the programs (orc_attn.replay):
 *   0  real arithmetic: scores, weights and sums in FP64 (the program values
 *      exact as computed); the softcap chain factor is cap RN32(1 / (cap
 *      sqrt D)).  Pinned against automatic differentiation.
 *   1  the method's rounding steps: the FP32 score path of the pages'
 *      attention kernels (QK^T accumulated in FP32, the softmax in FP32 with
 *      its exponential as exp2) and the BF16 operands of the P V, dS K and
 *      dS^T Q products (section 3.4: P cast to the value dtype before the
 *      product).  Every scalar step below is rounded to FP32 once (a fused
 *      multiply-add where one operation forms a product and a sum); P and dS
 *      are rounded to BF16 before they multiply V, dO, K or Q; the row sum l
 *      adds the FP32 P; the sums themselves are exact.
 *      Softcap forward: z = RN32(t c2 - m), c2 = RN32(cap log2 e), with the
 *      fixed reference m = ceil(RN32(c2 - 40)) when c2 <= 80 (every logit is
 *      bounded by cap, so one reference keeps each P in FP32's normal range);
 *      otherwise, and with a software exp2 core, z = RN32(t c2) split as
 *      2^floor(z) 2^(z - floor z), which makes each P independent of the
 *      reference up to an exact power of two.  P = RN32(2^z) (or the core's
 *      value).  lse = (m + log2 l) ln 2.
 *      Backward: P = 2^z with z = RN32(t c2 + RN32(-lse log2 e)) from the
 *      forward's FP32 log-sum-exp (through the same exp2 core, if any);
 *      Delta_i = RN32(dO_i . O_i), dP = RN32(dO_i . V_j);
 *      softcap dS = RN32(q' RN32(P RN32(dP - Delta))), q' the derivative
 *      value; sigmoid dS = RN32(dP g); dQ and dK scaled by RN32(1 / sqrt D)
 *      at the end.
 *
 * Backward (chain rule through O = P V):
 *   dV_j = sum_i P_ij dO_i;   dP_ij = dO_i . V_j;
 *   softcap: dS_ij = P_ij (dP_ij - Delta_i) ds/dS,  Delta_i = dO_i . O_i
 *   sigmoid: dS_ij = dP_ij dP/dS;
 *   dQ_i = sum_j dS_ij K_j;   dK_j = sum over query heads of the group and
 *   visible i of dS_ij Q_i.
 * Each output also gets a noise scale sqrt(sum of squared terms), and dQ / dK
 * two further scales (see pair_grad); these are diagnostics that do not
 * enter the values. */

static const double LOG2E = 1.4426950408889634074;
static const double LN2 = 0.69314718055994530942;

static double stable_sigmoid(double s)
{
    const double e = exp(-fabs(s));
    return s >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

/* Analytic derivative of the tanh program at x (bits of format f): the D3
 * with coefficients (j + 1) c_{j+1} in format f at |x|, 0 beyond the clamp. */
static uint16_t dtanh_prog(const fmt_ops *f, const orc_prog *tp, uint16_t x)
{
    uint16_t d[8];
    for (int j = 0; j < tp->degree; j++) {
        const double v = (double)(j + 1) * orc_bf16_to_f64(tp->c[j + 1]);
        d[j] = enc(f, v);
        if (f->order == ORC_ORDER_F16_FMA && orc_f16_to_f64(d[j]) != v) abort();
    }
    if (is_nan(f, x)) return x | f->quiet;
    const uint16_t t = x & 0x7FFF;
    if (val(f, t) > tp->Lc) return 0;
    uint16_t v = d[tp->degree - 1];
    for (int j = tp->degree - 2; j >= 0; j--) v = t_fma(f, v, t, d[j]);
    return v;
}

uint16_t orc_dtanh_prog(const orc_prog *tp, uint16_t x, int order)
{
    const fmt_ops f = ops_for(order);
    return dtanh_prog(&f, tp, x);
}

uint16_t orc_dtanh_prog_f16(const orc_prog *tp, uint16_t x)
{
    return orc_dtanh_prog(tp, x, ORC_ORDER_F16_FMA);
}

/* Two-region sigmoid-attention program at BF16 x: region 1 when x >= thr;
 * x clamped to [lo, hi]; v = c3; v = fma(x, v, c_j) for j = 2, 1, 0 in the
 * given order; P = max(v, +0); surrogate derivative P * fma(x, b, a). */
static uint16_t sig_eval(const fmt_ops *f, const orc_sig_prog *sp, uint16_t x,
                         uint16_t *grad)
{
    const double xv = orc_bf16_to_f64(x);
    const int r = xv >= orc_bf16_to_f64(sp->thr);
    uint16_t xc = x;
    if (xv > orc_bf16_to_f64(sp->hi)) xc = sp->hi;
    if (xv < orc_bf16_to_f64(sp->lo)) xc = sp->lo;
    uint16_t v = sp->c[r][3];
    for (int j = 2; j >= 0; j--) v = t_fma(f, xc, v, sp->c[r][j]);
    if (orc_bf16_to_f64(v) < 0.0) v = 0;
    if (grad) *grad = t_mul(f, v, t_fma(f, xc, sp->b[r], sp->a[r]));
    return v;
}

uint16_t orc_sig_prog_eval(const orc_sig_prog *sp, uint16_t x, int order, uint16_t *grad)
{
    const fmt_ops f = ops_for(order);
    return sig_eval(&f, sp, x, grad);
}

typedef struct {
    const orc_attn *a;
    fmt_ops ft;       /* format of the softcap program */
    fmt_ops fs;       /* replay order of the sigmoid program */
    float scale;      /* RN32 of the factor applied to S before rounding x */
    float c2;         /* RN32(cap log2 e) */
    float mref;       /* fixed reference of the softcap forward (c2 <= 80) */
    int sref;
    float rsd32;      /* RN32(1 / sqrt D) */
    float logn32;     /* RN32(ln S) */
    double rsd;       /* 1 / sqrt(D) */
    double logn;      /* ln S (sigmoid) */
} actx;

static int actx_init(actx *c, const orc_attn *a)
{
    if (a->H <= 0 || a->Hkv <= 0 || a->H % a->Hkv || a->S < 0 || a->D <= 0) return -2;
    if (a->replay < 0 || a->replay > 1) return -2;
    c->a = a;
    c->ft = ops_for(a->tanh_order ? a->tanh_order : ORC_ORDER_F32FMA_BF16);
    if (c->ft.order != ORC_ORDER_F16_FMA && c->ft.order != ORC_ORDER_F32FMA_BF16) return -3;
    c->fs = ops_for(a->order ? a->order : ORC_ORDER_F32FMA_BF16);
    c->rsd = 1.0 / sqrt((double)a->D);
    c->rsd32 = (float)c->rsd;
    c->logn = log((double)a->S);
    c->logn32 = (float)c->logn;
    c->c2 = (float)((double)a->cap * LOG2E);
    c->sref = c->c2 <= 80.0f;
    c->mref = ceilf(orc_add_f32(c->c2, -40.0f));
    switch (a->kind) {
    case ORC_ATTN_SOFTCAP_POLY:
    case ORC_ATTN_SOFTCAP_EXACT:
        if (!(a->cap > 0.0f)) return -2;
        c->scale = (float)(1.0 / ((double)a->cap * sqrt((double)a->D)));
        return 0;
    case ORC_ATTN_SIGMOID_POLY:
        if (!a->sig || a->sig->n != a->S) return -1;   /* the length guard */
        c->scale = c->rsd32;
        return 0;
    case ORC_ATTN_SIGMOID_EXACT:
        c->scale = c->rsd32;
        return 0;
    default:
        return -3;
    }
}

static int is_softcap(const orc_attn *a)
{
    return a->kind == ORC_ATTN_SOFTCAP_POLY || a->kind == ORC_ATTN_SOFTCAP_EXACT;
}

static double bf16r(double v)
{
    return orc_bf16_to_f64(orc_f64_to_bf16(v));
}

/* Softcap: tanh value t and derivative value q' (of t with respect to the
 * scaled score x) at raw score Sr. */
static void softcap_t(const actx *c, double Sr, double *t, double *dq)
{
    const orc_attn *a = c->a;
    if (a->kind == ORC_ATTN_SOFTCAP_POLY) {
        const uint16_t x = enc(&c->ft, (double)orc_mul_f32((float)Sr, c->scale));
        *t = val(&c->ft, eval_one(&c->ft, a->tanh_prog, x));
        *dq = val(&c->ft, dtanh_prog(&c->ft, a->tanh_prog, x));
    } else if (a->replay) {
        const float tt = (float)tanh((double)orc_mul_f32((float)Sr, c->scale));
        *t = tt;
        *dq = orc_fma_f32(-tt, tt, 1.0f);
    } else {
        *t = tanh(Sr / ((double)a->cap * sqrt((double)a->D)));
        *dq = 1.0 - *t * *t;
    }
}

/* 2^z in FP32 by the softmax's exponential: core 0 the exponential itself
 * (correctly rounded), else 2^floor(z) p(z - floor z) with the core p in
 * target precision (z clamped below at -16384).  The power of two is applied
 * relative to 2^ref (an integer). */
static double exp2_fp32(int core, float z, double ref)
{
    if (core == 0) return (double)(float)exp2((double)z - ref);
    if (z < -16384.0f) z = -16384.0f;
    const double n = floor((double)z);
    const float f = (float)((double)z - n);      /* exact */
    return (double)(float)ldexp((double)orc_exp2_core_target(core, f), (int)(n - ref));
}

/* Softmax weights of one softcap row (real-arithmetic model) with a
 * software exp2: 2^z = 2^floor(z) p(z - floor(z)), z = RN32(t RN32(cap
 * log2 e)), relative to the row's largest floor(z).  Returns the natural
 * log-sum-exp; w holds the normalised weights. */
static double exp2_core_weights(const actx *c, const double *t, double *w, int64_t nk)
{
    double M = -INFINITY;
    for (int64_t j = 0; j < nk; j++) {
        const double n = floor((double)orc_mul_f32((float)t[j], c->c2));
        if (n > M) M = n;
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; j++) {
        w[j] = exp2_fp32(c->a->exp2_core, orc_mul_f32((float)t[j], c->c2), M);
        l += w[j];
    }
    for (int64_t j = 0; j < nk; j++) w[j] /= l;
    return (M + log2(l)) * LN2;
}

/* Softmax of one softcap row in the replay model: P_j in FP32 (see the
 * header), l the sum of the FP32 P_j, w_j = RN_bf16(P_j) / l.  Returns the
 * natural log-sum-exp. */
static double softcap_row_replay(const actx *c, const double *t, double *w, int64_t nk)
{
    const int core = c->a->exp2_core;
    double ref = 0.0;
    if (core == 0 && c->sref) {
        for (int64_t j = 0; j < nk; j++)
            w[j] = (double)(float)exp2((double)orc_fma_f32((float)t[j], c->c2, -c->mref));
        ref = c->mref;
    } else {
        ref = -INFINITY;
        for (int64_t j = 0; j < nk; j++) {
            float z = orc_mul_f32((float)t[j], c->c2);
            if (z < -16384.0f) z = -16384.0f;
            const double n = floor((double)z);
            if (n > ref) ref = n;
        }
        for (int64_t j = 0; j < nk; j++)
            w[j] = exp2_fp32(core, orc_mul_f32((float)t[j], c->c2), ref);
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; j++) l += w[j];
    for (int64_t j = 0; j < nk; j++) w[j] = bf16r(w[j]) / l;
    return (ref + log2(l)) * LN2;
}

static double dot_bf16(const uint16_t *x, const uint16_t *y, int D)
{
    double s = 0.0;
    for (int d = 0; d < D; d++) s += orc_bf16_to_f64(x[d]) * orc_bf16_to_f64(y[d]);
    return s;
}

/* P of one sigmoid-attention score: the program value (BF16) or sigma. */
static double sigmoid_p(const actx *c, double Sr, uint16_t *g)
{
    const orc_attn *a = c->a;
    if (a->kind == ORC_ATTN_SIGMOID_POLY) {
        const uint16_t x = orc_f64_to_bf16((double)orc_mul_f32((float)Sr, c->scale));
        return orc_bf16_to_f64(sig_eval(&c->fs, a->sig, x, g));
    }
    if (a->replay)
        return (double)(float)stable_sigmoid((double)orc_fma_f32((float)Sr, c->scale, -c->logn32));
    return stable_sigmoid(Sr * c->rsd - c->logn);
}

int orc_attn_fwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const int64_t *rows, int64_t n_rows,
                      double *out, double *lse, double *noise)
{
    actx c;
    const int rc = actx_init(&c, a);
    if (rc) return rc;
    if (a->exp2_core && a->kind != ORC_ATTN_SOFTCAP_POLY) return -3;
    const int64_t S = a->S, D = a->D, G = a->H / a->Hkv;
#pragma omp parallel
    {
        double *w = malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < n_rows; ri++) {
            const int64_t r = rows[ri];
            const int64_t bh = r / S, i = r % S;
            const int64_t b = bh / a->H, h = bh % a->H;
            const int64_t kvb = (b * a->Hkv + h / G) * S * D;
            const int64_t nk = a->causal ? i + 1 : S;
            if (is_softcap(a)) {
                double dummy, ls;
                for (int64_t j = 0; j < nk; j++)
                    softcap_t(&c, dot_bf16(q + r * D, k + kvb + j * D, (int)D), &w[j], &dummy);
                if (a->replay) {
                    ls = softcap_row_replay(&c, w, w, nk);
                } else if (a->exp2_core) {
                    ls = exp2_core_weights(&c, w, w, nk);
                } else {
                    double m = -INFINITY, l = 0.0;
                    for (int64_t j = 0; j < nk; j++) {
                        w[j] *= (double)a->cap;
                        if (w[j] > m) m = w[j];
                    }
                    for (int64_t j = 0; j < nk; j++) { w[j] = exp(w[j] - m); l += w[j]; }
                    for (int64_t j = 0; j < nk; j++) w[j] /= l;
                    ls = m + log(l);
                }
                if (lse) lse[ri] = ls;
            } else {
                for (int64_t j = 0; j < nk; j++) {
                    const double p = sigmoid_p(&c, dot_bf16(q + r * D, k + kvb + j * D, (int)D), NULL);
                    w[j] = a->replay ? bf16r(p) : p;
                }
                if (lse) lse[ri] = NAN;
            }
            for (int64_t d = 0; d < D; d++) {
                double o = 0.0, n2 = 0.0;
                for (int64_t j = 0; j < nk; j++) {
                    const double vj = orc_bf16_to_f64(v[kvb + j * D + d]);
                    o += w[j] * vj;
                    n2 += w[j] * w[j] * vj * vj;
                }
                out[ri * D + d] = o;
                if (noise) noise[ri * D + d] = sqrt(n2);
            }
        }
        free(w);
    }
    return 0;
}

/* P_ij and dS_ij of one (query row, key row) pair as the products use them
 * (BF16-rounded in the replay model), and two scales of an FP32 evaluation
 * of dS:
 *   cs  |dS / (dP - Delta)| (softcap) or |dS / dP| (sigmoid) times the sum of
 *       the absolute products that form dP - Delta (or dP);
 *   sd  |dS / g|, g the transform's derivative before the chain factor: the
 *       sensitivity to an absolute error in g.
 * delta_i is Delta_i (RN32 of it in the replay model), lse_i the row's
 * log-sum-exp (softcap). */
static void pair_grad(const actx *c, const uint16_t *qi, const uint16_t *kj,
                      const uint16_t *vj, const uint16_t *doi, const double *oi,
                      double lse_i, double delta_i, double *P, double *dS, double *cs,
                      double *sd)
{
    const orc_attn *a = c->a;
    const int D = a->D;
    const double Sr = dot_bf16(qi, kj, D);
    const double dP = dot_bf16(doi, vj, D);
    double ab = 0.0;
    for (int d = 0; d < D; d++) {
        const double g = fabs(orc_bf16_to_f64(doi[d]));
        ab += g * fabs(orc_bf16_to_f64(vj[d]));
        if (oi) ab += g * fabs(oi[d]);
    }
    if (is_softcap(a)) {
        double t, dq;
        softcap_t(c, Sr, &t, &dq);
        if (a->replay) {
            const float nl = -orc_mul_f32((float)lse_i, (float)LOG2E);
            const float p = (float)exp2_fp32(a->exp2_core, orc_fma_f32((float)t, c->c2, nl), 0.0);
            const float u = orc_add_f32((float)dP, -(float)delta_i);
            const float ds = orc_mul_f32((float)dq, orc_mul_f32(p, u));
            *P = bf16r(p);
            *dS = bf16r(ds);
            *cs = fabs((double)p * dq) * ab;
            *sd = fabs((double)p * u);
        } else {
            /* the program sees RN32(S scale); the exact transform S itself */
            const double dval = a->kind == ORC_ATTN_SOFTCAP_POLY
                                    ? (double)a->cap * (double)c->scale * dq : dq * c->rsd;
            *P = exp((double)a->cap * t - lse_i);
            *dS = *P * (dP - delta_i) * dval;
            *cs = fabs(*P * dval) * ab;
            *sd = fabs(*P * (dP - delta_i)) * c->rsd;
        }
        return;
    }
    uint16_t g = 0;
    const double p = sigmoid_p(c, Sr, &g);
    double dval;
    if (a->kind == ORC_ATTN_SIGMOID_POLY) {
        dval = orc_bf16_to_f64(g);
        if (!a->replay) dval *= (double)c->scale;
    } else if (a->replay) {
        dval = orc_mul_f32((float)p, orc_add_f32(1.0f, -(float)p));
    } else {
        dval = p * (1.0 - p) * c->rsd;
    }
    if (a->replay) {
        *P = bf16r(p);
        *dS = bf16r(orc_mul_f32((float)dP, (float)dval));
    } else {
        *P = p;
        *dS = dP * dval;
    }
    *cs = fabs(dval) * ab;
    *sd = fabs(dP) * (a->replay ? 1.0 : c->rsd);
}

static double row_delta(const actx *c, const uint16_t *doi, const double *oi, int D)
{
    double s = 0.0;
    for (int d = 0; d < D; d++) s += orc_bf16_to_f64(doi[d]) * oi[d];
    return c->a->replay ? (double)(float)s : s;
}

int orc_attn_bwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const double *o, const uint16_t *dout,
                      const double *lse, const int64_t *qrows, int64_t nq,
                      const int64_t *krows, int64_t nk, double *dq, double *dk,
                      double *dv, double *nz_dq, double *nz_dk, double *nz_dv,
                      double *cs_dq, double *cs_dk, double *sd_dq, double *sd_dk)
{
    actx c;
    const int rc = actx_init(&c, a);
    if (rc) return rc;
    if (a->exp2_core && a->kind != ORC_ATTN_SOFTCAP_POLY) return -3;
    const int64_t S = a->S, D = a->D, G = a->H / a->Hkv;
    const int sc = is_softcap(a);
    /* replay: dQ, dK scaled by RN32(1 / sqrt D) at the end; the real model
     * carries the chain factor inside dS */
    const double fin = a->replay ? (double)c.rsd32 : 1.0;
    /* dQ rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nq; ri++) {
        const int64_t r = qrows[ri];
        const int64_t bh = r / S, i = r % S;
        const int64_t b = bh / a->H, h = bh % a->H;
        const int64_t kvb = (b * a->Hkv + h / G) * S * D;
        const double delta = sc ? row_delta(&c, dout + r * D, o + r * D, (int)D) : 0.0;
        const double li = sc ? lse[r] : 0.0;
        const int64_t n = a->causal ? i + 1 : S;
        for (int64_t d = 0; d < D; d++) {
            dq[ri * D + d] = 0.0;
            if (nz_dq) nz_dq[ri * D + d] = 0.0;
            if (cs_dq) cs_dq[ri * D + d] = 0.0;
            if (sd_dq) sd_dq[ri * D + d] = 0.0;
        }
        for (int64_t j = 0; j < n; j++) {
            double P, dS, cs, sd;
            pair_grad(&c, q + r * D, k + kvb + j * D, v + kvb + j * D, dout + r * D,
                      sc ? o + r * D : NULL, li, delta, &P, &dS, &cs, &sd);
            for (int64_t d = 0; d < D; d++) {
                const double kd = orc_bf16_to_f64(k[kvb + j * D + d]);
                const double t = dS * kd;
                dq[ri * D + d] += t;
                if (nz_dq) nz_dq[ri * D + d] += t * t;
                if (cs_dq) cs_dq[ri * D + d] += cs * fabs(kd);
                if (sd_dq) sd_dq[ri * D + d] += sd * fabs(kd);
            }
        }
        for (int64_t d = 0; d < D; d++) {
            dq[ri * D + d] *= fin;
            if (nz_dq) nz_dq[ri * D + d] = sqrt(nz_dq[ri * D + d]) * fin;
            if (cs_dq) cs_dq[ri * D + d] *= fin;
            if (sd_dq) sd_dq[ri * D + d] *= fin;
        }
    }
    /* dK, dV rows: key row r = (b Hkv + hk) S + j */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nk; ri++) {
        const int64_t r = krows[ri];
        const int64_t bk = r / S, j = r % S;
        const int64_t b = bk / a->Hkv, hk = bk % a->Hkv;
        for (int64_t d = 0; d < D; d++) {
            dk[ri * D + d] = dv[ri * D + d] = 0.0;
            if (nz_dk) nz_dk[ri * D + d] = 0.0;
            if (nz_dv) nz_dv[ri * D + d] = 0.0;
            if (cs_dk) cs_dk[ri * D + d] = 0.0;
            if (sd_dk) sd_dk[ri * D + d] = 0.0;
        }
        for (int64_t h = hk * G; h < (hk + 1) * G; h++) {
            const int64_t qb = (b * a->H + h) * S;
            for (int64_t i = a->causal ? j : 0; i < S; i++) {
                const int64_t qr = qb + i;
                const double delta = sc ? row_delta(&c, dout + qr * D, o + qr * D, (int)D) : 0.0;
                double P, dS, cs, sd;
                pair_grad(&c, q + qr * D, k + r * D, v + r * D, dout + qr * D,
                          sc ? o + qr * D : NULL, sc ? lse[qr] : 0.0, delta, &P, &dS, &cs,
                          &sd);
                for (int64_t d = 0; d < D; d++) {
                    const double qd = orc_bf16_to_f64(q[qr * D + d]);
                    const double tk = dS * qd;
                    if (cs_dk) cs_dk[ri * D + d] += cs * fabs(qd);
                    if (sd_dk) sd_dk[ri * D + d] += sd * fabs(qd);
                    const double tv = P * orc_bf16_to_f64(dout[qr * D + d]);
                    dk[ri * D + d] += tk;
                    dv[ri * D + d] += tv;
                    if (nz_dk) nz_dk[ri * D + d] += tk * tk;
                    if (nz_dv) nz_dv[ri * D + d] += tv * tv;
                }
            }
        }
        for (int64_t d = 0; d < D; d++) {
            dk[ri * D + d] *= fin;
            if (nz_dk) nz_dk[ri * D + d] = sqrt(nz_dk[ri * D + d]) * fin;
            if (nz_dv) nz_dv[ri * D + d] = sqrt(nz_dv[ri * D + d]);
            if (cs_dk) cs_dk[ri * D + d] *= fin;
            if (sd_dk) sd_dk[ri * D + d] *= fin;
        }
    }
    return 0;
}
