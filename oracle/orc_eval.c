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

/* Threads of the following parallel loops (n >= 1); the previous count. */
int orc_set_threads(int n)
{
    const int old = orc_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return old;
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
 *
 * Several results are correct.  The pages fix the precision of each step but
 * not the order in which an FP32 dot product accumulates, nor the last bit of
 * an FP32 exponential, so the replay model's rounding decisions (the program
 * input x, the BF16 P, the BF16 dS) can go either way where the value that
 * is rounded lies close to a rounding boundary.  The oracle therefore also
 * returns, per output, the spread: the largest change of that output that
 * admissible alternatives of those decisions can cause, each score taken on
 * its own (first order in l for the forward):
 *   raw score and dP: any FP32 value within 8 u sum |a_d b_d| of the exact
 *     dot product (u = 2^-24; an FP32 accumulation that rounds once per 16
 *     products, the depth of one BF16 matrix instruction);
 *   Delta: any FP32 value within 128 u sum |dO_d O_d| (any order);
 *   the hardware exponential 2^z: the correctly rounded FP32 value or a
 *     neighbour (1 ulp); the software exp2 cores are exact FP32 arithmetic;
 *   the comparators' tanh and sigma: within 4 ulps of the correctly rounded
 *     FP32 value.
 * The spread is 0 in the real-arithmetic model. */

#define U32 5.9604644775390625e-08   /* 2^-24 */
#define XC_MAX 64

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

static int is_softcap(const orc_attn *a)
{
    return a->kind == ORC_ATTN_SOFTCAP_POLY || a->kind == ORC_ATTN_SOFTCAP_EXACT;
}

static double bf16r(double v)
{
    return orc_bf16_to_f64(orc_f64_to_bf16(v));
}

/* Smallest FP32 value >= v and largest FP32 value <= v. */
static float ru32(double v)
{
    float f = (float)v;
    if ((double)f < v) f = nextafterf(f, INFINITY);
    return f;
}

static float rd32(double v)
{
    float f = (float)v;
    if ((double)f > v) f = nextafterf(f, -INFINITY);
    return f;
}

/* x +- k ulps of FP32 */
static float ulps32(float x, int k)
{
    for (int i = 0; i < (k < 0 ? -k : k); i++) x = nextafterf(x, k < 0 ? -INFINITY : INFINITY);
    return x;
}

/* Exact dot product of two BF16 rows and the sum of the absolute products. */
static double dot_bf16(const uint16_t *x, const uint16_t *y, int D, double *abs_sum)
{
    double s = 0.0, a = 0.0;
    for (int d = 0; d < D; d++) {
        const double p = orc_bf16_to_f64(x[d]) * orc_bf16_to_f64(y[d]);
        s += p;
        a += fabs(p);
    }
    if (abs_sum) *abs_sum = a;
    return s;
}

/* The admissible FP32 values of a dot product: RN32 of the exact value and
 * every FP32 value within eps of it. */
typedef struct { float v, lo, hi; } f32r;

static f32r fp32_range(double exact, double eps)
{
    f32r r;
    r.v = (float)exact;
    r.lo = ru32(exact - eps);
    r.hi = rd32(exact + eps);
    if (r.lo > r.v) r.lo = r.v;
    if (r.hi < r.v) r.hi = r.v;
    return r;
}

/* Order key of a 16-bit float pattern (monotone in value; +-0 -> 0). */
static int fkey(uint16_t b)
{
    return (b & 0x8000) ? -(int)(b & 0x7FFF) : (int)(b & 0x7FFF);
}

static uint16_t fbits(int k)
{
    return k >= 0 ? (uint16_t)k : (uint16_t)(0x8000 | (uint16_t)(-k));
}

/* The program inputs x in format f reachable from scaled scores in
 * [xs_lo, xs_hi] (RN to the format is monotone): every format value between
 * the two roundings, x0 first.  More than XC_MAX values occur only where the
 * range straddles zero, where every program in use is RN(c_1 t) to first
 * order and monotone, so the two ends stand for the rest.  Returns the count. */
static int x_cands(const fmt_ops *f, float xs0, float xs_lo, float xs_hi, uint16_t *out)
{
    const uint16_t x0 = enc(f, (double)xs0);
    const int k0 = fkey(enc(f, (double)xs_lo)), k1 = fkey(enc(f, (double)xs_hi));
    int n = 0;
    out[n++] = x0;
    if (k1 - k0 + 1 > XC_MAX) {
        if (fbits(k0) != x0) out[n++] = fbits(k0);
        if (fbits(k1) != x0) out[n++] = fbits(k1);
        return n;
    }
    for (int k = k0; k <= k1; k++)
        if (k != fkey(x0)) out[n++] = fbits(k);
    return n;
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

/* ---- real-arithmetic model ----------------------------------------------- */

/* Transformed score of raw score Sr: the logit (softcap) or the probability
 * (sigmoid), and its derivative with respect to Sr. */
static void score_real(const actx *c, double Sr, double *value, double *dval)
{
    const orc_attn *a = c->a;
    switch (a->kind) {
    case ORC_ATTN_SOFTCAP_POLY: {
        const uint16_t x = enc(&c->ft, (double)orc_mul_f32((float)Sr, c->scale));
        *value = (double)a->cap * val(&c->ft, eval_one(&c->ft, a->tanh_prog, x));
        *dval = (double)a->cap * (double)c->scale * val(&c->ft, dtanh_prog(&c->ft, a->tanh_prog, x));
        return;
    }
    case ORC_ATTN_SOFTCAP_EXACT: {
        const double t = tanh(Sr / ((double)a->cap * sqrt((double)a->D)));
        *value = (double)a->cap * t;
        *dval = (1.0 - t * t) * c->rsd;
        return;
    }
    case ORC_ATTN_SIGMOID_POLY: {
        const uint16_t x = orc_f64_to_bf16((double)orc_mul_f32((float)Sr, c->scale));
        uint16_t g;
        *value = orc_bf16_to_f64(sig_eval(&c->fs, a->sig, x, &g));
        *dval = orc_bf16_to_f64(g) * (double)c->scale;
        return;
    }
    default: {
        const double p = stable_sigmoid(Sr * c->rsd - c->logn);
        *value = p;
        *dval = p * (1.0 - p) * c->rsd;
        return;
    }
    }
}

/* 2^z in FP32 by the softmax's exponential: core 0 the exponential itself
 * (correctly rounded), else 2^floor(z) p(z - floor z) with the core p in
 * target precision (z clamped below at -16384).  The power of two is taken
 * relative to 2^ref (an integer). */
static double exp2_fp32(int core, float z, double ref)
{
    if (core == 0) return (double)(float)exp2((double)z - ref);
    if (z < -16384.0f) z = -16384.0f;
    const double n = floor((double)z);
    const float f = (float)((double)z - n);      /* exact */
    return (double)(float)ldexp((double)orc_exp2_core_target(core, f), (int)(n - ref));
}

/* ---- replay model: one score's rounding decisions --------------------------
 * cand_t: the softcap's tanh value t and derivative value q' for every
 * admissible program input (or comparator tanh); entry 0 is the primary. */
typedef struct { int n; double t[XC_MAX + 2], d[XC_MAX + 2]; } tcands;

static void softcap_cands(const actx *c, double S, double A, tcands *tc)
{
    const orc_attn *a = c->a;
    const f32r s = fp32_range(S, 8.0 * U32 * A);
    const float xs0 = orc_mul_f32(s.v, c->scale);
    const float xlo = orc_mul_f32(s.lo, c->scale), xhi = orc_mul_f32(s.hi, c->scale);
    if (a->kind == ORC_ATTN_SOFTCAP_POLY) {
        uint16_t xb[XC_MAX + 2];
        tc->n = x_cands(&c->ft, xs0, xlo, xhi, xb);
        for (int i = 0; i < tc->n; i++) {
            tc->t[i] = val(&c->ft, eval_one(&c->ft, a->tanh_prog, xb[i]));
            tc->d[i] = val(&c->ft, dtanh_prog(&c->ft, a->tanh_prog, xb[i]));
        }
        return;
    }
    /* comparator: FP32 tanh within 4 ulps; q' = RN32(1 - t^2) as one FMA */
    const float t0 = (float)tanh((double)xs0);
    const float tl = ulps32((float)tanh((double)xlo), -4), th = ulps32((float)tanh((double)xhi), 4);
    const float ts[4] = {t0, tl, th, 0.0f};
    tc->n = (tl < 0.0f && th > 0.0f) ? 4 : 3;
    for (int i = 0; i < tc->n; i++) {
        tc->t[i] = ts[i];
        tc->d[i] = orc_fma_f32(-ts[i], ts[i], 1.0f);
    }
}

/* FP32 P of the candidates: primary and [lo, hi], the hardware exponential
 * taken within 1 ulp.  z = RN32(t c2 + zoff) when fused, else RN32(t c2)
 * with the result relative to 2^ref. */
static void p_range(const actx *c, const tcands *tc, int fused, float zoff, double ref,
                    double *P0, double *Plo, double *Phi)
{
    const int core = c->a->exp2_core;
    *Plo = INFINITY;
    *Phi = -INFINITY;
    for (int i = 0; i < tc->n; i++) {
        const float z = fused ? orc_fma_f32((float)tc->t[i], c->c2, zoff)
                              : orc_mul_f32((float)tc->t[i], c->c2);
        const double p = exp2_fp32(core, z, ref);
        if (i == 0) *P0 = p;
        const double lo = core ? p : (double)ulps32((float)p, -1);
        const double hi = core ? p : (double)ulps32((float)p, 1);
        if (lo < *Plo) *Plo = lo;
        if (hi > *Phi) *Phi = hi;
    }
}

static double half_spread(double v0, double lo, double hi)
{
    return fmax(v0 - lo, hi - v0);
}

/* Sigmoid attention: P (primary, range) and derivative value g (primary,
 * range) of one score. */
static void sigmoid_cands(const actx *c, double S, double A, double *P0, double *Plo,
                          double *Phi, double *g0, double *glo, double *ghi)
{
    const orc_attn *a = c->a;
    const f32r s = fp32_range(S, 8.0 * U32 * A);
    if (a->kind == ORC_ATTN_SIGMOID_POLY) {
        uint16_t xb[XC_MAX + 2];
        const int n = x_cands(&c->fs, orc_mul_f32(s.v, c->scale), orc_mul_f32(s.lo, c->scale),
                              orc_mul_f32(s.hi, c->scale), xb);
        *Plo = *glo = INFINITY;
        *Phi = *ghi = -INFINITY;
        for (int i = 0; i < n; i++) {
            uint16_t gb;
            const double p = orc_bf16_to_f64(sig_eval(&c->fs, a->sig, xb[i], &gb));
            const double g = orc_bf16_to_f64(gb);
            if (i == 0) { *P0 = p; *g0 = g; }
            *Plo = fmin(*Plo, p); *Phi = fmax(*Phi, p);
            *glo = fmin(*glo, g); *ghi = fmax(*ghi, g);
        }
        return;
    }
    /* comparator: u = RN32(S scale - ln n) as one FMA, FP32 sigma within 4
     * ulps, g = RN32(P RN32(1 - P)) */
    const float u0 = orc_fma_f32(s.v, c->scale, -c->logn32);
    const float ul = orc_fma_f32(s.lo, c->scale, -c->logn32), uh = orc_fma_f32(s.hi, c->scale, -c->logn32);
    const float p0 = (float)stable_sigmoid((double)u0);
    const float pl = ulps32((float)stable_sigmoid((double)ul), -4);
    const float ph = ulps32((float)stable_sigmoid((double)uh), 4);
    *P0 = p0; *Plo = pl; *Phi = ph;
    const float ps[4] = {p0, pl, ph, 0.5f};
    const int n = (pl < 0.5f && ph > 0.5f) ? 4 : 3;
    *glo = INFINITY;
    *ghi = -INFINITY;
    for (int i = 0; i < n; i++) {
        const double g = orc_mul_f32(ps[i], orc_add_f32(1.0f, -ps[i]));
        if (i == 0) *g0 = g;
        *glo = fmin(*glo, g);
        *ghi = fmax(*ghi, g);
    }
}

/* ---- forward ------------------------------------------------------------- */

int orc_attn_fwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const int64_t *rows, int64_t n_rows,
                      double *out, double *lse, double *spread)
{
    actx c;
    const int rc = actx_init(&c, a);
    if (rc) return rc;
    if (a->exp2_core && a->kind != ORC_ATTN_SOFTCAP_POLY) return -3;
    const int64_t S = a->S, D = a->D, G = a->H / a->Hkv;
    const int sc = is_softcap(a);
#pragma omp parallel
    {
        const size_t nb = (size_t)(S > 0 ? S : 1);
        double *w = malloc(sizeof(double) * nb);    /* weight entering P V (over l) */
        double *dw = malloc(sizeof(double) * nb);   /* its admissible half-spread */
        double *dl = malloc(sizeof(double) * nb);   /* of the term's share of l */
        tcands *tc = malloc(sizeof(tcands));
#pragma omp for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < n_rows; ri++) {
            const int64_t r = rows[ri];
            const int64_t bh = r / S, i = r % S;
            const int64_t b = bh / a->H, h = bh % a->H;
            const int64_t kvb = (b * a->Hkv + h / G) * S * D;
            const int64_t nk = a->causal ? i + 1 : S;
            double l = 1.0;
            for (int64_t j = 0; j < nk; j++) dw[j] = dl[j] = 0.0;
            if (sc && !a->replay) {
                double m = -INFINITY, dummy;
                for (int64_t j = 0; j < nk; j++) {
                    score_real(&c, dot_bf16(q + r * D, k + kvb + j * D, (int)D, NULL), &w[j], &dummy);
                    if (w[j] > m) m = w[j];
                }
                if (a->exp2_core) {
                    /* 2^floor(z) p(frac z), z = RN32(t c2), relative to the
                     * row's largest floor(z) */
                    double M = -INFINITY;
                    for (int64_t j = 0; j < nk; j++) {
                        w[j] /= (double)a->cap;
                        M = fmax(M, floor((double)orc_mul_f32((float)w[j], c.c2)));
                    }
                    l = 0.0;
                    for (int64_t j = 0; j < nk; j++) {
                        w[j] = exp2_fp32(a->exp2_core, orc_mul_f32((float)w[j], c.c2), M);
                        l += w[j];
                    }
                    if (lse) lse[ri] = (M + log2(l)) * LN2;
                } else {
                    l = 0.0;
                    for (int64_t j = 0; j < nk; j++) { w[j] = exp(w[j] - m); l += w[j]; }
                    if (lse) lse[ri] = m + log(l);
                }
            } else if (sc) {
                /* replay: FP32 P_j (fixed reference, or 2^z split relative to
                 * the row's largest floor(z)), l = sum of the FP32 P_j */
                const int fused = a->exp2_core == 0 && c.sref;
                double ref = fused ? (double)c.mref : -INFINITY;
                double *P0 = w;
                if (!fused) {
                    for (int64_t j = 0; j < nk; j++) {
                        double A;
                        const double Sr = dot_bf16(q + r * D, k + kvb + j * D, (int)D, &A);
                        softcap_cands(&c, Sr, A, tc);
                        float z = orc_mul_f32((float)tc->t[0], c.c2);
                        if (z < -16384.0f) z = -16384.0f;
                        ref = fmax(ref, floor((double)z));
                    }
                }
                l = 0.0;
                for (int64_t j = 0; j < nk; j++) {
                    double A, Plo, Phi;
                    const double Sr = dot_bf16(q + r * D, k + kvb + j * D, (int)D, &A);
                    softcap_cands(&c, Sr, A, tc);
                    p_range(&c, tc, fused, fused ? -c.mref : 0.0f, fused ? 0.0 : ref, &P0[j], &Plo, &Phi);
                    l += P0[j];
                    dl[j] = half_spread(P0[j], Plo, Phi);
                    const double pb = bf16r(P0[j]);
                    dw[j] = half_spread(pb, bf16r(Plo), bf16r(Phi));
                    w[j] = pb;
                }
                if (lse) lse[ri] = (ref + log2(l)) * LN2;
            } else {
                l = 1.0;
                for (int64_t j = 0; j < nk; j++) {
                    double A, p0, plo, phi, g0, glo, ghi;
                    const double Sr = dot_bf16(q + r * D, k + kvb + j * D, (int)D, &A);
                    if (a->replay) {
                        sigmoid_cands(&c, Sr, A, &p0, &plo, &phi, &g0, &glo, &ghi);
                        w[j] = bf16r(p0);
                        dw[j] = half_spread(w[j], bf16r(plo), bf16r(phi));
                    } else {
                        double dummy;
                        score_real(&c, Sr, &w[j], &dummy);
                    }
                }
                if (lse) lse[ri] = NAN;
            }
            for (int64_t d = 0; d < D; d++) {
                double o = 0.0, sp = 0.0;
                for (int64_t j = 0; j < nk; j++) {
                    const double vj = orc_bf16_to_f64(v[kvb + j * D + d]);
                    o += w[j] * vj;
                    sp += dw[j] * fabs(vj);
                }
                o /= l;
                sp /= l;
                if (sc && a->replay)
                    for (int64_t j = 0; j < nk; j++) sp += dl[j] * fabs(o) / l;
                out[ri * D + d] = o;
                if (spread) spread[ri * D + d] = sp;
            }
        }
        free(w);
        free(dw);
        free(dl);
        free(tc);
    }
    return 0;
}

/* ---- backward ------------------------------------------------------------ */

/* Delta_i (RN32 of it in the replay model) and its admissible half-range. */
static double row_delta(const actx *c, const uint16_t *doi, const double *oi, int D,
                        double *lo, double *hi)
{
    double s = 0.0, A = 0.0;
    for (int d = 0; d < D; d++) {
        const double p = orc_bf16_to_f64(doi[d]) * oi[d];
        s += p;
        A += fabs(p);
    }
    if (!c->a->replay) {
        *lo = *hi = s;
        return s;
    }
    const f32r r = fp32_range(s, 128.0 * U32 * A);
    *lo = r.lo;
    *hi = r.hi;
    return r.v;
}

/* P_ij and dS_ij of one pair as the products use them (BF16 in the replay
 * model) and their admissible half-spreads (0 in the real model). */
static void pair_grad(const actx *c, tcands *tc, const uint16_t *qi, const uint16_t *kj,
                      const uint16_t *vj, const uint16_t *doi, double lse_i, double delta,
                      double dlo, double dhi, double *P, double *dS, double *sP, double *sS)
{
    const orc_attn *a = c->a;
    const int D = a->D;
    double A, AdP;
    const double Sr = dot_bf16(qi, kj, D, &A);
    const double dP = dot_bf16(doi, vj, D, &AdP);
    *sP = *sS = 0.0;
    if (!a->replay) {
        double val, dval;
        score_real(c, Sr, &val, &dval);
        if (is_softcap(a)) {
            *P = exp(val - lse_i);
            *dS = *P * (dP - delta) * dval;
        } else {
            *P = val;
            *dS = dP * dval;
        }
        return;
    }
    const f32r dp = fp32_range(dP, 8.0 * U32 * AdP);
    double P0, Plo, Phi, d0, dlo_, dhi_;
    if (is_softcap(a)) {
        softcap_cands(c, Sr, A, tc);
        const float nl = -orc_mul_f32((float)lse_i, (float)LOG2E);
        p_range(c, tc, 1, nl, 0.0, &P0, &Plo, &Phi);
        d0 = tc->d[0];
        dlo_ = dhi_ = d0;
        for (int i = 1; i < tc->n; i++) { dlo_ = fmin(dlo_, tc->d[i]); dhi_ = fmax(dhi_, tc->d[i]); }
        /* dS = RN32(q' RN32(P RN32(dP - Delta))) */
        const float u0 = orc_add_f32(dp.v, -(float)delta);
        const float ul = orc_add_f32(dp.lo, -(float)dhi), uh = orc_add_f32(dp.hi, -(float)dlo);
        const float ds0 = orc_mul_f32((float)d0, orc_mul_f32((float)P0, u0));
        double sl = INFINITY, sh = -INFINITY;
        const double pc[2] = {Plo, Phi}, uc[2] = {ul, uh}, dc[2] = {dlo_, dhi_};
        for (int x = 0; x < 2; x++)
            for (int y = 0; y < 2; y++)
                for (int z = 0; z < 2; z++) {
                    const double ds = orc_mul_f32((float)dc[z], orc_mul_f32((float)pc[x], (float)uc[y]));
                    sl = fmin(sl, ds);
                    sh = fmax(sh, ds);
                }
        *dS = bf16r(ds0);
        *sS = half_spread(*dS, bf16r(sl), bf16r(sh));
        *P = bf16r(P0);
        *sP = half_spread(*P, bf16r(Plo), bf16r(Phi));
        return;
    }
    /* sigmoid: dS = RN32(dP g) */
    sigmoid_cands(c, Sr, A, &P0, &Plo, &Phi, &d0, &dlo_, &dhi_);
    const float ds0 = orc_mul_f32(dp.v, (float)d0);
    double sl = INFINITY, sh = -INFINITY;
    const double uc[2] = {dp.lo, dp.hi}, gc[2] = {dlo_, dhi_};
    for (int x = 0; x < 2; x++)
        for (int y = 0; y < 2; y++) {
            const double ds = orc_mul_f32((float)uc[x], (float)gc[y]);
            sl = fmin(sl, ds);
            sh = fmax(sh, ds);
        }
    *dS = bf16r(ds0);
    *sS = half_spread(*dS, bf16r(sl), bf16r(sh));
    *P = bf16r(P0);
    *sP = half_spread(*P, bf16r(Plo), bf16r(Phi));
}

int orc_attn_bwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const double *o, const uint16_t *dout,
                      const double *lse, const int64_t *qrows, int64_t nq,
                      const int64_t *krows, int64_t nk, double *dq, double *dk,
                      double *dv, double *sp_dq, double *sp_dk, double *sp_dv)
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
#pragma omp parallel
    {
        tcands *tc = malloc(sizeof(tcands));
#pragma omp for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < nq; ri++) {
            const int64_t r = qrows[ri];
            const int64_t bh = r / S, i = r % S;
            const int64_t b = bh / a->H, h = bh % a->H;
            const int64_t kvb = (b * a->Hkv + h / G) * S * D;
            double dlo = 0.0, dhi = 0.0;
            const double delta = sc ? row_delta(&c, dout + r * D, o + r * D, (int)D, &dlo, &dhi) : 0.0;
            const double li = sc ? lse[r] : 0.0;
            const int64_t n = a->causal ? i + 1 : S;
            for (int64_t d = 0; d < D; d++) {
                dq[ri * D + d] = 0.0;
                if (sp_dq) sp_dq[ri * D + d] = 0.0;
            }
            for (int64_t j = 0; j < n; j++) {
                double P, dS, sP, sS;
                pair_grad(&c, tc, q + r * D, k + kvb + j * D, v + kvb + j * D, dout + r * D, li,
                          delta, dlo, dhi, &P, &dS, &sP, &sS);
                for (int64_t d = 0; d < D; d++) {
                    const double kd = orc_bf16_to_f64(k[kvb + j * D + d]);
                    dq[ri * D + d] += dS * kd;
                    if (sp_dq) sp_dq[ri * D + d] += sS * fabs(kd);
                }
            }
            for (int64_t d = 0; d < D; d++) {
                dq[ri * D + d] *= fin;
                if (sp_dq) sp_dq[ri * D + d] *= fin;
            }
        }
        free(tc);
    }
    /* dK, dV rows: key row r = (b Hkv + hk) S + j */
#pragma omp parallel
    {
        tcands *tc = malloc(sizeof(tcands));
#pragma omp for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < nk; ri++) {
            const int64_t r = krows[ri];
            const int64_t bk = r / S, j = r % S;
            const int64_t b = bk / a->Hkv, hk = bk % a->Hkv;
            for (int64_t d = 0; d < D; d++) {
                dk[ri * D + d] = dv[ri * D + d] = 0.0;
                if (sp_dk) sp_dk[ri * D + d] = 0.0;
                if (sp_dv) sp_dv[ri * D + d] = 0.0;
            }
            for (int64_t h = hk * G; h < (hk + 1) * G; h++) {
                const int64_t qb = (b * a->H + h) * S;
                for (int64_t i = a->causal ? j : 0; i < S; i++) {
                    const int64_t qr = qb + i;
                    double dlo = 0.0, dhi = 0.0;
                    const double delta =
                        sc ? row_delta(&c, dout + qr * D, o + qr * D, (int)D, &dlo, &dhi) : 0.0;
                    double P, dS, sP, sS;
                    pair_grad(&c, tc, q + qr * D, k + r * D, v + r * D, dout + qr * D,
                              sc ? lse[qr] : 0.0, delta, dlo, dhi, &P, &dS, &sP, &sS);
                    for (int64_t d = 0; d < D; d++) {
                        const double qd = orc_bf16_to_f64(q[qr * D + d]);
                        const double gd = orc_bf16_to_f64(dout[qr * D + d]);
                        dk[ri * D + d] += dS * qd;
                        dv[ri * D + d] += P * gd;
                        if (sp_dk) sp_dk[ri * D + d] += sS * fabs(qd);
                        if (sp_dv) sp_dv[ri * D + d] += sP * fabs(gd);
                    }
                }
            }
            for (int64_t d = 0; d < D; d++) {
                dk[ri * D + d] *= fin;
                if (sp_dk) sp_dk[ri * D + d] *= fin;
            }
        }
        free(tc);
    }
    return 0;
}
