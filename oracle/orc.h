/*
 * orc.h -- plain CPU oracle for the polynomial activation programs of
 * "Fast Polynomial Transcendentals for LLMs" (arXiv 2610.00049).
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load or call it.  The product
 * path (the HIP library and its Python binding) never does, and this code
 * shares nothing with it: no headers, no helpers, no tables, no generated
 * constants.  The oracle derives every coefficient itself, by the fitting
 * procedure the paper describes, and replays every operation of a program
 * with an explicitly correct rounding.
 *
 * Everything is written for clarity, not speed: each value is decoded to an
 * exact number, each operation is computed exactly (or with a library routine
 * that is correctly rounded by definition, e.g. C99 fmaf), and the result is
 * rounded once, to nearest-even, by a routine written from the definition of
 * the binary format.
 *
 * Pins (tests/test_oracle_*.py): formats against numpy / torch and exact
 * rationals; the fit against Table 2's printed sigmoid-derivative D4 bound
 * (reproduced bit for bit) and the least-squares normal equations; replay
 * against rounding-error bounds and the symmetry identities; attention rows
 * against a textbook FP64 attention, attention gradients against automatic
 * differentiation of textbook FP64 attention, the sigmoid-attention program
 * against sigma(s - ln n); the rotary embedding against an independent
 * least-squares solve, big-integer phases and an exact rational FP16 replay.
 * Parity unpinned: the selection of the
 * GELU D5 program (Table 2's 1.06e-3 is not reached under any reading) and of
 * the tanh-derivative D4 program (no printed value).
 */
#ifndef ORC_H
#define ORC_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Functions (paper section 3.1 / 3.3). */
enum { ORC_SIGMOID = 1, ORC_TANH = 2, ORC_SILU = 3, ORC_GELU = 4 };

/* Rounding orders used to replay a program (paper section 3.2, steps 4-5 and
 * the paragraph after the step list).
 *   ORC_ORDER_F16_FMA      FP16 arithmetic, one rounding per fused multiply-add
 *                          (packed FP16 FMA semantics);
 *   ORC_ORDER_BF16_FMA     BF16 arithmetic, one rounding per fused multiply-add
 *                          (the paper's packed BF16 FMA semantics);
 *   ORC_ORDER_F32FMA_BF16  FP32 fused multiply-add rounded to FP32, then rounded
 *                          to BF16 (how a machine without a packed BF16 FMA runs
 *                          the same chain: two roundings per stage);
 *   ORC_ORDER_BF16_SPLIT   BF16 arithmetic with multiply and add rounded
 *                          separately (the paper's search emulator).          */
enum { ORC_ORDER_F16_FMA = 1, ORC_ORDER_BF16_FMA = 2, ORC_ORDER_F32FMA_BF16 = 3,
       ORC_ORDER_BF16_SPLIT = 4 };

/* A fitted program: function, direction (deriv = 1 for a direct derivative
 * fit), degree D, fit interval Li, runtime clamp Lc and the BF16 bit patterns
 * of the monomial coefficients c_0..c_D in the half-domain variable t = |x|. */
typedef struct {
    int32_t func, deriv, degree, reserved;
    double Li, Lc;
    uint16_t c[8];
} orc_prog;

/* ---- binary formats (orc_fp.c) ---------------------------------------- */
double   orc_f16_to_f64(uint16_t h);
double   orc_bf16_to_f64(uint16_t b);
uint16_t orc_f64_to_f16(double x);    /* round to nearest even */
uint16_t orc_f64_to_bf16(double x);   /* round to nearest even */
uint16_t orc_f32_to_bf16(float x);    /* round to nearest even */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_fma_f16(uint16_t a, uint16_t b, uint16_t c);   /* RN(a*b+c), exact */
uint16_t orc_fma_bf16(uint16_t a, uint16_t b, uint16_t c);  /* RN(a*b+c), exact */
uint16_t orc_fma_f32_bf16(uint16_t a, uint16_t b, uint16_t c); /* RN16(RN32(a*b+c)) */
float    orc_fma_f32(float a, float b, float c);            /* RN(a*b+c) */
float    orc_add_f32(float a, float b);
float    orc_mul_f32(float a, float b);

/* ---- functions, fitting, selection (orc_fit.c) ------------------------ */
double orc_ref(int func, int deriv, double x);        /* FP64 function value */
double orc_residual(int func, int deriv, double t);   /* half-domain target  */
int    orc_fit(int func, int deriv, int degree, double Li, double *coef);
int    orc_make_prog(int func, int deriv, int degree, double Li, double Lc,
                     orc_prog *out);
double orc_prog_real(const orc_prog *p, double x);
double orc_table2_metric(const orc_prog *p);
double orc_search_objective(const orc_prog *p, int order, int *gates_ok);
int    orc_search(int func, int deriv, int degree, double Lc_fixed, double bound,
                  int order, orc_prog *out, double *objective, double *metric);

/* ---- program replay (orc_eval.c) -------------------------------------- */
uint16_t orc_prog_eval(const orc_prog *p, uint16_t x, int order);
uint16_t orc_prog_bwd(const orc_prog *p, uint16_t x, uint16_t g, int order);
void orc_act_fwd(const orc_prog *p, int order, const uint16_t *x, uint16_t *y,
                 int64_t n);
void orc_act_bwd(const orc_prog *p, int order, const uint16_t *x,
                 const uint16_t *g, uint16_t *dx, int64_t n);
void orc_swiglu_fwd(const orc_prog *sig, const uint16_t *gate, const uint16_t *up,
                    uint16_t *h, int64_t row_begin, int64_t row_end, int64_t cols,
                    int64_t ld_gate, int64_t ld_up, int64_t ld_h);
void orc_swiglu_bwd(const orc_prog *sig, const uint16_t *gate, const uint16_t *up,
                    const uint16_t *dh, uint16_t *dgate, uint16_t *dup,
                    int64_t row_begin, int64_t row_end, int64_t cols,
                    int64_t ld_gate, int64_t ld_up, int64_t ld_dh,
                    int64_t ld_dgate, int64_t ld_dup);
/* ---- attention with a transformed score (orc_eval.c) -------------------- */
enum { ORC_ATTN_SOFTCAP_POLY = 1, ORC_ATTN_SOFTCAP_EXACT = 2,
       ORC_ATTN_SIGMOID_POLY = 3, ORC_ATTN_SIGMOID_EXACT = 4 };

/* The two-region sigmoid-attention program (section 3.4 and Appendix C,
 * Listings 1-2): BF16 bit patterns of the region threshold, the clamp bounds,
 * the cubic coefficients c[r][j] of x^j for region r (r = 1 when x >= thr) and
 * the derivative factor a[r] + b[r] x; n is the one sequence length the
 * coefficients hold for. */
typedef struct {
    int32_t n;
    uint16_t thr, lo, hi;
    uint16_t c[2][4];
    uint16_t a[2], b[2];
} orc_sig_prog;

/* Fractional cores of a software exp2 (orc_exp2.c; Appendix B.1). */
enum { ORC_EXP2_EXACT = 0, ORC_EXP2_D1 = 1, ORC_EXP2_PWL2 = 2, ORC_EXP2_D2 = 3,
       ORC_EXP2_D3 = 4 };
double orc_exp2_core(int core, double a, double f);
void   orc_exp2_errors(int core, double a, double *max_rel, double *rms_rel);
double orc_exp2_fit(int core, int minimax);
float  orc_exp2_core_target(int core, float f);

typedef struct {
    int32_t kind;              /* ORC_ATTN_*                                   */
    int32_t B, H, Hkv, S, D;   /* Q [B, H, S, D]; K, V [B, Hkv, S, D]          */
    int32_t causal;
    int32_t order;             /* replay order of the sigmoid program (0: F32FMA_BF16) */
    int32_t exp2_core;         /* softcap: ORC_EXP2_* for the softmax's 2^z (0: exact) */
    float cap;                 /* softcap alpha                                 */
    const orc_prog *tanh_prog; /* D4 tanh program (SOFTCAP_POLY)                */
    const orc_sig_prog *sig;   /* SIGMOID_POLY                                  */
    int32_t tanh_order;        /* format of the softcap program and its
                                  derivative: ORC_ORDER_F32FMA_BF16 (the pages'
                                  BF16 path; also 0) or ORC_ORDER_F16_FMA      */
    int32_t replay;            /* 0: real arithmetic around the programs (FP64
                                  scores, weights and sums);
                                  1: the method's FP32 steps (scores, scaled
                                  scores, exponent arguments, dP - Delta, dS)
                                  rounded to FP32 and P / dS rounded to BF16
                                  before the products with V / K / Q / dO;
                                  sums exact                                    */
} orc_attn;

/* Returns 0, or -1 (sequence length differs from the sigmoid program's n),
 * -2 (bad shape), -3 (unknown kind).  spread (nullable): per output, the
 * largest change admissible alternatives of the replay model's rounding
 * decisions can cause (orc_eval.c); 0 in the real-arithmetic model. */
int orc_attn_fwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const int64_t *rows, int64_t n_rows,
                      double *out, double *lse, double *spread);
int orc_attn_bwd_rows(const orc_attn *a, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const double *o, const uint16_t *dout,
                      const double *lse, const int64_t *qrows, int64_t nq,
                      const int64_t *krows, int64_t nk, double *dq, double *dk,
                      double *dv, double *sp_dq, double *sp_dk, double *sp_dv);
/* The analytic derivative of the softcap tanh program at x (bits in the
 * format of `order`): the D3 with coefficients (j + 1) c_{j+1} (exact in
 * FP16; rounded to BF16 for the BF16 program) at |x|, 0 beyond the clamp. */
uint16_t orc_dtanh_prog(const orc_prog *tanh_prog, uint16_t x, int order);
uint16_t orc_dtanh_prog_f16(const orc_prog *tanh_prog, uint16_t x);
uint16_t orc_sig_prog_eval(const orc_sig_prog *sp, uint16_t x, int order, uint16_t *grad);
int orc_threads(void);
int orc_set_threads(int n);   /* threads of later parallel loops; returns the old count */

/* ---- paired sine / cosine and rotary embedding (orc_rope.c) ----------------
 * Appendix B.2: Q0.32 turn increments, signed Q15 half-turn coordinate,
 * packed FP16 D5 sine and D6 cosine on the shared square, rotation of the
 * interleaved pairs (the readings are listed in orc_rope.c). */
typedef struct {
    uint16_t sin_c[3];   /* BF16 a1, a3, a5: sin(pi u) ~ u (a1 + a3 u^2 + a5 u^4) */
    uint16_t cos_c[4];   /* BF16 b0, b2, b4, b6: cos(pi u) ~ b0 + b2 u^2 + ...   */
} orc_rope;
int  orc_lsq(int N, int m, double *A, double *r, double *x);   /* Householder QR */
int  orc_rope_fit(double *sin_coef, double *cos_coef);          /* FP64 a1,a3,a5; b0..b6 */
int  orc_rope_prog(orc_rope *out);                              /* the BF16-rounded fit */
void orc_rope_inc(int D, double base, uint32_t *inc);           /* D/2 turn increments */
uint16_t orc_rope_coord(uint32_t phase);                        /* u = RN16(v / 2^15) */
void orc_rope_sincos(const orc_rope *rp, uint32_t phase, uint16_t *s, uint16_t *c);
void orc_rope_rotate(uint16_t x0, uint16_t x1, uint16_t s, uint16_t c, uint16_t *y0, uint16_t *y1);
void orc_rope_rows(const orc_rope *rp, const uint32_t *inc, int D, const uint16_t *x,
                   const int64_t *pos, int64_t nrows, uint16_t *y);

#ifdef __cplusplus
}
#endif
#endif
