/*
 * polyact.h -- C ABI of the MI355X (gfx950) polynomial activation library.
 *
 * Short polynomial programs replace sigmoid, tanh, SiLU and exact GELU in the
 * forward pass and the sigmoid / tanh derivatives in the backward pass, as in
 * "Fast Polynomial Transcendentals for LLMs" (arXiv 2610.00049):
 *   - range reduction t = |x|, runtime clamp t^ = min(t, Lc)   (section 3.1, Eq. 2)
 *   - centered-odd sigmoid 1/2 + sign(x) p(t^), odd tanh        (Eq. 3)
 *   - SiLU / GELU as x/2 + t p(t^), t unclamped                 (Eqs. 4-6)
 *   - even direct derivative fits q(t^) for sigmoid', tanh'     (section 3.3)
 *   - Horner chains with BF16-rounded coefficients, one rounding per
 *     multiply-add in the target format, in deployed order     (section 3.2)
 *   - the same D3 sigmoid inside a fused SwiGLU forward / backward
 *     (section 3.3, section 3.4, Eq. 15) over dense or expert-grouped rows
 *   - the D4 tanh as the softcap alpha tanh(x / alpha) on attention logits
 *     inside a flash-attention forward, and its analytic derivative (a D3)
 *     in the backward (Eq. 1, Eq. 12, sections 3.3 and 5.2.2), in BF16 as
 *     the pages run it (section 3.4) or in packed FP16; the softmax's
 *     exponentials optionally by a software exp2 core (Appendix B.1)
 *   - sigmoid attention P = sigma(s - ln n) (Eq. 14) with the two-region
 *     cubic and its factored derivative surrogate of section 3.4, forward
 *     and backward.
 *
 * Arithmetic.  FP16 programs run on packed FP16 FMA (one IEEE rounding per
 * stage).  gfx950 has no packed BF16 FMA, so BF16 programs run each stage as
 * an FP32 FMA followed by round-to-nearest-even to BF16 (two roundings per
 * stage; pa_program.order = PA_ORDER_F32FMA_BF16).
 *
 * Special values.  NaN in -> the same NaN with its quiet bit set; +-inf is
 * clamped like any large input (sigmoid(+inf) = 1/2 + p(Lc)); SiLU / GELU map
 * -inf to -0 and +inf to +inf; signed zeros follow IEEE arithmetic of the
 * deployed sequence.  Backward: NaN x or NaN upstream gradient -> that NaN,
 * quieted.  Subnormals are preserved (no flush to zero).
 *
 * Conventions for every entry point below.
 *   Ownership  all data pointers are DEVICE pointers owned by the caller; the
 *              library never allocates, frees or retains caller memory and has
 *              no mutable global state (the program table is read-only).
 *   Streams    work is enqueued on `stream` (0 = the default stream) and runs
 *              asynchronously; nothing synchronises the device.
 *   Errors     argument errors are detected on the host before any launch and
 *              returned synchronously; nothing is enqueued then.  A failed
 *              launch returns PA_ERR_LAUNCH.  n == 0 (or rows == 0) returns
 *              PA_OK without a launch; negative sizes return PA_ERR_SHAPE.
 *   Layout     element arrays are contiguous 16-bit values (FP16 or BF16);
 *              pointers must be 2-byte aligned (PA_ERR_ALIGN otherwise).  The
 *              16-byte vector path runs on the aligned middle of the range;
 *              any misaligned head or ragged tail takes a scalar path.
 *   Aliasing   an output may alias an input exactly (same pointer); partial
 *              overlap of an output with any other buffer is PA_ERR_OVERLAP.
 */
#ifndef POLYACT_H
#define POLYACT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (the same typedef as hip_runtime_api.h). */
typedef struct ihipStream_t *hipStream_t;

#define PA_ABI_VERSION 5

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,     /* a required pointer is NULL                      */
    PA_ERR_SHAPE = 2,    /* negative size, ld < cols, bad head dimension ... */
    PA_ERR_DTYPE = 3,    /* unknown pa_dtype or dtype not supported here    */
    PA_ERR_FUNC = 4,     /* unknown pa_func / pa_impl or no such program    */
    PA_ERR_OVERLAP = 5,  /* an output partially overlaps another buffer     */
    PA_ERR_LAUNCH = 6,   /* the kernel launch failed (hipGetLastError)      */
    PA_ERR_ALIGN = 7     /* a pointer is not 2-byte aligned                 */
} pa_status;

/* The functions take the codes below as int32_t, so a caller may pass any
 * value: an unknown one is reported (PA_ERR_DTYPE / PA_ERR_FUNC), never
 * acted on.  The enums name the valid codes. */
typedef enum { PA_F16 = 1, PA_BF16 = 2 } pa_dtype;
typedef enum { PA_SIGMOID = 1, PA_TANH = 2, PA_SILU = 3, PA_GELU = 4 } pa_func;

/* Comparator implementations (the "native" path the programs replace).
 *   PA_IMPL_NATIVE         accurate FP32 evaluation from x: expf / tanhf / erfcf
 *                          without fast-math and an IEEE divide (for the
 *                          backward: the derivative recomputed from x);
 *   PA_IMPL_NATIVE_FROM_Y  backward from the saved forward output y:
 *                          g y (1 - y) for sigmoid, g (1 - y^2) for tanh
 *                          (Eqs. 10-11; the paper's native backward). */
typedef enum { PA_IMPL_POLY = 0, PA_IMPL_NATIVE = 1, PA_IMPL_NATIVE_FROM_Y = 2 } pa_impl;

/* Rounding order of a program (see "Arithmetic" above). */
typedef enum { PA_ORDER_F16_FMA = 1, PA_ORDER_F32FMA_BF16 = 3 } pa_order;

/* A deployed program: y = reconstruct(Horner(c_D..c_0, min(|x|, Lc))).
 * coeff_bits[j] is the BF16 bit pattern of the monomial coefficient c_j of
 * t^j, j = 0..degree (entries above degree are 0).  The FP16 path uses the
 * same values, each exactly representable in FP16. */
typedef struct {
    int32_t func;          /* pa_func                                        */
    int32_t deriv;         /* 0 forward program, 1 direct derivative program,
                              2 analytic derivative of the forward program
                              (PA_TANH only: the softcap attention backward;
                              coeff_bits are (j + 1) c_{j+1} as FP16 bit
                              patterns for PA_F16, exact, or rounded to BF16
                              for PA_BF16)                                  */
    int32_t degree;        /* D                                              */
    int32_t dtype;         /* pa_dtype the info was requested for            */
    float Li;              /* fit interval [0, Li] (section 3.2)             */
    float Lc;              /* runtime clamp                                  */
    uint16_t coeff_bits[8];
    int32_t order;         /* pa_order used for dtype                        */
} pa_program;

/* The two-region sigmoid-attention program (see poly_sigmoid_attn_fwd). */
typedef struct {
    int32_t n;                 /* sequence length the coefficients hold for */
    uint16_t thr;              /* region threshold (BF16)                   */
    uint16_t clamp_lo, clamp_hi;
    uint16_t coeff_bits[2][4]; /* [region][j], BF16                         */
    uint16_t a_bits[2], b_bits[2];
    int32_t order;             /* PA_ORDER_F32FMA_BF16                      */
} pa_sigmoid_attn_program;

/* The paired sine / cosine program of the rotary embedding (BF16 bit
 * patterns, see poly_rope): sin(pi u) ~ u (a1 + a3 u^2 + a5 u^4),
 * cos(pi u) ~ b0 + b2 u^2 + b4 u^4 + b6 u^6. */
typedef struct {
    uint16_t sin_bits[3];      /* a1, a3, a5     */
    uint16_t cos_bits[4];      /* b0, b2, b4, b6 */
} pa_rope_program;

/* y[i] = f~(x[i]), i < n.  f = PA_SIGMOID (D3), PA_TANH (D4), PA_SILU (D3,
 * reusing the sigmoid polynomial), PA_GELU (D5).  x, y: n elements of
 * dtype t.  Paper: section 3.1, Eqs. 2-6; Table 2 programs. */
pa_status poly_act_fwd(int32_t f, int32_t t, const void *x, void *y, int64_t n,
                       hipStream_t stream);

/* dx[i] = dy[i] * f~'(x[i]) with the direct derivative fit of f, evaluated
 * from x.  f = PA_SIGMOID or PA_TANH: an even D4 polynomial q(t^) (section
 * 3.3; section 4.2 backward from x; Table 3).  f = PA_SILU (D3) or PA_GELU
 * (D5): the centered-odd form 1/2 + sign(x) q(t^), which keeps
 * f~'(x) + f~'(-x) = 1 (Eq. 9); dx = RN(dy * RN(1/2 + (q xor sign))). */
pa_status poly_act_bwd(int32_t f, int32_t t, const void *x, const void *dy,
                       void *dx, int64_t n, hipStream_t stream);

/* Fused SwiGLU forward, BF16 only: h = SiLU~(g) * u with SiLU~(g) = g p(g)
 * and p the D3 sigmoid program (section 3.3, Eq. 15); p in BF16 (FP32 FMA +
 * BF16 rounding per stage), then h = RN_bf16(RN_f32(g p) * u) in FP32.
 * Matrices are row-major [rows x cols] with leading dimensions (elements).
 * Dense mode: row_offsets == NULL, rows [0, rows) are processed.
 * Grouped mode: row_offsets is a DEVICE int64 array of n_groups + 1
 * monotone offsets of an expert-sorted buffer; the kernel reads it on the
 * device and processes rows [row_offsets[0], row_offsets[n_groups]),
 * clipped to [0, rows): `rows` is the buffer's capacity, so the caller never
 * synchronises to learn the routed row count.  Rows outside are untouched. */
pa_status poly_swiglu_fwd(int32_t t, const void *gate, const void *up, void *h,
                          int64_t rows, int64_t cols, int64_t ld_gate, int64_t ld_up,
                          int64_t ld_h, const int64_t *row_offsets, int32_t n_groups,
                          hipStream_t stream);

/* Fused SwiGLU backward, BF16 only, both input gradients in one pass
 * (section 3.3: recompute p = sigma~(g); SiLU~' = p + g p (1 - p)):
 *   ds = RN_f32(g p (1 - p) + p),  dup = RN_bf16(dh * RN_f32(g p)),
 *   dgate = RN_bf16(RN_f32(RN_f32(dh u) * ds)).
 * Row selection as in poly_swiglu_fwd. */
pa_status poly_swiglu_bwd(int32_t t, const void *gate, const void *up, const void *dh,
                          void *dgate, void *dup, int64_t rows, int64_t cols,
                          int64_t ld_gate, int64_t ld_up, int64_t ld_dh,
                          int64_t ld_dgate, int64_t ld_dup, const int64_t *row_offsets,
                          int32_t n_groups, hipStream_t stream);

/* ---- attention (BF16 in/out, FP32 accumulation on MFMA, D = 128) -------
 * Layout: q, o, dout, dq: [B, H, S, D]; k, v, dk, dv: [B, Hkv, S, D], all
 * contiguous BF16 and 16-byte aligned; H must be a multiple of Hkv (query head
 * h uses key/value head h / (H / Hkv): grouped-query attention; Hkv = H is
 * plain multi-head attention).  D must be 128; 0 <= S <= 2^31 - 257 (the
 * kernels' tile counts stay in int32); causal != 0 masks
 * key j from query i when j > i.  lse and workspace: [B, H, S] FP32, 4-byte
 * aligned.  No output may overlap another output or an input
 * (PA_ERR_OVERLAP).  B * H * ceil(S / 128) must fit in int32. */

/* Softcapped attention forward, the pages' B2 program in BF16:
 *   S = Q K^T (FP32);  x = RN_bf16(RN_f32(S) * RN_f32(1 / (cap sqrt(D))));
 *   t = the D4 tanh program on x, each Horner stage an FP32 FMA rounded to
 *   BF16, t^ = min(|x|, Lc), sign restored;  s = cap t;  causal mask;
 *   P = softmax(s) in FP32 with exp2 (log2 e folded into RN_f32(cap log2 e));
 *   O = P V / l with P rounded to BF16 for the product, l the FP32 row sum.
 * The softmax runs against a fixed reference ceil(RN_f32(cap log2 e) - 40)
 * when cap log2 e <= 80 (every logit is bounded by cap, so all P stay normal
 * FP32), else against an integer running reference with 2^z evaluated as
 * 2^floor(z) 2^(z - floor z).
 * lse (nullable): the natural log-sum-exp of each row's softcapped logits,
 *   the input the backward needs.  cap > 0 and finite.
 * Paper: Eq. 1, section 3.4 (BF16 integrations), section 5.2.2 (the D4 tanh
 * softcap inside attention). */
pa_status poly_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                                int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D, float cap,
                                int32_t causal, hipStream_t stream);

/* The same with the tanh program in packed FP16 (the isolated sweep's
 * format, section 3.4): x = RN_f16(RN_f32(S) * RN_f32(1 / (cap sqrt(D)))), the
 * BF16-fitted coefficients as FP16 values, one FP16 rounding per stage. */
pa_status poly_softcap_attn_fwd_f16(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                    int32_t D, float cap, int32_t causal, hipStream_t stream);

/* poly_softcap_attn_fwd with the softmax's exponentials by a software exp2
 * (Appendix B.1, Eqs. 16-19): 2^z = 2^n p(f) with n = floor(z), f = z - n
 * in [0, 1), z = RN_f32(t * RN_f32(cap log2 e)) clamped below at -16384, and
 * the running reference kept an integer so that every rescale is an exact
 * power of two and the normalised weights do not depend on it.  Cores:
 *   PA_EXP2_HW     v_exp_f32 (the same kernel as poly_softcap_attn_fwd)
 *   PA_EXP2_D1     p = 1 + f (FP32)
 *   PA_EXP2_PWL2   p = 1 + a f + 2 (1 - a) max(f - 1/2, 0), a = 0.7978515625,
 *                  2 (1 - a) = 0.40380859375, packed FP16 (f rounded to FP16)
 *   PA_EXP2_D2     p = 1 + a f + (1 - a) f^2, a = RN_f32(0.6602339719), FP32 FMA
 *   PA_EXP2_D3     1 + 0.6951461434 f + 0.2275643945 f^2 + 0.0771190897 f^3
 *                  (the pages' reference cubic; p(1) != 2), FP32 FMA
 * D1, PWL2 and D2 keep p(0) = 1 and p(1) = 2 exactly after rounding (the
 * invariants online softmax needs).  lse as for poly_softcap_attn_fwd, with
 * the approximate exponentials.  Unknown core: PA_ERR_FUNC. */
typedef enum { PA_EXP2_HW = 0, PA_EXP2_D1 = 1, PA_EXP2_PWL2 = 2, PA_EXP2_D2 = 3,
               PA_EXP2_D3 = 4 } pa_exp2_core;
pa_status poly_softcap_attn_fwd_exp2(const void *q, const void *k, const void *v, void *o,
                                     float *lse, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                     int32_t D, float cap, int32_t causal, int32_t core,
                                     hipStream_t stream);

/* Softcapped attention backward of poly_softcap_attn_fwd: given the
 * forward's O and lse and the upstream gradient dout, writes dq, dk, dv:
 *   P = exp2(RN_f32(t RN_f32(cap log2 e) - RN_f32(lse log2 e))) recomputed
 *   with the forward's program;  dV = P^T dO;  dP = dO V^T;
 *   Delta_i = dO_i . O_i;  dS = RN_f32(q'(x) RN_f32(P RN_f32(dP - Delta)));
 *   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D) (summed over the query heads
 *   of a group),
 * where q'(x) is the analytic derivative of the D4 tanh program, the D3 with
 * coefficients (j + 1) c_{j+1} rounded to BF16 (poly_program_info(PA_TANH, 2,
 * PA_BF16)) evaluated like the forward program at |x|, and 0 where
 * |x| > Lc (the clamped forward program is constant there).  P and dS are
 * rounded to BF16 for the MFMA.  workspace: caller-owned scratch, 16-byte
 * aligned, of pa_attn_bwd_workspace_bytes(1, B, H, Hkv, S, D) bytes: B * H * S
 * floats each for Delta and for -lse log2(e) (each region rounded up to 16
 * bytes); when H > Hkv, FP32 dK and dV partials of every query head (summed
 * per group by a final pass in a fixed order); and, while they fit the limit
 * of pa_attn_bwd_ds_limit, the BF16 dS of every 32 x 32 block (B H x
 * 4 ceil(S/128) x ceil(S/32) x 2 KiB), which the dK/dV kernel stores so
 * that dQ is one product over them instead of a second pass of S, dP and
 * the transform (the same dQ either way); contents on return unspecified.
 * Paper: Eq. 12 and section 5.2.2 (the differentiated D3 at the recomputed
 * scaled score), section 3.3 (differentiated-polynomial backward). */
pa_status poly_softcap_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                float *workspace, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                int32_t D, float cap, int32_t causal, hipStream_t stream);

/* Backward of poly_softcap_attn_fwd_f16: the FP16 program and its FP16
 * derivative (coefficients exact in FP16; poly_program_info(PA_TANH, 2,
 * PA_F16)), 0 beyond the clamp; otherwise as poly_softcap_attn_bwd. */
pa_status poly_softcap_attn_bwd_f16(const void *q, const void *k, const void *v, const void *o,
                                    const void *dout, const float *lse, void *dq, void *dk,
                                    void *dv, float *workspace, int32_t B, int32_t H, int32_t Hkv,
                                    int32_t S, int32_t D, float cap, int32_t causal,
                                    hipStream_t stream);

/* Backward of poly_softcap_attn_fwd_exp2: P recomputed as 2^z with
 * z = RN_f32(t RN_f32(cap log2 e) - RN_f32(lse log2 e)) through the same exp2
 * core (2^floor(z) p(z - floor z)); otherwise as poly_softcap_attn_bwd.
 * Paper: Appendix B.1 (the cores inside the attention's forward and
 * backward). */
pa_status poly_softcap_attn_bwd_exp2(const void *q, const void *k, const void *v, const void *o,
                                     const void *dout, const float *lse, void *dq, void *dk,
                                     void *dv, float *workspace, int32_t B, int32_t H, int32_t Hkv,
                                     int32_t S, int32_t D, float cap, int32_t causal, int32_t core,
                                     hipStream_t stream);

/* poly_softcap_attn_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, serving loops,
 * harnesses that forbid allocation).  The scratch lives in one device array
 * of pa_attn_bwd_static_scratch_bytes() bytes (8 MiB) inside the library,
 * held by each GPU the library runs on until the process ends.  It runs the
 * recompute form of the backward (no stored dS blocks), whose scratch is
 * Delta and -lse log2(e) per query row and, with grouped heads, the FP32
 * dK / dV partials; shapes whose scratch exceeds the array return
 * PA_ERR_SHAPE (for example B H S <= 1,048,576 query rows when H == Hkv, and
 * B H S <= 8,128 rows with grouped heads).  The call allocates nothing.  Every
 * call on a GPU shares that GPU's array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  Results equal poly_softcap_attn_bwd's (bit for bit: both forms
 * give the same bits). */
pa_status poly_softcap_attn_bwd_static(const void *q, const void *k, const void *v,
                                       const void *o, const void *dout, const float *lse,
                                       void *dq, void *dk, void *dv, int32_t B, int32_t H,
                                       int32_t Hkv, int32_t S, int32_t D, float cap,
                                       int32_t causal, hipStream_t stream);

/* Size in bytes of poly_softcap_attn_bwd_static's device scratch array. */
int64_t pa_attn_bwd_static_scratch_bytes(void);

/* Sigmoid attention forward, O = P V with P = sigma(s - ln n) and
 * s = q.k / sqrt(D) (Eq. 14), n = S.  The program: x = RN_bf16(RN_f32(S_ij) *
 * RN_f32(1 / sqrt D)); region r = (x >= 1.25); x clamped to [-6, 6]; one
 * cubic per region with ln n and 1/n folded into its BF16 coefficients,
 * Horner with an FP32 FMA rounded to BF16 per stage; P = max(value, 0), used
 * directly (no normalisation).  The coefficients hold for n = 4096 only: any
 * other S > 0 returns PA_ERR_SHAPE (the runtime length guard).  The constants
 * are those printed for the paper's B3 evaluator (poly_sigmoid_attn_program).
 * Paper: section 3.4, section 5.2.3 (Eq. 14), Appendix C (Listing 1). */
pa_status poly_sigmoid_attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                                int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                hipStream_t stream);

/* Sigmoid attention backward: dV = P^T dO, dP = dO V^T, dS = dP g,
 * dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D), with g the factored derivative
 * surrogate P~(x) (a + b x) of the same region and clamped x (BF16 per
 * stage).  Same length guard.  workspace: as for the softcap backward,
 * pa_attn_bwd_workspace_bytes(0, ...) bytes; with H == Hkv NULL is allowed
 * too and selects the recompute form, which needs none.  Paper: section 3.4 (the coupled value / derivative
 * evaluator), Appendix C (Listing 2). */
pa_status poly_sigmoid_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                                void *dq, void *dk, void *dv, float *workspace, int32_t B,
                                int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                hipStream_t stream);

/* ---- rotary position embedding (FP16 in/out) ---------------------------- */

/* Rotary embedding of Q and K with the paired sine / cosine programs of the
 * paper's Appendix B.2 (the fused RoPE experiment).  For frequency
 * i < D / 2, w_i = base^(-2 i / D) and the host-side turn increment
 * inc_i = round(w_i 2^32 / (2 pi)) (a Q0.32 fraction of a turn); at position
 * s (0 .. S - 1) the phase is (s inc_i) mod 2^32, its top 16 bits read as a
 * signed integer v give the Q15 half-turn coordinate (angle pi v / 2^15), and
 * u = RN16(v) 2^-15, w = RN16(u u),
 *   sin = RN16(u RN16(fma(RN16(fma(a5, w, a3)), w, a1)))          (D5)
 *   cos = RN16(fma(RN16(fma(RN16(fma(b6, w, b4)), w, b2)), w, b0)) (D6)
 * with the coefficients of poly_rope_program, every step one packed FP16
 * operation.  Each interleaved pair (x_{2i}, x_{2i+1}) of a head row turns by
 * that angle: y0 = RN16(x0 cos - RN16(x1 sin)), y1 = RN16(x1 cos +
 * RN16(x0 sin)).  q: [B, S, Hq, D], k: [B, S, Hkv, D] FP16 in; q_out:
 * [B, Hq, S, D], k_out: [B, Hkv, S, D] FP16 out (transposed, as the
 * appendix's fused kernel writes them).  D a multiple of 8, 8 <= D <= 512;
 * base finite and >= 1.  All pointers device memory, 16-byte aligned, the
 * outputs overlapping no input.  Errors: PA_ERR_NULL, PA_ERR_ALIGN,
 * PA_ERR_SHAPE, PA_ERR_OVERLAP, PA_ERR_LAUNCH. */
pa_status poly_rope(const void *q, const void *k, void *q_out, void *k_out, int32_t B, int32_t S,
                    int32_t Hq, int32_t Hkv, int32_t D, double base, hipStream_t stream);

/* The same with accurate FP32 sinf / cosf of the same angle (RN32(pi / 2^15)
 * times v), rounded to FP16, computed on the fly (the appendix's native
 * on-the-fly variant; arguments and errors as poly_rope). */
pa_status native_rope(const void *q, const void *k, void *q_out, void *k_out, int32_t B, int32_t S,
                      int32_t Hq, int32_t Hkv, int32_t D, double base, hipStream_t stream);

/* The appendix's cached-table variant: table holds S * D / 2 words, word
 * s * D / 2 + i = (cos, sin) of frequency i at position s as two FP16 values
 * (cos in the low half), as pa_rope_table writes them; arguments and errors
 * otherwise as poly_rope (table 16-byte aligned, not overlapping the
 * outputs). */
pa_status native_rope_table(const void *q, const void *k, void *q_out, void *k_out,
                            const void *table, int32_t B, int32_t S, int32_t Hq, int32_t Hkv,
                            int32_t D, hipStream_t stream);

/* Writes the (cos, sin) table of native_rope_table: S * D / 2 words of
 * caller-owned device memory (16-byte aligned), the values native_rope
 * computes.  Errors: PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_SHAPE, PA_ERR_LAUNCH. */
pa_status pa_rope_table(void *table, int32_t S, int32_t D, double base, hipStream_t stream);

/* ---- matched comparators (same memory path, accurate FP32 math) -------- */

/* The "native" paths every timing in the paper divides by (Table 1's caption
 * calls native the unchanged implementation of the same function in the same
 * task; section 4.2 and
 * Eq. 13 time the isolated functions against it, Table 3).  They share the
 * launch shape and memory path of the poly_ entry points, so a speedup
 * measures the arithmetic alone.  Arguments, layout, ownership and errors as
 * the poly_ counterpart named beside each.
 *
 * Counterpart of poly_act_fwd: y = f(x) with accurate FP32 math (sigmoid
 * 1/(1+e^-|x|) in the overflow-safe form, tanhf, SiLU (x >= 0 ? x : x e) /
 * (1 + e) with e = expf(-|x|), GELU x erfc(-x / sqrt 2) / 2), rounded once to
 * dtype t. */
pa_status native_act_fwd(int32_t f, int32_t t, const void *x, void *y, int64_t n,
                         hipStream_t stream);

/* Counterpart of poly_act_bwd (section 4.2's backward timing, section 3.3).
 * impl = PA_IMPL_NATIVE: x_or_y is x and the derivative is recomputed
 * accurately from x (all four functions; SiLU' = sigma (1 + x sigma(-x)),
 * GELU' = Phi + x phi); impl = PA_IMPL_NATIVE_FROM_Y: x_or_y is the saved
 * forward output y (the derivatives in terms of y, Eqs. 10-11: section 4.2's
 * native sigmoid and tanh backward), PA_SIGMOID and PA_TANH only.  PA_ERR_FUNC for another impl or function. */
pa_status native_act_bwd(int32_t impl, int32_t f, int32_t t, const void *x_or_y,
                         const void *dy, void *dx, int64_t n, hipStream_t stream);

/* SwiGLU with accurate FP32 SiLU, the native side of the B1 dense-MLP and B4
 * routed-expert components (section 4.3, Table 4, sections 5.2.1 and 5.2.4);
 * arguments as poly_swiglu_fwd / _bwd. */
pa_status native_swiglu_fwd(int32_t t, const void *gate, const void *up, void *h,
                            int64_t rows, int64_t cols, int64_t ld_gate, int64_t ld_up,
                            int64_t ld_h, const int64_t *row_offsets, int32_t n_groups,
                            hipStream_t stream);
pa_status native_swiglu_bwd(int32_t t, const void *gate, const void *up, const void *dh,
                            void *dgate, void *dup, int64_t rows, int64_t cols,
                            int64_t ld_gate, int64_t ld_up, int64_t ld_dh,
                            int64_t ld_dgate, int64_t ld_dup, const int64_t *row_offsets,
                            int32_t n_groups, hipStream_t stream);

/* Attention comparators, the native side of the B2 softcap and B3 sigmoid
 * attention components (section 4.3, Table 4, sections 5.2.2 and 5.2.3);
 * arguments as the poly_ entry points: softcap with accurate FP32 tanhf on
 * the unrounded FP32 scaled score (Eq. 1) and, backward, 1 - tanh^2 (Eq. 12);
 * sigmoid with sigma(RN_f32(S) * RN_f32(1 / sqrt D) - RN_f32(ln S)) from expf
 * and an IEEE divide (Eq. 14), sigma (1 - sigma) backward, for any S. */
pa_status native_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                                  int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D,
                                  float cap, int32_t causal, hipStream_t stream);
pa_status native_softcap_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                  float *workspace, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                  int32_t D, float cap, int32_t causal, hipStream_t stream);
pa_status native_sigmoid_attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                                  int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                  hipStream_t stream);
pa_status native_sigmoid_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                                  void *dq, void *dk, void *dv, float *workspace, int32_t B,
                                  int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                  hipStream_t stream);

/* ---- measurement reference ---------------------------------------------- */

/* The elementwise streaming kernels with no arithmetic: y[i] = a[i] when b is
 * NULL (one read stream and one write stream, 4 bytes per 16-bit element),
 * y[i] = a[i] XOR b[i] bitwise otherwise (two read streams and one write
 * stream, 6 bytes per element).  Same launch configuration, 16-byte vector
 * body and scalar head / tail as poly_act_fwd / poly_act_bwd, so its rate is
 * the HBM rate that launch shape reaches with nothing to compute: the
 * ceiling the programs' rates are read against (no passage of the paper
 * defines it; section 4.2 reads its two endpoints as the L2-resident and the
 * HBM-streaming regime, and this is that regime's rate).  Arguments and errors as
 * poly_act_fwd (16-bit elements of any type; no dtype argument). */
pa_status pa_stream_copy(const void *a, const void *b, void *y, int64_t n, hipStream_t stream);

/* ---- host-only queries (no device work) -------------------------------- */

/* The program the kernels execute for (f, deriv, t): the fitted and
 * BF16-rounded coefficients, Li and Lc of section 3.2 (Table 2 prints their
 * maximum errors), deriv = 0 forward, 1 the direct derivative fit (section
 * 3.3, Eq. 9), 2 the differentiated D4 tanh the softcap backward uses (Eq. 12)
 * in the format t.  Returns PA_ERR_FUNC if there is none, PA_ERR_NULL if out
 * is NULL. */
pa_status poly_program_info(int32_t f, int32_t deriv, int32_t t, pa_program *out);

/* The sigmoid-attention program printed in the paper's Appendix C (packed
 * PTX listings) and described in section 3.4 (BF16 bit patterns): region
 * threshold, clamp bounds, coeff_bits[r][j] = coefficient of x^j in region r
 * (r = 1 when x >= thr), derivative factor a_bits[r] + b_bits[r] x, and the
 * sequence length n it holds for.  Returns PA_ERR_NULL if out is NULL. */
pa_status poly_sigmoid_attn_program(pa_sigmoid_attn_program *out);

/* The paired sine / cosine program poly_rope evaluates (Appendix B.2; fitted
 * like the other programs, section 3.2 and Eq. 8, with sin(pi) = 0,
 * cos(0) = 1 and cos(pi) = -1 imposed).  Returns PA_ERR_NULL if out is NULL. */
pa_status poly_rope_program(pa_rope_program *out);

/* Bytes of caller-owned workspace an attention backward needs (softcap != 0
 * for the softcap backward, 0 for sigmoid); -1 for an invalid shape.  The
 * paper defines the gradients (Eq. 12, section 3.3), not their storage: the
 * workspace is this library's split of the backward into kernels (the row
 * terms Delta and -lse log2 e, FP32 dK / dV partials per query head when
 * Hkv < H, and the stored dS blocks while their B H x 4 ceil(S/128) x
 * ceil(S/32) x 2 KiB is within pa_attn_bwd_ds_limit).  The size depends on
 * the limit in force: size the workspace under the limit the call will
 * see. */
int64_t pa_attn_bwd_workspace_bytes(int32_t softcap, int32_t B, int32_t H, int32_t Hkv,
                                    int32_t S, int32_t D);

/* The process-wide limit, in bytes, on the dS blocks an attention backward
 * stores (default 16 GiB; 0 makes every backward recompute S, dP and the
 * transform for dQ instead).  bytes >= 0 sets it and returns the previous
 * value; bytes < 0 only returns it.  Results do not depend on it; the
 * workspace size does, so a caller that raises it must size workspaces
 * after the change (a workspace sized under a higher limit serves any lower
 * one).  A storage choice of this library, not a passage of the paper. */
int64_t pa_attn_bwd_ds_limit(int64_t bytes);

/* Static description of a status code. */
const char *pa_status_str(pa_status s);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* POLYACT_H */
