// attn.hpp -- flash-attention forward with a transformed score, gfx950 MFMA.
//
// Two score transforms from "Fast Polynomial Transcendentals for LLMs":
//   softcap  s = cap tanh(x / cap) on the logits, then softmax (Eq. 1); the
//            polynomial variant evaluates the D4 tanh program (section 5.2.2
//            puts a packed D4 tanh inside the attention forward);
//   sigmoid  P = sigma(s - ln n), no normalisation (Eq. 14); the polynomial
//            variant evaluates the two-region cubic of section 3.4 with ln n
//            and 1 / n folded into its coefficients (one n only).
// Each has an accurate FP32 comparator (tanhf; expf and an IEEE divide).
//
// Arithmetic of the programs.  The pages run the attention integrations on
// the BF16 path (section 3.4).  gfx950 has no packed BF16 FMA, so a BF16
// program runs each Horner stage as an FP32 FMA rounded to BF16 (one
// v_cvt_pk_bf16_f32 per lane): the tanh program on x = RN_bf16(RN_f32(S) *
// RN_f32(1 / (cap sqrt D))) and the sigmoid program on x = RN_bf16(RN_f32(S) *
// RN_f32(1 / sqrt D)).  The tanh program is also offered in packed FP16
// (v_pk_fma_f16, two scores per instruction) on x = RN_f16(...), with the FP16
// values of the same BF16 coefficients: fewer VALU instructions, a different
// rounding of every stage.
//
// Layout: Q, O [B, H, S, D]; K, V [B, Hkv, S, D], H a multiple of Hkv (query
// head h reads key/value head h / (H / Hkv)); D = 128; BF16.
//
// Tiling (D = 128):
//   workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
//   queries q0 .. q0 + 31.  Blocks are numbered heaviest query tile first
//   across all heads (causal work grows with the query index).  Key/value
//   tiles of 64 rows go from HBM straight into LDS with global_load_lds_dwordx4
//   (no register staging), double buffered with one barrier per tile: tile
//   kt + 1 streams in while tile kt is consumed.  Rows are 256 B with the
//   16-byte chunks XOR-swizzled by row: chunk c of row r sits at slot
//   c ^ f(r), f(r) = 4 (r mod 4) + (r / 4 mod 4).  The row reads (16 lanes =
//   16 consecutive rows, one chunk) and the transposed reads (a half-wave =
//   4 consecutive rows x 4 consecutive chunks) then each touch 16 distinct
//   slots, i.e. all 64 banks once.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q held
//   in registers; the accumulator gives every lane one query (column) and 16
//   keys of each 32-key block, so the softmax row reductions need only a
//   swap with the lane 32 away.
//   O^T += V^T P^T: B = P^T comes straight from the score accumulator (the
//   contraction order over keys is permuted so that each lane's 8 B-operand
//   values are 8 consecutive accumulator entries); A = V^T is read from the
//   row-major V tile with ds_read_b64_tr_b16: within each 16-lane group the
//   instruction returns to lane i element (i mod 4) of the 4-element vectors
//   addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12, so lanes addressing
//   V[k0 + j/4][d0 + 4 (j mod 4)] deliver V[k0 .. k0 + 3][d0 + i] to lane i.
//   Softcap: online softmax in the log2 domain (cap * log2 e folded in).  The
//   running reference max is only moved when a row's max exceeds it by more
//   than 8 (so P <= 2^8): the O rescale (64 multiplies per lane) is skipped
//   for almost every tile and the result is unchanged up to rounding.  P is
//   rounded to BF16 for the MFMA, O^T accumulated in FP32, O = O^T / l, and
//   the natural log-sum-exp of each row is written for the backward.
//   Sigmoid: P (already BF16 for the program) goes straight into the MFMA;
//   O = O^T.
#pragma once
#include <type_traits>
#include <utility>

#include "ops.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int AT_D = 128;
constexpr int AT_BM = 128;          // queries per workgroup
constexpr int AT_BN = 64;           // keys per tile
constexpr int AT_TILE = AT_BN * AT_D;   // elements of one 64-row tile in LDS
constexpr float AT_RESCALE = 8.0f;  // log2 headroom before the reference max moves
constexpr float AT_LN2 = 0.693147180559945309f;
constexpr float AT_LOG2E = 1.442695040888963407f;

// score transforms: the softcap with the D4 tanh program in FP16 or BF16 or
// with accurate tanhf, the sigmoid with the two-region program or accurate
// sigma
enum { AM_SOFTCAP_POLY = 0, AM_SOFTCAP_NATIVE = 1, AM_SIGMOID_POLY = 2, AM_SIGMOID_NATIVE = 3,
       AM_SOFTCAP_POLY_BF16 = 4 };
__host__ __device__ constexpr bool am_softcap(int m)
{
    return m == AM_SOFTCAP_POLY || m == AM_SOFTCAP_NATIVE || m == AM_SOFTCAP_POLY_BF16;
}
__host__ __device__ constexpr bool am_softcap_poly(int m) { return m == AM_SOFTCAP_POLY || m == AM_SOFTCAP_POLY_BF16; }

// The D4 tanh program in BF16 (coefficient values as FP32) and, for the
// backward, its analytic derivative (a D3, coefficients (j + 1) c_{j+1}
// rounded to BF16); lc = Lc.
struct TanhBF16 {
    float c[5];
    float lc;
};

// two-region sigmoid program: threshold and clamp bounds as FP32 values of
// their BF16 constants; the coefficients as FP16 pairs (each BF16 coefficient
// is an FP16 value, checked at compile time), one pair of region r per word,
// so that one per-lane select fetches two of them
struct SigCoef {
    uint32_t c23[2];   // c2 (low half), c3 (high half)
    uint32_t c01[2];   // c0 (low), c1 (high)
    uint32_t ab[2];    // a (low), b (high) of the derivative surrogate
    float thr, lo, hi;
};

struct AttnArgs {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;        // softcap: natural log-sum-exp per query row (nullable)
    int32_t S, H, G;   // G = H / Hkv
    int32_t causal;
    float scale;       // softcap: RN_f32(1 / (cap sqrt D)); sigmoid: RN_f32(1 / sqrt D)
    float c2;          // softcap: RN_f32(cap * log2(e))
    float logn;        // sigmoid comparator: RN_f32(ln S)
    float mref;        // softcap, fixed reference (see SREF)
    CoefF16 tanh16;    // D4 tanh program, FP16 coefficients
    TanhBF16 tanhbf;   // the same program in BF16
    SigCoef sig;
};

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Buffer B (compile time, 0 or 1) of an LDS double buffer, held either as
// two LDS arrays (SPLIT) or as one [2][N] array.  The compiler gives every
// LDS variable its own alias scope: with two arrays it can tell that a
// global-to-LDS load into one buffer does not write what a read of the other
// buffer reads, and does not wait for the load before the read.  That frees
// the schedule (a gain where the kernel has registers to spare) but raises
// the register count (a loss, or spills, where it has none); the kernels
// choose per mode.  The unused declaration is dropped by the compiler.
template <int B, bool SPLIT, class T, int N>
__device__ __forceinline__ T *dbuf(T *b0, T *b1, T (&pair)[2][N])
{
    if constexpr (SPLIT) {
        if constexpr (B == 0) return b0;
        else return b1;
    } else {
        return pair[B];
    }
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t *p) { return *(const bf16x8 *)p; }

// slot of 16-byte chunk c of LDS row r (rows are 256 B, 16 chunks)
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 3) << 2) | ((r >> 2) & 3)); }

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3))) *)(p));
    return bc<u32x2>(r);
}

// A 64-row tile of a [rows, 128] BF16 matrix into LDS, rows past S repeating
// row S - 1 (finite data; those rows are masked).  16 wave instructions per
// tile, 4 per wave: instruction r of wave w fills LDS bytes [(4 w + r) KiB,
// +1 KiB): lane p writes slot p % 16 of row (4 w + r) * 4 + p / 16, so it
// fetches the chunk that belongs in that slot.
__device__ __forceinline__ void load_rows64(const uint16_t *src, uint16_t *lds, int row0, int S,
                                            int wave, int lane)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = (wave * 4 + r) * 4 + (lane >> 4);
        const int slot = lane & 15;
        int g = row0 + row;
        g = g < S ? g : S - 1;
        const int64_t off = (int64_t)g * AT_D + swz(row, slot) * 8;
        const int dst = __builtin_amdgcn_readfirstlane((wave * 4 + r) * 512);
        __builtin_amdgcn_global_load_lds((const void *)(src + off),
                                         (void __attribute__((address_space(3))) *)(lds + dst),
                                         16, 0, 0);
    }
}

// load_rows64 with the global-to-LDS loads issued from assembly.  The
// compiler cannot tell which buffer of a one-array LDS double buffer a
// builtin load writes, so it waits for every tile load in flight before the
// next LDS read; it does not see these loads and adds no such wait.  The
// caller waits (s_waitcnt vmcnt(0) and a barrier) before any wave reads the
// tile, and must have waited for its own earlier global loads before the
// first of these (the compiler counts only the loads it issued).  M0, the
// LDS base of the load, is saved and restored; one wait state separates its
// write from the load.
__device__ __forceinline__ void load_rows64_asm(const uint16_t *src, uint16_t *lds, int row0, int S,
                                                int wave, int lane)
{
    const uint32_t base = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = (wave * 4 + r) * 4 + (lane >> 4);
        const int slot = lane & 15;
        int g = row0 + row;
        g = g < S ? g : S - 1;
        const uint16_t *gp = src + (int64_t)g * AT_D + swz(row, slot) * 8;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (uint32_t)((wave * 4 + r) * 512) * 2u);
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(gp), "s"(dst) : "memory");
    }
}

// 8 BF16 of row `row`, chunk `chunk` of a swizzled LDS tile
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t *t, int row, int chunk)
{
    return ld_bf16x8(t + row * AT_D + swz(row, chunk) * 8);
}

// A operand (8 x 4 BF16 per lane as two tr16 reads) of X^T for the
// contraction step ks over 64 rows of a swizzled row-major tile, d block d0:
// lane (i16, g16) provides rows k0 .. k0 + 3 and k0 + 8 .. k0 + 11 of column
// d, where the contraction order matches the permuted B operand built from a
// 32x32 accumulator (see the header).
__device__ __forceinline__ bf16x8 lds_tr_a(const uint16_t *t, int ks, int db, int g16, int i16)
{
    const int d = db * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
    const int k0 = (ks >> 1) * 32 + (ks & 1) * 16 + (g16 >> 1) * 4 + (i16 >> 2);
    const u32x2 lo = ds_read_tr16(t + k0 * AT_D + swz(k0, d >> 3) * 8 + (d & 7));
    const u32x2 hi = ds_read_tr16(t + (k0 + 8) * AT_D + swz(k0 + 8, d >> 3) * 8 + (d & 7));
    const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
    return bc<bf16x8>(av);
}

// ---- score transforms on a pair of raw FP32 scores --------------------------

// softcap program: packed FP16 tanh~ of x = RN_f16(s * scale); returns the
// packed FP16 t and (through xabs) the packed |x| for the derivative program.
__device__ __forceinline__ uint32_t softcap_poly_pair(float s0, float s1, float scale,
                                                      const CoefF16 &k, uint32_t &aw)
{
    // the FP32 product rounded once to FP16 equals RN_f16(RN_f32(s * scale))
    // only through the explicit FP32 multiply (no contraction)
    h2 xh;
    xh[0] = (_Float16)fmaf(s0, scale, -0.0f);
    xh[1] = (_Float16)fmaf(s1, scale, -0.0f);
    const uint32_t xw = bc<uint32_t>(xh);
    aw = xw & 0x7FFF7FFFu;
    const h2 v = horner_f16<4, true>(bc<h2>(min_u16x2(aw, k.lc)), k);
    return bc<uint32_t>(v) ^ (xw ^ aw);
}

// softcap program in BF16 on a pair: x = RN_bf16(s * scale), x^ = x clamped
// to [-Lc, Lc] (one median of three; |x^| = min(|x|, Lc)), v = c4;
// v = RN_bf16(fma(v, |x^|, c_j)) for j = 3, 2, 1 (the absolute value is a free
// operand modifier); t = RN_bf16(v x^), which is RN_bf16(v |x^|) with x's sign
// (nearest even is symmetric; v > 0).  Returns t0, t1 (BF16 values as FP32)
// and x0, x1 (the rounded scaled scores, for the derivative program).
__device__ __forceinline__ void softcap_bf16_pair(float s0, float s1, float scale, const TanhBF16 &k,
                                                  float &t0, float &t1, float &x0, float &x1,
                                                  float &c0, float &c1)
{
    x0 = rn_bf16(s0 * scale);
    x1 = rn_bf16(s1 * scale);
    c0 = __builtin_amdgcn_fmed3f(x0, -k.lc, k.lc);
    c1 = __builtin_amdgcn_fmed3f(x1, -k.lc, k.lc);
    float v0 = rn_bf16(fmaf(k.c[4], fabsf(c0), k.c[3])), v1 = rn_bf16(fmaf(k.c[4], fabsf(c1), k.c[3]));
    v0 = rn_bf16(fmaf(v0, fabsf(c0), k.c[2]));
    v1 = rn_bf16(fmaf(v1, fabsf(c1), k.c[2]));
    v0 = rn_bf16(fmaf(v0, fabsf(c0), k.c[1]));
    v1 = rn_bf16(fmaf(v1, fabsf(c1), k.c[1]));
    t0 = rn_bf16(v0 * c0);
    t1 = rn_bf16(v1 * c1);
}
__device__ __forceinline__ void softcap_bf16_pair(float s0, float s1, float scale, const TanhBF16 &k,
                                                  float &t0, float &t1, float &x0, float &x1)
{
    float c0, c1;
    softcap_bf16_pair(s0, s1, scale, k, t0, t1, x0, x1, c0, c1);
}

// FP32 FMAs with FP16 operands taken from the halves of a packed word
// (v_fma_mix_f32: the halves convert to FP32 exactly, one rounding)
// t * high(w) + low(w)
__device__ __forceinline__ float fma_mix_pair(float t, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %2 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "=v"(r) : "v"(t), "v"(w));
    return r;
}
// t * v + high(w)
__device__ __forceinline__ float fma_mix_add_hi(float t, float v, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(r) : "v"(t), "v"(v), "v"(w));
    return r;
}
// t * v + low(w), clamped to [0, 1]
__device__ __forceinline__ float fma_mix_add_lo_clamp(float t, float v, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,0,1] clamp" : "=v"(r) : "v"(t), "v"(v), "v"(w));
    return r;
}

// sigmoid program on a pair: packed BF16 P~ (and, when GRAD, the BF16
// surrogate derivatives as FP32 values in g0, g1)
template <bool GRAD>
__device__ __forceinline__ uint32_t sigmoid_poly_pair(float s0, float s1, float scale,
                                                      const SigCoef &k, float *g0, float *g1)
{
    // every value BF16-rounded per lane (rn_bf16: one instruction, no unpack)
    const float x0 = rn_bf16(s0 * scale), x1 = rn_bf16(s1 * scale);
    const int r0 = x0 >= k.thr, r1 = x1 >= k.thr;
    // clamp to [lo, hi] as one median of three (lo < hi; the same value as
    // min(max(x, lo), hi) for every finite score)
    const float t0 = __builtin_amdgcn_fmed3f(x0, k.lo, k.hi);
    const float t1 = __builtin_amdgcn_fmed3f(x1, k.lo, k.hi);
    // Horner in FP32 FMAs with FP16 coefficient operands (exact conversions,
    // so each stage is the FP32 FMA of the BF16 constants), each rounded to
    // BF16: c3 t + c2, then + c1, then + c0.  The program's value lies below
    // 0.06 for every input, so the last FMA's [0, 1] clamp before its
    // rounding is max(value, 0) after it.
    const uint32_t w0 = r0 ? k.c23[1] : k.c23[0], w1 = r1 ? k.c23[1] : k.c23[0];
    const uint32_t u0 = r0 ? k.c01[1] : k.c01[0], u1 = r1 ? k.c01[1] : k.c01[0];
    float v0 = rn_bf16(fma_mix_pair(t0, w0)), v1 = rn_bf16(fma_mix_pair(t1, w1));
    v0 = rn_bf16(fma_mix_add_hi(t0, v0, u0));
    v1 = rn_bf16(fma_mix_add_hi(t1, v1, u1));
    v0 = rn_bf16(fma_mix_add_lo_clamp(t0, v0, u0));
    v1 = rn_bf16(fma_mix_add_lo_clamp(t1, v1, u1));
    if constexpr (GRAD) {
        const uint32_t z0 = r0 ? k.ab[1] : k.ab[0], z1 = r1 ? k.ab[1] : k.ab[0];
        const float f0 = rn_bf16(fma_mix_pair(t0, z0));   // b t + a
        const float f1 = rn_bf16(fma_mix_pair(t1, z1));
        *g0 = rn_bf16(v0 * f0);
        *g1 = rn_bf16(v1 * f1);
    }
    return pack_bf(v0, v1);   // exact: v0, v1 are BF16 values
}

// Split exp2 of the softmax (Appendix B.1, Eqs. 16-19): 2^z = 2^n p(f),
// n = floor(z), f = z - n, with the reference max m an integer so that
// 2^(z - m) = ldexp(p(f), n - m) exactly scales by a power of two and the
// normalised weights do not depend on m.  z is clamped below at -16384
// (masked keys, z = -inf, give 0).  Cores (p(0) = 1, p(1) = 2 after rounding
// except D3):
//   0 HW    p = 2^f by v_exp_f32 (the large-cap path of the hardware
//           exponential: each P is the same FP32 value up to an exact power of
//           two whatever the reference)
//   1 D1    p = f + 1                                         (FP32)
//   2 PWL2  p = 1 + a f + 2 (1 - a) max(f - 1/2, 0), a = 0.7978515625,
//           in packed FP16 (f rounded to FP16, one rounding per op)
//   3 D2    p = 1 + a f + (1 - a) f^2, a = RN32(0.6602339719)   (FP32 FMA)
//   4 D3    the pages' printed cubic                           (FP32 FMA)
constexpr float EXP2_D2_A = 0.6602339719f;
constexpr float EXP2_D3_C1 = 0.6951461434f, EXP2_D3_C2 = 0.2275643945f, EXP2_D3_C3 = 0.0771190897f;

template <int EXP>
__device__ __forceinline__ void exp2_core_pair(float z0, float z1, float m, float &p0, float &p1)
{
    z0 = fmaxf(z0, -16384.0f);
    z1 = fmaxf(z1, -16384.0f);
    const float n0 = floorf(z0), n1 = floorf(z1);
    const float f0 = z0 - n0, f1 = z1 - n1;
    float c0, c1;
    if constexpr (EXP == 0) {
        c0 = __builtin_amdgcn_exp2f(f0);
        c1 = __builtin_amdgcn_exp2f(f1);
    } else if constexpr (EXP == 1) {
        c0 = f0 + 1.0f;
        c1 = f1 + 1.0f;
    } else if constexpr (EXP == 2) {
        h2 fh;
        fh[0] = (_Float16)f0;
        fh[1] = (_Float16)f1;
        const h2 hinge = __builtin_elementwise_max(fh - h2{(_Float16)0.5f, (_Float16)0.5f},
                                                   h2{(_Float16)0.0f, (_Float16)0.0f});
        h2 p = __builtin_elementwise_fma(h2{(_Float16)0.7978515625f, (_Float16)0.7978515625f}, fh,
                                         h2{(_Float16)1.0f, (_Float16)1.0f});
        p = __builtin_elementwise_fma(h2{(_Float16)0.40380859375f, (_Float16)0.40380859375f}, hinge, p);
        c0 = (float)p[0];
        c1 = (float)p[1];
    } else if constexpr (EXP == 3) {
        constexpr float b = 1.0f - EXP2_D2_A;   // exact
        c0 = fmaf(fmaf(b, f0, EXP2_D2_A), f0, 1.0f);
        c1 = fmaf(fmaf(b, f1, EXP2_D2_A), f1, 1.0f);
    } else {
        c0 = fmaf(fmaf(fmaf(EXP2_D3_C3, f0, EXP2_D3_C2), f0, EXP2_D3_C1), f0, 1.0f);
        c1 = fmaf(fmaf(fmaf(EXP2_D3_C3, f1, EXP2_D3_C2), f1, EXP2_D3_C1), f1, 1.0f);
    }
    p0 = __builtin_amdgcn_ldexpf(c0, (int)(n0 - m));
    p1 = __builtin_amdgcn_ldexpf(c1, (int)(n1 - m));
}

// fma(t, b, c) with t the low / high FP16 half of a packed word, converted
// exactly (v_fma_mix_f32: one rounding, as fmaf((float)t, b, c))
__device__ __forceinline__ float fma_mix_lo(uint32_t w, float b, float c)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t w, float b, float c)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(b), "v"(c));
    return r;
}

// accurate sigmoid of u (the comparator)
__device__ __forceinline__ float sigmoid_acc(float u)
{
    const float e = expf(-fabsf(u));
    return (u >= 0.0f ? 1.0f : e) / (1.0f + e);
}

// EXP: 0 = hardware exp2 (v_exp_f32), 1-4 = the software cores above
// (softcap only).
// SREF (softcap with cap log2 e <= 80): the logits are bounded, |z| <= cap
// log2 e, so a fixed reference m = ceil(cap log2 e - 40) keeps every P in
// [2^-120, 2^40] -- normal FP32 and BF16, row sums far from overflow -- and
// the running max, its reductions and the rescales are not needed at all.
//
// Software pipeline.  Each wave walks its keys in units of 32 (one 32x32
// score block).  Stage j issues the QK^T MFMAs of unit j + 1 and the PV MFMAs
// of unit j - 1 and, independent of both, the VALU score transform of unit j,
// so the matrix cores and the vector ALU work on different units at the same
// time instead of taking turns.  K tiles therefore run one LDS tile ahead of
// V tiles: period p (stages 2p - 1 and 2p) reads K tile p and V tile p - 1
// from the two halves of each buffer while K tile p + 1 and V tile p stream
// in.  The order of every accumulation (over keys for S, O and the row sum)
// is the unpipelined one.  Steady-state stages are laid out as explicit
// scheduling slots (see `slotted`).
template <int MODE, int EXP = 0, bool SREF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_fwd(AttnArgs a)
{
    constexpr bool SOFTCAP = am_softcap(MODE);
    // K and V double buffers (see dbuf): separate arrays for sigmoid only;
    // the softcap with the hardware exponential runs 1-2 % slower with them,
    // and the BF16 softcap with a software exp2 core spills with them
    constexpr bool SPLIT_LDS = !SOFTCAP;
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[AT_TILE], Ks1[AT_TILE], Kp[2][AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[AT_TILE], Vs1[AT_TILE], Vp[2][AT_TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;     // 16-lane group, lane in group
    const int S = a.S;
    const int ntq = (S + AT_BM - 1) / AT_BM;
    const int nbh = (int)(gridDim.x / (unsigned)ntq);
    const int qrank = (int)blockIdx.x / nbh;          // 0 = heaviest query tile
    const int bh = (int)blockIdx.x - qrank * nbh;
    const int qt = a.causal ? ntq - 1 - qrank : qrank;
    const int64_t qbase = (int64_t)bh * S * AT_D;
    const int64_t kvbase = (int64_t)(bh / a.G) * S * AT_D;   // (b H + h) / G = b Hkv + h / G
    const uint16_t *Q = a.q + qbase, *K = a.k + kvbase, *V = a.v + kvbase;
    const int q0 = qt * AT_BM + wave * 32;
    const int my_q = q0 + col;

    // Q as the B operand of S^T = K Q^T: lane holds Q[my_q][ks*16 + h*8 + 0..7]
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (my_q < S) qf[ks] = ld_bf16x8(Q + (int64_t)my_q * AT_D + ks * 16 + h * 8);
        else qf[ks] = bf16x8{};
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m = SREF ? a.mref : -INFINITY;   // reference of the log2-domain score (softcap)
    float l = 0.0f;        // this lane's partial row sum (softcap)

    // keys of the workgroup and of this wave (units of 32 keys); the last
    // unit of a wave is the only one that can need a mask (the causal
    // diagonal, or the ragged end of S)
    const int kend = a.causal ? (qt * AT_BM + AT_BM < S ? qt * AT_BM + AT_BM : S) : S;
    const int nkt = (kend + AT_BN - 1) / AT_BN;
    const int wend = q0 >= S ? 0 : (a.causal ? (q0 + 32 < S ? q0 + 32 : S) : S);
    const int nu = (wend + 31) / 32;
    const bool last_masked = nu > 0 && (a.causal || wend < nu * 32);
    const int lim = a.causal ? (my_q < S - 1 ? my_q : S - 1) : S - 1;   // last visible key

    f32x16 sc[2];          // raw scores of an even / odd unit
    bf16x8 pf[2][2];       // P of an even / odd unit as two B-operand fragments

    // ---- the three parts of a stage ------------------------------------------
    // S^T of unit u from rows 32 * (u & 1) of a K tile
    auto qk = [&](f32x16 &s, const uint16_t *Kb, int half) __attribute__((always_inline)) {
        s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Kb, half * 32 + col, ks * 2 + h),
                                                        qf[ks], s, 0, 0, 0);
    };
    // O^T += V^T P^T for a unit from rows 32 * half of a V tile; contraction
    // index h*8 + e of step kk maps to key kk*16 + (e/4)*8 + h*4 + (e%4)
    auto pv = [&](const bf16x8 (&p)[2], const uint16_t *Vb, int half) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_a(Vb, half * 2 + kk, db, g16, i16),
                                                                p[kk], o[db], 0, 0, 0);
        }
    };
    // score transform of one unit, as NPC pieces run in order (the steady
    // state spreads them between its MFMAs): s[j*4 + i] is the score of key
    // ukey0 + j*8 + h*4 + i.  Masked keys get t = -inf (softcap) or P = 0
    // (sigmoid).  Softcap pieces 0-7 map the score pairs through the tanh
    // (packed FP16 words kept in st.w), then (online max only) one piece
    // moves the reference, then pieces for the pairs' exp2, row sums and BF16
    // words of P.  Sigmoid: one piece per pair.  For the online max the
    // factor st.corr rescales O once this stage's PV product has landed.
    constexpr int NPC = SOFTCAP ? (SREF ? 16 : 17) : 8;
    struct TState {
        float tf[16];      // t of the BF16 softcap program
        uint32_t w[8];     // packed FP16 t (FP16 softcap program), then the BF16 P words
        uint32_t mx;       // packed FP16 running max of t (FP16 softcap poly, online max)
        float tmax;        // running max of t (BF16 softcap poly, comparator; online max)
        float corr;
    };
    auto piece = [&](auto pc, f32x16 &s, TState &st, int ukey0, auto masked) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        constexpr bool MASKED = decltype(masked)::value;
        if constexpr (SOFTCAP) {
            if constexpr (P < 8) {
                constexpr int e = 2 * P;
                if constexpr (MODE == AM_SOFTCAP_POLY) {
                    uint32_t aw;
                    uint32_t w = softcap_poly_pair(s[e], s[e + 1], a.scale, a.tanh16, aw);
                    if constexpr (MASKED) {
                        const int k0 = ukey0 + (e >> 2) * 8 + h * 4 + (e & 3);
                        const uint32_t mlo = k0 > lim ? 0x0000FFFFu : 0u;
                        const uint32_t mhi = k0 + 1 > lim ? 0xFFFF0000u : 0u;
                        w = sel(mlo | mhi, 0xFC00FC00u, w);
                    }
                    if constexpr (!SREF) st.mx = bc<uint32_t>(__builtin_elementwise_max(bc<h2>(st.mx), bc<h2>(w)));
                    st.w[P] = w;
                } else if constexpr (MODE == AM_SOFTCAP_POLY_BF16) {
                    // t as FP32 values (masked keys: -inf)
                    float t0, t1, x0, x1;
                    softcap_bf16_pair(s[e], s[e + 1], a.scale, a.tanhbf, t0, t1, x0, x1);
                    if constexpr (MASKED) {
                        const int k0 = ukey0 + (e >> 2) * 8 + h * 4 + (e & 3);
                        t0 = k0 > lim ? -INFINITY : t0;
                        t1 = k0 + 1 > lim ? -INFINITY : t1;
                    }
                    if constexpr (!SREF) st.tmax = fmaxf(st.tmax, fmaxf(t0, t1));
                    st.tf[e] = t0;
                    st.tf[e + 1] = t1;
                } else {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        float t = tanhf(s[e + i] * a.scale);
                        if constexpr (MASKED) {
                            const int k0 = ukey0 + (e >> 2) * 8 + h * 4 + (e & 3) + i;
                            t = k0 > lim ? -INFINITY : t;
                        }
                        s[e + i] = t;
                        if constexpr (!SREF) st.tmax = fmaxf(st.tmax, t);
                    }
                }
            } else if constexpr (!SREF && P == 8) {
                // lazy rescale: move the reference only when the row max
                // outgrows it by more than AT_RESCALE
                float tmax = MODE == AM_SOFTCAP_POLY ? fmaxf(f16_lo(st.mx), f16_hi(st.mx)) : st.tmax;
                if (tmax == -INFINITY) tmax = -1.0f;   // every key masked: any reference
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                const float zmax = tmax * a.c2;
                const bool grow = zmax > m + AT_RESCALE;
                // integer reference; the rescale is an exact power of two
                const float m_new = grow ? ceilf(zmax) : m;
                st.corr = !grow ? 1.0f
                                : (m == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, (int)(m - m_new)));
                l *= st.corr;
                m = m_new;
            } else {
                // P of pair e2, the row sum, the BF16 word: with the fixed
                // reference P = exp2(RN32(t c2 - m)) in one FMA; otherwise
                // z = RN32(t c2) through the split exp2 (its core, or 2^frac
                // by v_exp_f32), relative to the integer reference
                constexpr int e2 = P - (SREF ? 8 : 9);
                constexpr int e = 2 * e2;
                float t0, t1;
                if constexpr (MODE == AM_SOFTCAP_NATIVE) {
                    t0 = s[e];
                    t1 = s[e + 1];
                } else if constexpr (MODE == AM_SOFTCAP_POLY_BF16) {
                    t0 = st.tf[e];
                    t1 = st.tf[e + 1];
                }
                float p0, p1;
                if constexpr (MODE == AM_SOFTCAP_POLY) {
                    // the FP16 t feed the FMA directly (no conversions)
                    const uint32_t w = st.w[e2];
                    if constexpr (EXP == 0 && SREF) {
                        p0 = __builtin_amdgcn_exp2f(fma_mix_lo(w, a.c2, -m));
                        p1 = __builtin_amdgcn_exp2f(fma_mix_hi(w, a.c2, -m));
                    } else {
                        exp2_core_pair<EXP>(fma_mix_lo(w, a.c2, -0.0f), fma_mix_hi(w, a.c2, -0.0f), m, p0, p1);
                    }
                } else if constexpr (EXP == 0 && SREF) {
                    p0 = __builtin_amdgcn_exp2f(fmaf(t0, a.c2, -m));
                    p1 = __builtin_amdgcn_exp2f(fmaf(t1, a.c2, -m));
                } else {
                    exp2_core_pair<EXP>(t0 * a.c2, t1 * a.c2, m, p0, p1);
                }
                l += p0;
                l += p1;
                st.w[e2] = pack_bf(p0, p1);
            }
        } else {
            // sigmoid: P of pair P directly, as a BF16 word
            constexpr int e = 2 * P;
            uint32_t w;
            if constexpr (MODE == AM_SIGMOID_POLY) {
                w = sigmoid_poly_pair<false>(s[e], s[e + 1], a.scale, a.sig, nullptr, nullptr);
            } else {
                w = pack_bf(sigmoid_acc(fmaf(s[e], a.scale, -a.logn)),
                            sigmoid_acc(fmaf(s[e + 1], a.scale, -a.logn)));
            }
            if constexpr (MASKED) {
                const int k0 = ukey0 + (e >> 2) * 8 + h * 4 + (e & 3);
                const uint32_t mlo = k0 > lim ? 0x0000FFFFu : 0u;
                const uint32_t mhi = k0 + 1 > lim ? 0xFFFF0000u : 0u;
                w &= ~(mlo | mhi);
            }
            st.w[P] = w;
        }
    };
    auto tstate = [&]() __attribute__((always_inline)) {
        TState st;
        st.mx = 0xFC00FC00u;   // packed FP16 -inf
        st.tmax = -INFINITY;
        st.corr = 1.0f;
        return st;
    };
    // P as the two B-operand fragments of the PV product
    auto finish = [&](const TState &st, bf16x8 (&p)[2]) __attribute__((always_inline)) {
        p[0] = bc<bf16x8>(u32x4{st.w[0], st.w[1], st.w[2], st.w[3]});
        p[1] = bc<bf16x8>(u32x4{st.w[4], st.w[5], st.w[6], st.w[7]});
    };
    auto transform = [&](f32x16 &s, bf16x8 (&p)[2], int ukey0, auto masked) __attribute__((always_inline)) -> float {
        TState st = tstate();
        static_for<NPC>([&](auto pc) __attribute__((always_inline)) { piece(pc, s, st, ukey0, masked); });
        finish(st, p);
        return st.corr;
    };
    auto rescale = [&](float corr) __attribute__((always_inline)) {
        if constexpr (SOFTCAP && !SREF) {
            if (__builtin_amdgcn_ballot_w64(corr != 1.0f)) {
#pragma unroll
                for (int db = 0; db < 4; ++db) o[db] *= corr;
            }
        }
    };

    // ---- the steady-state stage as explicit slots --------------------------
    // The 16 MFMAs of a stage alternate QK^T (even m, contraction step m / 2)
    // and PV (odd m, d block m / 4, key step (m / 2) & 1); every accumulator
    // sees its terms in the order above.  Slot t issues the LDS reads of the
    // operands of slot t + 1, its own MFMAs and its share of the transform
    // pieces; a scheduling fence closes each slot, so every LDS read runs one
    // slot ahead of its MFMA (the compiler otherwise waits for each operand
    // right before its MFMA) and the VALU work is spread evenly between the
    // matrix instructions.  FP16 softcap and comparator with the hardware
    // exponential: 16 slots (one MFMA and one piece each); sigmoid, the BF16
    // softcap and the software exp2 cores: 8 slots of two MFMAs, whose two
    // pieces (or pair) the scheduler can interleave, filling the stalls
    // between dependent steps of one chain (the exp2 cores 1.035-1.05x and
    // the BF16 softcap 1.03-1.04x faster than with 16 slots, 4 slots no
    // better; the FP16 softcap 1-2 % slower).  Reading the operands two or
    // three slots ahead instead of one made the 16-slot layouts 1-2 % slower
    // (more registers live across each MFMA).  Outputs are bit-identical
    // either way.
    constexpr int AT_SLOTS = (SOFTCAP && EXP == 0 && MODE != AM_SOFTCAP_POLY_BF16) ? 16 : 8, AT_AHEAD = 1;
    auto slotted = [&](f32x16 &sn, f32x16 &scur, bf16x8 (&pc)[2], const bf16x8 (&pp)[2],
                       const uint16_t *Kb, const uint16_t *Vb, int ukey0, auto halfc) __attribute__((always_inline)) {
        constexpr int HALF = decltype(halfc)::value;
        constexpr int MPS = 16 / AT_SLOTS;    // MFMAs per slot
        bf16x8 op[16];
        auto load_op = [&](auto mc) __attribute__((always_inline)) {
            constexpr int mm = decltype(mc)::value;
            if constexpr ((mm & 1) == 0) op[mm] = lds_row8(Kb, HALF * 32 + col, mm + h);
            else op[mm] = lds_tr_a(Vb, HALF * 2 + ((mm >> 1) & 1), mm >> 2, g16, i16);
        };
        auto mfma_op = [&](auto mc) __attribute__((always_inline)) {
            constexpr int mm = decltype(mc)::value;
            if constexpr ((mm & 1) == 0)
                sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[mm], qf[mm >> 1], mm == 0 ? f32x16{} : sn, 0, 0, 0);
            else
                o[mm >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[mm], pp[(mm >> 1) & 1], o[mm >> 2], 0, 0, 0);
        };
        TState st = tstate();
        static_for<AT_AHEAD * MPS>([&](auto mc) __attribute__((always_inline)) { load_op(mc); });
        static_for<AT_SLOTS>([&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            static_for<MPS>([&](auto ic) __attribute__((always_inline)) {
                constexpr int mm = (t + AT_AHEAD) * MPS + decltype(ic)::value;
                if constexpr (mm < 16) load_op(std::integral_constant<int, mm>{});
            });
            static_for<MPS>([&](auto ic) __attribute__((always_inline)) {
                mfma_op(std::integral_constant<int, t * MPS + decltype(ic)::value>{});
            });
            constexpr int p0 = t * NPC / AT_SLOTS, p1 = (t + 1) * NPC / AT_SLOTS;
            // FP16 softcap: the slot's transform piece at raised wave
            // priority, so the SIMD's other wave yields to it (measured on
            // MI355X: 1.025x; the BF16 program, sigmoid, the comparator and
            // the exp2 cores are slower with it, and so is raising it for
            // the MFMAs instead)
            if constexpr (MODE == AM_SOFTCAP_POLY) __builtin_amdgcn_s_setprio(1);
            static_for<p1 - p0>([&](auto ic) __attribute__((always_inline)) {
                piece(std::integral_constant<int, p0 + decltype(ic)::value>{}, scur, st, ukey0, std::false_type{});
            });
            if constexpr (MODE == AM_SOFTCAP_POLY) __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        });
        finish(st, pc);
        rescale(st.corr);
    };

    // ---- stage j of period p: HALF = j & 1 ... written out for the two
    // halves so that every register and LDS offset is a constant.
    // Stage j (HALF = (j + 1) & 1 is the K half of unit j + 1 and the V half
    // of unit j - 1): QK^T(j + 1) from Kb, transform(j), PV(j - 1) from Vb.
    auto stage = [&](int j, const uint16_t *Kb, const uint16_t *Vb, auto halfc) __attribute__((always_inline)) {
        constexpr int HALF = decltype(halfc)::value;   // = (j + 1) & 1
        constexpr int SN = HALF;                      // S(j + 1) lives in sc[(j + 1) & 1]
        constexpr int SC = HALF ^ 1;                  // S(j) in sc[j & 1]
        constexpr int PC = HALF ^ 1;                  // P(j) into pf[j & 1]
        constexpr int PP = HALF;                      // P(j - 1) from pf[(j - 1) & 1]
        if (j >= 1 && j + 1 < nu) {
            // steady state: all three parts, no mask, one basic block
            slotted(sc[SN], sc[SC], pf[PC], pf[PP], Kb, Vb, j * 32, halfc);
            return;
        }
        if (j + 1 < nu) qk(sc[SN], Kb, HALF);
        float corr = 1.0f;
        if (j >= 0 && j < nu) {
            if (j == nu - 1 && last_masked) corr = transform(sc[SC], pf[PC], j * 32, std::true_type{});
            else corr = transform(sc[SC], pf[PC], j * 32, std::false_type{});
        }
        if (j >= 1 && j <= nu) pv(pf[PP], Vb, HALF);
        rescale(corr);
    };

    // ---- periods: p = 0 .. nkt; period p runs stages 2p - 1 and 2p --------
    // tile loads from assembly for the BF16 program (measured on MI355X:
    // its forward 1.04x, with an exp2 core 1.04x; the FP16 program and the
    // comparator ran 2 % slower with them and keep the builtin loads)
    constexpr bool ASM_LOADS = MODE == AM_SOFTCAP_POLY_BF16;
    auto load_tile = [&](const uint16_t *src, uint16_t *lds, int row0) __attribute__((always_inline)) {
        if constexpr (ASM_LOADS) load_rows64_asm(src, lds, row0, S, wave, lane);
        else load_rows64(src, lds, row0, S, wave, lane);
    };
    // vmcnt(0) with lgkmcnt and expcnt left alone: the Q loads have landed,
    // so no wait on them is left for the loop to find
    if constexpr (ASM_LOADS) __builtin_amdgcn_s_waitcnt(0x0F70);
    load_tile(K, dbuf<0, SPLIT_LDS>(Ks0, Ks1, Kp), 0);
    auto period = [&](int p, auto bufc) __attribute__((always_inline)) {
        constexpr int kb = decltype(bufc)::value;    // K tile p in buffer kb, V tile p - 1 in buffer kb ^ 1
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of K p / V p - 1 landed
        __syncthreads();   // everybody's landed; nobody reads K buffer kb ^ 1 / V buffer kb any more
        uint16_t *const Kc = dbuf<kb, SPLIT_LDS>(Ks0, Ks1, Kp), *const Kn = dbuf<kb ^ 1, SPLIT_LDS>(Ks0, Ks1, Kp);
        uint16_t *const Vc = dbuf<kb ^ 1, SPLIT_LDS>(Vs0, Vs1, Vp), *const Vn = dbuf<kb, SPLIT_LDS>(Vs0, Vs1, Vp);
        if (p + 1 < nkt) load_tile(K, Kn, (p + 1) * AT_BN);
        if (p < nkt) load_tile(V, Vn, p * AT_BN);
        if (2 * p - 1 > nu) return;   // this wave is done (still takes part in the barriers)
        stage(2 * p - 1, Kc, Vc, std::integral_constant<int, 0>{});
        stage(2 * p, Kc, Vc, std::integral_constant<int, 1>{});
    };
    for (int p = 0; p <= nkt; p += 2) {
        period(p, std::integral_constant<int, 0>{});
        if (p + 1 <= nkt) period(p + 1, std::integral_constant<int, 1>{});
    }

    if (my_q >= S) return;
    float inv = 1.0f;
    if constexpr (SOFTCAP) {
        const float lt = l + __shfl_xor(l, 32);
        inv = 1.0f / lt;
        if (a.lse && h == 0) a.lse[(int64_t)bh * S + my_q] = (m + __log2f(lt)) * AT_LN2;
    }
    uint16_t *orow = a.o + qbase + (int64_t)my_q * AT_D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + j * 8 + h * 4;
            u32x2 w;
            w.x = pack_bf(o[db][j * 4 + 0] * inv, o[db][j * 4 + 1] * inv);
            w.y = pack_bf(o[db][j * 4 + 2] * inv, o[db][j * 4 + 3] * inv);
            *(u32x2 *)(orow + d) = w;
        }
    }
}

}  // namespace pa
