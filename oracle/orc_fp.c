/*
 * orc_fp.c -- binary16 / bfloat16 / binary32 values and correctly rounded
 * operations, written from the definitions of the formats.
 *
 * Test infrastructure (see orc.h).  Every routine here computes the exact
 * real result of an operation and rounds it once to nearest, ties to even,
 * with gradual underflow and overflow to infinity, as IEEE 754 prescribes.
 * The paper's programs execute as chains of such operations in FP16 or BF16
 * ("Fast Polynomial Transcendentals for LLMs", section 3.2: every multiply-add
 * is rounded to the target format; section 3.4: packed FP16/BF16 FMA).
 */
#include "orc.h"

#include <math.h>
#include <string.h>

/* Round a real value held exactly in a double to a binary format with
 * `mbits` stored fraction bits and `ebits` exponent bits (FP16: 10/5,
 * BF16: 7/8).  Returns the bit pattern.  Method: pick the quantum (the
 * weight of the last stored bit) from the binade of |x|, clamped at the
 * subnormal binade; |x| / quantum is then an exact double whose
 * round-to-nearest-even integer (nearbyint in the default rounding mode)
 * is the rounded significand. */
static uint32_t round_fmt(double x, int mbits, int ebits)
{
    const uint32_t sign = signbit(x) ? 1u : 0u;
    const int sshift = mbits + ebits;
    const uint32_t emask = (1u << ebits) - 1u;
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias, emax = bias;

    if (isnan(x))
        return (sign << sshift) | (emask << mbits) | (1u << (mbits - 1));
    double a = fabs(x);
    if (isinf(a))
        return (sign << sshift) | (emask << mbits);
    if (a == 0.0)
        return sign << sshift;

    int e;
    (void)frexp(a, &e);
    e -= 1;                                   /* 2^e <= a < 2^(e+1) */
    const int qexp = (e < emin ? emin : e) - mbits;
    const double r = nearbyint(ldexp(a, -qexp));  /* ties to even */
    if (r == 0.0)
        return sign << sshift;                /* underflow to a signed zero */
    const double v = ldexp(r, qexp);          /* the rounded magnitude */
    if (v >= ldexp(1.0, emax + 1))
        return (sign << sshift) | (emask << mbits);   /* overflow */
    int e2;
    (void)frexp(v, &e2);
    e2 -= 1;
    if (e2 < emin)                            /* subnormal: r < 2^mbits */
        return (sign << sshift) | (uint32_t)r;
    const uint32_t frac = (uint32_t)ldexp(v, mbits - e2) - (1u << mbits);
    return (sign << sshift) | ((uint32_t)(e2 + bias) << mbits) | frac;
}

/* Value of a bit pattern, from the definition of the format. */
static double decode_fmt(uint32_t bits, int mbits, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t s = (bits >> (mbits + ebits)) & 1u;
    const uint32_t ef = (bits >> mbits) & ((1u << ebits) - 1u);
    const uint32_t m = bits & ((1u << mbits) - 1u);
    double v;
    if (ef == (1u << ebits) - 1u)
        v = m ? NAN : INFINITY;
    else if (ef == 0)
        v = ldexp((double)m, 1 - bias - mbits);
    else
        v = ldexp((double)(m + (1u << mbits)), (int)ef - bias - mbits);
    return s ? -v : v;
}

double orc_f16_to_f64(uint16_t h) { return decode_fmt(h, 10, 5); }
double orc_bf16_to_f64(uint16_t b) { return decode_fmt(b, 7, 8); }
uint16_t orc_f64_to_f16(double x) { return (uint16_t)round_fmt(x, 10, 5); }
uint16_t orc_f64_to_bf16(double x) { return (uint16_t)round_fmt(x, 7, 8); }
uint16_t orc_f32_to_bf16(float x) { return (uint16_t)round_fmt((double)x, 7, 8); }
float orc_bf16_to_f32(uint16_t b) { return (float)decode_fmt(b, 7, 8); }

/* ---- FP16 fused multiply-add, exact integer arithmetic --------------------
 * Every finite FP16 value is an integer multiple of 2^-24, so every product
 * of two is an integer multiple of 2^-48 below 2^32 in magnitude, and every
 * sum a*b + c is an integer M times 2^-48 with |M| < 2^81.  M is computed
 * exactly in a 128-bit integer and rounded once. */
typedef __int128 i128;

static void f16_parts(uint16_t h, int *neg, int64_t *m, int *e)
{
    const int ef = (h >> 10) & 31;
    const int64_t fr = h & 1023;
    *neg = (h >> 15) & 1;
    if (ef == 0) { *m = fr; *e = -24; }
    else { *m = fr + 1024; *e = ef - 25; }
}

static int bitlen128(i128 v)   /* v > 0 */
{
    int n = 0;
    while (v) { v >>= 1; n++; }
    return n;
}

/* Round |M| * 2^-48 (M != 0) to FP16 and attach the sign. */
static uint16_t f16_round_units(int neg, i128 M)
{
    /* quantum in units of 2^-48: 2^24 in the subnormal binade, else
     * 2^(bitlen - 11) so that 11 significant bits remain */
    const int bl = bitlen128(M);
    int shift = bl - 11;
    if (shift < 24) shift = 24;
    i128 r = M >> shift;
    const i128 rem = M - (r << shift);
    const i128 half = (i128)1 << (shift - 1);
    if (rem > half || (rem == half && (r & 1))) r++;
    const uint16_t s = neg ? 0x8000 : 0;
    if (r == 0) return s;
    const i128 val = r << shift;
    const int vb = bitlen128(val);
    const int E = vb - 1 - 48;                /* 2^E <= value < 2^(E+1) */
    if (E > 15) return s | 0x7C00;           /* overflow */
    if (E < -14) return s | (uint16_t)(val >> 24);   /* subnormal */
    const uint16_t frac = (uint16_t)((val >> (E + 48 - 10)) - 1024);
    return s | (uint16_t)((E + 15) << 10) | frac;
}

uint16_t orc_fma_f16(uint16_t a, uint16_t b, uint16_t c)
{
    const double da = orc_f16_to_f64(a), db = orc_f16_to_f64(b),
                 dc = orc_f16_to_f64(c);
    /* Non-finite operands: IEEE 754 rules; an invalid operation produces
     * the canonical quiet NaN 0x7E00. */
    if (isnan(da) || isnan(db) || isnan(dc)) return 0x7E00;
    const int sp = ((a ^ b) >> 15) & 1;      /* sign of the product */
    if (isinf(da) || isinf(db)) {
        if (da == 0.0 || db == 0.0) return 0x7E00;   /* inf * 0 */
        if (isinf(dc) && (((c >> 15) & 1) != sp)) return 0x7E00; /* inf - inf */
        return sp ? 0xFC00 : 0x7C00;
    }
    if (isinf(dc)) return c;

    int na, nb, nc, ea, eb, ec;
    int64_t ma, mb, mc;
    f16_parts(a, &na, &ma, &ea);
    f16_parts(b, &nb, &mb, &eb);
    f16_parts(c, &nc, &mc, &ec);
    i128 P = (i128)(ma * mb) << (ea + eb + 48);
    i128 C = (i128)mc << (ec + 48);
    if (sp) P = -P;
    if (nc) C = -C;
    const i128 S = P + C;
    if (S == 0) {
        /* exact zero: -0 only when both addends are negative zeros, or a
         * negative product of zero plus -0; an exact cancellation of nonzero
         * terms is +0 under round-to-nearest */
        const int pzero = (ma == 0 || mb == 0), czero = (mc == 0);
        if (pzero && czero) return (sp && nc) ? 0x8000 : 0x0000;
        return 0x0000;
    }
    return S < 0 ? f16_round_units(1, -S) : f16_round_units(0, S);
}

/* ---- BF16 fused multiply-add -------------------------------------------
 * The product of two BF16 values has at most 16 significant bits and lies
 * within the normal double range, so it is exact in a double.  The sum with
 * c is formed with Knuth's TwoSum (s + err is exact), then rounded to odd
 * at double precision; a double rounded to odd carries 53 >= 8 + 2 bits, so
 * one further round-to-nearest gives the correctly rounded BF16 result
 * (S. Boldo and G. Melquiond, "Emulation of FMA and correctly rounded sums:
 * proved algorithms using rounding to odd", IEEE Trans. Computers, 2008). */
static double round_to_odd_sum(double p, double c)
{
    const double s = p + c;
    const double bb = s - p;
    const double err = (p - (s - bb)) + (c - bb);
    if (err == 0.0) return s;
    uint64_t bits;
    memcpy(&bits, &s, sizeof bits);
    if (bits & 1u) return s;                  /* already odd */
    return nextafter(s, err > 0 ? INFINITY : -INFINITY);
}

uint16_t orc_fma_bf16(uint16_t a, uint16_t b, uint16_t c)
{
    const double da = orc_bf16_to_f64(a), db = orc_bf16_to_f64(b),
                 dc = orc_bf16_to_f64(c);
    if (isnan(da) || isnan(db) || isnan(dc)) return 0x7FC0;
    const double p = da * db;                 /* exact (or inf / NaN) */
    if (isnan(p)) return 0x7FC0;
    if (isinf(p) || isinf(dc)) {
        const double s = p + dc;
        return isnan(s) ? 0x7FC0 : orc_f64_to_bf16(s);
    }
    if (p == 0.0 && dc == 0.0)
        return orc_f64_to_bf16(p + dc);       /* IEEE signed-zero sum */
    return orc_f64_to_bf16(round_to_odd_sum(p, dc));
}

/* ---- binary32 ----------------------------------------------------------
 * C99 fmaf is defined to compute a*b + c rounded once; add and multiply are
 * expressed through it so that each is one correctly rounded operation. */
float orc_fma_f32(float a, float b, float c) { return fmaf(a, b, c); }
float orc_add_f32(float a, float b) { return fmaf(a, 1.0f, b); }
float orc_mul_f32(float a, float b) { return fmaf(a, b, -0.0f); }

uint16_t orc_fma_f32_bf16(uint16_t a, uint16_t b, uint16_t c)
{
    return orc_f32_to_bf16(fmaf(orc_bf16_to_f32(a), orc_bf16_to_f32(b),
                                orc_bf16_to_f32(c)));
}
