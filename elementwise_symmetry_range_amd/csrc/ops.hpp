// ops.hpp -- per-register-pair element programs for gfx950.
//
// Every operator here maps one 32-bit register holding two 16-bit lanes (a
// packed FP16 or BF16 pair) to its result pair.  The polynomial programs follow
// "Fast Polynomial Transcendentals for LLMs" (arXiv 2610.00049):
//   t = |x| (sign-bit clear), t^ = min(t, Lc)                    section 3.1, Eq. 2
//   Horner: v = c_D; v = fma(v, t^, c_j) for j = D-1..1; then
//           v = v t^ (c_0 = 0) or fma(v, t^, c_0)               section 3.2
//   sigmoid  y = 1/2 + (v with x's sign bit xor-ed in)           Eq. 3
//   tanh     y = v xor sign(x)                                   section 3.1
//   SiLU/GELU y = fma(t, v, x * 1/2), t unclamped               Eqs. 4-6
//   sigmoid', tanh' (direct fits, even)  dx = g * v             section 3.3
//   SiLU', GELU' (direct fits, centered odd)
//            dx = g * (1/2 + (v xor sign(x)))                      Eq. 9
//
// FP16: one v_pk_fma_f16 / v_pk_mul_f16 / v_pk_add_f16 per stage for both
// lanes (IEEE single rounding).  BF16: gfx950 has no packed BF16 FMA, so each
// lane runs v_fma_f32 and the pair is rounded to BF16 with one
// v_cvt_pk_bf16_f32 (nearest even) per stage; the rounded pair is unpacked
// back to FP32 with a shift and a mask.
//
// The clamp is an unsigned integer minimum on the sign-cleared bits: for
// non-negative IEEE values integer order equals numeric order, and +inf
// clamps to Lc.  NaN lanes are replaced at the end by the input NaN with its
// quiet bit set (detected without compares: a sign-cleared half is NaN iff
// adding 0x03FF (FP16) / 0x007F (BF16) carries into its top bit).  SiLU and
// GELU map -inf to -0 with one more select.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { F_SIGMOID = 1, F_TANH = 2, F_SILU = 3, F_GELU = 4 };

template <class T, class F>
__device__ __forceinline__ T bc(F f) { return __builtin_bit_cast(T, f); }

// ---- lane-mask helpers ----------------------------------------------------
__device__ __forceinline__ uint32_t fill_sign16(uint32_t w)
{   // 0xFFFF in each half whose top bit is set, else 0 (v_pk_ashrrev_i16)
    return bc<uint32_t>(bc<i16x2>(w) >> (short)15);
}
__device__ __forceinline__ uint32_t sel(uint32_t mask, uint32_t a, uint32_t b)
{   // a where mask bits are set, else b (v_bfi_b32)
    return (a & mask) | (b & ~mask);
}
__device__ __forceinline__ uint32_t min_u16x2(uint32_t a, uint32_t b)
{
    return bc<uint32_t>(__builtin_elementwise_min(bc<u16x2>(a), bc<u16x2>(b)));
}
__device__ __forceinline__ uint32_t addsat_u16x2(uint32_t a, uint32_t b)
{
    return bc<uint32_t>(__builtin_elementwise_add_sat(bc<u16x2>(a), bc<u16x2>(b)));
}
// halves of |x| that are NaN: FP16 exponent all ones with nonzero fraction
__device__ __forceinline__ uint32_t nan_mask_f16(uint32_t aw) { return fill_sign16(aw + 0x03FF03FFu); }
__device__ __forceinline__ uint32_t nan_mask_bf16(uint32_t aw) { return fill_sign16(aw + 0x007F007Fu); }
// halves that are NOT -inf (xor with -inf leaves zero only there)
__device__ __forceinline__ uint32_t not_ninf_f16(uint32_t xw)
{
    return fill_sign16(addsat_u16x2(xw ^ 0xFC00FC00u, 0x7FFF7FFFu));
}
__device__ __forceinline__ uint32_t not_ninf_bf16(uint32_t xw)
{
    return fill_sign16(addsat_u16x2(xw ^ 0xFF80FF80u, 0x7FFF7FFFu));
}

// ---- BF16 pair helpers ----------------------------------------------------
__device__ __forceinline__ float lo_f(uint32_t w) { return bc<float>(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return bc<float>(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf(float a, float b)
{   // round both lanes to nearest even BF16 (v_cvt_pk_bf16_f32)
    bf2 r = {(__bf16)a, (__bf16)b};
    return bc<uint32_t>(r);
}

// ---- coefficients, passed by value as kernel arguments (SGPRs) -----------
struct CoefF16 {
    uint32_t c[8];   // FP16 coefficient duplicated into both halves
    uint32_t lc;     // FP16 Lc duplicated
};
struct CoefBF16 {
    float c[8];      // BF16 coefficient values as FP32
    uint32_t lc;     // FP32 bit pattern of Lc
};

// ---- FP16 programs ----------------------------------------------------------
template <int D, bool C0_ZERO>
__device__ __forceinline__ h2 horner_f16(h2 th, const CoefF16 &k)
{
    h2 v = bc<h2>(k.c[D]);
#pragma unroll
    for (int j = D - 1; j >= 1; --j) v = __builtin_elementwise_fma(v, th, bc<h2>(k.c[j]));
    if constexpr (C0_ZERO) return v * th;
    else return __builtin_elementwise_fma(v, th, bc<h2>(k.c[0]));
}

template <int FUNC, int D>
struct PolyFwdF16 {
    CoefF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw) const
    {
        const uint32_t aw = xw & 0x7FFF7FFFu;
        const uint32_t sw = xw ^ aw;
        const h2 v = horner_f16<D, true>(bc<h2>(min_u16x2(aw, k.lc)), k);
        uint32_t y;
        if constexpr (FUNC == F_SIGMOID) {
            y = bc<uint32_t>(bc<h2>(0x38003800u) + bc<h2>(bc<uint32_t>(v) ^ sw));
        } else if constexpr (FUNC == F_TANH) {
            y = bc<uint32_t>(v) ^ sw;
        } else {
            const h2 xh = bc<h2>(xw) * bc<h2>(0x38003800u);
            y = bc<uint32_t>(__builtin_elementwise_fma(bc<h2>(aw), v, xh));
            y = sel(not_ninf_f16(xw), y, 0x80008000u);
        }
        return sel(nan_mask_f16(aw), xw | 0x02000200u, y);
    }
};

template <int D>
struct PolyBwdF16 {   // even direct-derivative program, dx = g * q(t^)
    CoefF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw, uint32_t gw) const
    {
        const uint32_t aw = xw & 0x7FFF7FFFu;
        const h2 v = horner_f16<D, false>(bc<h2>(min_u16x2(aw, k.lc)), k);
        uint32_t y = bc<uint32_t>(bc<h2>(gw) * v);
        y = sel(nan_mask_f16(gw & 0x7FFF7FFFu), gw | 0x02000200u, y);
        return sel(nan_mask_f16(aw), xw | 0x02000200u, y);
    }
};

template <int D>
struct PolyBwdOddF16 {   // centered-odd direct-derivative program, dx = g (1/2 + sign q)
    CoefF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw, uint32_t gw) const
    {
        const uint32_t aw = xw & 0x7FFF7FFFu;
        const h2 v = horner_f16<D, true>(bc<h2>(min_u16x2(aw, k.lc)), k);
        const h2 ds = bc<h2>(0x38003800u) + bc<h2>(bc<uint32_t>(v) ^ (xw ^ aw));
        uint32_t y = bc<uint32_t>(bc<h2>(gw) * ds);
        y = sel(nan_mask_f16(gw & 0x7FFF7FFFu), gw | 0x02000200u, y);
        return sel(nan_mask_f16(aw), xw | 0x02000200u, y);
    }
};

// ---- BF16 programs ----------------------------------------------------------
// v rounded to nearest even BF16, as an FP32 value: v_cvt_pk_bf16_f32 with a
// zero low lane puts RN_bf16(v) in the high half, which is that FP32 value,
// so one instruction per lane replaces a packed convert and an unpack.
__device__ __forceinline__ float rn_bf16(float v)
{
    float r;   // the compiler would build {0, v} with a convert and a permute
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Horner stages D-1 .. 1 for the two lanes' clamped |x|: v0, v1 end as the
// BF16-rounded chain values (each stage one FP32 FMA and one rounding).
template <int D>
__device__ __forceinline__ void horner_bf16_mid(float t0, float t1, const CoefBF16 &k, float &v0, float &v1)
{
    v0 = k.c[D];
    v1 = k.c[D];
#pragma unroll
    for (int j = D - 1; j >= 1; --j) {
        v0 = rn_bf16(fmaf(v0, t0, k.c[j]));
        v1 = rn_bf16(fmaf(v1, t1, k.c[j]));
    }
}

// Returns the packed BF16 Horner value for the two lanes' clamped |x|.
template <int D, bool C0_ZERO>
__device__ __forceinline__ uint32_t horner_bf16(float t0, float t1, const CoefBF16 &k)
{
    float v0, v1;
    horner_bf16_mid<D>(t0, t1, k, v0, v1);
    if constexpr (C0_ZERO) return pack_bf(v0 * t0, v1 * t1);
    else return pack_bf(fmaf(v0, t0, k.c[0]), fmaf(v1, t1, k.c[0]));
}

// The forward program without the NaN select (used inside fused kernels,
// where a NaN gate already makes the product NaN).
template <int FUNC, int D>
__device__ __forceinline__ uint32_t poly_fwd_bf16_core(uint32_t xw, const CoefBF16 &k)
{
    const uint32_t aw = xw & 0x7FFF7FFFu;
    const uint32_t sw = xw ^ aw;
    const uint32_t a0 = aw << 16, a1 = aw & 0xFFFF0000u;
    const float t0 = bc<float>(a0 < k.lc ? a0 : k.lc);
    const float t1 = bc<float>(a1 < k.lc ? a1 : k.lc);
    if constexpr (FUNC == F_SIGMOID) {
        const uint32_t r = horner_bf16<D, true>(t0, t1, k) ^ sw;
        return pack_bf(0.5f + lo_f(r), 0.5f + hi_f(r));
    } else if constexpr (FUNC == F_TANH) {
        return horner_bf16<D, true>(t0, t1, k) ^ sw;
    } else {
        // x/2 + t v with v = RN(v t^) and x/2 rounded, each per lane
        float v0, v1;
        horner_bf16_mid<D>(t0, t1, k, v0, v1);
        v0 = rn_bf16(v0 * t0);
        v1 = rn_bf16(v1 * t1);
        const uint32_t y = pack_bf(fmaf(bc<float>(a0), v0, rn_bf16(lo_f(xw) * 0.5f)),
                                   fmaf(bc<float>(a1), v1, rn_bf16(hi_f(xw) * 0.5f)));
        return sel(not_ninf_bf16(xw), y, 0x80008000u);
    }
}

template <int FUNC, int D>
struct PolyFwdBF16 {
    CoefBF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw) const
    {
        const uint32_t y = poly_fwd_bf16_core<FUNC, D>(xw, k);
        return sel(nan_mask_bf16(xw & 0x7FFF7FFFu), xw | 0x00400040u, y);
    }
};

template <int D>
struct PolyBwdBF16 {
    CoefBF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw, uint32_t gw) const
    {
        const uint32_t aw = xw & 0x7FFF7FFFu;
        const uint32_t a0 = aw << 16, a1 = aw & 0xFFFF0000u;
        const float t0 = bc<float>(a0 < k.lc ? a0 : k.lc);
        const float t1 = bc<float>(a1 < k.lc ? a1 : k.lc);
        float v0, v1;
        horner_bf16_mid<D>(t0, t1, k, v0, v1);
        v0 = rn_bf16(fmaf(v0, t0, k.c[0]));
        v1 = rn_bf16(fmaf(v1, t1, k.c[0]));
        uint32_t y = pack_bf(lo_f(gw) * v0, hi_f(gw) * v1);
        y = sel(nan_mask_bf16(gw & 0x7FFF7FFFu), gw | 0x00400040u, y);
        return sel(nan_mask_bf16(aw), xw | 0x00400040u, y);
    }
};

template <int D>
struct PolyBwdOddBF16 {
    CoefBF16 k;
    __device__ __forceinline__ uint32_t operator()(uint32_t xw, uint32_t gw) const
    {
        const uint32_t aw = xw & 0x7FFF7FFFu;
        const uint32_t a0 = aw << 16, a1 = aw & 0xFFFF0000u;
        const float t0 = bc<float>(a0 < k.lc ? a0 : k.lc);
        const float t1 = bc<float>(a1 < k.lc ? a1 : k.lc);
        const uint32_t r = horner_bf16<D, true>(t0, t1, k) ^ (xw ^ aw);
        const uint32_t ds = pack_bf(0.5f + lo_f(r), 0.5f + hi_f(r));
        uint32_t y = pack_bf(lo_f(gw) * lo_f(ds), hi_f(gw) * hi_f(ds));
        y = sel(nan_mask_bf16(gw & 0x7FFF7FFFu), gw | 0x00400040u, y);
        return sel(nan_mask_bf16(aw), xw | 0x00400040u, y);
    }
};

// ---- accurate FP32 comparators ---------------------------------------------
// expf / tanhf / erfcf are the device library's accurate routines (no
// fast-math); 1.0f / d is the IEEE correctly rounded divide.
template <int FUNC>
__device__ __forceinline__ float native_fwd(float x)
{
    if constexpr (FUNC == F_SIGMOID) {
        const float e = expf(-fabsf(x));
        const float r = 1.0f / (1.0f + e);
        return x >= 0.0f ? r : e * r;
    } else if constexpr (FUNC == F_TANH) {
        return tanhf(x);
    } else if constexpr (FUNC == F_SILU) {
        // overflow-safe form: 1 + e stays in (1, 2]
        const float e = expf(-fabsf(x));
        const float r = 1.0f / (1.0f + e);
        return x == -INFINITY ? -0.0f : (x >= 0.0f ? x : x * e) * r;
    } else {
        return x == -INFINITY ? -0.0f : 0.5f * x * erfcf(-x * 0.70710678118654752440f);
    }
}

template <int FUNC, bool FROM_Y>
__device__ __forceinline__ float native_bwd(float xy, float g)
{
    if constexpr (FROM_Y) {
        if constexpr (FUNC == F_SIGMOID) return g * (xy * (1.0f - xy));
        else return g * (1.0f - xy * xy);
    } else {
        if constexpr (FUNC == F_SIGMOID) {   // sigma' = e / (1 + e)^2, e = exp(-|x|)
            const float e = expf(-fabsf(xy));
            const float r = 1.0f / (1.0f + e);
            return g * (e * r * r);
        } else if constexpr (FUNC == F_TANH) {   // tanh' = 4 e / (1 + e)^2, e = exp(-2|x|)
            const float e = expf(-2.0f * fabsf(xy));
            const float r = 1.0f / (1.0f + e);
            return g * (4.0f * e * r * r);
        } else if constexpr (FUNC == F_SILU) {   // s' = sigma (1 + x (1 - sigma))
            const float e = expf(-fabsf(xy));
            const float r = 1.0f / (1.0f + e);
            const float sg = xy >= 0.0f ? r : e * r;     // sigma(x)
            const float sn = xy >= 0.0f ? e * r : r;     // 1 - sigma(x) = sigma(-x)
            return g * (sg * fmaf(xy, sn, 1.0f));
        } else {                                 // GELU' = Phi(x) + x phi(x)
            const float phi = expf(-0.5f * xy * xy) * 0.39894228040143267794f;
            return g * fmaf(xy, phi, 0.5f * erfcf(-xy * 0.70710678118654752440f));
        }
    }
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)bc<h2>(w)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)bc<h2>(w)[1]; }
__device__ __forceinline__ uint32_t pack_f16(float a, float b)
{
    h2 r = {(_Float16)a, (_Float16)b};
    return bc<uint32_t>(r);
}

template <int FUNC, bool BF>
struct NativeFwd {
    __device__ __forceinline__ uint32_t operator()(uint32_t xw) const
    {
        if constexpr (BF) return pack_bf(native_fwd<FUNC>(lo_f(xw)), native_fwd<FUNC>(hi_f(xw)));
        else return pack_f16(native_fwd<FUNC>(f16_lo(xw)), native_fwd<FUNC>(f16_hi(xw)));
    }
};

template <int FUNC, bool BF, bool FROM_Y>
struct NativeBwd {
    __device__ __forceinline__ uint32_t operator()(uint32_t xw, uint32_t gw) const
    {
        if constexpr (BF)
            return pack_bf(native_bwd<FUNC, FROM_Y>(lo_f(xw), lo_f(gw)),
                           native_bwd<FUNC, FROM_Y>(hi_f(xw), hi_f(gw)));
        else
            return pack_f16(native_bwd<FUNC, FROM_Y>(f16_lo(xw), f16_lo(gw)),
                            native_bwd<FUNC, FROM_Y>(f16_hi(xw), f16_hi(gw)));
    }
};

}  // namespace pa
