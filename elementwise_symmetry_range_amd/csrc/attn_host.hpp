// attn_host.hpp -- argument validation and launches of the attention kernels.
#pragma once
#include <atomic>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "../../include/polyact.h"
#include "attn.hpp"
#include "attn_bwd.hpp"
#include "attn_programs.hpp"
#include "programs.hpp"

namespace pa {

struct Span {
    const void *p;
    int64_t bytes;
};

inline bool spans_overlap(const Span &a, const Span &b)
{
    if (a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
    return x < y + (uintptr_t)b.bytes && y < x + (uintptr_t)a.bytes;
}

// Every output against every other buffer (outputs and inputs).
inline bool any_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins)
{
    for (const Span *o = outs.begin(); o != outs.end(); ++o) {
        for (const Span *p = outs.begin(); p != outs.end(); ++p)
            if (p != o && spans_overlap(*o, *p)) return true;
        for (const Span &i : ins)
            if (spans_overlap(*o, i)) return true;
    }
    return false;
}

inline bool aligned16(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if ((uintptr_t)p & 15u) return false;
    return true;
}

// Shape rules shared by every attention entry point.
inline pa_status attn_shape(int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D)
{
    // S + 255 must fit int32 (the kernels' tile counts)
    if (B < 0 || H < 0 || Hkv < 0 || S < 0 || S > 0x7FFFFFFF - 256 || D != AT_D) return PA_ERR_SHAPE;
    if ((int64_t)B * H > 0 && (Hkv == 0 || H % Hkv != 0)) return PA_ERR_SHAPE;
    const int64_t tiles = ((int64_t)S + AT_BM - 1) / AT_BM;
    if ((int64_t)B * H * tiles > 0x7FFFFFFF) return PA_ERR_SHAPE;
    return PA_OK;
}

inline bool cap_ok(float cap) { return cap > 0.0f && cap != INFINITY; }

inline uint32_t f16_dup(float v)
{
    const _Float16 h = (_Float16)v;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return (uint32_t)b | ((uint32_t)b << 16);
}

inline float bf16_value(uint16_t bits)
{
    const uint32_t w = (uint32_t)bits << 16;
    float v;
    std::memcpy(&v, &w, 4);
    return v;
}

// Round an FP32 value to the nearest BF16 value, ties to even (finite input).
inline float bf16_round(float v)
{
    uint32_t w;
    std::memcpy(&w, &v, 4);
    w = (w + 0x7FFFu + ((w >> 16) & 1u)) & 0xFFFF0000u;
    float r;
    std::memcpy(&r, &w, 4);
    return r;
}

// The D4 tanh program and its analytic derivative (coefficients (j + 1)
// c_{j+1}, all exact in FP16) in FP16.
inline void tanh_coefs(CoefF16 &fwd, CoefF16 &der)
{
    const ProgramDef *p = find_program(PA_TANH, 0);
    fwd = CoefF16{};
    der = CoefF16{};
    for (int j = 0; j <= p->degree; ++j) fwd.c[j] = f16_dup(bf16_value(p->coeff[j]));
    for (int j = 0; j < p->degree; ++j) der.c[j] = f16_dup((float)(j + 1) * bf16_value(p->coeff[j + 1]));
    fwd.lc = der.lc = f16_dup(p->Lc);
}

// The same program in BF16, and its derivative with the coefficients
// (j + 1) c_{j+1} rounded to BF16 (3 c_3 needs more than 8 bits).
inline void tanh_coefs_bf16(TanhBF16 &fwd, TanhBF16 &der)
{
    const ProgramDef *p = find_program(PA_TANH, 0);
    fwd = TanhBF16{};
    der = TanhBF16{};
    for (int j = 0; j <= p->degree && j < 5; ++j) fwd.c[j] = bf16_value(p->coeff[j]);
    for (int j = 0; j < p->degree && j < 4; ++j) der.c[j] = bf16_round((float)(j + 1) * bf16_value(p->coeff[j + 1]));
    fwd.lc = der.lc = p->Lc;
}

// The FP16 encoding of a BF16 value, or -1 when FP16 cannot hold it exactly.
// A finite nonzero BF16 value is (128 + m) 2^(e - 7) with a 7-bit m; FP16
// holds it as a normal number for -14 <= e <= 15 and, below, as a multiple
// of 2^-24 when the low bits that would fall off are zero.
constexpr int32_t bf16_as_f16(uint16_t b)
{
    const uint32_t s = uint32_t(b >> 15), E = (b >> 7) & 0xFFu, m = b & 0x7Fu;
    if (E == 0 && m == 0) return int32_t(s << 15);
    if (E == 0 || E == 0xFF) return -1;
    const int e = int(E) - 127;
    if (e > 15) return -1;
    if (e >= -14) return int32_t((s << 15) | (uint32_t(e + 15) << 10) | (m << 3));
    uint32_t n = 128 + m;              // units of 2^(e - 7); FP16 subnormals count 2^-24
    const int sh = e - 7 + 24;
    if (sh >= 0) {
        n <<= sh;
    } else {
        if (n & ((1u << -sh) - 1)) return -1;
        n >>= -sh;
    }
    return int32_t((s << 15) | n);     // n < 1024 here
}

constexpr bool sigmoid_coefs_are_f16()
{
    for (int r = 0; r < 2; ++r) {
        for (int j = 0; j < 4; ++j)
            if (bf16_as_f16(kSigmoidAttn.c[r][j]) < 0) return false;
        if (bf16_as_f16(kSigmoidAttn.a[r]) < 0 || bf16_as_f16(kSigmoidAttn.b[r]) < 0) return false;
    }
    return true;
}
static_assert(sigmoid_coefs_are_f16(), "the sigmoid kernels read the coefficients as FP16");
static_assert(bf16_as_f16(0x3F80) == 0x3C00 && bf16_as_f16(0x37E8) == 0x01D0 &&
              bf16_as_f16(0xB380) == 0x8001 && bf16_as_f16(0x3381) == -1,
              "BF16 to FP16: normal, subnormal and inexact cases");

inline SigCoef sigmoid_coefs()
{
    const SigmoidAttnDef &d = kSigmoidAttn;
    auto pair = [](uint16_t lo, uint16_t hi) {
        return uint32_t(uint16_t(bf16_as_f16(lo))) | (uint32_t(uint16_t(bf16_as_f16(hi))) << 16);
    };
    SigCoef k{};
    for (int r = 0; r < 2; ++r) {
        k.c23[r] = pair(d.c[r][2], d.c[r][3]);
        k.c01[r] = pair(d.c[r][0], d.c[r][1]);
        k.ab[r] = pair(d.a[r], d.b[r]);
    }
    k.thr = bf16_value(d.thr);
    k.lo = bf16_value(d.lo);
    k.hi = bf16_value(d.hi);
    return k;
}

inline pa_status attn_launched() { return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

template <int MODE, int EXP, bool SREF>
inline void attn_fwd_launch(const AttnArgs &a, dim3 grid, hipStream_t stream)
{
    hipLaunchKernelGGL((k_attn_fwd<MODE, EXP, SREF>), grid, dim3(256), 0, stream, a);
}

// exp2_core: 0 the hardware exponential, 1-4 a software core (the BF16
// softcap program only).
inline pa_status attn_fwd(int mode, const void *q, const void *k, const void *v, void *o, float *lse,
                          int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D, float cap,
                          int32_t causal, hipStream_t stream, int exp2_core = 0)
{
    if (exp2_core < 0 || exp2_core > 4 || (exp2_core && mode != AM_SOFTCAP_POLY_BF16)) return PA_ERR_FUNC;
    if (!q || !k || !v || !o) return PA_ERR_NULL;
    if (!aligned16({q, k, v, o}) || ((uintptr_t)lse & 3u)) return PA_ERR_ALIGN;
    pa_status st = attn_shape(B, H, Hkv, S, D);
    if (st != PA_OK) return st;
    const bool softcap = am_softcap(mode);
    if (softcap && !cap_ok(cap)) return PA_ERR_SHAPE;
    if (mode == AM_SIGMOID_POLY && S != kSigmoidAttn.n && (int64_t)B * H * S > 0) return PA_ERR_SHAPE;
    const int64_t qb = (int64_t)B * H * S * D * 2, kb = (int64_t)B * Hkv * S * D * 2;
    const int64_t lb = lse ? (int64_t)B * H * S * 4 : 0;
    if (any_overlap({{o, qb}, {lse, lb}}, {{q, qb}, {k, kb}, {v, kb}})) return PA_ERR_OVERLAP;
    if ((int64_t)B * H == 0 || S == 0) return PA_OK;
    AttnArgs a{};
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (uint16_t *)o;
    a.lse = softcap ? lse : nullptr;
    a.S = S;
    a.H = H;
    a.G = H / Hkv;
    a.causal = causal ? 1 : 0;
    if (softcap) {
        a.scale = (float)(1.0 / ((double)cap * std::sqrt((double)D)));
        a.c2 = (float)((double)cap * 1.4426950408889634074);
        CoefF16 der;
        tanh_coefs(a.tanh16, der);
        TanhBF16 derb;
        tanh_coefs_bf16(a.tanhbf, derb);
    } else {
        a.scale = (float)(1.0 / std::sqrt((double)D));
        a.logn = (float)std::log((double)S);
        a.sig = sigmoid_coefs();
    }
    const dim3 grid((unsigned)(((S + AT_BM - 1) / AT_BM) * (B * H)));
    // the fixed reference while every logit's exponent fits (cap log2 e <= 80)
    const bool sref = softcap && a.c2 <= 80.0f;
    if (sref) a.mref = std::ceil(a.c2 - 40.0f);
    switch (mode) {
    case AM_SOFTCAP_POLY_BF16:
        switch (exp2_core * 2 + (sref ? 1 : 0)) {
        case 0: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 0, false>(a, grid, stream); break;
        case 1: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 0, true>(a, grid, stream); break;
        case 2: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 1, false>(a, grid, stream); break;
        case 3: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 1, true>(a, grid, stream); break;
        case 4: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 2, false>(a, grid, stream); break;
        case 5: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 2, true>(a, grid, stream); break;
        case 6: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 3, false>(a, grid, stream); break;
        case 7: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 3, true>(a, grid, stream); break;
        case 8: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 4, false>(a, grid, stream); break;
        default: attn_fwd_launch<AM_SOFTCAP_POLY_BF16, 4, true>(a, grid, stream); break;
        }
        break;
    case AM_SOFTCAP_POLY:
        if (sref) attn_fwd_launch<AM_SOFTCAP_POLY, 0, true>(a, grid, stream);
        else attn_fwd_launch<AM_SOFTCAP_POLY, 0, false>(a, grid, stream);
        break;
    case AM_SOFTCAP_NATIVE:
        if (sref) attn_fwd_launch<AM_SOFTCAP_NATIVE, 0, true>(a, grid, stream);
        else attn_fwd_launch<AM_SOFTCAP_NATIVE, 0, false>(a, grid, stream);
        break;
    case AM_SIGMOID_POLY: attn_fwd_launch<AM_SIGMOID_POLY, 0, false>(a, grid, stream); break;
    default: attn_fwd_launch<AM_SIGMOID_NATIVE, 0, false>(a, grid, stream); break;
    }
    return attn_launched();
}

// Bytes of the BF16 dS blocks of a backward: B H x 4 ceil(nqb / 4) x nqb
// blocks of 32 x 32, nqb = ceil(S / 32) (every block of the square, the
// query blocks padded to groups of four, so the size does not depend on the
// causal flag; a causal call writes and reads the lower triangle only).
inline int64_t attn_bwd_ds_bytes(int32_t B, int32_t H, int32_t S)
{
    const int64_t nqb = ((int64_t)S + 31) / 32;
    const double est = (double)B * H * (double)((nqb + 3) / 4 * 4) * (double)nqb * 2048.0;
    if (est > 4.0e18) return INT64_MAX;   // beyond any limit (and int64)
    return (int64_t)B * H * ((nqb + 3) / 4 * 4) * nqb * 2048;
}

// The backward stores dS for dQ (dK/dV kernel, then a dQ product over the
// stored blocks: the score transform runs once) when the blocks take at
// most the process-wide limit (16 GiB unless pa_attn_bwd_ds_limit changes
// it); above that the dQ kernel recomputes S, dP and the transform (twice
// the transform, no quadratic storage).  Both give the same dQ, dK and dV.
inline std::atomic<int64_t> &attn_ds_limit()
{
    static std::atomic<int64_t> limit{int64_t(16) << 30};
    return limit;
}
inline bool attn_bwd_use_ds(int32_t B, int32_t H, int32_t S)
{
    const int64_t b = attn_bwd_ds_bytes(B, H, S);
    return b != INT64_MAX && b <= attn_ds_limit().load(std::memory_order_relaxed);
}

// Workspace of a backward call, in floats: Delta and -lse log2(e) per query
// row (softcap; each region padded to 16 bytes), then, for grouped query
// heads, FP32 dK and dV partials per query head, then (ds) the dS blocks.
// 0 when none is needed.
inline int64_t attn_bwd_ws_floats(bool softcap, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                  int32_t D, bool ds)
{
    const int64_t rows = (int64_t)B * H * S;
    int64_t n = softcap ? 2 * ((rows + 3) / 4 * 4) : 0;
    if (Hkv > 0 && H > Hkv) n += 2 * rows * D;
    if (ds) n += attn_bwd_ds_bytes(B, H, S) / 4;
    return n;
}

template <int MODE, int EXP = 0>
inline void attn_bwd_launch(const AttnBwdArgs &a, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                            hipStream_t stream)
{
    const dim3 gq((unsigned)(((S + AT_BM - 1) / AT_BM) * (B * H)));
    if (!a.dsb) {
        hipLaunchKernelGGL((k_attn_bwd_dq<MODE, EXP>), gq, dim3(256), 0, stream, a);
    } else if (am_softcap(MODE)) {
        const int64_t rows = (int64_t)B * H * S;
        hipLaunchKernelGGL(k_attn_bwd_rows, dim3((unsigned)((rows + 127) / 128)), dim3(256), 0, stream, a, rows);
    }
    const int ntk = (S + AT_BK - 1) / AT_BK;
    if (H == Hkv) {
        hipLaunchKernelGGL((k_attn_bwd_dkdv<MODE, false, EXP>), dim3((unsigned)(ntk * B * Hkv)), dim3(512), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((k_attn_bwd_dkdv<MODE, true, EXP>), dim3((unsigned)(ntk * B * H)), dim3(512), 0,
                           stream, a);
        const int64_t n8 = (int64_t)B * Hkv * S * AT_D / 8;
        hipLaunchKernelGGL(k_attn_bwd_reduce, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a, n8,
                           (int64_t)S * AT_D);
    }
    if (a.dsb) {
        // 4 waves (128 queries) per workgroup: 8 waves, which halve the K
        // tile reads per query, measured the same on MI355X
        constexpr int NW = 4;
        const dim3 gd((unsigned)(((S + NW * 32 - 1) / (NW * 32)) * (B * H)));
        hipLaunchKernelGGL(k_attn_bwd_dq_ds<NW>, gd, dim3(NW * 64), 0, stream, a);
    }
}

// o, lse and ws are used by the softcap modes only.
inline pa_status attn_bwd(int mode, const void *q, const void *k, const void *v, const void *o,
                          const void *dout, const float *lse, void *dq, void *dk, void *dv, float *ws,
                          int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D, float cap,
                          int32_t causal, hipStream_t stream, int exp2_core = 0, bool allow_ds = true)
{
    if (exp2_core < 0 || exp2_core > 4 || (exp2_core && mode != AM_SOFTCAP_POLY_BF16)) return PA_ERR_FUNC;
    const bool softcap = am_softcap(mode);
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return PA_ERR_NULL;
    if (softcap && (!o || !lse)) return PA_ERR_NULL;
    pa_status st = attn_shape(B, H, Hkv, S, D);
    if (st != PA_OK) return st;
    // no workspace (allowed for sigmoid with H == Hkv): the recompute form
    const bool ds = allow_ds && ws && attn_bwd_use_ds(B, H, S);
    const int64_t wsn = attn_bwd_ws_floats(softcap, B, H, Hkv, S, D, ds);
    if (wsn > 0 && !ws) return PA_ERR_NULL;
    if (!aligned16({q, k, v, dout, dq, dk, dv, ws}) || (softcap && !aligned16({o})) ||
        ((uintptr_t)lse & 3u))
        return PA_ERR_ALIGN;
    if (softcap && !cap_ok(cap)) return PA_ERR_SHAPE;
    if (mode == AM_SIGMOID_POLY && S != kSigmoidAttn.n && (int64_t)B * H * S > 0) return PA_ERR_SHAPE;
    if ((int64_t)B * Hkv * ((S + AT_BK - 1) / AT_BK) > 0x7FFFFFFF) return PA_ERR_SHAPE;
    const int64_t qb = (int64_t)B * H * S * D * 2, kb = (int64_t)B * Hkv * S * D * 2;
    const int64_t rb = softcap ? (int64_t)B * H * S * 4 : 0;
    if (any_overlap({{dq, qb}, {dk, kb}, {dv, kb}, {ws, wsn * 4}},
                    {{q, qb}, {k, kb}, {v, kb}, {o, softcap ? qb : 0}, {dout, qb}, {lse, rb}}))
        return PA_ERR_OVERLAP;
    if ((int64_t)B * H == 0 || S == 0) return PA_OK;
    AttnBwdArgs a{};
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (const uint16_t *)o;
    a.dout = (const uint16_t *)dout;
    a.lse = lse;
    const int64_t rows4 = ((int64_t)B * H * S + 3) / 4 * 4;
    a.delta = softcap ? ws : nullptr;
    a.nlse = softcap ? ws + rows4 : nullptr;
    a.part = H > Hkv ? ws + (softcap ? 2 * rows4 : 0) : nullptr;
    a.dsb = ds ? (uint16_t *)(ws + attn_bwd_ws_floats(softcap, B, H, Hkv, S, D, false)) : nullptr;
    a.nqb = (S + 31) / 32;
    a.dq = (uint16_t *)dq;
    a.dk = (uint16_t *)dk;
    a.dv = (uint16_t *)dv;
    a.S = S;
    a.H = H;
    a.G = H / Hkv;
    a.causal = causal ? 1 : 0;
    a.rsd = (float)(1.0 / std::sqrt((double)D));
    if (softcap) {
        a.scale = (float)(1.0 / ((double)cap * std::sqrt((double)D)));
        a.c2 = (float)((double)cap * 1.4426950408889634074);
        tanh_coefs(a.tanh16, a.dtanh16);
        tanh_coefs_bf16(a.tanhbf, a.dtanhbf);
    } else {
        a.scale = a.rsd;
        a.logn = (float)std::log((double)S);
        a.sig = sigmoid_coefs();
    }
    switch (mode) {
    case AM_SOFTCAP_POLY_BF16:
        switch (exp2_core) {
        case 1: attn_bwd_launch<AM_SOFTCAP_POLY_BF16, 1>(a, B, H, Hkv, S, stream); break;
        case 2: attn_bwd_launch<AM_SOFTCAP_POLY_BF16, 2>(a, B, H, Hkv, S, stream); break;
        case 3: attn_bwd_launch<AM_SOFTCAP_POLY_BF16, 3>(a, B, H, Hkv, S, stream); break;
        case 4: attn_bwd_launch<AM_SOFTCAP_POLY_BF16, 4>(a, B, H, Hkv, S, stream); break;
        default: attn_bwd_launch<AM_SOFTCAP_POLY_BF16, 0>(a, B, H, Hkv, S, stream); break;
        }
        break;
    case AM_SOFTCAP_POLY: attn_bwd_launch<AM_SOFTCAP_POLY>(a, B, H, Hkv, S, stream); break;
    case AM_SOFTCAP_NATIVE: attn_bwd_launch<AM_SOFTCAP_NATIVE>(a, B, H, Hkv, S, stream); break;
    case AM_SIGMOID_POLY: attn_bwd_launch<AM_SIGMOID_POLY>(a, B, H, Hkv, S, stream); break;
    default: attn_bwd_launch<AM_SIGMOID_NATIVE>(a, B, H, Hkv, S, stream); break;
    }
    return attn_launched();
}

}  // namespace pa
