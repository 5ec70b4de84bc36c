// polyact.hip -- C ABI of the gfx950 polynomial activation library: argument
// validation, program lookup and kernel dispatch.  See include/polyact.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/polyact.h"
#include "attn_host.hpp"
#include "ops.hpp"
#include "programs.hpp"
#include "rope.hpp"
#include "stream_launch.hpp"
#include "swiglu.hpp"

using namespace pa;

namespace {

pa_status launched()
{
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status check_ptr(const void *p)
{
    if (!p) return PA_ERR_NULL;
    if ((uintptr_t)p & 1u) return PA_ERR_ALIGN;
    return PA_OK;
}

// [a, a + na) and [b, b + nb) bytes overlap but are not the same range start
bool partial_overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    if (x == y) return false;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}
bool any_overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

CoefF16 coef_f16(const ProgramDef &p)
{
    CoefF16 k{};
    for (int j = 0; j <= p.degree; ++j) {
        uint32_t fbits = (uint32_t)p.coeff[j] << 16;
        float v;
        std::memcpy(&v, &fbits, 4);
        const _Float16 h = (_Float16)v;   // exact: the fitted values fit FP16
        uint16_t hb;
        std::memcpy(&hb, &h, 2);
        k.c[j] = (uint32_t)hb | ((uint32_t)hb << 16);
    }
    const _Float16 l = (_Float16)p.Lc;
    uint16_t lb;
    std::memcpy(&lb, &l, 2);
    k.lc = (uint32_t)lb | ((uint32_t)lb << 16);
    return k;
}

CoefBF16 coef_bf16(const ProgramDef &p)
{
    CoefBF16 k{};
    for (int j = 0; j <= p.degree; ++j) {
        uint32_t fbits = (uint32_t)p.coeff[j] << 16;
        std::memcpy(&k.c[j], &fbits, 4);
    }
    std::memcpy(&k.lc, &p.Lc, 4);
    return k;
}

pa_status check_unary(int32_t t, const void *x, const void *y, int64_t n)
{
    if (t != PA_F16 && t != PA_BF16) return PA_ERR_DTYPE;
    if (n < 0) return PA_ERR_SHAPE;
    pa_status s = check_ptr(x);
    if (s != PA_OK) return s;
    if ((s = check_ptr(y)) != PA_OK) return s;
    if (partial_overlap(y, 2 * n, x, 2 * n)) return PA_ERR_OVERLAP;
    return PA_OK;
}

pa_status check_binary(int32_t t, const void *x, const void *g, const void *y, int64_t n)
{
    pa_status s = check_unary(t, x, y, n);
    if (s != PA_OK) return s;
    if ((s = check_ptr(g)) != PA_OK) return s;
    if (partial_overlap(y, 2 * n, g, 2 * n)) return PA_ERR_OVERLAP;
    return PA_OK;
}

template <int F, int D>
pa_status poly_fwd_dispatch(const ProgramDef &p, int32_t t, const void *x, void *y, int64_t n,
                            hipStream_t st)
{
    if (t == PA_F16) return run_map1(x, y, n, st, PolyFwdF16<F, D>{coef_f16(p)});
    return run_map1(x, y, n, st, PolyFwdBF16<F, D>{coef_bf16(p)});
}

template <int F, bool FROM_Y>
pa_status native_bwd_dispatch(int32_t t, const void *x, const void *g, void *y, int64_t n,
                              hipStream_t st)
{
    if (t == PA_F16) return run_map2(x, g, y, n, st, NativeBwd<F, false, FROM_Y>{});
    return run_map2(x, g, y, n, st, NativeBwd<F, true, FROM_Y>{});
}

// ---- SwiGLU -------------------------------------------------------------------
pa_status check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld)
{
    pa_status s = check_ptr(p);
    if (s != PA_OK) return s;
    if (ld < cols) return PA_ERR_SHAPE;
    (void)rows;
    return PA_OK;
}
int64_t extent_bytes(int64_t rows, int64_t cols, int64_t ld)
{
    return rows == 0 ? 0 : 2 * ((rows - 1) * ld + cols);
}

bool vec_ok(const SwiArgs &a, bool bwd)
{
    if (a.cols % 8) return false;
    const int64_t lds[6] = {a.ld_g, a.ld_u, bwd ? a.ld_dh : 8, bwd ? a.ld_dg : a.ld_h,
                            bwd ? a.ld_du : 8, 8};
    for (int64_t ld : lds)
        if (ld % 8) return false;
    const void *ps[5] = {a.g, a.u, bwd ? (const void *)a.dh : (const void *)a.g,
                         bwd ? (const void *)a.dg : (const void *)a.h,
                         bwd ? (const void *)a.du : (const void *)a.g};
    for (const void *p : ps)
        if ((uintptr_t)p & 15u) return false;
    return true;
}
bool flat(const SwiArgs &a, bool bwd)
{
    if (bwd)
        return a.ld_g == a.cols && a.ld_u == a.cols && a.ld_dh == a.cols && a.ld_dg == a.cols &&
               a.ld_du == a.cols;
    return a.ld_g == a.cols && a.ld_u == a.cols && a.ld_h == a.cols;
}

template <class Op>
pa_status swiglu_fwd_launch(const SwiArgs &a, hipStream_t st, const Op &op)
{
    if (vec_ok(a, false)) {
        const int64_t chunks = a.rows * (a.cols / 8);
        const bool small = chunks <= kSmallChunks;
        const int bs = small ? kSmallBS : kMap2BS;
        const dim3 grid((unsigned)grid_tiles(chunks, (int64_t)bs * kMap2U));
        if (small && flat(a, false))
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kSmallBS, kMap2U, true>), grid, dim3(bs), 0, st, a, op);
        else if (small)
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kSmallBS, kMap2U, false>), grid, dim3(bs), 0, st, a, op);
        else if (flat(a, false))
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kMap2BS, kMap2U, true>), grid, dim3(bs), 0, st, a, op);
        else
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kMap2BS, kMap2U, false>), grid, dim3(bs), 0, st, a, op);
    } else {
        hipLaunchKernelGGL((k_swiglu_fwd_scalar<Op>), dim3((unsigned)grid_for(a.rows * a.cols, 1)),
                           dim3(kThreads), 0, st, a, op);
    }
    return launched();
}

template <class Op>
pa_status swiglu_bwd_launch(const SwiArgs &a, hipStream_t st, const Op &op)
{
    if (vec_ok(a, true)) {
        const int64_t chunks = a.rows * (a.cols / 8);
        const bool small = chunks <= kSmallChunks;
        const int bs = small ? kSmallBS : kMap2BS;
        const dim3 grid((unsigned)grid_tiles(chunks, (int64_t)bs * kMap2U));
        if (small && flat(a, true))
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kSmallBS, kMap2U, true>), grid, dim3(bs), 0, st, a, op);
        else if (small)
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kSmallBS, kMap2U, false>), grid, dim3(bs), 0, st, a, op);
        else if (flat(a, true))
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kMap2BS, kMap2U, true>), grid, dim3(bs), 0, st, a, op);
        else
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kMap2BS, kMap2U, false>), grid, dim3(bs), 0, st, a, op);
    } else {
        hipLaunchKernelGGL((k_swiglu_bwd_scalar<Op>), dim3((unsigned)grid_for(a.rows * a.cols, 1)),
                           dim3(kThreads), 0, st, a, op);
    }
    return launched();
}

pa_status swiglu_fwd_check(int32_t t, const void *gate, const void *up, void *h, int64_t rows,
                           int64_t cols, int64_t ldg, int64_t ldu, int64_t ldh,
                           const int64_t *off, int32_t ng)
{
    if (t != PA_BF16) return PA_ERR_DTYPE;
    if (rows < 0 || cols < 0) return PA_ERR_SHAPE;
    pa_status s;
    if ((s = check_matrix(gate, rows, cols, ldg)) != PA_OK) return s;
    if ((s = check_matrix(up, rows, cols, ldu)) != PA_OK) return s;
    if ((s = check_matrix(h, rows, cols, ldh)) != PA_OK) return s;
    if (off && ng < 0) return PA_ERR_SHAPE;
    if (off && ((uintptr_t)off & 7u)) return PA_ERR_ALIGN;
    const int64_t eg = extent_bytes(rows, cols, ldg), eu = extent_bytes(rows, cols, ldu),
                  eh = extent_bytes(rows, cols, ldh);
    if (any_overlap(h, eh, gate, eg) && !(h == gate && ldh == ldg)) return PA_ERR_OVERLAP;
    if (any_overlap(h, eh, up, eu) && !(h == up && ldh == ldu)) return PA_ERR_OVERLAP;
    return PA_OK;
}

pa_status swiglu_bwd_check(int32_t t, const void *gate, const void *up, const void *dh,
                           void *dgate, void *dup, int64_t rows, int64_t cols, int64_t ldg,
                           int64_t ldu, int64_t lddh, int64_t lddg, int64_t lddu,
                           const int64_t *off, int32_t ng)
{
    if (t != PA_BF16) return PA_ERR_DTYPE;
    if (rows < 0 || cols < 0) return PA_ERR_SHAPE;
    pa_status s;
    if ((s = check_matrix(gate, rows, cols, ldg)) != PA_OK) return s;
    if ((s = check_matrix(up, rows, cols, ldu)) != PA_OK) return s;
    if ((s = check_matrix(dh, rows, cols, lddh)) != PA_OK) return s;
    if ((s = check_matrix(dgate, rows, cols, lddg)) != PA_OK) return s;
    if ((s = check_matrix(dup, rows, cols, lddu)) != PA_OK) return s;
    if (off && ng < 0) return PA_ERR_SHAPE;
    if (off && ((uintptr_t)off & 7u)) return PA_ERR_ALIGN;
    const void *in[3] = {gate, up, dh};
    const int64_t inld[3] = {ldg, ldu, lddh};
    void *out[2] = {dgate, dup};
    const int64_t outld[2] = {lddg, lddu};
    if (any_overlap(dgate, extent_bytes(rows, cols, lddg), dup, extent_bytes(rows, cols, lddu)))
        return PA_ERR_OVERLAP;
    for (int o = 0; o < 2; ++o)
        for (int i = 0; i < 3; ++i)
            if (any_overlap(out[o], extent_bytes(rows, cols, outld[o]), in[i],
                            extent_bytes(rows, cols, inld[i])) &&
                !(out[o] == in[i] && outld[o] == inld[i]))
                return PA_ERR_OVERLAP;
    return PA_OK;
}

SwiArgs swi_args(const void *gate, const void *up, const void *dh, void *h, void *dg, void *du,
                 int64_t rows, int64_t cols, int64_t ldg, int64_t ldu, int64_t lddh, int64_t ldh,
                 int64_t lddg, int64_t lddu, const int64_t *off, int32_t ng)
{
    SwiArgs a;
    a.g = (const uint16_t *)gate;
    a.u = (const uint16_t *)up;
    a.dh = (const uint16_t *)dh;
    a.h = (uint16_t *)h;
    a.dg = (uint16_t *)dg;
    a.du = (uint16_t *)du;
    a.rows = rows;
    a.cols = cols;
    a.ld_g = ldg;
    a.ld_u = ldu;
    a.ld_dh = lddh;
    a.ld_h = ldh;
    a.ld_dg = lddg;
    a.ld_du = lddu;
    a.off = off;
    a.n_groups = ng;
    return a;
}

const ProgramDef &sigmoid_d3() { return *find_program(PA_SIGMOID, 0); }

}  // namespace

namespace {
// No arithmetic: the streaming kernels' own HBM rate (pa_stream_copy).
struct CopyOp {
    __device__ __forceinline__ uint32_t operator()(uint32_t aw) const { return aw; }
};
struct XorOp {
    __device__ __forceinline__ uint32_t operator()(uint32_t aw, uint32_t bw) const { return aw ^ bw; }
};
}  // namespace

// =============================================================================
namespace {

// FP16 value of a BF16 coefficient, duplicated into both halves (exact: the
// rotary coefficients have at most 8 significant bits and FP16 exponents)
uint32_t bf16_coef_f16x2(uint16_t b)
{
    uint32_t fbits = (uint32_t)b << 16;
    float v;
    std::memcpy(&v, &fbits, 4);
    const _Float16 h = (_Float16)v;
    uint16_t hb;
    std::memcpy(&hb, &h, 2);
    return (uint32_t)hb | ((uint32_t)hb << 16);
}

// shape checks shared by the rotary entry points; fills the sizes and the
// turn increments inc_i = round(w_i 2^32 / (2 pi)), w_i = base^(-2 i / D)
pa_status rope_args(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, double base, bool need_base,
                    RopeArgs &a)
{
    if (B < 0 || S < 0 || Hq < 0 || Hkv < 0) return PA_ERR_SHAPE;
    if (D < 8 || D > RP_MAX_D || D % 8) return PA_ERR_SHAPE;
    if (need_base && !(std::isfinite(base) && base >= 1.0)) return PA_ERR_SHAPE;
    const int64_t rows = (int64_t)B * S;
    if (rows > ((int64_t)1 << 40) || (int64_t)(Hq > Hkv ? Hq : Hkv) * D > ((int64_t)1 << 24)) return PA_ERR_SHAPE;
    if ((rows * ((Hq + Hkv + RP_HPG - 1) / RP_HPG) * (D / 8) + 255) / 256 > 0x7FFFFFFF) return PA_ERR_SHAPE;
    a = RopeArgs{};
    a.rows = rows;
    a.S = S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    for (int j = 0; j < 3; ++j) a.sc[j] = bf16_coef_f16x2(kRopeSin[j]);
    for (int j = 0; j < 4; ++j) a.cc[j] = bf16_coef_f16x2(kRopeCos[j]);
    if (need_base) {
        const double turn = 4294967296.0 / (2.0 * 3.14159265358979323846);
        for (int i = 0; i < D / 2; ++i)
            a.inc[i] = (uint32_t)std::llround(std::pow(base, -2.0 * i / (double)D) * turn);
    }
    return PA_OK;
}

pa_status rope_run(int var, const void *q, const void *k, void *q_out, void *k_out, const void *table,
                   int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, double base, hipStream_t stream)
{
    RopeArgs a;
    pa_status st = rope_args(B, S, Hq, Hkv, D, base, var != RP_TABLE, a);
    if (st != PA_OK) return st;
    if (!q || !k || !q_out || !k_out || (var == RP_TABLE && !table)) return PA_ERR_NULL;
    if (!aligned16({q, k, q_out, k_out}) || (var == RP_TABLE && !aligned16({table}))) return PA_ERR_ALIGN;
    const int64_t qb = a.rows * Hq * D * 2, kb = a.rows * Hkv * D * 2;
    const int64_t tb = var == RP_TABLE ? (int64_t)S * (D / 2) * 4 : 0;
    if (pa::any_overlap({{q_out, qb}, {k_out, kb}}, {{q, qb}, {k, kb}, {table, tb}}) ||
        (qb > 0 && kb > 0 && pa::any_overlap({{q_out, qb}}, {{k_out, kb}})))
        return PA_ERR_OVERLAP;
    if (a.rows == 0 || (Hq == 0 && Hkv == 0)) return PA_OK;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.qo = (uint16_t *)q_out;
    a.ko = (uint16_t *)k_out;
    a.table = (const uint32_t *)table;
    const int64_t ng = (Hq + Hkv + RP_HPG - 1) / RP_HPG;
    const dim3 grid((unsigned)((a.rows * ng * (D / 8) + 255) / 256));
    switch (var) {
    case RP_POLY: hipLaunchKernelGGL(k_rope<RP_POLY>, grid, dim3(256), 0, stream, a); break;
    case RP_NATIVE: hipLaunchKernelGGL(k_rope<RP_NATIVE>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(k_rope<RP_TABLE>, grid, dim3(256), 0, stream, a); break;
    }
    return launched();
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char *pa_status_str(pa_status s)
{
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "invalid shape or size";
    case PA_ERR_DTYPE: return "unsupported dtype";
    case PA_ERR_FUNC: return "unknown function or program";
    case PA_ERR_OVERLAP: return "output partially overlaps another buffer";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_ALIGN: return "pointer not 2-byte aligned";
    }
    return "unknown status";
}

pa_status poly_program_info(int32_t f, int32_t deriv, int32_t t, pa_program *out)
{
    if (!out) return PA_ERR_NULL;
    if (t != PA_F16 && t != PA_BF16) return PA_ERR_DTYPE;
    if (deriv == 2) {
        // the analytic derivative of the D4 tanh program (softcap attention
        // backward): FP16 coefficients (exact), or BF16 ones (rounded)
        if (f != PA_TANH) return PA_ERR_FUNC;
        const ProgramDef *p = find_program(PA_TANH, 0);
        std::memset(out, 0, sizeof *out);
        out->func = PA_TANH;
        out->deriv = 2;
        out->degree = p->degree - 1;
        out->dtype = t;
        out->Li = p->Li;
        out->Lc = p->Lc;
        if (t == PA_F16) {
            CoefF16 fwd, der;
            tanh_coefs(fwd, der);
            for (int j = 0; j < p->degree; ++j) out->coeff_bits[j] = (uint16_t)(der.c[j] & 0xFFFFu);
            out->order = PA_ORDER_F16_FMA;
        } else {
            TanhBF16 fwd, der;
            tanh_coefs_bf16(fwd, der);
            for (int j = 0; j < p->degree; ++j) {
                uint32_t w;
                std::memcpy(&w, &der.c[j], 4);
                out->coeff_bits[j] = (uint16_t)(w >> 16);
            }
            out->order = PA_ORDER_F32FMA_BF16;
        }
        return PA_OK;
    }
    const ProgramDef *p = find_program((int)f, deriv ? 1 : 0);
    if (!p || deriv < 0 || deriv > 1) return PA_ERR_FUNC;
    std::memset(out, 0, sizeof *out);
    out->func = p->func;
    out->deriv = p->deriv;
    out->degree = p->degree;
    out->dtype = t;
    out->Li = p->Li;
    out->Lc = p->Lc;
    for (int j = 0; j <= p->degree; ++j) out->coeff_bits[j] = p->coeff[j];
    out->order = t == PA_F16 ? PA_ORDER_F16_FMA : PA_ORDER_F32FMA_BF16;
    return PA_OK;
}

pa_status poly_act_fwd(int32_t f, int32_t t, const void *x, void *y, int64_t n,
                       hipStream_t stream)
{
    pa_status s = check_unary(t, x, y, n);
    if (s != PA_OK) return s;
    const ProgramDef *p = find_program((int)f, 0);
    if (!p) return PA_ERR_FUNC;
    if (n == 0) return PA_OK;
    switch (f) {
    case PA_SIGMOID: return poly_fwd_dispatch<F_SIGMOID, 3>(*p, t, x, y, n, stream);
    case PA_TANH: return poly_fwd_dispatch<F_TANH, 4>(*p, t, x, y, n, stream);
    case PA_SILU: return poly_fwd_dispatch<F_SILU, 3>(*p, t, x, y, n, stream);
    case PA_GELU: return poly_fwd_dispatch<F_GELU, 5>(*p, t, x, y, n, stream);
    }
    return PA_ERR_FUNC;
}

pa_status poly_act_bwd(int32_t f, int32_t t, const void *x, const void *dy, void *dx, int64_t n,
                       hipStream_t stream)
{
    pa_status s = check_binary(t, x, dy, dx, n);
    if (s != PA_OK) return s;
    const ProgramDef *p = find_program((int)f, 1);
    if (!p) return PA_ERR_FUNC;
    if (n == 0) return PA_OK;
    const bool h = t == PA_F16;
    switch (f) {
    case PA_SIGMOID:
    case PA_TANH:   // even direct fits, D4
        return h ? run_map2(x, dy, dx, n, stream, PolyBwdF16<4>{coef_f16(*p)})
                 : run_map2(x, dy, dx, n, stream, PolyBwdBF16<4>{coef_bf16(*p)});
    case PA_SILU:   // centered-odd direct fit, D3
        return h ? run_map2(x, dy, dx, n, stream, PolyBwdOddF16<3>{coef_f16(*p)})
                 : run_map2(x, dy, dx, n, stream, PolyBwdOddBF16<3>{coef_bf16(*p)});
    case PA_GELU:   // centered-odd direct fit, D5
        return h ? run_map2(x, dy, dx, n, stream, PolyBwdOddF16<5>{coef_f16(*p)})
                 : run_map2(x, dy, dx, n, stream, PolyBwdOddBF16<5>{coef_bf16(*p)});
    }
    return PA_ERR_FUNC;
}

pa_status native_act_fwd(int32_t f, int32_t t, const void *x, void *y, int64_t n,
                         hipStream_t stream)
{
    pa_status s = check_unary(t, x, y, n);
    if (s != PA_OK) return s;
    if (f < PA_SIGMOID || f > PA_GELU) return PA_ERR_FUNC;
    if (n == 0) return PA_OK;
    const bool bf = t == PA_BF16;
    switch (f) {
    case PA_SIGMOID:
        return bf ? run_map1(x, y, n, stream, NativeFwd<F_SIGMOID, true>{})
                  : run_map1(x, y, n, stream, NativeFwd<F_SIGMOID, false>{});
    case PA_TANH:
        return bf ? run_map1(x, y, n, stream, NativeFwd<F_TANH, true>{})
                  : run_map1(x, y, n, stream, NativeFwd<F_TANH, false>{});
    case PA_SILU:
        return bf ? run_map1(x, y, n, stream, NativeFwd<F_SILU, true>{})
                  : run_map1(x, y, n, stream, NativeFwd<F_SILU, false>{});
    case PA_GELU:
        return bf ? run_map1(x, y, n, stream, NativeFwd<F_GELU, true>{})
                  : run_map1(x, y, n, stream, NativeFwd<F_GELU, false>{});
    }
    return PA_ERR_FUNC;
}

pa_status pa_stream_copy(const void *a, const void *b, void *y, int64_t n, hipStream_t stream)
{
    pa_status s = b ? check_binary(PA_F16, a, b, y, n) : check_unary(PA_F16, a, y, n);
    if (s != PA_OK) return s;
    if (n == 0) return PA_OK;
    return b ? run_map2(a, b, y, n, stream, XorOp{}) : run_map1(a, y, n, stream, CopyOp{});
}

pa_status native_act_bwd(int32_t impl, int32_t f, int32_t t, const void *x_or_y, const void *dy,
                         void *dx, int64_t n, hipStream_t stream)
{
    pa_status s = check_binary(t, x_or_y, dy, dx, n);
    if (s != PA_OK) return s;
    if (impl != PA_IMPL_NATIVE && impl != PA_IMPL_NATIVE_FROM_Y) return PA_ERR_FUNC;
    if (f < PA_SIGMOID || f > PA_GELU) return PA_ERR_FUNC;
    const bool from_y = impl == PA_IMPL_NATIVE_FROM_Y;
    if (from_y && f != PA_SIGMOID && f != PA_TANH) return PA_ERR_FUNC;   // no rule from y
    if (n == 0) return PA_OK;
    switch (f) {
    case PA_SIGMOID:
        return from_y ? native_bwd_dispatch<F_SIGMOID, true>(t, x_or_y, dy, dx, n, stream)
                      : native_bwd_dispatch<F_SIGMOID, false>(t, x_or_y, dy, dx, n, stream);
    case PA_TANH:
        return from_y ? native_bwd_dispatch<F_TANH, true>(t, x_or_y, dy, dx, n, stream)
                      : native_bwd_dispatch<F_TANH, false>(t, x_or_y, dy, dx, n, stream);
    case PA_SILU: return native_bwd_dispatch<F_SILU, false>(t, x_or_y, dy, dx, n, stream);
    case PA_GELU: return native_bwd_dispatch<F_GELU, false>(t, x_or_y, dy, dx, n, stream);
    }
    return PA_ERR_FUNC;
}

pa_status poly_swiglu_fwd(int32_t t, const void *gate, const void *up, void *h, int64_t rows,
                          int64_t cols, int64_t ld_gate, int64_t ld_up, int64_t ld_h,
                          const int64_t *row_offsets, int32_t n_groups, hipStream_t stream)
{
    pa_status s = swiglu_fwd_check(t, gate, up, h, rows, cols, ld_gate, ld_up, ld_h, row_offsets,
                                   n_groups);
    if (s != PA_OK) return s;
    if (rows == 0 || cols == 0) return PA_OK;
    const SwiArgs a = swi_args(gate, up, nullptr, h, nullptr, nullptr, rows, cols, ld_gate, ld_up,
                               0, ld_h, 0, 0, row_offsets, n_groups);
    return swiglu_fwd_launch(a, stream, SwiPolyFwd{coef_bf16(sigmoid_d3())});
}

pa_status poly_swiglu_bwd(int32_t t, const void *gate, const void *up, const void *dh,
                          void *dgate, void *dup, int64_t rows, int64_t cols, int64_t ld_gate,
                          int64_t ld_up, int64_t ld_dh, int64_t ld_dgate, int64_t ld_dup,
                          const int64_t *row_offsets, int32_t n_groups, hipStream_t stream)
{
    pa_status s = swiglu_bwd_check(t, gate, up, dh, dgate, dup, rows, cols, ld_gate, ld_up, ld_dh,
                                   ld_dgate, ld_dup, row_offsets, n_groups);
    if (s != PA_OK) return s;
    if (rows == 0 || cols == 0) return PA_OK;
    const SwiArgs a = swi_args(gate, up, dh, nullptr, dgate, dup, rows, cols, ld_gate, ld_up,
                               ld_dh, 0, ld_dgate, ld_dup, row_offsets, n_groups);
    return swiglu_bwd_launch(a, stream, SwiPolyBwd{coef_bf16(sigmoid_d3())});
}

pa_status native_swiglu_fwd(int32_t t, const void *gate, const void *up, void *h, int64_t rows,
                            int64_t cols, int64_t ld_gate, int64_t ld_up, int64_t ld_h,
                            const int64_t *row_offsets, int32_t n_groups, hipStream_t stream)
{
    pa_status s = swiglu_fwd_check(t, gate, up, h, rows, cols, ld_gate, ld_up, ld_h, row_offsets,
                                   n_groups);
    if (s != PA_OK) return s;
    if (rows == 0 || cols == 0) return PA_OK;
    const SwiArgs a = swi_args(gate, up, nullptr, h, nullptr, nullptr, rows, cols, ld_gate, ld_up,
                               0, ld_h, 0, 0, row_offsets, n_groups);
    return swiglu_fwd_launch(a, stream, SwiNativeFwd{});
}

pa_status native_swiglu_bwd(int32_t t, const void *gate, const void *up, const void *dh,
                            void *dgate, void *dup, int64_t rows, int64_t cols, int64_t ld_gate,
                            int64_t ld_up, int64_t ld_dh, int64_t ld_dgate, int64_t ld_dup,
                            const int64_t *row_offsets, int32_t n_groups, hipStream_t stream)
{
    pa_status s = swiglu_bwd_check(t, gate, up, dh, dgate, dup, rows, cols, ld_gate, ld_up, ld_dh,
                                   ld_dgate, ld_dup, row_offsets, n_groups);
    if (s != PA_OK) return s;
    if (rows == 0 || cols == 0) return PA_OK;
    const SwiArgs a = swi_args(gate, up, dh, nullptr, dgate, dup, rows, cols, ld_gate, ld_up,
                               ld_dh, 0, ld_dgate, ld_dup, row_offsets, n_groups);
    return swiglu_bwd_launch(a, stream, SwiNativeBwd{});
}

pa_status poly_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                                int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D, float cap,
                                int32_t causal, hipStream_t stream)
{
    return attn_fwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, lse, B, H, Hkv, S, D, cap, causal, stream);
}

pa_status poly_softcap_attn_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                                    int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D, float cap,
                                    int32_t causal, hipStream_t stream)
{
    return attn_fwd(AM_SOFTCAP_POLY, q, k, v, o, lse, B, H, Hkv, S, D, cap, causal, stream);
}

pa_status poly_softcap_attn_fwd_exp2(const void *q, const void *k, const void *v, void *o,
                                     float *lse, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                     int32_t D, float cap, int32_t causal, int32_t core,
                                     hipStream_t stream)
{
    return attn_fwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, lse, B, H, Hkv, S, D, cap, causal, stream,
                    (int)core);
}

pa_status native_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                                  int32_t B, int32_t H, int32_t Hkv, int32_t S, int32_t D,
                                  float cap, int32_t causal, hipStream_t stream)
{
    return attn_fwd(AM_SOFTCAP_NATIVE, q, k, v, o, lse, B, H, Hkv, S, D, cap, causal, stream);
}

pa_status poly_softcap_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                float *workspace, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                int32_t D, float cap, int32_t causal, hipStream_t stream)
{
    return attn_bwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, S,
                    D, cap, causal, stream);
}

pa_status poly_softcap_attn_bwd_f16(const void *q, const void *k, const void *v, const void *o,
                                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                    float *workspace, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                    int32_t D, float cap, int32_t causal, hipStream_t stream)
{
    return attn_bwd(AM_SOFTCAP_POLY, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, S, D,
                    cap, causal, stream);
}

pa_status poly_softcap_attn_bwd_exp2(const void *q, const void *k, const void *v, const void *o,
                                     const void *dout, const float *lse, void *dq, void *dk,
                                     void *dv, float *workspace, int32_t B, int32_t H, int32_t Hkv,
                                     int32_t S, int32_t D, float cap, int32_t causal, int32_t core,
                                     hipStream_t stream)
{
    return attn_bwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, S,
                    D, cap, causal, stream, (int)core);
}

pa_status native_softcap_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                  float *workspace, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                  int32_t D, float cap, int32_t causal, hipStream_t stream)
{
    return attn_bwd(AM_SOFTCAP_NATIVE, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, S,
                    D, cap, causal, stream);
}

pa_status poly_sigmoid_attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                                int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                hipStream_t stream)
{
    return attn_fwd(AM_SIGMOID_POLY, q, k, v, o, nullptr, B, H, Hkv, S, D, 0.0f, causal, stream);
}

pa_status native_sigmoid_attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                                  int32_t H, int32_t Hkv, int32_t S, int32_t D, int32_t causal,
                                  hipStream_t stream)
{
    return attn_fwd(AM_SIGMOID_NATIVE, q, k, v, o, nullptr, B, H, Hkv, S, D, 0.0f, causal, stream);
}

pa_status poly_sigmoid_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                                void *dq, void *dk, void *dv, float *workspace, int32_t B, int32_t H,
                                int32_t Hkv, int32_t S, int32_t D, int32_t causal, hipStream_t stream)
{
    return attn_bwd(AM_SIGMOID_POLY, q, k, v, nullptr, dout, nullptr, dq, dk, dv, workspace, B, H, Hkv, S,
                    D, 0.0f, causal, stream);
}

pa_status native_sigmoid_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                                  void *dq, void *dk, void *dv, float *workspace, int32_t B, int32_t H,
                                  int32_t Hkv, int32_t S, int32_t D, int32_t causal, hipStream_t stream)
{
    return attn_bwd(AM_SIGMOID_NATIVE, q, k, v, nullptr, dout, nullptr, dq, dk, dv, workspace, B, H, Hkv, S,
                    D, 0.0f, causal, stream);
}

int64_t pa_attn_bwd_workspace_bytes(int32_t softcap, int32_t B, int32_t H, int32_t Hkv,
                                    int32_t S, int32_t D)
{
    if (attn_shape(B, H, Hkv, S, D) != PA_OK) return -1;
    return 4 * attn_bwd_ws_floats(softcap != 0, B, H, Hkv, S, D, attn_bwd_use_ds(B, H, S));
}

int64_t pa_attn_bwd_ds_limit(int64_t bytes)
{
    if (bytes < 0) return attn_ds_limit().load();
    return attn_ds_limit().exchange(bytes);
}

pa_status poly_sigmoid_attn_program(pa_sigmoid_attn_program *out)
{
    if (!out) return PA_ERR_NULL;
    const SigmoidAttnDef &d = kSigmoidAttn;
    std::memset(out, 0, sizeof *out);
    out->n = d.n;
    out->thr = d.thr;
    out->clamp_lo = d.lo;
    out->clamp_hi = d.hi;
    for (int r = 0; r < 2; ++r) {
        for (int j = 0; j < 4; ++j) out->coeff_bits[r][j] = d.c[r][j];
        out->a_bits[r] = d.a[r];
        out->b_bits[r] = d.b[r];
    }
    out->order = PA_ORDER_F32FMA_BF16;
    return PA_OK;
}

pa_status poly_rope(const void *q, const void *k, void *q_out, void *k_out, int32_t B, int32_t S,
                    int32_t Hq, int32_t Hkv, int32_t D, double base, hipStream_t stream)
{
    return rope_run(RP_POLY, q, k, q_out, k_out, nullptr, B, S, Hq, Hkv, D, base, stream);
}

pa_status native_rope(const void *q, const void *k, void *q_out, void *k_out, int32_t B, int32_t S,
                      int32_t Hq, int32_t Hkv, int32_t D, double base, hipStream_t stream)
{
    return rope_run(RP_NATIVE, q, k, q_out, k_out, nullptr, B, S, Hq, Hkv, D, base, stream);
}

pa_status native_rope_table(const void *q, const void *k, void *q_out, void *k_out,
                            const void *table, int32_t B, int32_t S, int32_t Hq, int32_t Hkv,
                            int32_t D, hipStream_t stream)
{
    return rope_run(RP_TABLE, q, k, q_out, k_out, table, B, S, Hq, Hkv, D, 1.0, stream);
}

pa_status pa_rope_table(void *table, int32_t S, int32_t D, double base, hipStream_t stream)
{
    RopeArgs a;
    const pa_status st = rope_args(1, S, 0, 0, D, base, true, a);
    if (st != PA_OK) return st;
    if (!table) return PA_ERR_NULL;
    if (!aligned16({table})) return PA_ERR_ALIGN;
    const int64_t n = (int64_t)S * (D / 2);
    if (n == 0) return PA_OK;
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, (uint32_t *)table, a);
    return launched();
}

pa_status poly_rope_program(pa_rope_program *out)
{
    if (!out) return PA_ERR_NULL;
    for (int j = 0; j < 3; ++j) out->sin_bits[j] = kRopeSin[j];
    for (int j = 0; j < 4; ++j) out->cos_bits[j] = kRopeCos[j];
    return PA_OK;
}

}  // extern "C"

// ---- allocation-free softcap backward -----------------------------------
// The backward's scratch (Delta and -lse log2(e) per query row, and the FP32
// dK / dV partials of grouped query heads) lives in one file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends; its device address comes from
// hipGetSymbolAddress once per device (the array's name is only a host-side
// stand-in in host code) and is kept here.  Every call writes all the scratch
// it reads before reading it, so nothing needs clearing between calls.
namespace {
constexpr int64_t kStaticScratchFloats = int64_t(2) << 20;   // 8 MiB
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) float scratch[kStaticScratchFloats];

// The device address of this device's scratch array, or nullptr.
static float *static_scratch(pa_status &st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        st = PA_ERR_LAUNCH;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            st = PA_ERR_LAUNCH;
            return nullptr;
        }
        g_scratch_ptr[dev] = (float *)p;
    }
    st = PA_OK;
    return g_scratch_ptr[dev];
}

int64_t pa_attn_bwd_static_scratch_bytes(void) { return kStaticScratchFloats * 4; }

pa_status poly_softcap_attn_bwd_static(const void *q, const void *k, const void *v, const void *o,
                                       const void *dout, const float *lse, void *dq, void *dk,
                                       void *dv, int32_t B, int32_t H, int32_t Hkv, int32_t S,
                                       int32_t D, float cap, int32_t causal, hipStream_t stream)
{
    pa_status st = attn_shape(B, H, Hkv, S, D);
    if (st != PA_OK) return st;
    const int64_t need = attn_bwd_ws_floats(true, B, H, Hkv, S, D, false);
    if (need > kStaticScratchFloats) return PA_ERR_SHAPE;
    if ((int64_t)B * H == 0 || S == 0) {
        return attn_bwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, Hkv,
                        S, D, cap, causal, stream, 0, false);
    }
    float *ws = static_scratch(st);
    if (!ws) return st;
    return attn_bwd(AM_SOFTCAP_POLY_BF16, q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, Hkv, S, D,
                    cap, causal, stream, 0, false);
}
