// polyact.hip -- C ABI of the gfx950 polynomial activation library: argument
// validation, program lookup and kernel dispatch.  See include/polyact.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/polyact.h"
#include "attn.hpp"
#include "ops.hpp"
#include "programs.hpp"
#include "stream.hpp"
#include "swiglu.hpp"

using namespace pa;

namespace {

constexpr int kThreads = 256;       // scalar kernels
// Streaming tiles (threads per block, 16-byte chunks per thread).  A sweep of
// block sizes 128-1024 and 1-4 chunks per thread on MI355X put one chunk per
// thread and the most blocks first for every stream shape: 6.49 TB/s for one
// input and one output, 6.52 TB/s for two inputs and one output, 6.20 TB/s
// for three inputs and two outputs.
constexpr int kMap1BS = 512, kMap1U = 1;   // x -> y
constexpr int kMap2BS = 1024, kMap2U = 1;  // x, g -> y; SwiGLU fwd and bwd
constexpr int64_t kMaxGrid = 0x7FFFFFFF;
constexpr int kBlocksPerCU = 8;     // scalar kernels: blocks per compute unit

int cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// one block per tile of tile_items work items (capped by the launch limit)
int64_t grid_tiles(int64_t work_items, int64_t tile_items)
{
    const int64_t need = (work_items + tile_items - 1) / tile_items;
    return need < 1 ? 1 : (need < kMaxGrid ? need : kMaxGrid);
}

int64_t grid_for(int64_t work_items, int per_thread)
{
    const int64_t need = (work_items + (int64_t)kThreads * per_thread - 1) /
                         ((int64_t)kThreads * per_thread);
    const int64_t cap = (int64_t)cu_count() * kBlocksPerCU;
    return need < 1 ? 1 : (need < cap ? need : cap);
}

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

// Split [0, n) of 16-bit elements into a scalar head, a 16-byte vector body
// and a scalar tail, given the byte addresses of all streams.
struct Split {
    int64_t head, nvec, tail0, n;
};
Split split_range(int64_t n, std::initializer_list<const void *> ptrs)
{
    Split s{n, 0, n, n};
    uintptr_t mis = (uintptr_t)(*ptrs.begin()) & 15u;
    for (const void *p : ptrs)
        if (((uintptr_t)p & 15u) != mis) return s;   // different phases: all scalar
    int64_t head = (int64_t)(((16u - mis) & 15u) / 2u);
    if (head > n) head = n;
    s.head = head;
    s.nvec = (n - head) / 8;
    s.tail0 = head + s.nvec * 8;
    return s;
}

template <class Op>
pa_status run_map1(const void *x, void *y, int64_t n, hipStream_t st, const Op &op)
{
    const Split sp = split_range(n, {x, y});
    const uint16_t *xs = (const uint16_t *)x;
    uint16_t *ys = (uint16_t *)y;
    if (sp.nvec > 0) {
        const int64_t grid = grid_tiles(sp.nvec, (int64_t)kMap1BS * kMap1U);
        hipLaunchKernelGGL((k_map1<Op, kMap1BS, kMap1U>), dim3((unsigned)grid), dim3(kMap1BS), 0, st,
                           (const u32x4 *)(xs + sp.head), (u32x4 *)(ys + sp.head), sp.nvec, op);
        if (launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    const int64_t rest = sp.head + (n - sp.tail0);
    if (rest > 0) {
        hipLaunchKernelGGL((k_scalar1<Op>), dim3((unsigned)grid_for(rest, 1)), dim3(kThreads), 0,
                           st, xs, ys, (int64_t)0, sp.head, sp.tail0, n, op);
        if (launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

template <class Op>
pa_status run_map2(const void *x, const void *g, void *y, int64_t n, hipStream_t st, const Op &op)
{
    const Split sp = split_range(n, {x, g, y});
    const uint16_t *xs = (const uint16_t *)x, *gs = (const uint16_t *)g;
    uint16_t *ys = (uint16_t *)y;
    if (sp.nvec > 0) {
        const int64_t grid = grid_tiles(sp.nvec, (int64_t)kMap2BS * kMap2U);
        hipLaunchKernelGGL((k_map2<Op, kMap2BS, kMap2U>), dim3((unsigned)grid), dim3(kMap2BS), 0, st,
                           (const u32x4 *)(xs + sp.head), (const u32x4 *)(gs + sp.head),
                           (u32x4 *)(ys + sp.head), sp.nvec, op);
        if (launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    const int64_t rest = sp.head + (n - sp.tail0);
    if (rest > 0) {
        hipLaunchKernelGGL((k_scalar2<Op>), dim3((unsigned)grid_for(rest, 1)), dim3(kThreads), 0,
                           st, xs, gs, ys, (int64_t)0, sp.head, sp.tail0, n, op);
        if (launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

pa_status check_unary(pa_dtype t, const void *x, const void *y, int64_t n)
{
    if (t != PA_F16 && t != PA_BF16) return PA_ERR_DTYPE;
    if (n < 0) return PA_ERR_SHAPE;
    pa_status s = check_ptr(x);
    if (s != PA_OK) return s;
    if ((s = check_ptr(y)) != PA_OK) return s;
    if (partial_overlap(y, 2 * n, x, 2 * n)) return PA_ERR_OVERLAP;
    return PA_OK;
}

pa_status check_binary(pa_dtype t, const void *x, const void *g, const void *y, int64_t n)
{
    pa_status s = check_unary(t, x, y, n);
    if (s != PA_OK) return s;
    if ((s = check_ptr(g)) != PA_OK) return s;
    if (partial_overlap(y, 2 * n, g, 2 * n)) return PA_ERR_OVERLAP;
    return PA_OK;
}

template <int F, int D>
pa_status poly_fwd_dispatch(const ProgramDef &p, pa_dtype t, const void *x, void *y, int64_t n,
                            hipStream_t st)
{
    if (t == PA_F16) return run_map1(x, y, n, st, PolyFwdF16<F, D>{coef_f16(p)});
    return run_map1(x, y, n, st, PolyFwdBF16<F, D>{coef_bf16(p)});
}

template <int F, bool FROM_Y>
pa_status native_bwd_dispatch(pa_dtype t, const void *x, const void *g, void *y, int64_t n,
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
        const int64_t grid = grid_tiles(a.rows * (a.cols / 8), (int64_t)kMap2BS * kMap2U);
        if (flat(a, false))
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kMap2BS, kMap2U, true>), dim3((unsigned)grid),
                               dim3(kMap2BS), 0, st, a, op);
        else
            hipLaunchKernelGGL((k_swiglu_fwd_vec<Op, kMap2BS, kMap2U, false>), dim3((unsigned)grid),
                               dim3(kMap2BS), 0, st, a, op);
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
        const int64_t grid = grid_tiles(a.rows * (a.cols / 8), (int64_t)kMap2BS * kMap2U);
        if (flat(a, true))
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kMap2BS, kMap2U, true>), dim3((unsigned)grid),
                               dim3(kMap2BS), 0, st, a, op);
        else
            hipLaunchKernelGGL((k_swiglu_bwd_vec<Op, kMap2BS, kMap2U, false>), dim3((unsigned)grid),
                               dim3(kMap2BS), 0, st, a, op);
    } else {
        hipLaunchKernelGGL((k_swiglu_bwd_scalar<Op>), dim3((unsigned)grid_for(a.rows * a.cols, 1)),
                           dim3(kThreads), 0, st, a, op);
    }
    return launched();
}

pa_status swiglu_fwd_check(pa_dtype t, const void *gate, const void *up, void *h, int64_t rows,
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

pa_status swiglu_bwd_check(pa_dtype t, const void *gate, const void *up, const void *dh,
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

// =============================================================================
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

pa_status poly_program_info(pa_func f, int32_t deriv, pa_dtype t, pa_program *out)
{
    if (!out) return PA_ERR_NULL;
    if (t != PA_F16 && t != PA_BF16) return PA_ERR_DTYPE;
    const ProgramDef *p = find_program((int)f, deriv ? 1 : 0);
    if (!p) return PA_ERR_FUNC;
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

pa_status poly_act_fwd(pa_func f, pa_dtype t, const void *x, void *y, int64_t n,
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

pa_status poly_act_bwd(pa_func f, pa_dtype t, const void *x, const void *dy, void *dx, int64_t n,
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

pa_status native_act_fwd(pa_func f, pa_dtype t, const void *x, void *y, int64_t n,
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

pa_status native_act_bwd(pa_impl impl, pa_func f, pa_dtype t, const void *x_or_y, const void *dy,
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

pa_status poly_swiglu_fwd(pa_dtype t, const void *gate, const void *up, void *h, int64_t rows,
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

pa_status poly_swiglu_bwd(pa_dtype t, const void *gate, const void *up, const void *dh,
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

pa_status native_swiglu_fwd(pa_dtype t, const void *gate, const void *up, void *h, int64_t rows,
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

pa_status native_swiglu_bwd(pa_dtype t, const void *gate, const void *up, const void *dh,
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

pa_status poly_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                                int32_t H, int32_t S, int32_t D, float cap, int32_t causal,
                                hipStream_t stream)
{
    const ProgramDef *p = find_program(PA_TANH, 0);
    return attn_fwd(q, k, v, o, B, H, S, D, cap, causal, true, coef_f16(*p), stream);
}

pa_status native_softcap_attn_fwd(const void *q, const void *k, const void *v, void *o,
                                  int32_t B, int32_t H, int32_t S, int32_t D, float cap,
                                  int32_t causal, hipStream_t stream)
{
    const ProgramDef *p = find_program(PA_TANH, 0);
    return attn_fwd(q, k, v, o, B, H, S, D, cap, causal, false, coef_f16(*p), stream);
}

}  // extern "C"
