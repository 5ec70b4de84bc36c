// swiglu.hpp -- fused SwiGLU forward / backward over dense or expert-grouped
// row ranges (BF16 in and out, FP32 combine).
//
// "Fast Polynomial Transcendentals for LLMs" (arXiv 2610.00049): section 3.3
// (recompute the D3 sigmoid p(g), SiLU~ = g p, derivative p + g p (1 - p)),
// section 3.4 (activation and gating fused in forward; both projected-input
// gradients in one backward kernel, no intermediate tensor) and Eq. 15 (the
// routed-expert form Y = SiLU~(X Wg) * (X Wu) over expert-grouped rows).
//
// Per element (g gate, u up, dh upstream gradient):
//   p  = sigma~(g)                (D3 program in BF16: FP32 FMA + BF16 per stage)
//   gp = RN32(g p)                (exact: 8 x 8 significant bits)
//   h  = RN16(RN32(gp u))
//   ds = RN32(gp (1 - p) + p)     (one FMA; 1 - p exact in FP32)
//   du = RN16(RN32(dh gp)),  dg = RN16(RN32(RN32(dh u) ds))
//
// Rows: dense mode processes [0, rows); grouped mode reads the device offsets
// and processes [off[0], off[n_groups]) clipped to [0, rows), so the row
// count never travels to the host.  The vector path needs cols and every
// leading dimension divisible by 8 and 16-byte aligned bases; when all
// leading dimensions equal cols the range is one flat stream.
#pragma once
#include "ops.hpp"
#include "stream.hpp"

namespace pa {

struct SwiArgs {
    const uint16_t *g, *u, *dh;
    uint16_t *h, *dg, *du;
    int64_t rows, cols;
    int64_t ld_g, ld_u, ld_dh, ld_h, ld_dg, ld_du;
    const int64_t *off;
    int32_t n_groups;
};

__device__ __forceinline__ void row_range(const SwiArgs &a, int64_t &r0, int64_t &r1)
{
    if (a.off) {
        int64_t s = a.off[0], e = a.off[a.n_groups];
        s = s < 0 ? 0 : (s > a.rows ? a.rows : s);
        e = e < s ? s : (e > a.rows ? a.rows : e);
        r0 = s;
        r1 = e;
    } else {
        r0 = 0;
        r1 = a.rows;
    }
}

// ---- pair operators --------------------------------------------------------
struct SwiPolyFwd {
    CoefBF16 k;   // the D3 sigmoid program
    __device__ __forceinline__ uint32_t operator()(uint32_t gw, uint32_t uw) const
    {
        const uint32_t p = poly_fwd_bf16_core<F_SIGMOID, 3>(gw, k);
        const float gp0 = lo_f(gw) * lo_f(p), gp1 = hi_f(gw) * hi_f(p);
        return pack_bf(gp0 * lo_f(uw), gp1 * hi_f(uw));
    }
};

struct SwiPolyBwd {
    CoefBF16 k;
    __device__ __forceinline__ void operator()(uint32_t gw, uint32_t uw, uint32_t dw,
                                               uint32_t &dgw, uint32_t &duw) const
    {
        const uint32_t p = poly_fwd_bf16_core<F_SIGMOID, 3>(gw, k);
        const float p0 = lo_f(p), p1 = hi_f(p);
        const float gp0 = lo_f(gw) * p0, gp1 = hi_f(gw) * p1;
        const float ds0 = fmaf(gp0, 1.0f - p0, p0), ds1 = fmaf(gp1, 1.0f - p1, p1);
        const float d0 = lo_f(dw), d1 = hi_f(dw);
        duw = pack_bf(d0 * gp0, d1 * gp1);
        dgw = pack_bf((d0 * lo_f(uw)) * ds0, (d1 * hi_f(uw)) * ds1);
    }
};

// accurate FP32 SiLU: e = exp(-|g|), r = 1 / (1 + e), sigma = g >= 0 ? r : e r
__device__ __forceinline__ void native_silu(float g, float &sig, float &silu)
{
    const float e = expf(-fabsf(g));
    const float r = 1.0f / (1.0f + e);
    sig = g >= 0.0f ? r : e * r;
    silu = g == -INFINITY ? -0.0f : (g >= 0.0f ? g : g * e) * r;
}

struct SwiNativeFwd {
    __device__ __forceinline__ uint32_t operator()(uint32_t gw, uint32_t uw) const
    {
        float s0, s1, a0, a1;
        native_silu(lo_f(gw), s0, a0);
        native_silu(hi_f(gw), s1, a1);
        return pack_bf(a0 * lo_f(uw), a1 * hi_f(uw));
    }
};

struct SwiNativeBwd {
    __device__ __forceinline__ void operator()(uint32_t gw, uint32_t uw, uint32_t dw,
                                               uint32_t &dgw, uint32_t &duw) const
    {
        float s0, s1, a0, a1;
        const float g0 = lo_f(gw), g1 = hi_f(gw);
        native_silu(g0, s0, a0);
        native_silu(g1, s1, a1);
        const float ds0 = s0 + a0 * (1.0f - s0), ds1 = s1 + a1 * (1.0f - s1);
        const float d0 = lo_f(dw), d1 = hi_f(dw);
        duw = pack_bf(d0 * a0, d1 * a1);
        dgw = pack_bf(d0 * lo_f(uw) * ds0, d1 * hi_f(uw) * ds1);
    }
};

// ---- kernels ----------------------------------------------------------------
// Chunk c of the selected rows -> element offset for a matrix with leading
// dimension ld.  FLAT: all leading dimensions equal cols.
template <bool FLAT>
__device__ __forceinline__ int64_t chunk_elem(int64_t r0, int64_t c, int64_t cpr, int64_t ld,
                                              int64_t cols)
{
    if constexpr (FLAT) return r0 * cols + c * 8;
    else {
        const int64_t r = c / cpr;
        return (r0 + r) * ld + (c - r * cpr) * 8;
    }
}

// One block per tile of BS * U chunks of the selected rows (the tiling of the
// streaming kernels); the host sizes the grid for the capacity `rows`, and
// blocks past the device-side row range exit at once.
template <class Op, int BS, int U, bool FLAT>
__global__ __launch_bounds__(BS) void k_swiglu_fwd_vec(SwiArgs a, Op op)
{
    int64_t r0, r1;
    row_range(a, r0, r1);
    const int64_t cpr = a.cols >> 3;
    const int64_t n = (r1 - r0) * cpr;
    const int64_t tile = (int64_t)BS * U;
    for (int64_t t0 = (int64_t)blockIdx.x * tile; t0 < n; t0 += (int64_t)gridDim.x * tile) {
        u32x4 g[U], u[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t c = t0 + k * BS + threadIdx.x;
            if (c < n) {
                g[k] = ld16<true>((const u32x4 *)(a.g + chunk_elem<FLAT>(r0, c, cpr, a.ld_g, a.cols)));
                u[k] = ld16<true>((const u32x4 *)(a.u + chunk_elem<FLAT>(r0, c, cpr, a.ld_u, a.cols)));
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t c = t0 + k * BS + threadIdx.x;
            if (c < n)
                st16<true>((u32x4 *)(a.h + chunk_elem<FLAT>(r0, c, cpr, a.ld_h, a.cols)),
                           map4(op, g[k], u[k]));
        }
    }
}

template <class Op>
__device__ __forceinline__ void bwd_chunk(const Op &op, u32x4 g, u32x4 u, u32x4 d, u32x4 &dg,
                                          u32x4 &du)
{
    uint32_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) op(g[i], u[i], d[i], a[i], b[i]);
    dg = u32x4{a[0], a[1], a[2], a[3]};
    du = u32x4{b[0], b[1], b[2], b[3]};
}

template <class Op, int BS, int U, bool FLAT>
__global__ __launch_bounds__(BS) void k_swiglu_bwd_vec(SwiArgs a, Op op)
{
    int64_t r0, r1;
    row_range(a, r0, r1);
    const int64_t cpr = a.cols >> 3;
    const int64_t n = (r1 - r0) * cpr;
    const int64_t tile = (int64_t)BS * U;
    for (int64_t t0 = (int64_t)blockIdx.x * tile; t0 < n; t0 += (int64_t)gridDim.x * tile) {
        u32x4 g[U], u[U], d[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t c = t0 + k * BS + threadIdx.x;
            if (c < n) {
                g[k] = ld16<true>((const u32x4 *)(a.g + chunk_elem<FLAT>(r0, c, cpr, a.ld_g, a.cols)));
                u[k] = ld16<true>((const u32x4 *)(a.u + chunk_elem<FLAT>(r0, c, cpr, a.ld_u, a.cols)));
                d[k] = ld16<true>((const u32x4 *)(a.dh + chunk_elem<FLAT>(r0, c, cpr, a.ld_dh, a.cols)));
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t c = t0 + k * BS + threadIdx.x;
            if (c < n) {
                u32x4 dg, du;
                bwd_chunk(op, g[k], u[k], d[k], dg, du);
                st16<true>((u32x4 *)(a.dg + chunk_elem<FLAT>(r0, c, cpr, a.ld_dg, a.cols)), dg);
                st16<true>((u32x4 *)(a.du + chunk_elem<FLAT>(r0, c, cpr, a.ld_du, a.cols)), du);
            }
        }
    }
}

// One element per thread, any alignment and any cols.
template <class Op>
__global__ __launch_bounds__(256) void k_swiglu_fwd_scalar(SwiArgs a, Op op)
{
    int64_t r0, r1;
    row_range(a, r0, r1);
    const int64_t n = (r1 - r0) * a.cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = r0 + i / a.cols, c = i % a.cols;
        const uint32_t g = a.g[r * a.ld_g + c], u = a.u[r * a.ld_u + c];
        a.h[r * a.ld_h + c] = (uint16_t)op(g | (g << 16), u | (u << 16));
    }
}

template <class Op>
__global__ __launch_bounds__(256) void k_swiglu_bwd_scalar(SwiArgs a, Op op)
{
    int64_t r0, r1;
    row_range(a, r0, r1);
    const int64_t n = (r1 - r0) * a.cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = r0 + i / a.cols, c = i % a.cols;
        const uint32_t g = a.g[r * a.ld_g + c], u = a.u[r * a.ld_u + c], d = a.dh[r * a.ld_dh + c];
        uint32_t dg, du;
        op(g | (g << 16), u | (u << 16), d | (d << 16), dg, du);
        a.dg[r * a.ld_dg + c] = (uint16_t)dg;
        a.du[r * a.ld_du + c] = (uint16_t)du;
    }
}

}  // namespace pa
