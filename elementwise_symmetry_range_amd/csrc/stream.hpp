// stream.hpp -- HBM streaming kernels for the elementwise programs.
//
// The vector kernels move 16 bytes (8 x 16-bit values = four packed pairs) per
// thread per access with global_load_dwordx4 / global_store_dwordx4, the
// analogue of the paper's one-int4-chunk-per-thread packed path ("Fast
// Polynomial Transcendentals for LLMs", section 3.4).  Each thread keeps U
// independent chunks in flight (loads issued first, then compute, then
// stores).  No LDS, no MFMA: the work is bound by HBM bandwidth (4 bytes per
// element forward, 6 backward).
//
// A scalar kernel handles the elements outside the 16-byte-aligned middle
// (a misaligned head and a ragged tail), one element per thread, by feeding
// the pair operator a duplicated lane.
#pragma once
#include "ops.hpp"

namespace pa {

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4 *p, u32x4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <class Op>
__device__ __forceinline__ u32x4 map4(const Op &op, u32x4 a)
{
    u32x4 r;
    r.x = op(a.x);
    r.y = op(a.y);
    r.z = op(a.z);
    r.w = op(a.w);
    return r;
}
template <class Op>
__device__ __forceinline__ u32x4 map4(const Op &op, u32x4 a, u32x4 b)
{
    u32x4 r;
    r.x = op(a.x, b.x);
    r.y = op(a.y, b.y);
    r.z = op(a.z, b.z);
    r.w = op(a.w, b.w);
    return r;
}

// Tiling.  Block b owns the tile of BS * U consecutive 16-byte chunks
// starting at b * BS * U; chunk t0 + u * BS + threadIdx.x is thread
// threadIdx.x's u-th chunk, so every load and store instruction of a wave
// covers 1 KiB of contiguous memory.  The grid is one block per tile (no
// persistent loop): blocks are spread round-robin over the eight XCDs, which
// interleaves neighbouring tiles across the whole memory system, and the
// occupancy of many small blocks keeps the loads in flight.  Measured on
// MI355X this beats a persistent grid-stride walk and an XCD-contiguous
// block order by 10-25 %.  Loads and stores are nontemporal: each byte is
// touched once.  The loop only runs again for grids capped by the launch
// limit.
template <class Op, int BS, int U>
__global__ __launch_bounds__(BS) void k_map1(const u32x4 *x, u32x4 *y, int64_t nvec, Op op)
{
    const int64_t tile = (int64_t)BS * U;
    for (int64_t t0 = (int64_t)blockIdx.x * tile; t0 < nvec; t0 += (int64_t)gridDim.x * tile) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = t0 + u * BS + threadIdx.x;
            if (i < nvec) v[u] = ld16<true>(x + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = t0 + u * BS + threadIdx.x;
            if (i < nvec) st16<true>(y + i, map4(op, v[u]));
        }
    }
}

template <class Op, int BS, int U>
__global__ __launch_bounds__(BS) void k_map2(const u32x4 *x, const u32x4 *g, u32x4 *y,
                                             int64_t nvec, Op op)
{
    const int64_t tile = (int64_t)BS * U;
    for (int64_t t0 = (int64_t)blockIdx.x * tile; t0 < nvec; t0 += (int64_t)gridDim.x * tile) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = t0 + u * BS + threadIdx.x;
            if (i < nvec) {
                a[u] = ld16<true>(x + i);
                b[u] = ld16<true>(g + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = t0 + u * BS + threadIdx.x;
            if (i < nvec) st16<true>(y + i, map4(op, a[u], b[u]));
        }
    }
}

// Elements [a0, a1) and [b0, b1), one per thread.
template <class Op>
__global__ __launch_bounds__(256) void k_scalar1(const uint16_t *x, uint16_t *y, int64_t a0,
                                                 int64_t a1, int64_t b0, int64_t b1, Op op)
{
    const int64_t na = a1 - a0, total = na + (b1 - b0);
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * 256) {
        const int64_t i = k < na ? a0 + k : b0 + (k - na);
        const uint32_t w = x[i];
        y[i] = (uint16_t)op(w | (w << 16));
    }
}

template <class Op>
__global__ __launch_bounds__(256) void k_scalar2(const uint16_t *x, const uint16_t *g,
                                                 uint16_t *y, int64_t a0, int64_t a1,
                                                 int64_t b0, int64_t b1, Op op)
{
    const int64_t na = a1 - a0, total = na + (b1 - b0);
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * 256) {
        const int64_t i = k < na ? a0 + k : b0 + (k - na);
        const uint32_t w = x[i], v = g[i];
        y[i] = (uint16_t)op(w | (w << 16), v | (v << 16));
    }
}

}  // namespace pa
