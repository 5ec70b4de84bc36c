// stream_launch.hpp -- launch configuration of the elementwise streaming
// kernels (stream.hpp): tile sizes, grids, and the split of a range into a
// scalar head, a 16-byte vector body and a scalar tail.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "../../include/polyact.h"
#include "stream.hpp"

namespace pa {
namespace {

constexpr int kThreads = 256;       // scalar kernels
// Streaming tiles (threads per block, 16-byte chunks per thread).  Sweeps of
// block sizes 128-1024 and 1-8 chunks per thread on MI355X put one chunk per
// thread first for every stream shape (6.5 TB/s for one input and one
// output, 6.5 TB/s for two inputs and one output, 6.2 TB/s for three inputs
// and two outputs at 268,435,456 elements, with 512 threads for one input
// and 1024 for two or three).  Below 2^23 chunks per stream (128 MiB) a
// 256-thread block is faster -- the grid is small there: 25 % for two inputs
// at 4M elements, 10 % for the BF16 SiLU at 58.7M -- while above it 256
// threads lose 2-6 %, so the block size follows the size.
constexpr int kMap1BS = 512, kMap2BS = 1024, kSmallBS = 256;
constexpr int kMap1U = 1, kMap2U = 1;
constexpr int64_t kSmallChunks = int64_t(1) << 23;   // 16-byte chunks per stream
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

inline pa_status stream_launched()
{
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
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
        const u32x4 *xv = (const u32x4 *)(xs + sp.head);
        u32x4 *yv = (u32x4 *)(ys + sp.head);
        if (sp.nvec <= kSmallChunks)
            hipLaunchKernelGGL((k_map1<Op, kSmallBS, 1>), dim3((unsigned)grid_tiles(sp.nvec, kSmallBS)),
                               dim3(kSmallBS), 0, st, xv, yv, sp.nvec, op);
        else
            hipLaunchKernelGGL((k_map1<Op, kMap1BS, kMap1U>),
                               dim3((unsigned)grid_tiles(sp.nvec, (int64_t)kMap1BS * kMap1U)), dim3(kMap1BS),
                               0, st, xv, yv, sp.nvec, op);
        if (stream_launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    const int64_t rest = sp.head + (n - sp.tail0);
    if (rest > 0) {
        hipLaunchKernelGGL((k_scalar1<Op>), dim3((unsigned)grid_for(rest, 1)), dim3(kThreads), 0,
                           st, xs, ys, (int64_t)0, sp.head, sp.tail0, n, op);
        if (stream_launched() != PA_OK) return PA_ERR_LAUNCH;
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
        const u32x4 *xv = (const u32x4 *)(xs + sp.head), *gv = (const u32x4 *)(gs + sp.head);
        u32x4 *yv = (u32x4 *)(ys + sp.head);
        if (sp.nvec <= kSmallChunks)
            hipLaunchKernelGGL((k_map2<Op, kSmallBS, 1>), dim3((unsigned)grid_tiles(sp.nvec, kSmallBS)),
                               dim3(kSmallBS), 0, st, xv, gv, yv, sp.nvec, op);
        else
            hipLaunchKernelGGL((k_map2<Op, kMap2BS, kMap2U>),
                               dim3((unsigned)grid_tiles(sp.nvec, (int64_t)kMap2BS * kMap2U)), dim3(kMap2BS),
                               0, st, xv, gv, yv, sp.nvec, op);
        if (stream_launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    const int64_t rest = sp.head + (n - sp.tail0);
    if (rest > 0) {
        hipLaunchKernelGGL((k_scalar2<Op>), dim3((unsigned)grid_for(rest, 1)), dim3(kThreads), 0,
                           st, xs, gs, ys, (int64_t)0, sp.head, sp.tail0, n, op);
        if (stream_launched() != PA_OK) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

}  // namespace
}  // namespace pa
