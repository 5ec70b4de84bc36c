// rope.hpp -- rotary position embedding with paired sine / cosine programs
// ("Fast Polynomial Transcendentals for LLMs", Appendix B.2).
//
// The angle of frequency i at position s is a Q0.32 fraction of a turn,
// phase = (s * inc_i) mod 2^32 with inc_i = round(w_i 2^32 / (2 pi)) stored
// by the host; its top 16 bits, read as a signed integer v, are the Q15
// half-turn coordinate (angle pi v / 2^15).  Per thread: one position and 8
// consecutive head dimensions = 4 frequencies (two packed FP16 pairs), whose
// sine and cosine are formed once and reused for every query and key head
// of that position:
//   RP_POLY    u = RN16(v) 2^-15, w = u u; sine u (a1 + w (a3 + w a5)) (D5),
//              cosine b0 + w (b2 + w (b4 + w b6)) (D6), every step a packed
//              FP16 multiply or FMA;
//   RP_NATIVE  accurate FP32 sinf / cosf of the same angle, rounded to FP16
//              (the comparator computed on the fly);
//   RP_TABLE   the comparator's values read from a [S, D / 2] table of
//              (cos, sin) FP16 pairs built once by k_rope_table.
// The rotation of each interleaved pair (x0, x1) is one packed product and
// one packed FMA: y0 = RN16(x0 c - RN16(x1 s)), y1 = RN16(x1 c + RN16(x0 s)).
// Layouts: Q [B, S, Hq, D] and K [B, S, Hkv, D] in, Q [B, Hq, S, D] and
// K [B, Hkv, S, D] out (FP16).  A thread takes one position, 8 consecutive
// head dimensions and a group of 8 heads (queries, then keys); consecutive
// threads take the 16-byte chunks of a row, then consecutive positions of
// the same head group, so a workgroup (16 positions at D = 128) reads runs
// of 8 whole head rows per position and writes 4 KiB runs of each output
// head.  Measured on MI355X at 1 x 4096 x 32 (8) x 128: 13.7 us, the rate of
// a plain copy of the same bytes, against 15.3 us with the positions outer
// (each output head written in 256-byte runs) and 4 heads per thread.
#pragma once
#include <cmath>

#include "ops.hpp"

namespace pa {

// The programs (read-only data): a D5 sine and a D6 cosine of the signed
// Q15 half-turn coordinate u (angle pi u), fitted by the workflow of section
// 3.2 (least squares on Chebyshev nodes over [0, 1] in FP64 with the endpoint
// values sin(pi) = 0, cos(0) = 1 and cos(pi) = -1 imposed, Eq. 8), every
// coefficient rounded to BF16; BF16 bit patterns:
//   sin(pi u) ~ u (a1 + a3 u^2 + a5 u^4)      {a1, a3, a5}
//   cos(pi u) ~ b0 + b2 u^2 + b4 u^4 + b6 u^6  {b0, b2, b4, b6}
// The test suite re-derives them with an independent CPU fitter.
constexpr uint16_t kRopeSin[3] = {0x4046, 0xC098, 0x3FD3};
constexpr uint16_t kRopeCos[4] = {0x3F80, 0xC09D, 0x4075, 0xBF70};

enum { RP_POLY = 0, RP_NATIVE = 1, RP_TABLE = 2 };
constexpr int RP_MAX_D = 512;

struct RopeArgs {
    const uint16_t *q, *k;
    uint16_t *qo, *ko;
    const uint32_t *table;    // RP_TABLE: [S][D / 2] words, cos low half, sin high half
    int64_t rows;             // B * S
    int32_t S, Hq, Hkv, D;
    uint32_t sc[3];           // FP16 a1, a3, a5, duplicated into both halves
    uint32_t cc[4];           // FP16 b0, b2, b4, b6
    uint32_t inc[RP_MAX_D / 2];
};

// signed Q15 half-turn coordinate of a phase: v = top 16 bits as int16
__device__ __forceinline__ int rope_q15(uint32_t phase) { return (int)(int16_t)(uint16_t)(phase >> 16); }

// accurate (cos, sin) of the angle pi v / 2^15 as an FP16 pair word
__device__ __forceinline__ uint32_t rope_native(int v)
{
    const float th = (float)v * 9.58737992428525768e-5f;   // RN32(pi / 2^15); (float)v is exact
    float sn, cs;
    sincosf(th, &sn, &cs);
    const h2 r = {(_Float16)cs, (_Float16)sn};
    return bc<uint32_t>(r);
}

// y0 = RN16(x0 c - RN16(x1 s)), y1 = RN16(x1 c + RN16(x0 s)) for the pair word x
__device__ __forceinline__ uint32_t rope_rot(uint32_t xw, _Float16 sn, _Float16 cs)
{
    const h2 x = bc<h2>(xw);
    const h2 xs = {x[1], x[0]};
    const h2 t = xs * h2{sn, sn};
    const h2 y = __builtin_elementwise_fma(x, h2{cs, cs}, h2{-t[0], t[1]});
    return bc<uint32_t>(y);
}

constexpr int RP_HPG = 8;   // heads per thread (of the Hq query then Hkv key heads)

template <int VAR>
__global__ __launch_bounds__(256) void k_rope(RopeArgs a)
{
    const int ch = a.D >> 3;                                   // 16-byte chunks per row
    const int ng = (a.Hq + a.Hkv + RP_HPG - 1) / RP_HPG;       // head groups
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t ps = gid / ch;                               // (b ng + g) S + s
    const int64_t bg = ps / a.S;
    const int64_t b = bg / ng;
    if (b * a.S >= a.rows) return;
    const int c = (int)(gid - ps * ch);
    const int s = (int)(ps - bg * a.S);
    const int g = (int)(bg - b * ng);
    const int64_t row = b * a.S + s;

    // (cos, sin) of frequencies 4c .. 4c + 3 as FP16 pairs: lane l of word j
    // is frequency 4c + 2j + l
    h2 sn[2], cs[2];
    if constexpr (VAR == RP_TABLE) {
        const u32x4 tw = *(const u32x4 *)(a.table + (int64_t)s * (a.D >> 1) + 4 * c);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const h2 t0 = bc<h2>(tw[2 * j]), t1 = bc<h2>(tw[2 * j + 1]);
            cs[j] = h2{t0[0], t1[0]};
            sn[j] = h2{t0[1], t1[1]};
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = 4 * c + 2 * j;
            const int v0 = rope_q15((uint32_t)s * a.inc[i]), v1 = rope_q15((uint32_t)s * a.inc[i + 1]);
            if constexpr (VAR == RP_POLY) {
                const h2 scale = {(_Float16)0x1p-15f, (_Float16)0x1p-15f};
                const h2 u = h2{(_Float16)v0, (_Float16)v1} * scale;   // exact scaling by 2^-15
                const h2 w = u * u;
                h2 q = __builtin_elementwise_fma(bc<h2>(a.sc[2]), w, bc<h2>(a.sc[1]));
                q = __builtin_elementwise_fma(q, w, bc<h2>(a.sc[0]));
                sn[j] = q * u;
                h2 p = __builtin_elementwise_fma(bc<h2>(a.cc[3]), w, bc<h2>(a.cc[2]));
                p = __builtin_elementwise_fma(p, w, bc<h2>(a.cc[1]));
                cs[j] = __builtin_elementwise_fma(p, w, bc<h2>(a.cc[0]));
            } else {
                const h2 t0 = bc<h2>(rope_native(v0)), t1 = bc<h2>(rope_native(v1));
                cs[j] = h2{t0[0], t1[0]};
                sn[j] = h2{t0[1], t1[1]};
            }
        }
    }

    // heads RP_HPG g .. + RP_HPG - 1 of the query heads followed by the key
    // heads; all their loads in flight before any store (the outputs never
    // alias the inputs)
    const uint16_t *__restrict__ src[RP_HPG];
    uint16_t *__restrict__ dst[RP_HPG];
    bool live[RP_HPG];
#pragma unroll
    for (int e = 0; e < RP_HPG; ++e) {
        const int h = g * RP_HPG + e;
        live[e] = h < a.Hq + a.Hkv;
        const bool isq = h < a.Hq;
        const int H = isq ? a.Hq : a.Hkv, hh = isq ? h : h - a.Hq;
        src[e] = (isq ? a.q : a.k) + (row * H + hh) * a.D + 8 * c;
        dst[e] = (isq ? a.qo : a.ko) + ((b * H + hh) * a.S + s) * a.D + 8 * c;
    }
    u32x4 x[RP_HPG];
#pragma unroll
    for (int e = 0; e < RP_HPG; ++e)
        if (live[e]) x[e] = __builtin_nontemporal_load((const u32x4 *)src[e]);
#pragma unroll
    for (int e = 0; e < RP_HPG; ++e) {
        if (!live[e]) break;
        u32x4 y;
#pragma unroll
        for (int m = 0; m < 4; ++m) y[m] = rope_rot(x[e][m], sn[m >> 1][m & 1], cs[m >> 1][m & 1]);
        __builtin_nontemporal_store(y, (u32x4 *)dst[e]);
    }
}

// the comparator's (cos, sin) table: word [s][i] for frequency i at position s
__global__ __launch_bounds__(256) void k_rope_table(uint32_t *table, RopeArgs a)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int half = a.D >> 1;
    if (gid >= (int64_t)a.S * half) return;
    const int s = (int)(gid / half), i = (int)(gid - (int64_t)s * half);
    table[gid] = rope_native(rope_q15((uint32_t)s * a.inc[i]));
}

}  // namespace pa
