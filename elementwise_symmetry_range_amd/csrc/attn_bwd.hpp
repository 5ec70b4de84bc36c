// attn_bwd.hpp -- flash-attention backward with a transformed score, gfx950 MFMA.
//
// The chain rule through O = P V for the two transforms of attn.hpp
// ("Fast Polynomial Transcendentals for LLMs"):
//   dV = P^T dO,  dP = dO V^T,
//   softcap  dS = P (dP - Delta) ds/dS,  Delta_i = dO_i . O_i, P recomputed
//            from the saved natural log-sum-exp (with the forward's exp2: the
//            hardware exponential or a software core); the polynomial variant
//            uses the analytic derivative of the D4 tanh program, a D3 with
//            coefficients (j + 1) c_{j+1} (BF16-rounded for the BF16 program,
//            exact in FP16 for the FP16 one), in the program's format at |x|,
//            and 0 beyond the clamp, where the clamped forward program is
//            constant (sections 3.3 and 5.2.2); the comparator uses
//            1 - tanh^2 recomputed with tanhf (Eq. 12);
//   sigmoid  dS = dP dP~/ds; the polynomial variant uses the factored
//            surrogate P~ (a + b x) of section 3.4 from the same region,
//            clamp and Horner value as the forward; the comparator
//            sigma (1 - sigma);
//   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D) (summed over the query heads
//   that share a key/value head).
//
// Two kernels, no atomics:
//   k_attn_bwd_dq    one workgroup per 128 queries of one head (4 waves x 32
//                    queries, lane = query as in the forward).  It computes
//                    Delta for its rows first (softcap) and stores it, with
//                    -lse log2(e), in the caller's workspace, then streams
//                    K / V tiles of 64 keys
//                    through LDS: S^T = K Q^T and dP^T = V dO^T with Q and dO
//                    held in registers, the transform, dQ^T += K^T dS^T with
//                    K^T read transposed from the K tile.
//   k_attn_bwd_dkdv  one workgroup per 128 keys of one key/value head (4
//                    waves x 32 keys, lane = key); it loops over the query
//                    heads of the group and the query tiles of 64 rows that
//                    see its keys, with Q / dO tiles (and the rows'
//                    -lse log2(e) and Delta) streamed through LDS: S = Q K^T and dP = dO V^T
//                    with K and V held in registers, the transform,
//                    dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//                    transposed from the tiles.
// Both run after the forward has written O and the LSE; dkdv after dq (it
// reads Delta).  Every MFMA is v_mfma_f32_32x32x16_bf16 with the operand
// layouts described in attn.hpp; P and dS are rounded to BF16 for the MFMA.
#pragma once
#include <type_traits>

#include "attn.hpp"

namespace pa {

struct AttnBwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;      // softcap: natural log-sum-exp per query row
    float *delta;          // softcap: workspace, Delta per query row
    float *nlse;           // softcap: workspace, -lse * log2(e) per query row
    float *part;           // grouped query heads: FP32 dK, dV partials per query head
    uint16_t *dq, *dk, *dv;
    int32_t S, H, G;       // G = H / Hkv
    int32_t causal;
    float scale;           // as AttnArgs
    float c2;
    float logn;
    float rsd;             // RN_f32(1 / sqrt D)
    CoefF16 tanh16;        // D4 tanh program
    CoefF16 dtanh16;       // its derivative, D3 (FP16 coefficients)
    TanhBF16 tanhbf;       // the D4 tanh program in BF16
    TanhBF16 dtanhbf;      // its derivative, D3 (BF16 coefficients)
    SigCoef sig;
};

// The D3 derivative program in BF16 at |x|, 0 where |x| > Lc.
__device__ __forceinline__ float dtanh_bf16(float x, const TanhBF16 &d)
{
    const float th = fabsf(__builtin_amdgcn_fmed3f(x, -d.lc, d.lc));
    float v = rn_bf16(fmaf(d.c[3], th, d.c[2]));
    v = rn_bf16(fmaf(v, th, d.c[1]));
    v = rn_bf16(fmaf(v, th, d.c[0]));
    return fabsf(x) > d.lc ? 0.0f : v;
}

// P = 2^z of the backward for a pair, z the exponent arguments, with the
// forward's exponential: v_exp_f32 (EXP = 0) or 2^floor(z) p(z - floor z)
// by a software core.
template <int EXP>
__device__ __forceinline__ void bwd_exp2(float z0, float z1, float &p0, float &p1)
{
    if constexpr (EXP == 0) {
        p0 = __builtin_amdgcn_exp2f(z0);
        p1 = __builtin_amdgcn_exp2f(z1);
    } else {
        exp2_core_pair<EXP>(z0, z1, 0.0f, p0, p1);
    }
}

// dS and P of a pair of scores; s0, s1 raw scores, dp0, dp1 = dO . V,
// nl0, nl1 = -lse * log2(e) (softcap), dl0, dl1 = Delta (softcap).  P comes
// back as the packed BF16 pair the dV product takes (the sigmoid program
// produces it in that form), dS as FP32.
template <int MODE, int EXP = 0>
__device__ __forceinline__ void bwd_pair(const AttnBwdArgs &a, float s0, float s1, float dp0,
                                         float dp1, float nl0, float nl1, float dl0, float dl1,
                                         uint32_t &pw, float &ds0, float &ds1)
{
    if constexpr (MODE == AM_SOFTCAP_POLY) {
        uint32_t aw;
        const uint32_t tw = softcap_poly_pair(s0, s1, a.scale, a.tanh16, aw);
        uint32_t dw = bc<uint32_t>(horner_f16<3, false>(bc<h2>(min_u16x2(aw, a.dtanh16.lc)), a.dtanh16));
        // 0 where |x| > Lc: the sign of the 16-bit Lc - |x| (no overflow:
        // both are at most 0x7FFF)
        dw &= ~fill_sign16(bc<uint32_t>(bc<i16x2>(a.dtanh16.lc) - bc<i16x2>(aw)));
        float p0, p1;
        bwd_exp2<EXP>(fma_mix_lo(tw, a.c2, nl0), fma_mix_hi(tw, a.c2, nl1), p0, p1);
        ds0 = fma_mix_lo(dw, p0 * (dp0 - dl0), -0.0f);
        ds1 = fma_mix_hi(dw, p1 * (dp1 - dl1), -0.0f);
        pw = pack_bf(p0, p1);
    } else if constexpr (MODE == AM_SOFTCAP_POLY_BF16) {
        float t0, t1, x0, x1;
        softcap_bf16_pair(s0, s1, a.scale, a.tanhbf, t0, t1, x0, x1);
        const float d0 = dtanh_bf16(x0, a.dtanhbf), d1 = dtanh_bf16(x1, a.dtanhbf);
        float p0, p1;
        bwd_exp2<EXP>(fmaf(t0, a.c2, nl0), fmaf(t1, a.c2, nl1), p0, p1);
        ds0 = d0 * (p0 * (dp0 - dl0));
        ds1 = d1 * (p1 * (dp1 - dl1));
        pw = pack_bf(p0, p1);
    } else if constexpr (MODE == AM_SOFTCAP_NATIVE) {
        const float t0 = tanhf(s0 * a.scale), t1 = tanhf(s1 * a.scale);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(t0, a.c2, nl0));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(t1, a.c2, nl1));
        ds0 = p0 * (dp0 - dl0) * fmaf(-t0, t0, 1.0f);
        ds1 = p1 * (dp1 - dl1) * fmaf(-t1, t1, 1.0f);
        pw = pack_bf(p0, p1);
    } else if constexpr (MODE == AM_SIGMOID_POLY) {
        float g0, g1;
        pw = sigmoid_poly_pair<true>(s0, s1, a.scale, a.sig, &g0, &g1);
        ds0 = dp0 * g0;
        ds1 = dp1 * g1;
    } else {
        const float p0 = sigmoid_acc(fmaf(s0, a.scale, -a.logn));
        const float p1 = sigmoid_acc(fmaf(s1, a.scale, -a.logn));
        ds0 = dp0 * (p0 * (1.0f - p0));
        ds1 = dp1 * (p1 * (1.0f - p1));
        pw = pack_bf(p0, p1);
    }
}

template <int MODE, int EXP = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bwd_dq(AttnBwdArgs a)
{
    constexpr bool SOFTCAP = am_softcap(MODE);
    // one [2][tile] array each (see dbuf: separate arrays make this kernel spill)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][AT_TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int S = a.S;
    const int ntq = (S + AT_BM - 1) / AT_BM;
    const int nbh = (int)(gridDim.x / (unsigned)ntq);
    const int qrank = (int)blockIdx.x / nbh;
    const int bh = (int)blockIdx.x - qrank * nbh;
    const int qt = a.causal ? ntq - 1 - qrank : qrank;
    const int64_t qbase = (int64_t)bh * S * AT_D;
    const int64_t kvbase = (int64_t)(bh / a.G) * S * AT_D;
    const uint16_t *Q = a.q + qbase, *dO = a.dout + qbase;
    const uint16_t *K = a.k + kvbase, *V = a.v + kvbase;
    const int q0 = qt * AT_BM + wave * 32;
    const int my_q = q0 + col;
    const bool valid = my_q < S;

    // Q and dO as B operands: lane holds row my_q, columns ks*16 + h*8 + 0..7
    bf16x8 qf[8], df[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        qf[ks] = valid ? ld_bf16x8(Q + (int64_t)my_q * AT_D + ks * 16 + h * 8) : bf16x8{};
        df[ks] = valid ? ld_bf16x8(dO + (int64_t)my_q * AT_D + ks * 16 + h * 8) : bf16x8{};
    }
    float nl = 0.0f, dl = 0.0f;
    if constexpr (SOFTCAP) {
        float acc = 0.0f;
        if (valid) {
            const uint16_t *orow = a.o + qbase + (int64_t)my_q * AT_D;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 ov = ld_bf16x8(orow + ks * 16 + h * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)df[ks][e], (float)ov[e], acc);
            }
        }
        dl = acc + __shfl_xor(acc, 32);
        if (valid) {
            nl = -a.lse[(int64_t)bh * S + my_q] * AT_LOG2E;
            if (h == 0) {
                a.delta[(int64_t)bh * S + my_q] = dl;
                a.nlse[(int64_t)bh * S + my_q] = nl;   // the dK/dV kernel streams it
            }
        }
    }

    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

    const int kend = a.causal ? (qt * AT_BM + AT_BM < S ? qt * AT_BM + AT_BM : S) : S;
    const int nkt = (kend + AT_BN - 1) / AT_BN;

    load_rows64(K, Ks[0], 0, S, wave, lane);
    load_rows64(V, Vs[0], 0, S, wave, lane);
    auto tile = [&](int kt, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 1 < nkt) {
            load_rows64(K, Ks[buf ^ 1], (kt + 1) * AT_BN, S, wave, lane);
            load_rows64(V, Vs[buf ^ 1], (kt + 1) * AT_BN, S, wave, lane);
        }
        const int key0 = kt * AT_BN;
        if (a.causal && key0 > q0 + 31) return;
        if (q0 >= S) return;
        const uint16_t *Kb = Ks[buf];
        const uint16_t *Vb = Vs[buf];

        // one 32-key block at a time (keeps two accumulators live, not four)
        const bool need_mask = (a.causal && key0 + AT_BN - 1 > q0) || key0 + AT_BN > S;
        const int lim = a.causal ? (my_q < S - 1 ? my_q : S - 1) : S - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Kb, kb * 32 + col, ks * 2 + h), qf[ks],
                                                            s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Vb, kb * 32 + col, ks * 2 + h), df[ks],
                                                             dp, 0, 0, 0);
            }
            // dS^T of the block, as BF16 B operands in the permuted key order
            bf16x8 dsf[2];
            auto transform = [&](auto masked) {
                constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    u32x4 fw;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int e = jj * 8 + e2 * 2;
                        uint32_t pw;   // P is not needed here
                        float d0, d1;
                        bwd_pair<MODE, EXP>(a, s[e], s[e + 1], dp[e], dp[e + 1], nl, nl, dl, dl, pw, d0, d1);
                        uint32_t w = pack_bf(d0, d1);
                        if constexpr (MASKED) {
                            const int k0 = key0 + kb * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
                            const uint32_t mlo = k0 > lim ? 0x0000FFFFu : 0u;
                            const uint32_t mhi = k0 + 1 > lim ? 0xFFFF0000u : 0u;
                            w &= ~(mlo | mhi);
                        }
                        fw[e2] = w;
                    }
                    dsf[jj] = bc<bf16x8>(fw);
                }
            };
            if (need_mask) transform(std::true_type{});
            else transform(std::false_type{});

            // dQ^T += K^T dS^T over this block's two contraction steps
#pragma unroll
            for (int db = 0; db < 4; ++db) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_a(Kb, kb * 2 + jj, db, g16, i16),
                                                                     dsf[jj], dq[db], 0, 0, 0);
            }
        }
    };
    for (int kt = 0; kt < nkt; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nkt) tile(kt + 1, std::integral_constant<int, 1>{});
    }

    if (!valid) return;
    uint16_t *row = a.dq + qbase + (int64_t)my_q * AT_D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + j * 8 + h * 4;
            u32x2 w;
            w.x = pack_bf(dq[db][j * 4 + 0] * a.rsd, dq[db][j * 4 + 1] * a.rsd);
            w.y = pack_bf(dq[db][j * 4 + 2] * a.rsd, dq[db][j * 4 + 3] * a.rsd);
            *(u32x2 *)(row + d) = w;
        }
    }
}

constexpr int AT_BK = 128;   // keys per dK/dV workgroup
constexpr int AT_BQ = 64;    // query rows per streamed tile

// SPLIT (grouped query heads): one workgroup per (query head, key tile)
// instead of per (key/value head, key tile), so a group's heads run in
// parallel; each writes its FP32 dK, dV contribution to a.part and
// k_attn_bwd_reduce sums the group.  Without the split the workgroups of a
// causal launch differ G-fold more in work and there are G times fewer.
template <int MODE, bool SPLIT, int EXP = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_bwd_dkdv(AttnBwdArgs a)
{
    constexpr bool SOFTCAP = am_softcap(MODE);
    // double buffers (see dbuf): separate arrays except for the softcap
    // comparator, whose tanh needs the registers (it spills with them)
    constexpr bool SPLIT_LDS = MODE != AM_SOFTCAP_NATIVE;
    __shared__ __attribute__((aligned(16))) uint16_t Qs0[AT_TILE], Qs1[AT_TILE], Qp[2][AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ds0[AT_TILE], Ds1[AT_TILE], Dp[2][AT_TILE];
    __shared__ __attribute__((aligned(16))) float Ls0[AT_BQ], Ls1[AT_BQ], Lp[2][AT_BQ];   // -lse * log2(e)
    __shared__ __attribute__((aligned(16))) float Es0[AT_BQ], Es1[AT_BQ], Ep[2][AT_BQ];   // Delta

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int S = a.S, G = a.G;
    const int ntk = (S + AT_BK - 1) / AT_BK;
    const int nbk = (int)(gridDim.x / (unsigned)ntk);       // B * Hkv, or B * H (SPLIT)
    const int krank = (int)blockIdx.x / nbk;                 // 0 = heaviest key tile
    const int bx = (int)blockIdx.x - krank * nbk;            // b Hkv + hk, or b H + h (SPLIT)
    const int bk = SPLIT ? bx / G : bx;                      // key/value head
    const int kt = krank;                                    // causal: key tile 0 sees the most queries
    const int64_t kvbase = (int64_t)bk * S * AT_D;
    const int k0 = kt * AT_BK + wave * 32;
    const int my_k = k0 + col;
    const bool valid = my_k < S;

    // K and V as B operands of S = Q K^T and dP = dO V^T: lane holds row my_k
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        kf[ks] = valid ? ld_bf16x8(a.k + kvbase + (int64_t)my_k * AT_D + ks * 16 + h * 8) : bf16x8{};
        vf[ks] = valid ? ld_bf16x8(a.v + kvbase + (int64_t)my_k * AT_D + ks * 16 + h * 8) : bf16x8{};
    }
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};

    // query tiles: every head of the group, rows from the first one that can
    // see this workgroup's keys
    const int qstart = a.causal ? kt * AT_BK : 0;
    const int nqt = (S - qstart + AT_BQ - 1) / AT_BQ;
    const int ntile = SPLIT ? nqt : G * nqt;

    auto head_of = [&](int t) { return SPLIT ? (int64_t)bx : (int64_t)bk * G + t / nqt; };
    auto load = [&](int t, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        const int64_t bh = head_of(t);
        const int r0 = qstart + (t % nqt) * AT_BQ;
        load_rows64(a.q + bh * S * AT_D, dbuf<buf, SPLIT_LDS>(Qs0, Qs1, Qp), r0, S, wave, lane);
        load_rows64(a.dout + bh * S * AT_D, dbuf<buf, SPLIT_LDS>(Ds0, Ds1, Dp), r0, S, wave, lane);
        if constexpr (SOFTCAP) {
            const int wv = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
            int r = r0 + lane;
            r = r < S ? r : S - 1;
            // one fixed destination array per load (keeps its alias scope)
            if (wv == 0)
                __builtin_amdgcn_global_load_lds((const void *)(a.nlse + bh * S + r),
                                                 (void __attribute__((address_space(3))) *)dbuf<buf, SPLIT_LDS>(Ls0, Ls1, Lp), 4, 0, 0);
            else if (wv == 1)
                __builtin_amdgcn_global_load_lds((const void *)(a.delta + bh * S + r),
                                                 (void __attribute__((address_space(3))) *)dbuf<buf, SPLIT_LDS>(Es0, Es1, Ep), 4, 0, 0);
        }
    };

    // ---- an unmasked tile as explicit scheduling slots -----------------------
    // With one wave per SIMD nothing else hides a wave's latencies, so the 64
    // MFMAs of a tile (m < 32: S and dP, query block m / 16, contraction step
    // (m % 16) / 2, S for even m; m >= 32: n = m - 32, fragment n / 8, d block
    // (n % 8) / 2, dV for even n) run two per slot with every LDS operand read
    // AT_BW_AHEAD slots ahead, and the transform of query block 0 runs beside
    // the S / dP MFMAs of block 1 (slots 8-15), that of block 1 beside the
    // dV / dK MFMAs of fragments 0 and 1 (slots 16-23), one score pair per
    // slot.  A scheduling fence closes each slot.  Every accumulator sees its
    // terms in the order of the masked path below, so the outputs are those
    // of the unslotted tile bit for bit (measured on MI355X: softcap backward
    // 1.085x, sigmoid 1.07x, the comparators 1.09-1.13x).
    constexpr int AT_BW_AHEAD = 2;   // 1 and 3 measured within 1 %
    auto slotted_tile = [&](const uint16_t *Qb, const uint16_t *Db, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        f32x16 s[2], dp[2];
        bf16x8 pf[4], dsf[4];
        uint32_t pw[4][4], dw[4][4];   // P and dS words of fragment f
        bf16x8 op[64];
        f32x4 nlb[2], dlb[2];          // -lse log2(e) and Delta of a group of 4 query rows
        auto load_op = [&](auto mc) __attribute__((always_inline)) {
            constexpr int M = decltype(mc)::value;
            if constexpr (M < 32) {
                constexpr int qb = M >> 4, ks = (M & 15) >> 1;
                op[M] = lds_row8((M & 1) ? Db : Qb, qb * 32 + col, ks * 2 + h);
            } else {
                constexpr int n = M - 32;
                op[M] = lds_tr_a((n & 1) ? Qb : Db, n >> 3, (n & 7) >> 1, g16, i16);
            }
        };
        auto mfma_op = [&](auto mc) __attribute__((always_inline)) {
            constexpr int M = decltype(mc)::value;
            if constexpr (M < 32) {
                constexpr int qb = M >> 4, ks = (M & 15) >> 1;
                if constexpr ((M & 1) == 0)
                    s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[M], kf[ks], ks == 0 ? f32x16{} : s[qb], 0, 0, 0);
                else
                    dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[M], vf[ks], ks == 0 ? f32x16{} : dp[qb], 0, 0, 0);
            } else {
                constexpr int n = M - 32, f = n >> 3, db = (n & 7) >> 1;
                if constexpr ((n & 1) == 0)
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[M], pf[f], dv[db], 0, 0, 0);
                else
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[M], dsf[f], dk[db], 0, 0, 0);
            }
        };
        // LSE / Delta of group g = 4 qb + j (query rows qb*32 + j*8 + h*4 .. + 3)
        auto group_load = [&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value, qb = g >> 2, j = g & 3;
            if constexpr (SOFTCAP) {
                nlb[g & 1] = *(const f32x4 *)(&dbuf<buf, SPLIT_LDS>(Ls0, Ls1, Lp)[qb * 32 + j * 8 + h * 4]);
                dlb[g & 1] = *(const f32x4 *)(&dbuf<buf, SPLIT_LDS>(Es0, Es1, Ep)[qb * 32 + j * 8 + h * 4]);
            }
        };
        // score pair P: query block P / 8, rows j*8 + h*4 + i, i + 1 with
        // j = (P % 8) / 2, i = 2 (P % 2)
        auto pair = [&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value, qb = P >> 3, j = (P & 7) >> 1, i = (P & 1) * 2;
            constexpr int e = j * 4 + i;
            float nl0 = 0.0f, nl1 = 0.0f, dl0 = 0.0f, dl1 = 0.0f;
            if constexpr (SOFTCAP) {
                nl0 = nlb[j & 1][i];
                nl1 = nlb[j & 1][i + 1];
                dl0 = dlb[j & 1][i];
                dl1 = dlb[j & 1][i + 1];
            }
            float d0, d1;
            constexpr int f = qb * 2 + (j >> 1), w = (j & 1) * 2 + (i >> 1);
            bwd_pair<MODE, EXP>(a, s[qb][e], s[qb][e + 1], dp[qb][e], dp[qb][e + 1], nl0, nl1, dl0, dl1,
                                pw[f][w], d0, d1);
            dw[f][w] = pack_bf(d0, d1);
            if constexpr (w == 3) {
                pf[f] = bc<bf16x8>(u32x4{pw[f][0], pw[f][1], pw[f][2], pw[f][3]});
                dsf[f] = bc<bf16x8>(u32x4{dw[f][0], dw[f][1], dw[f][2], dw[f][3]});
            }
        };
        static_for<2 * AT_BW_AHEAD>([&](auto mc) __attribute__((always_inline)) { load_op(mc); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<32>([&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            static_for<2>([&](auto ic) __attribute__((always_inline)) {
                constexpr int M = 2 * (t + AT_BW_AHEAD) + decltype(ic)::value;
                if constexpr (M < 64) load_op(std::integral_constant<int, M>{});
            });
            // the group's LSE / Delta one slot before its first pair
            if constexpr (t >= 7 && t < 23 && ((t - 7) & 1) == 0)
                group_load(std::integral_constant<int, (t - 7) / 2>{});
            mfma_op(std::integral_constant<int, 2 * t>{});
            mfma_op(std::integral_constant<int, 2 * t + 1>{});
            if constexpr (t >= 8 && t < 24) pair(std::integral_constant<int, t - 8>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    load(0, std::integral_constant<int, 0>{});
    auto tile = [&](int t, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < ntile) load(t + 1, std::integral_constant<int, buf ^ 1>{});
        const int r0 = qstart + (t % nqt) * AT_BQ;
        if (a.causal && r0 + AT_BQ - 1 < k0) return;   // every row of the tile precedes these keys
        if (k0 >= S) return;
        const uint16_t *Qb = dbuf<buf, SPLIT_LDS>(Qs0, Qs1, Qp);
        const uint16_t *Db = dbuf<buf, SPLIT_LDS>(Ds0, Ds1, Dp);
        const bool need_mask = (a.causal && r0 < k0 + 31) || r0 + AT_BQ > S;
        if (!need_mask) {
            slotted_tile(Qb, Db, bufc);
            return;
        }

        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            s[qb] = f32x16{};
            dp[qb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Qb, qb * 32 + col, ks * 2 + h),
                                                                kf[ks], s[qb], 0, 0, 0);
                dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Db, qb * 32 + col, ks * 2 + h),
                                                                 vf[ks], dp[qb], 0, 0, 0);
            }
        }

        // a masked tile (the causal diagonal or the ragged end; every other
        // tile takes slotted_tile): s[qb][j*4 + i] is query r0 + qb*32 + j*8 +
        // h*4 + i of this lane's key
        bf16x8 pf[4] = {}, dsf[4] = {};
        {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 nl4 = {}, dl4 = {};
                    if constexpr (SOFTCAP) {
                        nl4 = *(const f32x4 *)(&dbuf<buf, SPLIT_LDS>(Ls0, Ls1, Lp)[qb * 32 + j * 8 + h * 4]);
                        dl4 = *(const f32x4 *)(&dbuf<buf, SPLIT_LDS>(Es0, Es1, Ep)[qb * 32 + j * 8 + h * 4]);
                    }
                    uint32_t pw[2], dw[2];
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const int e = j * 4 + i;
                        uint32_t pk;
                        float d0, d1;
                        bwd_pair<MODE, EXP>(a, s[qb][e], s[qb][e + 1], dp[qb][e], dp[qb][e + 1], nl4[i],
                                            nl4[i + 1], dl4[i], dl4[i + 1], pk, d0, d1);
                        uint32_t dk2 = pack_bf(d0, d1);
                        const int q = r0 + qb * 32 + j * 8 + h * 4 + i;
                        const bool vis0 = q < S && (!a.causal || q >= my_k);
                        const bool vis1 = q + 1 < S && (!a.causal || q + 1 >= my_k);
                        const uint32_t keep = (vis0 ? 0x0000FFFFu : 0u) | (vis1 ? 0xFFFF0000u : 0u);
                        pk &= keep;
                        dk2 &= keep;
                        pw[i >> 1] = pk;
                        dw[i >> 1] = dk2;
                    }
                    // B-operand fragment ks = 2 qb + j / 2 holds accumulator
                    // entries (j % 2) * 8 .. + 7
                    const int f = qb * 2 + (j >> 1);
                    const int half = (j & 1) * 2;
                    u32x4 pv = bc<u32x4>(pf[f]), dv4 = bc<u32x4>(dsf[f]);
                    pv[half] = pw[0];
                    pv[half + 1] = pw[1];
                    dv4[half] = dw[0];
                    dv4[half + 1] = dw[1];
                    pf[f] = bc<bf16x8>(pv);
                    dsf[f] = bc<bf16x8>(dv4);
                }
            }
        }

        // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_a(Db, ks, db, g16, i16), pf[ks],
                                                                 dv[db], 0, 0, 0);
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_a(Qb, ks, db, g16, i16), dsf[ks],
                                                                 dk[db], 0, 0, 0);
            }
        }
    };
    for (int t = 0; t < ntile; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntile) tile(t + 1, std::integral_constant<int, 1>{});
    }

    if (!valid) return;
    if constexpr (SPLIT) {
        // FP32 partials of this query head: part[0][bx][my_k][:] = dK (before
        // the 1/sqrt(D) factor), part[1][bx][my_k][:] = dV
        const int64_t plane = (int64_t)gridDim.x / ntk * S * AT_D;   // B H S D
        float *pk = a.part + (int64_t)bx * S * AT_D + (int64_t)my_k * AT_D;
        float *pv = pk + plane;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = db * 32 + j * 8 + h * 4;
                *(f32x4 *)(pk + d) = f32x4{dk[db][j * 4], dk[db][j * 4 + 1], dk[db][j * 4 + 2], dk[db][j * 4 + 3]};
                *(f32x4 *)(pv + d) = f32x4{dv[db][j * 4], dv[db][j * 4 + 1], dv[db][j * 4 + 2], dv[db][j * 4 + 3]};
            }
        }
        return;
    }
    uint16_t *krow = a.dk + kvbase + (int64_t)my_k * AT_D;
    uint16_t *vrow = a.dv + kvbase + (int64_t)my_k * AT_D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + j * 8 + h * 4;
            u32x2 w;
            w.x = pack_bf(dk[db][j * 4 + 0] * a.rsd, dk[db][j * 4 + 1] * a.rsd);
            w.y = pack_bf(dk[db][j * 4 + 2] * a.rsd, dk[db][j * 4 + 3] * a.rsd);
            *(u32x2 *)(krow + d) = w;
            w.x = pack_bf(dv[db][j * 4 + 0], dv[db][j * 4 + 1]);
            w.y = pack_bf(dv[db][j * 4 + 2], dv[db][j * 4 + 3]);
            *(u32x2 *)(vrow + d) = w;
        }
    }
}

// dK, dV of a key/value head = the sum of its G query heads' FP32 partials
// (the group's heads in order, so the result does not depend on scheduling);
// one thread per 8 consecutive elements of a [B Hkv S D] output.
__global__ __launch_bounds__(256) void k_attn_bwd_reduce(AttnBwdArgs a, int64_t n8, int64_t SD)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const int64_t e = i * 8;                 // element of [B Hkv S D]
    const int64_t bk = e / SD, r = e - bk * SD;
    const int64_t plane = n8 * 8 * a.G;      // B H S D
    const float *pk = a.part + (bk * a.G) * SD + r;
    f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
    for (int g = 0; g < a.G; ++g) {
        const float *p = pk + (int64_t)g * SD;
        k0 += *(const f32x4 *)p;
        k1 += *(const f32x4 *)(p + 4);
        v0 += *(const f32x4 *)(p + plane);
        v1 += *(const f32x4 *)(p + plane + 4);
    }
    u32x4 wk, wv;
    wk[0] = pack_bf(k0[0] * a.rsd, k0[1] * a.rsd);
    wk[1] = pack_bf(k0[2] * a.rsd, k0[3] * a.rsd);
    wk[2] = pack_bf(k1[0] * a.rsd, k1[1] * a.rsd);
    wk[3] = pack_bf(k1[2] * a.rsd, k1[3] * a.rsd);
    wv[0] = pack_bf(v0[0], v0[1]);
    wv[1] = pack_bf(v0[2], v0[3]);
    wv[2] = pack_bf(v1[0], v1[1]);
    wv[3] = pack_bf(v1[2], v1[3]);
    *(u32x4 *)(a.dk + e) = wk;
    *(u32x4 *)(a.dv + e) = wv;
}

}  // namespace pa
