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
// Two forms, no atomics, the same dQ, dK and dV bits.  With the dS blocks
// stored (while they fit the workspace limit): k_attn_bwd_rows (Delta and
// -lse log2(e) per row), k_attn_bwd_dkdv, which also stores the BF16 dS it
// forms (2 KiB per 32 x 32 block), and k_attn_bwd_dq_ds, dQ^T += K^T dS^T
// over the stored blocks, so the transform runs once.  Without them:
//   k_attn_bwd_dq    one workgroup per 128 queries of one head (4 waves x 32
//                    queries, lane = query as in the forward).  It computes
//                    Delta for its rows first (softcap) and stores it, with
//                    -lse log2(e), in the caller's workspace, then streams
//                    K / V tiles of 64 keys
//                    through LDS: S^T = K Q^T and dP^T = V dO^T with Q and dO
//                    held in registers, the transform, dQ^T += K^T dS^T with
//                    K^T read transposed from the K tile.
//   k_attn_bwd_dkdv  one workgroup per 128 keys of one key/value head (8
//                    waves: 4 groups of 32 keys, lane = key, times the two
//                    32-row halves of each query tile); it loops over the
//                    query heads of the group and the query tiles of 64 rows
//                    that see its keys, with Q / dO tiles (and the rows'
//                    -lse log2(e) and Delta) streamed through LDS: S = Q K^T
//                    and dP = dO V^T with K and V held in LDS, the
//                    transform, dV^T += dO^T P and dK^T += Q^T dS with dO^T
//                    and Q^T read transposed from the tiles.
// Both run after the forward has written O and the LSE; dkdv after dq (it
// reads Delta); in the stored form dkdv after the row pass and dq_ds last.
// Every MFMA is v_mfma_f32_32x32x16_bf16 with the operand layouts described
// in attn.hpp; P and dS are rounded to BF16 for the MFMA.
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
    uint16_t *dsb;         // BF16 dS blocks the dK/dV kernel stores for dQ, or nullptr
    int32_t nqb;           // 32-row blocks per head, ceil(S / 32)
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

// The D3 derivative program in BF16 at |c|, c = x clamped to [-Lc, Lc] by
// the forward program (the derivative shares its clamp), 0 where |x| > Lc.
__device__ __forceinline__ float dtanh_bf16(float x, float c, const TanhBF16 &d)
{
    float v = rn_bf16(fmaf(d.c[3], fabsf(c), d.c[2]));
    v = rn_bf16(fmaf(v, fabsf(c), d.c[1]));
    v = rn_bf16(fmaf(v, fabsf(c), d.c[0]));
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
        float t0, t1, x0, x1, c0, c1;
        softcap_bf16_pair(s0, s1, a.scale, a.tanhbf, t0, t1, x0, x1, c0, c1);
        const float d0 = dtanh_bf16(x0, c0, a.dtanhbf), d1 = dtanh_bf16(x1, c1, a.dtanhbf);
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

// Delta_i = dO_i . O_i and -lse_i log2(e) of every query row, for the dK/dV
// kernel when dQ is formed from stored dS blocks: the dQ kernel's arithmetic
// (the same FP32 FMAs in the same order, the halves summed by one add), one
// wave per 32 rows, lane = row and half h of each 16-column chunk.
__global__ __launch_bounds__(256) void k_attn_bwd_rows(AttnBwdArgs a, int64_t rows)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int64_t r = ((int64_t)blockIdx.x * 4 + wave) * 32 + col;
    const bool valid = r < rows;
    float acc = 0.0f;
    if (valid) {
        const uint16_t *orow = a.o + r * AT_D, *drow = a.dout + r * AT_D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 dv = ld_bf16x8(drow + ks * 16 + h * 8);
            const bf16x8 ov = ld_bf16x8(orow + ks * 16 + h * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)dv[e], (float)ov[e], acc);
        }
    }
    const float dl = acc + __shfl_xor(acc, 32);
    if (valid && h == 0) {
        a.delta[r] = dl;
        a.nlse[r] = -a.lse[r] * AT_LOG2E;
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

    // tile loads from assembly for the BF16 program (the compiler would wait
    // for the tile in flight at the next LDS read; measured on MI355X: its
    // backward 1.02x, no gain for the other modes, which keep the builtin)
    constexpr bool ASM_LOADS = MODE == AM_SOFTCAP_POLY_BF16;
    auto load_tile = [&](const uint16_t *src, uint16_t *lds, int row0) __attribute__((always_inline)) {
        if constexpr (ASM_LOADS) load_rows64_asm(src, lds, row0, S, wave, lane);
        else load_rows64(src, lds, row0, S, wave, lane);
    };
    // vmcnt(0), lgkmcnt and expcnt left alone: the Q, dO, O loads have landed
    if constexpr (ASM_LOADS) __builtin_amdgcn_s_waitcnt(0x0F70);
    load_tile(K, Ks[0], 0);
    load_tile(V, Vs[0], 0);
    auto tile = [&](int kt, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 1 < nkt) {
            load_tile(K, Ks[buf ^ 1], (kt + 1) * AT_BN);
            load_tile(V, Vs[buf ^ 1], (kt + 1) * AT_BN);
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

// Index of the stored dS block (query block qb, key block kb) of head bh:
// four query blocks (a dQ workgroup's 128 rows) side by side per key block,
// so that a dQ workgroup's two key blocks are 16 KiB in one piece and a
// dK/dV workgroup's tile is four pieces of 4 KiB.  ceil(nqb / 4) groups of
// four rows per head (the last group padded).
__device__ __forceinline__ int64_t ds_block(int64_t bh, int qb, int kb, int nqb)
{
    const int64_t nqg = (nqb + 3) / 4;
    return ((bh * nqg + (qb >> 2)) * nqb + kb) * 4 + (qb & 3);
}

constexpr int AT_BK = 128;   // keys per dK/dV workgroup
constexpr int AT_BQ = 64;    // query rows per streamed tile

// dK / dV kernel with two waves per SIMD: eight waves per workgroup of 128
// keys; wave w owns keys 32 (w % 4) .. + 31 of the workgroup and the query
// half w / 4 (rows 32 (w / 4) .. + 31) of every streamed 64-row Q / dO tile,
// so a wave keeps only its dK, dV accumulators (128 registers) and one
// 32 x 32 score block, and the two waves of a key group sum their partials
// through LDS at the end (half 0 + half 1, a fixed order).  K and V of the
// workgroup's keys sit in LDS for the whole kernel (B operands of S and dP).
// Measured on MI355X against the earlier form (four waves, one per SIMD,
// K and V in registers, all 64 rows per wave): softcap backward 1.046x
// (BF16 program), 1.01x (FP16), 1.15x (comparator); sigmoid 1.03x, 1.05x.
//
// SPLIT (grouped query heads): one workgroup per (query head, key tile)
// instead of per (key/value head, key tile), so a group's heads run in
// parallel; each writes its FP32 dK, dV contribution to a.part and
// k_attn_bwd_reduce sums the group.  Without the split the workgroups of a
// causal launch differ G-fold more in work and there are G times fewer.
template <int MODE, bool SPLIT, int EXP = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bwd_dkdv(AttnBwdArgs a)
{
    constexpr bool SOFTCAP = am_softcap(MODE);
    constexpr int AH = 1;   // operand reads ahead, in slots (2 measured no faster)
    __shared__ __attribute__((aligned(16))) uint16_t Kt[2 * AT_TILE], Vt[2 * AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Qs0[AT_TILE], Qs1[AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ds0[AT_TILE], Ds1[AT_TILE];
    __shared__ __attribute__((aligned(16))) float Ls0[AT_BQ], Ls1[AT_BQ];   // -lse * log2(e)
    __shared__ __attribute__((aligned(16))) float Es0[AT_BQ], Es1[AT_BQ];   // Delta

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kg = wave & 3, qh = wave >> 2;
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
    const int k0 = kt * AT_BK + kg * 32;
    const int my_k = k0 + col;
    const bool valid = my_k < S;

    // the workgroup's 128 K and V rows (rows past S repeat row S - 1)
    load_rows64(a.k + kvbase, Kt, kt * AT_BK, S, wave, lane);
    load_rows64(a.v + kvbase, Vt, kt * AT_BK, S, wave, lane);

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};

    const int qstart = a.causal ? kt * AT_BK : 0;
    const int nqt = (S - qstart + AT_BQ - 1) / AT_BQ;
    const int ntile = SPLIT ? nqt : G * nqt;

    // byte offsets of the lane's reads in the swizzled tiles: row chunk
    // h of row 32 qh + col (Q, dO) and 32 kg + col (K, V), and the
    // transposed read of rows 32 qh + 4 (g16 / 2) + i16 / 4, chunk
    // 2 (g16 % 2) + (i16 / 2) % 2, half 8 (i16 % 2) bytes
    const uint32_t fr = (uint32_t)swz(col, 0);
    const uint32_t bq0 = (uint32_t)(qh * 32 + col) * 256u + (((uint32_t)h ^ fr) << 4);
    const uint32_t bkv0 = (uint32_t)(kg * 32 + col) * 256u + (((uint32_t)h ^ fr) << 4);
    const int tr_r = (g16 >> 1) * 4 + (i16 >> 2), tr_c = (g16 & 1) * 2 + ((i16 >> 1) & 1);
    const uint32_t btr0 = (uint32_t)(qh * 32 + tr_r) * 256u + ((uint32_t)swz(tr_r, tr_c) << 4) +
                          (uint32_t)(i16 & 1) * 8u;
    auto head_of = [&](int t) { return SPLIT ? (int64_t)bx : (int64_t)bk * G + t / nqt; };
    // waves 0-3 load the Q tile, waves 4-7 the dO tile; waves 0 and 4 the
    // rows' -lse log2(e) and Delta
    auto load = [&](int t, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        const int64_t bh = head_of(t);
        const int r0 = qstart + (t % nqt) * AT_BQ;
        const int wv = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
        if (wv < 4) load_rows64(a.q + bh * S * AT_D, buf ? Qs1 : Qs0, r0, S, wv, lane);
        else load_rows64(a.dout + bh * S * AT_D, buf ? Ds1 : Ds0, r0, S, wv - 4, lane);
        if constexpr (SOFTCAP) {
            int r = r0 + lane;
            r = r < S ? r : S - 1;
            if (wv == 0)
                __builtin_amdgcn_global_load_lds((const void *)(a.nlse + bh * S + r),
                                                 (void __attribute__((address_space(3))) *)(buf ? Ls1 : Ls0), 4, 0, 0);
            else if (wv == 4)
                __builtin_amdgcn_global_load_lds((const void *)(a.delta + bh * S + r),
                                                 (void __attribute__((address_space(3))) *)(buf ? Es1 : Es0), 4, 0, 0);
        }
    };

    load(0, std::integral_constant<int, 0>{});
    // the dS block of a tile is stored at the start of the next one, after
    // its wait: that wait counts stores too, and a store issued at the end of
    // a tile would hold it for the store's whole latency
    u32x4 pend0 = {}, pend1 = {};
    uint16_t *pend = nullptr;
    auto flush = [&]() __attribute__((always_inline)) {
        if (pend) {
            __builtin_nontemporal_store(pend0, (u32x4 *)pend);
            __builtin_nontemporal_store(pend1, (u32x4 *)(pend + 512));
            pend = nullptr;
        }
    };
    auto tile = [&](int t, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < ntile) load(t + 1, std::integral_constant<int, buf ^ 1>{});
        flush();
        const int r0 = qstart + (t % nqt) * AT_BQ + qh * 32;   // this wave's first row
        if (a.causal && r0 + 31 < k0) return;   // every row of the half precedes these keys
        if (k0 >= S || r0 >= S) return;
        const uint16_t *Qb = buf ? Qs1 : Qs0;
        const uint16_t *Db = buf ? Ds1 : Ds0;
        const float *Lb = buf ? Ls1 : Ls0;
        const float *Eb = buf ? Es1 : Es0;
        // keys past S are masked too: their dS entries are stored for dQ
        const bool need_mask = (a.causal && r0 < k0 + 31) || r0 + 32 > S || k0 + 32 > S;
        // the lane's byte offsets (per tile, so the compiler does not hold
        // every derived address for the whole loop)
        uint32_t bq = bq0, bkv = bkv0, btr = btr0;
        asm volatile("" : "+v"(bq), "+v"(bkv), "+v"(btr));

        // S = Q K^T, dP = dO V^T of the half (lane holds key my_k, rows
        // r0 + j*8 + h*4 + i in entry j*4 + i) as 8 fenced slots (S and dP
        // of one contraction step) with the operands read one slot ahead.  Row chunk c of a swizzled tile row r
        // sits at byte r * 256 + ((c ^ f(r)) << 4), so step ks of a lane's
        // row is its step-0 offset XOR (ks << 5): one XOR per read from a
        // per-lane base instead of one held address per step
        f32x16 s = {}, dp = {};
        {
            bf16x8 qa[AH + 1], ka[AH + 1], da[AH + 1], va[AH + 1];
            auto ld = [&](auto kc) __attribute__((always_inline)) {
                constexpr int ks = decltype(kc)::value, b = ks % (AH + 1);
                const uint32_t oq = bq ^ (uint32_t)(ks << 5), ok = bkv ^ (uint32_t)(ks << 5);
                qa[b] = ld_bf16x8((const uint16_t *)((const char *)Qb + oq));
                da[b] = ld_bf16x8((const uint16_t *)((const char *)Db + oq));
                ka[b] = ld_bf16x8((const uint16_t *)((const char *)Kt + ok));
                va[b] = ld_bf16x8((const uint16_t *)((const char *)Vt + ok));
            };
            static_for<AH>([&](auto kc) __attribute__((always_inline)) { ld(kc); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<8>([&](auto kc) __attribute__((always_inline)) {
                constexpr int ks = decltype(kc)::value, b = ks % (AH + 1);
                if constexpr (ks + AH < 8) ld(std::integral_constant<int, ks + AH>{});
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[b], ka[b], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[b], va[b], dp, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        // P and dS as the B operands of the two contraction steps: fragment
        // f holds entries j = f (words 0-1) and j = f + 2 (words 2-3), i.e.
        // rows 8 f + .. of the half and the rows 16 further on
        u32x4 pw4[2], dw4[2];
        f32x4 nl4[4], dl4[4];
        auto pair = [&](auto jc, auto ic, auto masked) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value, i = decltype(ic)::value;
            constexpr bool MASKED = decltype(masked)::value;
            constexpr int e = j * 4 + i, f = j & 1, w = (j >> 1) * 2 + (i >> 1);
            if constexpr (SOFTCAP && i == 0) {
                nl4[j] = *(const f32x4 *)(&Lb[qh * 32 + j * 8 + h * 4]);
                dl4[j] = *(const f32x4 *)(&Eb[qh * 32 + j * 8 + h * 4]);
            }
            float nl0 = 0.0f, nl1 = 0.0f, dl0 = 0.0f, dl1 = 0.0f;
            if constexpr (SOFTCAP) {
                nl0 = nl4[j][i];
                nl1 = nl4[j][i + 1];
                dl0 = dl4[j][i];
                dl1 = dl4[j][i + 1];
            }
            uint32_t pk;
            float d0, d1;
            bwd_pair<MODE, EXP>(a, s[e], s[e + 1], dp[e], dp[e + 1], nl0, nl1, dl0, dl1, pk, d0, d1);
            uint32_t dk2 = pack_bf(d0, d1);
            if constexpr (MASKED) {
                const int q = r0 + j * 8 + h * 4 + i;
                const bool vis0 = valid && q < S && (!a.causal || q >= my_k);
                const bool vis1 = valid && q + 1 < S && (!a.causal || q + 1 >= my_k);
                const uint32_t keep = (vis0 ? 0x0000FFFFu : 0u) | (vis1 ? 0xFFFF0000u : 0u);
                pk &= keep;
                dk2 &= keep;
            }
            pw4[f][w] = pk;
            dw4[f][w] = dk2;
        };

        // this wave's 32 x 32 dS block for dQ: block (r0 / 32, k0 / 32) of
        // the head, at ds_block; 2 KiB: dw4[0] of lanes 0..63, then dw4[1]
        // (16 bytes per lane, so each store fills 1 KiB)
        uint16_t *dsp = nullptr;
        if (a.dsb) dsp = a.dsb + ds_block(head_of(t), r0 / 32, k0 / 32, a.nqb) * 1024 + lane * 8;

        // dV^T += dO^T P,  dK^T += Q^T dS over the half's two contraction
        // steps f, in slots (d block db) with the operands read one slot
        // ahead.  A transposed read covers rows 8 f + .. of the half and the
        // rows 16 further on (the same swizzle, so a fixed offset); d block
        // db is the chunk offset XOR (db << 6) and step f adds 8 rows, i.e.
        // XOR (1 << 5) and + 2048 bytes.  The transform of fragment 1 runs
        // one pair per slot beside the MFMAs of fragment 0.
        bf16x8 oa[AH + 1], qa[AH + 1];
        auto ld = [&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value, f = n >> 2, db = n & 3, b = n % (AH + 1);
            const uint32_t o = (btr ^ (uint32_t)((db << 6) | (f << 5))) + (uint32_t)(f * 2048);
            const u32x2 ol = ds_read_tr16((const uint16_t *)((const char *)Db + o));
            const u32x2 oh = ds_read_tr16((const uint16_t *)((const char *)Db + o + 4096));
            const u32x2 ql = ds_read_tr16((const uint16_t *)((const char *)Qb + o));
            const u32x2 qh2 = ds_read_tr16((const uint16_t *)((const char *)Qb + o + 4096));
            oa[b] = bc<bf16x8>(u32x4{ol.x, ol.y, oh.x, oh.y});
            qa[b] = bc<bf16x8>(u32x4{ql.x, ql.y, qh2.x, qh2.y});
        };
        auto run = [&](auto masked) __attribute__((always_inline)) {
            using I0 = std::integral_constant<int, 0>;
            using I2 = std::integral_constant<int, 2>;
            // fragment 0 (entries 0 and 2)
            pair(I0{}, I0{}, masked);
            pair(I0{}, I2{}, masked);
            pair(I2{}, I0{}, masked);
            pair(I2{}, I2{}, masked);
            const bf16x8 pf0 = bc<bf16x8>(pw4[0]), ds0 = bc<bf16x8>(dw4[0]);
            static_for<AH>([&](auto nc) __attribute__((always_inline)) { ld(nc); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<8>([&](auto nc) __attribute__((always_inline)) {
                constexpr int n = decltype(nc)::value, f = n >> 2, db = n & 3, b = n % (AH + 1);
                if constexpr (n + AH < 8) ld(std::integral_constant<int, n + AH>{});
                if constexpr (f == 0) {
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[b], pf0, dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[b], ds0, dk[db], 0, 0, 0);
                    // fragment 1 (entries 1 and 3), one pair per slot
                    pair(std::integral_constant<int, 1 + 2 * (db >> 1)>{}, std::integral_constant<int, 2 * (db & 1)>{},
                         masked);
                } else {
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[b], bc<bf16x8>(pw4[1]), dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[b], bc<bf16x8>(dw4[1]), dk[db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        if (need_mask) run(std::true_type{});
        else run(std::false_type{});
        if (dsp) {
            pend0 = dw4[0];
            pend1 = dw4[1];
            pend = dsp;
        }
    };
    for (int t = 0; t < ntile; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntile) tile(t + 1, std::integral_constant<int, 1>{});
    }
    flush();

    // half 1 hands its partials to half 0 through LDS (16 KB per array per
    // key group: the Q / dO buffers take dK, K / V take dV)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float *xk = (float *)(kg == 0 ? Qs0 : kg == 1 ? Qs1 : kg == 2 ? Ds0 : Ds1);
    float *xv = (float *)(kg < 2 ? Kt : Vt) + (kg & 1) * 4096;
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = (db * 4 + j) * 64 + lane;
                *(f32x4 *)(xk + c * 4) = f32x4{dk[db][j * 4], dk[db][j * 4 + 1], dk[db][j * 4 + 2], dk[db][j * 4 + 3]};
                *(f32x4 *)(xv + c * 4) = f32x4{dv[db][j * 4], dv[db][j * 4 + 1], dv[db][j * 4 + 2], dv[db][j * 4 + 3]};
            }
        }
    }
    __syncthreads();
    if (qh == 1 || !valid) return;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = (db * 4 + j) * 64 + lane;
            const f32x4 ok = *(const f32x4 *)(xk + c * 4), ov = *(const f32x4 *)(xv + c * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dk[db][j * 4 + e] += ok[e];
                dv[db][j * 4 + e] += ov[e];
            }
        }
    }
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

// dQ from the dS blocks the dK/dV kernel stored: the dQ kernel's workgroups,
// key tiles and products (dQ^T += K^T dS^T, the same operands in the same
// order, so the same dQ) with dS^T read from LDS instead of recomputed.
// The kernel streams 2 KiB of dS per 32 x 32 block (nontemporal, so the
// stream does not push K out of L2) and is bound by that stream, about
// 5 TB/s on MI355X.  Both operands come through registers (K loaded one
// tile ahead, dS two tiles ahead) and are written to LDS at the start of
// their tile, one barrier per tile, 48 KiB of LDS per workgroup: K double
// buffered (all waves read it), the dS blocks single buffered per wave (a
// wave reads only the blocks it wrote, in program order).  (Loading both
// with global-to-LDS loads into double buffers measured the same.)  The
// workgroup's dS of a tile is 16 KiB in one piece (ds_block).
// A wave's two 32 x 32 blocks of a 64-key tile are stored as the
// dK/dV kernel's fragments: 1 KiB per dword group f, 16 bytes per lane,
// lane (key c, half h') holding queries 8 f + 4 h' + i and 16 further on.
// Each B operand (lane: query q, keys 16 jj + 4 h + r and 8 further on) is
// two transposed reads: in a 16-lane group, lane m addresses the four
// consecutive queries 4 (m % 4) + 16 (g16 % 2) .. + 3 of key row
// 16 jj + 4 h + m / 4 (+ 8), so that lane j receives query j + 16 (g16 % 2)
// of the four keys.  Causal blocks above the diagonal are neither stored nor
// multiplied (their dS is zero); their loads read a stored block instead,
// as do the loads past the last tile, so that every tile issues the same
// loads.
template <int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_bwd_dq_ds(AttnBwdArgs a)
{
    constexpr int QBM = NW * 32;              // queries per workgroup
    constexpr int CH = AT_TILE / 8 / (NW * 64);   // 16-byte K chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[AT_TILE], Ks1[AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Dl[NW][2048];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int S = a.S, nqb = a.nqb;
    const int ntq = (S + QBM - 1) / QBM;
    const int nbh = (int)(gridDim.x / (unsigned)ntq);
    const int qrank = (int)blockIdx.x / nbh;
    const int bh = (int)blockIdx.x - qrank * nbh;
    const int qt = a.causal ? ntq - 1 - qrank : qrank;
    const int64_t qbase = (int64_t)bh * S * AT_D;
    const int64_t kvbase = (int64_t)(bh / a.G) * S * AT_D;
    const uint16_t *K = a.k + kvbase;
    const int q0 = qt * QBM + wave * 32;
    const int qb = q0 / 32;
    const int my_q = q0 + col;
    const bool valid = my_q < S;
    const int qbc = qb < nqb ? qb : nqb - 1;
    const int kbmax = a.causal ? qbc : nqb - 1;   // last stored block of the row
    const uint16_t *dsrow = a.dsb + ds_block(bh, qb, 0, nqb) * 1024 + lane * 8;   // key block 0
    auto has_block = [&](int kb) { return q0 < S && kb <= kbmax; };

    const int kend = a.causal ? (qt * QBM + QBM < S ? qt * QBM + QBM : S) : S;
    const int nkt = (kend + AT_BN - 1) / AT_BN;

    // K tile kt (clamped to the last): thread tid holds chunk idx % 16 of
    // row idx / 16 for idx = tid + 64 NW i (rows past S repeat row S - 1)
    auto load_k = [&](int kt, u32x4 (&r)[CH]) __attribute__((always_inline)) {
        kt = kt < nkt ? kt : nkt - 1;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + NW * 64 * i, row = idx >> 4, c = idx & 15;
            int g = kt * AT_BN + row;
            g = g < S ? g : S - 1;
            r[i] = *(const u32x4 *)(K + (int64_t)g * AT_D + c * 8);
        }
    };
    auto store_k = [&](uint16_t *lds, const u32x4 (&r)[CH]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + NW * 64 * i, row = idx >> 4, c = idx & 15;
            *(u32x4 *)(lds + row * AT_D + swz(row, c) * 8) = r[i];
        }
    };
    // the lane's 2 x 16 bytes of this wave's blocks 2 kt and 2 kt + 1 (a
    // stored block in their place where they do not exist)
    auto load_d = [&](int kt, u32x4 (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            int kb = kt * 2 + b;
            kb = kb <= kbmax ? kb : kbmax;
            const uint16_t *p = dsrow + (int64_t)kb * 4096;
            r[2 * b] = __builtin_nontemporal_load((const u32x4 *)p);
            r[2 * b + 1] = __builtin_nontemporal_load((const u32x4 *)(p + 512));
        }
    };

    // In LDS a fragment (dword group f, 16 bytes of stored lane L) sits at
    // 16-byte slot L ^ ((2 f + L / 32) << 2) of its 1 KiB (bits 2-3 of the
    // slot swizzled, so that the 16 lanes of a transposed read hit 16
    // different slots: without it four of them shared each bank).  The
    // lane's read for key row 16 jj + 8 half + 4 h + r (r = i16 / 4) of
    // stored lane key + 32 (u % 2) in group f = u / 2 (u = i16 % 4), half
    // g16 % 2: slot bits 2-3 are (2 half + h) ^ u.
    const int u = i16 & 3;
    const uint32_t trb = (uint32_t)((u >> 1) * 1024 + (32 * (u & 1) + (i16 >> 2)) * 16 + (g16 & 1) * 8);
    const uint32_t tlo = trb + (uint32_t)((h ^ u) * 64), thi = trb + (uint32_t)(((h ^ u) ^ 2) * 64);
    uint16_t *dl = Dl[wave];

    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

    // tiles held in registers (measured on MI355X: 1-3 K tiles and 1-3 dS
    // tiles within 2 %, more registers slower)
    constexpr int KD = 1, DD = 2;
    u32x4 kr[KD][CH], dr[DD][4];
#pragma unroll
    for (int j = 0; j < KD; ++j) load_k(j, kr[j]);
#pragma unroll
    for (int j = 0; j < DD; ++j) load_d(j, dr[j]);
    auto tile = [&](int kt, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        uint16_t *Kb = buf ? Ks1 : Ks0;
        store_k(Kb, kr[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(u32x4 *)(dl + (i >> 1) * 1024 + (i & 1) * 512 + (lane ^ ((2 * (i & 1) + (lane >> 5)) << 2)) * 8) =
                dr[0][i];
        __syncthreads();
#pragma unroll
        for (int j = 0; j + 1 < KD; ++j)
#pragma unroll
            for (int i = 0; i < CH; ++i) kr[j][i] = kr[j + 1][i];
        load_k(kt + KD, kr[KD - 1]);
#pragma unroll
        for (int j = 0; j + 1 < DD; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) dr[j][i] = dr[j + 1][i];
        load_d(kt + DD, dr[DD - 1]);
        const int key0 = kt * AT_BN;
        if (a.causal && key0 > q0 + 31) return;
        if (q0 >= S) return;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!has_block(kt * 2 + kb)) continue;
            const char *blk = (const char *)dl + kb * 2048;
            bf16x8 dsf[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const u32x2 lo = ds_read_tr16((const uint16_t *)(blk + tlo + jj * 256));
                const u32x2 hi = ds_read_tr16((const uint16_t *)(blk + thi + jj * 256));
                dsf[jj] = bc<bf16x8>(u32x4{lo.x, lo.y, hi.x, hi.y});
            }
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
