// attn.hpp -- softcapped flash-attention forward on gfx950 MFMA.
//
// Scores are transformed by the softcap alpha tanh(x / alpha) ("Fast
// Polynomial Transcendentals for LLMs", Eq. 1) inside the attention tile;
// the polynomial variant evaluates the D4 tanh program (section 5.2.2 puts a
// packed D4 tanh inside the attention forward).  On gfx950 the packed 16-bit
// FMA is FP16 (v_pk_fma_f16); there is no packed BF16 FMA.  The program
// therefore runs in packed FP16 on x = RN_f16(RN_f32(S) * RN_f32(1/(cap sqrt D))),
// two scores per instruction, with the FP16 coefficients of the same BF16 fit.
// The comparator uses accurate FP32 tanhf on the unrounded FP32 x.
//
// Layout and tiling (D = 128):
//   workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
//   queries q0 .. q0 + 31.  Key/value tiles of 64 rows are staged in LDS
//   (K row-major, V transposed to Vt[d][key]) and the next tile is prefetched
//   into registers while the current one is consumed.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q held
//   in registers; the accumulator gives every lane one query (column) and 16
//   keys of each 32-key block, so the softmax row reductions need only a
//   swap with the lane 32 away.
//   O^T += V^T P^T: B = P^T comes straight from the score accumulator (the
//   contraction order over keys is permuted so that each lane's 8 B-operand
//   values are 8 consecutive accumulator entries), A = V^T from LDS.
//   Online softmax in the log2 domain (scale cap * log2 e folded in), P
//   rounded to BF16 for the MFMA, O^T accumulated in FP32, O = O^T / l.
#pragma once
#include "ops.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int AT_D = 128;
constexpr int AT_BM = 128;          // queries per workgroup
constexpr int AT_BN = 64;           // keys per tile
constexpr int AT_KS = AT_D + 8;     // K row stride in LDS (elements): 272 B
constexpr int AT_VS = AT_BN + 4;    // Vt row stride in LDS (elements): 136 B

struct AttnArgs {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    int32_t S;
    int32_t causal;
    float scale;       // RN_f32(1 / (cap sqrt(D)))
    float c2;          // RN_f32(cap * log2(e))
    CoefF16 tanh16;    // D4 tanh program, FP16 coefficients
};

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t *p) { return *(const bf16x8 *)p; }

template <bool POLY>
__global__ __launch_bounds__(256) void k_attn_fwd(AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ks[AT_BN * AT_KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[AT_D * AT_VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int S = a.S;
    const int ntq = (S + AT_BM - 1) / AT_BM;
    const int qt = a.causal ? ntq - 1 - (int)blockIdx.x : (int)blockIdx.x;  // heavy tiles first
    const int64_t base = (int64_t)blockIdx.y * S * AT_D;
    const uint16_t *Q = a.q + base, *K = a.k + base, *V = a.v + base;
    const int q0 = qt * AT_BM + wave * 32;
    const int my_q = q0 + col;

    // Q as the B operand of S^T = K Q^T: lane holds Q[my_q][ks*16 + h*8 + 0..7]
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (my_q < S) qf[ks] = ld_bf16x8(Q + (int64_t)my_q * AT_D + ks * 16 + h * 8);
        else qf[ks] = bf16x8{};
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m = -INFINITY;   // running max of the log2-domain score
    float l = 0.0f;        // this lane's partial row sum

    const int kend = a.causal ? (qt * AT_BM + AT_BM < S ? qt * AT_BM + AT_BM : S) : S;
    const int nkt = (kend + AT_BN - 1) / AT_BN;

    // global -> register staging of one K/V tile: 4 x 16 B each per thread
    u32x4 kr[4], vr[4];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = tid + r * 256;
            const int kk = c >> 4, kd = (c & 15) * 8;         // K: 16 threads per row
            const int vk = c & 63, vd = (c >> 6) * 8;         // V: consecutive keys per wave
            const int gk = kt * AT_BN + kk, gv = kt * AT_BN + vk;
            kr[r] = gk < S ? *(const u32x4 *)(K + (int64_t)gk * AT_D + kd) : u32x4{0, 0, 0, 0};
            vr[r] = gv < S ? *(const u32x4 *)(V + (int64_t)gv * AT_D + vd) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = tid + r * 256;
            const int kk = c >> 4, kd = (c & 15) * 8;
            *(u32x4 *)(Ks + kk * AT_KS + kd) = kr[r];
            const int vk = c & 63, vd = (c >> 6) * 8;
            const uint32_t w[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Vt[(vd + 2 * i) * AT_VS + vk] = (uint16_t)(w[i] & 0xFFFFu);
                Vt[(vd + 2 * i + 1) * AT_VS + vk] = (uint16_t)(w[i] >> 16);
            }
        }
    };

    load_tile(0);
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < nkt) load_tile(kt + 1);

        const int key0 = kt * AT_BN;
        if (key0 > q0 + 31 && a.causal) continue;   // tile entirely above this wave's rows
        if (q0 >= S) continue;

        // ---- S^T for two 32-key blocks ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 af = ld_bf16x8(Ks + (kb * 32 + col) * AT_KS + ks * 16 + h * 8);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], s[kb], 0, 0, 0);
            }
        }

        // ---- score transform: z = log2(e) * cap * tanh(x) -----------------
        // s[kb][j*4 + i] is the score of key key0 + kb*32 + j*8 + h*4 + i
        const bool need_mask = (a.causal && key0 + AT_BN - 1 > q0) || key0 + AT_BN > S;
        float zmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                float t0, t1;
                if constexpr (POLY) {
                    const uint32_t xw = pack_f16(s[kb][e] * a.scale, s[kb][e + 1] * a.scale);
                    const uint32_t aw = xw & 0x7FFF7FFFu;
                    const h2 v = horner_f16<4, true>(bc<h2>(min_u16x2(aw, a.tanh16.lc)), a.tanh16);
                    const uint32_t tw = bc<uint32_t>(v) ^ (xw ^ aw);
                    t0 = f16_lo(tw);
                    t1 = f16_hi(tw);
                } else {
                    t0 = tanhf(s[kb][e] * a.scale);
                    t1 = tanhf(s[kb][e + 1] * a.scale);
                }
                float z0 = t0 * a.c2, z1 = t1 * a.c2;
                if (need_mask) {
                    const int k0 = key0 + kb * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
                    if ((a.causal && k0 > my_q) || k0 >= S) z0 = -INFINITY;
                    if ((a.causal && k0 + 1 > my_q) || k0 + 1 >= S) z1 = -INFINITY;
                }
                s[kb][e] = z0;
                s[kb][e + 1] = z1;
                zmax = fmaxf(zmax, fmaxf(z0, z1));
            }
        }
        zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
        const float m_new = fmaxf(m, zmax);
        const float corr = exp2f(m - m_new);
        m = m_new;

        // ---- P = exp2(z - m), row sums, BF16 B operands ---------------------
        bf16x8 pf[4];
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                bf16x8 frag;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = exp2f(s[kb][jj * 8 + e] - m_new);
                    lsum += p;
                    frag[e] = (__bf16)p;
                }
                pf[kb * 2 + jj] = frag;
            }
        }
        l = l * corr + lsum;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= corr;

        // ---- O^T += V^T P^T ------------------------------------------------
        // contraction index h*8 + e of step ks maps to key
        // kb*32 + jj*16 + (e/4)*8 + h*4 + (e%4)   (ks = 2 kb + jj)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const uint16_t *vrow = Vt + (db * 32 + col) * AT_VS;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kofs = (ks >> 1) * 32 + (ks & 1) * 16 + h * 4;
                const u32x2 lo = *(const u32x2 *)(vrow + kofs);
                const u32x2 hi = *(const u32x2 *)(vrow + kofs + 8);
                const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bc<bf16x8>(av), pf[ks], o[db], 0, 0, 0);
            }
        }
    }

    if (my_q >= S) return;
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.0f / lt;
    uint16_t *orow = a.o + base + (int64_t)my_q * AT_D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + j * 8 + h * 4;
            u32x2 w;
            w.x = pack_bf(o[db][j * 4 + 0] * inv, o[db][j * 4 + 1] * inv);
            w.y = pack_bf(o[db][j * 4 + 2] * inv, o[db][j * 4 + 3] * inv);
            *(u32x2 *)(orow + d) = w;
        }
    }
}

inline pa_status attn_fwd(const void *q, const void *k, const void *v, void *o, int32_t B,
                          int32_t H, int32_t S, int32_t D, float cap, int32_t causal, bool poly,
                          const CoefF16 &tanh16, hipStream_t stream)
{
    if (!q || !k || !v || !o) return PA_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)o})
        if ((uintptr_t)p & 15u) return PA_ERR_ALIGN;
    if (B < 0 || H < 0 || S < 0 || D != AT_D) return PA_ERR_SHAPE;
    if (!(cap > 0.0f) || cap == INFINITY) return PA_ERR_SHAPE;
    const int64_t bytes = (int64_t)B * H * S * D * 2;
    for (const void *p : {q, k, v})
        if ((uintptr_t)o < (uintptr_t)p + (uintptr_t)bytes && (uintptr_t)p < (uintptr_t)o + (uintptr_t)bytes)
            return PA_ERR_OVERLAP;   // O is written while Q, K, V are still read
    if ((int64_t)B * H == 0 || S == 0) return PA_OK;
    if ((int64_t)B * H > 65535) return PA_ERR_SHAPE;
    AttnArgs a;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (uint16_t *)o;
    a.S = S;
    a.causal = causal ? 1 : 0;
    a.scale = (float)(1.0 / ((double)cap * sqrt((double)D)));
    a.c2 = (float)((double)cap * 1.4426950408889634074);
    a.tanh16 = tanh16;
    const dim3 grid((unsigned)((S + AT_BM - 1) / AT_BM), (unsigned)(B * H));
    if (poly) hipLaunchKernelGGL(k_attn_fwd<true>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_attn_fwd<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
