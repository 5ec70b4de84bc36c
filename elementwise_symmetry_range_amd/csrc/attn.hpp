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
//   queries q0 .. q0 + 31.  Blocks are numbered heaviest query tile first
//   across all heads (causal work grows with the query index).  Key/value
//   tiles of 64 rows go from HBM straight into LDS with global_load_lds_dwordx4
//   (no register staging), double buffered with one barrier per tile: tile
//   kt + 1 streams in while tile kt is consumed.  Rows are 256 B with the
//   16-byte chunks XOR-swizzled by row: chunk c of row r sits at slot
//   c ^ f(r), f(r) = 4 (r mod 4) + (r / 4 mod 4).  The K reads (16 lanes =
//   16 consecutive rows, one chunk) and the transposed V reads (a half-wave =
//   4 consecutive rows x 4 consecutive chunks) then each touch 16 distinct
//   slots, i.e. all 64 banks once.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q held
//   in registers; the accumulator gives every lane one query (column) and 16
//   keys of each 32-key block, so the softmax row reductions need only a
//   swap with the lane 32 away.
//   O^T += V^T P^T: B = P^T comes straight from the score accumulator (the
//   contraction order over keys is permuted so that each lane's 8 B-operand
//   values are 8 consecutive accumulator entries); A = V^T is read from the
//   row-major V tile with ds_read_b64_tr_b16: within each 16-lane group the
//   instruction returns to lane i element (i mod 4) of the 4-element vectors
//   addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12, so lanes addressing
//   V[k0 + j/4][d0 + 4 (j mod 4)] deliver V[k0 .. k0 + 3][d0 + i] to lane i.
//   Online softmax in the log2 domain (cap * log2 e folded in).  The running
//   reference max is only moved when a row's max exceeds it by more than 8
//   (so P <= 2^8): the O rescale (64 multiplies per lane) is skipped for
//   almost every tile and the result is unchanged up to rounding.  P is
//   rounded to BF16 for the MFMA, O^T accumulated in FP32, O = O^T / l.
#pragma once
#include <type_traits>

#include "ops.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int AT_D = 128;
constexpr int AT_BM = 128;          // queries per workgroup
constexpr int AT_BN = 64;           // keys per tile
constexpr int AT_TILE = AT_BN * AT_D;   // elements of one K or V tile in LDS
constexpr float AT_RESCALE = 8.0f;  // log2 headroom before the reference max moves

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

// slot of 16-byte chunk c of LDS row r (rows are 256 B, 16 chunks)
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 3) << 2) | ((r >> 2) & 3)); }

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3))) *)(p));
    return bc<u32x2>(r);
}

template <bool POLY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_fwd(AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][AT_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][AT_TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;     // 16-lane group, lane in group
    const int S = a.S;
    const int ntq = (S + AT_BM - 1) / AT_BM;
    const int nbh = (int)(gridDim.x / (unsigned)ntq);
    const int qrank = (int)blockIdx.x / nbh;          // 0 = heaviest query tile
    const int bh = (int)blockIdx.x - qrank * nbh;
    const int qt = a.causal ? ntq - 1 - qrank : qrank;
    const int64_t base = (int64_t)bh * S * AT_D;
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
    float m = -INFINITY;   // reference max of the log2-domain score
    float l = 0.0f;        // this lane's partial row sum

    const int kend = a.causal ? (qt * AT_BM + AT_BM < S ? qt * AT_BM + AT_BM : S) : S;
    const int nkt = (kend + AT_BN - 1) / AT_BN;

    // One tile = 64 rows x 16 chunks of 16 B for each of K and V: 16 wave
    // instructions each, 4 per wave.  Instruction r of wave w fills LDS bytes
    // [(4 w + r) KiB, +1 KiB): lane p writes slot p % 16 of row (4 w + r) * 4 +
    // p / 16, so it fetches the chunk that belongs in that slot.  Rows past S
    // repeat row S - 1 (finite data; those keys are masked).
    auto load_tile = [&](int kt, int buf) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (wave * 4 + r) * 4 + (lane >> 4);
            const int slot = lane & 15;
            int g = kt * AT_BN + row;
            g = g < S ? g : S - 1;
            const int64_t src = (int64_t)g * AT_D + swz(row, slot) * 8;
            const int dst = __builtin_amdgcn_readfirstlane((wave * 4 + r) * 512);
            __builtin_amdgcn_global_load_lds((const void *)(K + src),
                                             (void __attribute__((address_space(3))) *)(&Ks[buf][dst]),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(V + src),
                                             (void __attribute__((address_space(3))) *)(&Vs[buf][dst]),
                                             16, 0, 0);
        }
    };

    load_tile(0, 0);
    // One tile; BUF is the LDS buffer holding it (a constant: the loop below
    // is unrolled by two so that buffer bases become immediate offsets).
    auto tile = [&](int kt, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's share of tile kt landed
        __syncthreads();   // all of tile kt landed; nobody reads buffer buf ^ 1 any more
        if (kt + 1 < nkt) load_tile(kt + 1, buf ^ 1);

        const int key0 = kt * AT_BN;
        if (a.causal && key0 > q0 + 31) return;   // tile entirely above this wave's rows
        if (q0 >= S) return;
        const uint16_t *Kb = Ks[buf];
        const uint16_t *Vb = Vs[buf];

        // ---- S^T for two 32-key blocks ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int row = kb * 32 + col;
                const bf16x8 af = ld_bf16x8(Kb + row * AT_D + swz(row, ks * 2 + h) * 8);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], s[kb], 0, 0, 0);
            }
        }

        // ---- score transform: t = tanh(x), z = t * cap * log2(e) ------------
        // s[kb][j*4 + i] is the score of key key0 + kb*32 + j*8 + h*4 + i.
        // Masked keys (beyond the query, or beyond S) get t = -inf.  Tiles
        // that need no mask (all but the diagonal and the ragged end) take a
        // branch-free pass without the key arithmetic.
        const bool need_mask = (a.causal && key0 + AT_BN - 1 > q0) || key0 + AT_BN > S;
        const int lim = a.causal ? (my_q < S - 1 ? my_q : S - 1) : S - 1;   // last visible key
        float tmax;
        auto transform = [&](auto masked) {
            constexpr bool MASKED = decltype(masked)::value;
            if constexpr (POLY) {
                uint32_t mx = 0xFC00FC00u;   // packed FP16 -inf
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        // x = RN_f16(s * scale): the FP32 product rounded once to
                        // FP16 equals RN_f16(RN_f32(s * scale)) (24 >= 2 * 11 + 2)
                        h2 xh;
                        xh[0] = (_Float16)fmaf(s[kb][e], a.scale, -0.0f);
                        xh[1] = (_Float16)fmaf(s[kb][e + 1], a.scale, -0.0f);
                        const uint32_t xw = bc<uint32_t>(xh);
                        const uint32_t aw = xw & 0x7FFF7FFFu;
                        const h2 v = horner_f16<4, true>(bc<h2>(min_u16x2(aw, a.tanh16.lc)), a.tanh16);
                        uint32_t w = bc<uint32_t>(v) ^ (xw ^ aw);
                        if constexpr (MASKED) {
                            const int k0 = key0 + kb * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
                            const uint32_t mlo = k0 > lim ? 0x0000FFFFu : 0u;
                            const uint32_t mhi = k0 + 1 > lim ? 0xFFFF0000u : 0u;
                            w = sel(mlo | mhi, 0xFC00FC00u, w);
                        }
                        mx = bc<uint32_t>(__builtin_elementwise_max(bc<h2>(mx), bc<h2>(w)));
                        s[kb][e] = f16_lo(w);
                        s[kb][e + 1] = f16_hi(w);
                    }
                }
                tmax = fmaxf(f16_lo(mx), f16_hi(mx));
            } else {
                tmax = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float t = tanhf(s[kb][e] * a.scale);
                        if constexpr (MASKED) {
                            const int k0 = key0 + kb * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
                            t = k0 > lim ? -INFINITY : t;
                        }
                        s[kb][e] = t;
                        tmax = fmaxf(tmax, t);
                    }
                }
            }
        };
        if (need_mask) transform(std::true_type{});
        else transform(std::false_type{});
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float zmax = tmax * a.c2;

        // lazy rescale: move the reference only when the row max outgrows it
        const bool grow = zmax > m + AT_RESCALE;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? zmax : m;
            const float corr = __builtin_amdgcn_exp2f(m - m_new);
            l *= corr;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= corr;
            m = m_new;
        }

        // ---- P = exp2(t c2 - m), row sums, BF16 B operands ------------------
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                bf16x8 frag;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][jj * 8 + e], a.c2, -m));
                    l += p;
                    frag[e] = (__bf16)p;
                }
                pf[kb * 2 + jj] = frag;
            }
        }

        // ---- O^T += V^T P^T ------------------------------------------------
        // contraction index h*8 + e of step ks maps to key
        // kb*32 + jj*16 + (e/4)*8 + h*4 + (e%4)   (ks = 2 kb + jj)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = db * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k0 = (ks >> 1) * 32 + (ks & 1) * 16 + (g16 >> 1) * 4 + (i16 >> 2);
                const u32x2 lo = ds_read_tr16(Vb + k0 * AT_D + swz(k0, d >> 3) * 8 + (d & 7));
                const u32x2 hi = ds_read_tr16(Vb + (k0 + 8) * AT_D + swz(k0 + 8, d >> 3) * 8 + (d & 7));
                const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bc<bf16x8>(av), pf[ks], o[db], 0, 0, 0);
            }
        }
    };
    for (int kt = 0; kt < nkt; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nkt) tile(kt + 1, std::integral_constant<int, 1>{});
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
    if ((int64_t)B * H * ((S + AT_BM - 1) / AT_BM) > 0x7FFFFFFF) return PA_ERR_SHAPE;
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
    const dim3 grid((unsigned)(((S + AT_BM - 1) / AT_BM) * (B * H)));
    if (poly) hipLaunchKernelGGL(k_attn_fwd<true>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_attn_fwd<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
