// Per-chunk preparation for the single-chain-wave state pass (bf16 inputs,
// one step per token): everything about a chunk that does not depend on the
// state, computed in parallel over chunks (msj19 "gated_deltaproduct"
// test.py with r = 1: gated_chunk_scaled_dot_kkt_fwd_kernel, solve_tril and
// the block merges, and the intra-chunk scores of
// gated_chunk_linear_attn_fwd_kernel_o).  Per chunk of C tokens:
//
//   G       chunk-local cumsum of the log-decay (kept in log2 units)
//   A       [s<t] beta_t (k_t . k_s) e^{G_t - G_s}       (fp32, LDS)
//   T       (I + A)^-1: 16x16 diagonal blocks by forward substitution, then
//           block rows T_ij = -T_ii sum_m A_im T_mj; stored as T diag(beta)
//           without its diagonal (the state pass forms V_new = T diag(beta)
//           (V - e^G K S) from exact V and K and applies the diagonal, beta,
//           in fp32), columns in the permuted k order              -> bf16
//   P       [s<=t] (q_t . k_s) e^{G_t - G_s} of the lower 16x16 tiles, as
//           hi/lo bf16 MFMA fragments (lane l: row t = 16 ti + l%16,
//           columns s = 16 tj + 4 (l/16) + e)
//   gates   e^{G_t}, e^{G_L - G_t}, e^{G_L}, beta_t                   -> fp32
//
// Persistent workgroups of 4 waves walk the chunks with a stride of the
// grid; the next chunk's K, Q, beta and g are loaded into registers while the
// current one is solved, so the global-load latency stays hidden.  Wave 0
// inverts I + A alone (forward substitution, then the block rows: no
// barriers) while waves 1..3 compute the P tiles.
#pragma once

#include "chunk_kernels.h"

namespace gdn {

template <int KD, int C>
struct Prep1Shape {
    static constexpr int NTT = C / 16;        // 16-token tiles (= diagonal blocks)
    static constexpr int NLOW = NTT * (NTT + 1) / 2;
    static constexpr int NKS = KD / 32;       // 32-wide k steps over the key dim
    static constexpr int LDK = KD + 8;        // Ks [C][KD] bf16
    static constexpr int LDA = C + 4;         // As, Ts [C][C] fp32
    static constexpr int NKV = C * KD / 8;    // 16-byte vectors of K per chunk
    static constexpr int PK = (NKV + 255) / 256;
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_AS = OFF_KS + al(C * LDK * 2);
    static constexpr int OFF_TS = OFF_AS + al(C * LDA * 4);
    static constexpr int OFF_G = OFF_TS + al(C * LDA * 4);
    static constexpr int BYTES = OFF_G + al(2 * C * 4);   // beta, G2
    static_assert(C % 32 == 0 && C <= 64 && KD % 32 == 0 && KD <= 256, "shape");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
    // P row tiles while wave 0 inverts (waves 1..3):
    // wave w takes rows prow0(w) and prow1(w) (-1: none).
    static constexpr int prow0(int w) {
        return NTT == 4 ? (w == 1 ? 3 : w == 2 ? 2 : w == 3 ? 1 : -1) : (w == 1 ? 1 : w == 2 ? 0 : -1);
    }
    static constexpr int prow1(int w) { return NTT == 4 && w == 2 ? 0 : -1; }
};

template <int KD, int C>
__global__ __launch_bounds__(256) void chunk_prep1_kernel(ChunkArgs args) {
    using S = Prep1Shape<KD, C>;
    constexpr int NTT = S::NTT, NLOW = S::NLOW, NKS = S::NKS, LDK = S::LDK, LDA = S::LDA;
    constexpr int NKV = S::NKV, PK = S::PK;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    u16 *Ks = reinterpret_cast<u16 *>(smem + S::OFF_KS);
    float *As = reinterpret_cast<float *>(smem + S::OFF_AS);
    float *Ts = reinterpret_cast<float *>(smem + S::OFF_TS);
    float *betas = reinterpret_cast<float *>(smem + S::OFF_G);
    float *G2 = betas + C;

    const int tid = threadIdx.x, l = tid & 63, c16 = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, H = args.H;
    const int NT = (T + C - 1) / C;
    const int total = args.B * H * NT;
    const u16 *kg = reinterpret_cast<const u16 *>(args.k);
    const u16 *qg = reinterpret_cast<const u16 *>(args.q);

    // ---- registers of the next chunk ----
    u32x4 rk[PK];
    bf16x8 qf[NKS], qf1[NKS];                 // Q fragments of P row tiles prow0(w), prow1(w)
    float rb = 0.f, rg = 0.f;
    const int pr0 = S::prow0(w), pr1 = S::prow1(w);
    auto prefetch = [&](int ci) {
        const int bh = ci / NT, c = ci % NT, b = bh / H, h = bh % H, t0 = c * C;
        const size_t row0 = (size_t)b * T * H + h;
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            const int idx = min(tid + 256 * q, NKV - 1);
            const int tt = min(t0 + idx / (KD / 8), T - 1);
            rk[q] = *reinterpret_cast<const u32x4 *>(kg + (row0 + (size_t)tt * H) * KD + (idx % (KD / 8)) * 8);
        }
        if (pr0 >= 0) {                         // Q rows of the P row tiles of this wave
            const int tq = min(t0 + pr0 * 16 + c16, T - 1);
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                qf[m] = *reinterpret_cast<const bf16x8 *>(qg + (row0 + (size_t)tq * H) * KD + m * 32 + 8 * g);
        }
        if (pr1 >= 0) {
            const int tq = min(t0 + pr1 * 16 + c16, T - 1);
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                qf1[m] = *reinterpret_cast<const bf16x8 *>(qg + (row0 + (size_t)tq * H) * KD + m * 32 + 8 * g);
        }
        if (w == 0) {
            const int tt = min(t0 + l, T - 1);
            rb = args.beta[row0 + (size_t)tt * H];
            rg = args.g[row0 + (size_t)tt * H];
        }
    };

    if ((int)blockIdx.x < total) prefetch(blockIdx.x);
    for (int ci = blockIdx.x; ci < total; ci += gridDim.x) {
        const int bh = ci / NT, c = ci % NT, t0 = c * C;

        // ---- K rows (zero past T), beta, cumsum ----
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            const int idx = tid + 256 * q;
            if (idx < NKV) {
                const int t = idx / (KD / 8);
                *reinterpret_cast<u32x4 *>(Ks + t * LDK + (idx % (KD / 8)) * 8) =
                    t0 + t < T ? rk[q] : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (w == 0) {
            const bool ok = l < C && t0 + l < T;
            float gs = ok ? rg : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(gs, off, 64);
                if (l >= off) gs += y;
            }
            const float g2 = gs * LOG2E;
            const float g2l = __shfl(g2, C - 1, 64);
            if (l < C) {
                const float bt = ok ? rb : 0.f;
                const float eg = fast_exp2(g2);
                betas[l] = bt;
                G2[l] = g2;
                float *gt = reinterpret_cast<float *>(args.gtab) + ((size_t)bh * NT + c) * gate_table_len<C>();
                gt[l] = eg;                          // e^{G_t}
                gt[C + l] = fast_exp2(g2l - g2);     // e^{G_L - G_t}
                if (l < 4) gt[2 * C + l] = l == 0 ? fast_exp2(g2l) : 0.f;   // e^{G_L}
                gt[2 * C + 4 + l] = bt;              // beta_t
            }
        }
        __syncthreads();

        // ---- gram tiles (round robin): As[t][s] = [s<t] beta_t (k_t.k_s) e^{G_t-G_s} ----
#pragma unroll
        for (int kk = 0; kk < NLOW; ++kk) {
            if (kk % 4 != w) continue;
            int ti = 0, p = kk;
            while (p > ti) { p -= ti + 1; ++ti; }
            const int tj = p;
            floatx4 acc = zero4();
            const u16 *ar = Ks + (ti * 16 + c16) * LDK, *br = Ks + (tj * 16 + c16) * LDK;
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld8(ar + m * 32 + 8 * g), ld8(br + m * 32 + 8 * g), acc,
                                                              0, 0, 0);
            const int s = tj * 16 + c16;
            const float g2s = G2[s];
            const floatx4 g2t = *reinterpret_cast<const floatx4 *>(G2 + ti * 16 + 4 * g);
            const floatx4 bt = *reinterpret_cast<const floatx4 *>(betas + ti * 16 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = ti * 16 + 4 * g + e;
                As[t * LDA + s] = s < t ? bt[e] * acc[e] * fast_exp2(fminf(g2t[e] - g2s, 0.f)) : 0.f;
            }
        }
        __syncthreads();

        // ---- wave 0: T = (I + A)^-1 (diagonal blocks by forward substitution,
        //      then the block rows, without barriers); waves 1..3: P ----
        if (w == 0) {
            const int ib = l >> 4, col = l & 15;
            if (ib < NTT) {
                const float *Ab = As + (ib * 16) * LDA + ib * 16;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
                    for (int j4 = 0; j4 < i; j4 += 4) {        // row i of the block, 4 entries per read
                        const floatx4 a4 = *reinterpret_cast<const floatx4 *>(Ab + i * LDA + j4);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (j4 + e < i) acc -= a4[e] * x[j4 + e];
                    }
                    x[i] = acc;
                }
                float *Tc = Ts + (ib * 16) * LDA + ib * 16 + col;
#pragma unroll
                for (int i = 0; i < 16; ++i) Tc[i * LDA] = x[i];
            }
            // block rows T_ij = -T_ii sum_{j<=m<i} A_im T_mj, by growing distance
            // i - j; everything this wave reads it wrote itself (LDS is in order)
#pragma unroll
            for (int st = 1; st < NTT; ++st) {
#pragma unroll
                for (int jb = 0; jb + st < NTT; ++jb) {
                    const int ib = jb + st;
                    floatx4 y = zero4();
#pragma unroll
                    for (int m = jb; m < ib; ++m)
                        mma_f32_bn(y, As + (ib * 16) * LDA + m * 16, LDA, Ts + (m * 16) * LDA + jb * 16, LDA, 16);
                    // -T_ii Y with Y straight from the accumulator: lane (g, j) holds
                    // Y[4g+e][j], fed as B[k][j] with k = 4g + s in step s, so the
                    // A operand of step s is T_ii[row][4g + s]
                    const floatx4 trow = *reinterpret_cast<const floatx4 *>(Ts + (ib * 16 + c16) * LDA + ib * 16 + 4 * g);
                    floatx4 z = zero4();
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) z = __builtin_amdgcn_mfma_f32_16x16x4f32(trow[s4], y[s4], z, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Ts[(ib * 16 + 4 * g + e) * LDA + jb * 16 + c16] = -z[e];
                }
            }
        } else {
            // P row tiles of this wave (fragments to the work space)
            auto p_row = [&](int ti, const bf16x8 (&q)[NKS]) {
                const float g2t = G2[ti * 16 + c16];
                uint4 *dst = reinterpret_cast<uint4 *>(args.pfrag) + ((size_t)bh * NT + c) * NLOW * 64 +
                             (ti * (ti + 1) / 2) * 64 + l;
                for (int tj = 0; tj <= ti; ++tj) {
                    floatx4 acc = zero4();
                    const u16 *krow = Ks + (tj * 16 + c16) * LDK;
#pragma unroll
                    for (int m = 0; m < NKS; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                                       ld8(krow + m * 32 + 8 * g), q[m], acc, 0, 0, 0);
                    const floatx4 g2s = *reinterpret_cast<const floatx4 *>(G2 + tj * 16 + 4 * g);
                    float pv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = tj * 16 + 4 * g + e;
                        pv[e] = s <= ti * 16 + c16 ? acc[e] * fast_exp2(fminf(g2t - g2s[e], 0.f)) : 0.f;
                    }
                    uint4 f;
                    split2_bf16(pv[0], pv[1], f.x, f.z);
                    split2_bf16(pv[2], pv[3], f.y, f.w);
                    dst[tj * 64] = f;
                }
            };
            if (pr0 >= 0) p_row(pr0, qf);
            if (pr1 >= 0) p_row(pr1, qf1);
        }
        // registers are free: start loading the next chunk
        if (ci + (int)gridDim.x < total) prefetch(ci + gridDim.x);
        __syncthreads();

        // ---- T diag(beta) (zero above the block diagonal), bf16, columns in the
        //      permuted order: 16-byte piece 4m + g of a row holds columns
        //      32m + 4g + {0..3} and 32m + 16 + 4g + {0..3} ----
        {
            u16 *out = reinterpret_cast<u16 *>(args.tmat) + ((size_t)bh * NT + c) * C * C;
            for (int idx = tid; idx < C * C / 8; idx += 256) {
                const int i = idx / (C / 8), pc = idx % (C / 8), j0 = (pc >> 2) * 32 + 4 * (pc & 3), j1 = j0 + 16;
                floatx4 x0 = *reinterpret_cast<const floatx4 *>(Ts + i * LDA + j0);
                floatx4 x1 = *reinterpret_cast<const floatx4 *>(Ts + i * LDA + j1);
                const floatx4 b0 = *reinterpret_cast<const floatx4 *>(betas + j0);
                const floatx4 b1 = *reinterpret_cast<const floatx4 *>(betas + j1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[e] *= b0[e];
                    x1[e] *= b1[e];
                }
                if ((j0 >> 4) > (i >> 4)) x0 = zero4();
                if ((j1 >> 4) > (i >> 4)) x1 = zero4();
#pragma unroll
                for (int e = 0; e < 4; ++e) {       // the diagonal (beta) is applied in fp32 by the state pass
                    if (j0 + e == i) x0[e] = 0.f;
                    if (j1 + e == i) x1[e] = 0.f;
                }
                *reinterpret_cast<uint4 *>(out + (size_t)i * C + pc * 8) =
                    uint4{cvt2_bf16(x0[0], x0[1]), cvt2_bf16(x0[2], x0[3]), cvt2_bf16(x1[0], x1[1]),
                          cvt2_bf16(x1[2], x1[3])};
            }
        }
        __syncthreads();                       // Ks, As, Ts are rewritten by the next chunk
    }
}

}  // namespace gdn
