// Per-chunk preparation for the state pass (bf16 inputs, one step per
// token), one wave per chunk: everything about a chunk that does not depend
// on the state (msj19 "gated_deltaproduct" test.py with r = 1:
// gated_chunk_scaled_dot_kkt_fwd_kernel, solve_tril and the block merges,
// and the intra-chunk scores of gated_chunk_linear_attn_fwd_kernel_o).  Per
// chunk of C tokens:
//
//   G       chunk-local cumsum of the log-decay (kept in log2 units)
//   A       [s<t] beta_t (k_t . k_s) e^{G_t - G_s}       (fp32, LDS)
//   T       (I + A)^-1: 16x16 diagonal blocks by forward substitution, then
//           block rows T_ij = -T_ii sum_m A_im T_mj (bf16 hi/lo MFMAs, T
//           blocks in registers), each block row written over A once it is
//           complete; stored as T diag(beta) without its diagonal (the
//           state pass forms V_new = T diag(beta) (V - e^G K S) and applies
//           the diagonal, beta, in fp32), columns in the permuted k order:
//           16-byte piece 4m + g of a row holds columns 32m + 4g + {0..3}
//           and 32m + 16 + 4g + {0..3}                                -> bf16
//   P       [s<=t] (q_t . k_s) e^{G_t - G_s} of the lower 16x16 tiles, as
//           hi/lo bf16 MFMA fragments (lane l: row t = 16 ti + l%16,
//           columns s = 16 tj + 4 (l/16) + e)
//   gates   e^{G_t}, e^{G_L - G_t}, e^{G_L}, beta_t                   -> fp32
//
// BWD (the backward of the rule) writes, in place of P, the same scores as
// the A operand of P^T (lane l: row s = 16 tj + l%16, columns t = 16 ti +
// 4 (l/16) + e), and also T^T without its diagonal, unscaled, rows s and
// columns t in the permuted k order (tmatT); with atil and atilT also A~ in
// that transposed layout (for the DeltaProduct backward's error gradient).
//
// A wave needs no other wave: K and Q come straight from global memory as
// MFMA fragments (the gram matrix K K^T and the scores K Q^T take both
// operands from the same row fragments), A and T live in the wave's own LDS
// slice, and no barrier is needed (LDS operations of one wave complete in
// order; compiler fences keep the cross-lane reads after the writes they
// depend on).  Four waves per workgroup, two workgroups per CU; waves walk
// the chunks with a stride of the grid.
#pragma once

#include "chunk_kernels.h"

namespace gdn {

template <int KD, int C>
struct Prep2Shape {
    static constexpr int NTT = C / 16;        // 16-token tiles (= diagonal blocks)
    static constexpr int NLOW = NTT * (NTT + 1) / 2;
    static constexpr int NKS = KD / 32;       // 32-wide k steps over the key dim
    static constexpr int LDA = C + 4;         // As [C][C] fp32 (A, then T)
    static constexpr int WAVE_BYTES = C * LDA * 4 + 2 * C * 4;   // As, G2, beta
    static constexpr int NWAVE = 4;
    static constexpr int BYTES = NWAVE * WAVE_BYTES;
    static_assert(C % 32 == 0 && C <= 64 && KD % 32 == 0 && KD <= 256, "shape");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
};

// compiler fence: LDS accesses stay in program order across it (the hardware
// keeps one wave's LDS operations in order)
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <int KD, int C, bool BWD = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void chunk_prep2_kernel(ChunkArgs args) {
    using S = Prep2Shape<KD, C>;
    constexpr int NTT = S::NTT, NLOW = S::NLOW, NKS = S::NKS, LDA = S::LDA;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    const int tid = threadIdx.x, l = tid & 63, c16 = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *As = reinterpret_cast<float *>(smem + w * S::WAVE_BYTES);
    float *G2 = As + C * LDA, *betas = G2 + C;

    const int T = args.T, H = args.H;
    const int NT = (T + C - 1) / C;
    const int per_sub = args.B * H * NT, total = per_sub * args.nsub;
    const u16 *kg = reinterpret_cast<const u16 *>(args.k);
    const u16 *qg = reinterpret_cast<const u16 *>(args.q);

    for (int cs = blockIdx.x * S::NWAVE + w; cs < total; cs += gridDim.x * S::NWAVE) {
        // work item cs: sub-key sub = cs / per_sub, chunk ci of it
        const int sub = cs / per_sub, ci = cs - sub * per_sub;
        const int bh = ci / NT, c = ci % NT, b = bh / H, h = bh % H, t0 = c * C;
        const size_t row0 = (size_t)b * T * H + h;
        const int koff = args.koff + sub * args.kw, boff = args.boff + sub;
        char *const wsa = static_cast<char *>(args.tmat) + sub * args.subws;   // this sub-key's work space
        void *const pfrag = static_cast<char *>(args.pfrag) + sub * args.subws;
        void *const gtab = static_cast<char *>(args.gtab) + sub * args.subws;

        // ---- K and Q rows as MFMA fragments: lane (g, j) of (tt, m) holds
        //      row 16 tt + j, key features 32m + 8g + {0..7}; zero past T ----
        // (features past the key width kw <= KD read as zero)
        const int kw = args.kw;
        bf16x8 kf[NTT][NKS], qf[NTT][NKS];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = t0 + tt * 16 + c16;
            const size_t off = (row0 + (size_t)min(t, T - 1) * H) * args.kst + koff;
            if (kw == KD) {                     // (wave-uniform) no padded key features
#pragma unroll
                for (int m = 0; m < NKS; ++m) {
                    const int f = m * 32 + 8 * g;
                    kf[tt][m] = *reinterpret_cast<const bf16x8 *>(kg + off + f);
                    qf[tt][m] = *reinterpret_cast<const bf16x8 *>(qg + off + f);
                    if (t >= T) kf[tt][m] = qf[tt][m] = bf16x8{};
                }
            } else {
#pragma unroll
                for (int m = 0; m < NKS; ++m) {
                    const int f = m * 32 + 8 * g;
                    const bool pad = f >= kw;
                    kf[tt][m] = *reinterpret_cast<const bf16x8 *>(kg + off + (pad ? 0 : f));
                    qf[tt][m] = *reinterpret_cast<const bf16x8 *>(qg + off + (pad ? 0 : f));
                    if (t >= T || pad) kf[tt][m] = qf[tt][m] = bf16x8{};
                }
            }
        }

        // ---- gates: cumsum of g (lane = token), beta ----
        {
            const int t = t0 + l;
            const bool ok = l < C && t < T;
            float gs = ok ? args.g[row0 + (size_t)t * H] : 0.f;
            const float bt = ok ? args.beta[(row0 + (size_t)t * H) * args.bst + boff] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(gs, off, 64);
                if (l >= off) gs += y;
            }
            const float g2 = gs * LOG2E;
            const float g2l = __shfl(g2, C - 1, 64);
            if (l < C) {
                G2[l] = g2;
                betas[l] = bt;
                float *gt = reinterpret_cast<float *>(gtab) + (size_t)ci * gate_table_len<C>();
                gt[l] = fast_exp2(g2);               // e^{G_t}
                gt[C + l] = fast_exp2(g2l - g2);     // e^{G_L - G_t}
                if (l < 4) gt[2 * C + l] = l == 0 ? fast_exp2(g2l) : 0.f;   // e^{G_L}
                gt[2 * C + 4 + l] = bt;              // beta_t
            }
        }
        lds_fence();

        // ---- A: tile (tt, ss <= tt); lane (g, j) gets row t = 16 tt + j and
        //      columns s = 16 ss + 4g + e (one 16-byte store).  With atil,
        //      A without beta (the decay-masked gram) also goes out as hi/lo
        //      MFMA fragments in P's layout ----
        uint4 *adst = args.atil && sub == 0 ? reinterpret_cast<uint4 *>(args.atil) + (size_t)ci * NLOW * 64 + l : nullptr;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = tt * 16 + c16;
            const float g2t = G2[t], btt = betas[t];
#pragma unroll
            for (int ss = 0; ss <= tt; ++ss) {
                floatx4 acc = zero4();
#pragma unroll
                for (int m = 0; m < NKS; ++m) acc = mfma32(kf[ss][m], kf[tt][m], acc);
                const floatx4 g2s = *reinterpret_cast<const floatx4 *>(G2 + ss * 16 + 4 * g);
                floatx4 a, at;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = ss * 16 + 4 * g + e;
                    at[e] = s < t ? acc[e] * fast_exp2(fminf(g2t - g2s[e], 0.f)) : 0.f;
                    a[e] = btt * at[e];
                }
                *reinterpret_cast<floatx4 *>(As + t * LDA + ss * 16 + 4 * g) = a;
                if (adst) {
                    uint4 f;
                    split2_bf16(at[0], at[1], f.x, f.z);
                    split2_bf16(at[2], at[3], f.y, f.w);
                    adst[(tt * (tt + 1) / 2 + ss) * 64] = f;
                }
            }
        }

        // ---- P tiles (ti, tj <= ti), fragments to the work space ----
        {
            uint4 *dst = reinterpret_cast<uint4 *>(pfrag) + (size_t)ci * NLOW * 64 + l;
#pragma unroll
            for (int ti = 0; ti < NTT; ++ti) {
                const float g2t = G2[ti * 16 + c16];
#pragma unroll
                for (int tj = 0; tj <= ti; ++tj) {
                    floatx4 acc = zero4();
                    float pv[4];
                    if constexpr (BWD) {
                        // Q rows as the A operand: lane (g, j) gets rows t = 16 ti + 4g + e, column s = 16 tj + j
#pragma unroll
                        for (int m = 0; m < NKS; ++m) acc = mfma32(qf[ti][m], kf[tj][m], acc);
                        const floatx4 g2r = *reinterpret_cast<const floatx4 *>(G2 + ti * 16 + 4 * g);
                        const float g2c = G2[tj * 16 + c16];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = ti * 16 + 4 * g + e;
                            pv[e] = tj * 16 + c16 <= t ? acc[e] * fast_exp2(fminf(g2r[e] - g2c, 0.f)) : 0.f;
                        }
                    } else {
#pragma unroll
                        for (int m = 0; m < NKS; ++m) acc = mfma32(kf[tj][m], qf[ti][m], acc);
                        const floatx4 g2s = *reinterpret_cast<const floatx4 *>(G2 + tj * 16 + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = tj * 16 + 4 * g + e;
                            pv[e] = s <= ti * 16 + c16 ? acc[e] * fast_exp2(fminf(g2t - g2s[e], 0.f)) : 0.f;
                        }
                    }
                    uint4 f;
                    split2_bf16(pv[0], pv[1], f.x, f.z);
                    split2_bf16(pv[2], pv[3], f.y, f.w);
                    dst[(ti * (ti + 1) / 2 + tj) * 64] = f;
                }
            }
        }
        if constexpr (BWD) {
            // A~ again as the A operand of its transpose (tile (tt, ss), lane (g, j):
            // rows t = 16 tt + 4g + e, column s = 16 ss + j), after the scores so that
            // the Q fragments are no longer held
            if (adst && args.atilT) {
                uint4 *tdst = reinterpret_cast<uint4 *>(args.atilT) + (size_t)ci * NLOW * 64 + l;
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    const floatx4 g2r = *reinterpret_cast<const floatx4 *>(G2 + tt * 16 + 4 * g);
#pragma unroll
                    for (int ss = 0; ss <= tt; ++ss) {
                        floatx4 tr = zero4();
#pragma unroll
                        for (int m = 0; m < NKS; ++m) tr = mfma32(kf[tt][m], kf[ss][m], tr);
                        const float g2c = G2[ss * 16 + c16];
                        float tv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            tv[e] = ss * 16 + c16 < tt * 16 + 4 * g + e ? tr[e] * fast_exp2(fminf(g2r[e] - g2c, 0.f)) : 0.f;
                        uint4 ft;
                        split2_bf16(tv[0], tv[1], ft.x, ft.z);
                        split2_bf16(tv[2], tv[3], ft.y, ft.w);
                        tdst[(tt * (tt + 1) / 2 + ss) * 64] = ft;
                    }
                }
            }
        }
        lds_fence();

        // ---- T = (I + A)^-1: diagonal blocks by forward substitution (lane
        //      (ib, col) forms column col of T_ii), written over A_ii once
        //      every lane has read its rows ----
        {
            const int ib = l >> 4, col = l & 15;
            float x[16];
            if (ib < NTT) {
                const float *Ab = As + (ib * 16) * LDA + ib * 16;
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
            }
            lds_fence();
            if (ib < NTT) {
                float *Tc = As + (ib * 16) * LDA + ib * 16 + col;
#pragma unroll
                for (int i = 0; i < 16; ++i) Tc[i * LDA] = x[i];
            }
            lds_fence();
        }
        // ---- block rows, row by row, columns ascending:
        //      T_ij = -T_ii sum_{j<=m<i} A_im T_mj.  T blocks stay in registers
        //      in accumulator layout (lane (g, c) holds rows 4g + e, column
        //      c), which is the B operand layout of a 16-deep bf16 MFMA step;
        //      the A operands (rows of A_im, T_ii) are read from LDS.  Every
        //      product takes its operands as hi + lo bf16 (three MFMAs: the
        //      lo x lo term is below fp32 rounding of the result's use). ----
        {
            floatx4 tb[NTT][NTT];              // T_mj, m >= j (accumulator layout)
#pragma unroll
            for (int jb = 0; jb < NTT; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) tb[jb][jb][e] = As[(jb * 16 + 4 * g + e) * LDA + jb * 16 + c16];
            // hi/lo B operands of T_mj, formed once
            shortx4 th[NTT][NTT], tl[NTT][NTT];
            auto split_t = [&](int m, int jb) { split4(tb[m][jb], th[m][jb], tl[m][jb]); };
#pragma unroll
            for (int jb = 0; jb < NTT; ++jb) split_t(jb, jb);
            // hi/lo A operand: row c16 of a 16x16 block at `p`, columns 4g..4g+3
            auto a_op = [&](const float *p, shortx4 &hi, shortx4 &lo) {
                split4(*reinterpret_cast<const floatx4 *>(p + c16 * LDA + 4 * g), hi, lo);
            };
#pragma unroll
            for (int ib = 1; ib < NTT; ++ib) {
                shortx4 dh, dl;                 // T_ii as A operand
                a_op(As + (ib * 16) * LDA + ib * 16, dh, dl);
#pragma unroll
                for (int jb = 0; jb < ib; ++jb) {
                    floatx4 y = zero4();
#pragma unroll
                    for (int m = jb; m < ib; ++m) {
                        shortx4 ah, al;
                        a_op(As + (ib * 16) * LDA + m * 16, ah, al);
                        y = mfma16(ah, th[m][jb], y);
                        y = mfma16(ah, tl[m][jb], y);
                        y = mfma16(al, th[m][jb], y);
                    }
                    shortx4 yh, yl;
                    split4(y, yh, yl);
                    floatx4 z = zero4();
                    z = mfma16(dh, yh, z);
                    z = mfma16(dh, yl, z);
                    z = mfma16(dl, yh, z);
#pragma unroll
                    for (int e = 0; e < 4; ++e) tb[ib][jb][e] = -z[e];
                    split_t(ib, jb);
                }
                // row ib is done: A_ib* is read no more, T_ib* goes over it
                lds_fence();
#pragma unroll
                for (int jb = 0; jb < ib; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) As[(ib * 16 + 4 * g + e) * LDA + jb * 16 + c16] = tb[ib][jb][e];
                lds_fence();
            }
        }

        // ---- T diag(beta) without its diagonal, zero above the block
        //      diagonal, bf16, columns in the permuted order ----
        {
            u16 *out = reinterpret_cast<u16 *>(wsa) + (size_t)ci * C * C;
#pragma unroll
            for (int k = 0; k < C * C / 8 / 64; ++k) {
                const int idx = k * 64 + l;
                const int i = idx / (C / 8), pc = idx % (C / 8), j0 = (pc >> 2) * 32 + 4 * (pc & 3), j1 = j0 + 16;
                floatx4 x0 = *reinterpret_cast<const floatx4 *>(As + i * LDA + j0);
                floatx4 x1 = *reinterpret_cast<const floatx4 *>(As + i * LDA + j1);
                const floatx4 b0 = *reinterpret_cast<const floatx4 *>(betas + j0);
                const floatx4 b1 = *reinterpret_cast<const floatx4 *>(betas + j1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[e] = (j0 >> 4) > (i >> 4) || j0 + e == i ? 0.f : x0[e] * b0[e];
                    x1[e] = (j1 >> 4) > (i >> 4) || j1 + e == i ? 0.f : x1[e] * b1[e];
                }
                *reinterpret_cast<uint4 *>(out + (size_t)i * C + pc * 8) =
                    uint4{cvt2_bf16(x0[0], x0[1]), cvt2_bf16(x0[2], x0[3]), cvt2_bf16(x1[0], x1[1]),
                          cvt2_bf16(x1[2], x1[3])};
            }
        }
        if constexpr (BWD) {
            // T^T without its diagonal, unscaled: row s holds T[t][s] for t > s (T's
            // strictly lower part, read down the columns of the LDS copy), columns in
            // the permuted order
            u16 *out = reinterpret_cast<u16 *>(static_cast<char *>(args.tmatT) + sub * args.subws) + (size_t)ci * C * C;
#pragma unroll
            for (int k = 0; k < C * C / 8 / 64; ++k) {
                const int idx = k * 64 + l;
                const int s = idx / (C / 8), pc = idx % (C / 8), j0 = (pc >> 2) * 32 + 4 * (pc & 3), j1 = j0 + 16;
                float x0[4], x1[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[e] = j0 + e > s ? As[(j0 + e) * LDA + s] : 0.f;
                    x1[e] = j1 + e > s ? As[(j1 + e) * LDA + s] : 0.f;
                }
                *reinterpret_cast<uint4 *>(out + (size_t)s * C + pc * 8) =
                    uint4{cvt2_bf16(x0[0], x0[1]), cvt2_bf16(x0[2], x0[3]), cvt2_bf16(x1[0], x1[1]),
                          cvt2_bf16(x1[2], x1[3])};
            }
        }
        lds_fence();                            // the next chunk rewrites this wave's slice
    }
}

}  // namespace gdn
