// Chunkwise gated delta rule / gated DeltaProduct forward for gfx950.
//
// Method: msj19 "gated_deltaproduct" test.py - chunk-local cumsum of the
// log-decay; the intra-chunk matrix of gated_chunk_scaled_dot_kkt_fwd_kernel;
// (I + A)^-1 from 16x16 diagonal blocks (solve_tril_16x16_kernel) and block
// merges (merge_16x16_to_{32x32,64x64}_inverse_kernel, taken as the exact
// block inverse); the WY form (gated_fwd_recompute_w_u_kernel,
// preprocess_qkw); the inter-chunk state pass
// (gated_chunk_delta_rule_fwd_kernel_h) and the output
// (gated_chunk_linear_attn_fwd_kernel_o), summed over the r sub-keys.
//
// Design (one kernel, no workspace): one 256-thread workgroup owns one
// (batch, head, 16-column slice of the value dimension) and walks the chunks
// of that sequence in order.  The (Dk x 16) fp32 slice of the state lives in
// MFMA accumulator registers for the whole sequence.  Per chunk:
//
//   load     K, Q (C x KD) and V (C x 16) to LDS, gates to LDS
//   cumsum   G_t = sum_{t' <= t} g_t' inside the chunk (one wave, shuffles)
//   gram     A[(t,a),(s,b)] = [s<t] beta_{t,a} M[a][b] (k_{t,b}.k_{s,b}) e^{G_t-G_s}
//            P_b[t][s]      = [s<=t] (q_{t,b}.k_{s,b}) e^{G_t-G_s}
//            (bf16 MFMA on the exact inputs, fp32 accumulation)
//   solve    T = (I + A)^-1: 16x16 diagonal blocks by forward substitution
//            (one lane per column), then block rows T_ij = -T_ii sum A_im T_mj
//            (fp32 MFMA)
//   chain    X_b = K_b S_b;  R = diag(beta) (V - diag(e^G) sum_b M X_b);
//            V_new = T R;  S_b <- e^{G_L} S_b + K_b^T diag(e^{G_L-G}) V_new_b
//   output   O = scale (diag(e^G) Q S_start + sum_b P_b V_new_b)
//
// V_new = T diag(beta) (V - diag(e^G) E S) is the page's u - w h with
// w = T diag(beta e^G) E and u = T diag(beta) V, regrouped so that W is never
// formed: the state only enters through the product K S.
//
// Virtual rows j = t*R + a (token-major) carry the R steps of each token.
//
// Precision (bf16 inputs): products of exact bf16 inputs use one bf16 MFMA;
// fp32 operands derived inside the kernel are split into hi + lo bf16 pairs
// (3 or 2 MFMAs) except T and the state in K S, which are rounded to bf16
// once.  fp32 inputs use fp32 MFMA throughout.
#pragma once

#include "gdn_common.h"

namespace gdn {

struct ChunkArgs {
    const void *q, *k, *v;
    const float *beta, *g;
    const float *h0;
    float *hT;
    void *o;
    int B, T, H, Dv;
    int out_bf16;
    float scale;
    float mask[4];   // R x R step mask, row-major
};

template <bool F32IN, int KD, int C, int R>
struct ChunkCfg {
    static constexpr int BV = 16;
    static constexpr int DK = KD / R;
    static constexpr int NR = C * R;           // virtual rows per chunk
    static constexpr int NB = NR / 16;         // 16-row blocks of the solve
    static constexpr int ESZ = F32IN ? 4 : 2;  // operand element size
    static constexpr int PAD = F32IN ? 4 : 8;  // row padding (elements)
    static constexpr int NLO = F32IN ? 0 : 1;  // number of "lo" copies
    static constexpr int LDK = KD + PAD;       // Ks, Qs:  [C][KD]
    static constexpr int LDKT = C + PAD;       // KsT:     [KD][C]
    static constexpr int LDA = NR + 4;         // As, Ts:  [NR][NR] fp32
    static constexpr int LDTB = NR + PAD;      // Tb:      [NR][NR]
    static constexpr int LDPQ = C + PAD;       // Pq:      [R][C][C]
    static constexpr int LDST = KD + PAD;      // St:      [BV][KD]
    static constexpr int LDRT = NR + PAD;      // RT:      [BV][NR]
    static constexpr int LDVT = C + PAD;       // VnT/VtT: [R][BV][C]
    static constexpr int LDY = 17;             // merge scratch [16][17] fp32

    // byte sizes
    static constexpr int SZ_KS = C * LDK * ESZ;
    static constexpr int SZ_KST = F32IN ? 0 : KD * LDKT * ESZ;
    static constexpr int SZ_QS = C * LDK * ESZ;
    static constexpr int SZ_VS = C * BV * 4;
    static constexpr int SZ_GATE = (C * R + 3 * C + 4) * 4;
    static constexpr int SZ_AS = NR * LDA * 4;
    static constexpr int SZ_TS = NR * LDA * 4;
    static constexpr int SZ_TB = F32IN ? 0 : NR * LDTB * ESZ;
    static constexpr int SZ_PQ = R * C * LDPQ * ESZ * (1 + NLO);
    static constexpr int SZ_ST = BV * LDST * ESZ * (1 + NLO);
    static constexpr int SZ_XS = R * C * BV * 4;
    static constexpr int SZ_RT = BV * LDRT * ESZ * (1 + NLO);
    static constexpr int SZ_VT = R * BV * LDVT * ESZ * (1 + NLO);
    static constexpr int SZ_Y = 4 * 16 * LDY * 4;
    static constexpr int SZ_CHAIN = SZ_XS + SZ_RT + 2 * SZ_VT;
    static constexpr int SZ_UNION = (SZ_AS > SZ_CHAIN ? SZ_AS : SZ_CHAIN);

    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_KST = OFF_KS + al(SZ_KS);
    static constexpr int OFF_QS = OFF_KST + al(SZ_KST);
    static constexpr int OFF_VS = OFF_QS + al(SZ_QS);
    static constexpr int OFF_GATE = OFF_VS + al(SZ_VS);
    static constexpr int OFF_TS = OFF_GATE + al(SZ_GATE);
    static constexpr int OFF_TB = OFF_TS + al(SZ_TS);
    static constexpr int OFF_PQ = OFF_TB + al(SZ_TB);
    static constexpr int OFF_ST = OFF_PQ + al(SZ_PQ);
    static constexpr int OFF_Y = OFF_ST + al(SZ_ST);
    static constexpr int OFF_U = OFF_Y + al(SZ_Y);      // As | (Xs, RT, VnT, VtT)
    static constexpr int BYTES = OFF_U + al(SZ_UNION);

    static_assert(KD % R == 0, "key width must split into R sub-keys");
    static_assert(DK % 16 == 0 && C % 16 == 0, "sizes must be multiples of 16");
    static_assert(NR <= 64, "the solve handles at most 64 virtual rows per chunk");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

template <bool F32IN>
struct OpType { typedef u16 type; };
template <>
struct OpType<true> { typedef float type; };

template <bool F32IN>
__device__ __forceinline__ void store_op(typename OpType<F32IN>::type *hi,
                                         typename OpType<F32IN>::type *lo, int idx, float x) {
    if constexpr (F32IN) {
        hi[idx] = x;
    } else {
        u16 a, b;
        split_bf16(x, a, b);
        hi[idx] = a;
        lo[idx] = b;
    }
}

template <bool F32IN, int KD, int C, int R>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkArgs args) {
    using Cfg = ChunkCfg<F32IN, KD, C, R>;
    using Op = typename OpType<F32IN>::type;
    constexpr int BV = Cfg::BV, DK = Cfg::DK, NR = Cfg::NR, NB = Cfg::NB;
    constexpr int LDK = Cfg::LDK, LDKT = Cfg::LDKT, LDA = Cfg::LDA, LDTB = Cfg::LDTB;
    constexpr int LDPQ = Cfg::LDPQ, LDST = Cfg::LDST, LDRT = Cfg::LDRT, LDVT = Cfg::LDVT;
    constexpr int LDY = Cfg::LDY;
    constexpr int NST = KD / 16;                 // state row tiles
    constexpr int NSTW = (NST + 3) / 4;          // state tiles per wave (max)

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::BYTES];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int nvb = args.Dv / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vb = slot % nvb;
    const int bh = (slot / nvb) * 8 + xcd;      // all value slices of one head share an XCD
    if (bh >= args.B * args.H) return;
    const int b = bh / args.H, h = bh % args.H;
    const int v0 = vb * BV;
    const int T = args.T, H = args.H, Dv = args.Dv;

    Op *Ks = reinterpret_cast<Op *>(smem + Cfg::OFF_KS);
    Op *KsT = reinterpret_cast<Op *>(smem + Cfg::OFF_KST);
    Op *Qs = reinterpret_cast<Op *>(smem + Cfg::OFF_QS);
    float *Vs = reinterpret_cast<float *>(smem + Cfg::OFF_VS);
    float *betas = reinterpret_cast<float *>(smem + Cfg::OFF_GATE);   // [C][R]
    float *Gs = betas + C * R;                                         // [C]
    float *eG = Gs + C;                                                // e^{G_t}
    float *eGLm = eG + C;                                              // e^{G_L - G_t}
    float *gLs = eGLm + C;                                             // e^{G_L}
    float *Ts = reinterpret_cast<float *>(smem + Cfg::OFF_TS);
    Op *Tb = reinterpret_cast<Op *>(smem + Cfg::OFF_TB);
    Op *PqH = reinterpret_cast<Op *>(smem + Cfg::OFF_PQ);
    Op *PqL = PqH + R * C * LDPQ;
    Op *StH = reinterpret_cast<Op *>(smem + Cfg::OFF_ST);
    Op *StL = StH + BV * LDST;
    float *Ys = reinterpret_cast<float *>(smem + Cfg::OFF_Y) + w * 16 * LDY;
    float *As = reinterpret_cast<float *>(smem + Cfg::OFF_U);
    float *Xs = reinterpret_cast<float *>(smem + Cfg::OFF_U);
    Op *RtH = reinterpret_cast<Op *>(smem + Cfg::OFF_U + Cfg::SZ_XS);
    Op *RtL = RtH + BV * LDRT;
    Op *VnH = reinterpret_cast<Op *>(smem + Cfg::OFF_U + Cfg::SZ_XS + Cfg::SZ_RT);
    Op *VnL = VnH + R * BV * LDVT;
    Op *VtH = reinterpret_cast<Op *>(smem + Cfg::OFF_U + Cfg::SZ_XS + Cfg::SZ_RT + Cfg::SZ_VT);
    Op *VtL = VtH + R * BV * LDVT;

    // ---- one-time set-up: zero the blocks above the diagonal of P and T ----
    {
        Op z = Op(0);
        for (int i = tid; i < R * C * LDPQ; i += 256) {
            PqH[i] = z;
            if constexpr (!F32IN) PqL[i] = z;
        }
        if constexpr (!F32IN)
            for (int i = tid; i < NR * LDTB; i += 256) Tb[i] = z;
        for (int i = tid; i < NR * LDA; i += 256) Ts[i] = 0.f;
    }

    // state slice: tile n of wave w covers rows (w + 4n)*16 .. +15, columns v0 .. v0+15
    floatx4 Sreg[NSTW];
#pragma unroll
    for (int n = 0; n < NSTW; ++n) {
        Sreg[n] = zero4();
        const int ts = w + 4 * n;
        if (ts < NST && args.h0) {
            const float *hp = args.h0 + ((size_t)bh * KD) * Dv + v0 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) Sreg[n][e] = hp[(size_t)(ts * 16 + 4 * (l >> 4) + e) * Dv];
        }
    }
    auto write_state_operand = [&]() {
#pragma unroll
        for (int n = 0; n < NSTW; ++n) {
            const int ts = w + 4 * n;
            if (ts < NST) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    store_op<F32IN>(StH, StL, (l & 15) * LDST + ts * 16 + 4 * (l >> 4) + e, Sreg[n][e]);
            }
        }
    };
    write_state_operand();

    const int nchunks = (T + C - 1) / C;
    const size_t tok_stride = (size_t)H;   // tokens of one (b, h) are H rows apart
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        // ---------------- load ----------------
        {
            constexpr int VEC = 16 / Cfg::ESZ;        // elements per 16-byte vector
            constexpr int NV = KD / VEC;              // vectors per row
            for (int idx = tid; idx < 2 * C * NV; idx += 256) {
                const int which = idx / (C * NV);     // 0 = k, 1 = q
                const int rem = idx % (C * NV);
                const int t = rem / NV, cv = rem % NV;
                const int tt = t0 + t;
                U16x8 raw;
                if (tt < T) {
                    const unsigned char *src = reinterpret_cast<const unsigned char *>(which ? args.q : args.k);
                    const size_t row = ((size_t)b * T + tt) * tok_stride + h;
                    raw = *reinterpret_cast<const U16x8 *>(src + (row * KD + cv * VEC) * Cfg::ESZ);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) raw.v[e] = 0;
                }
                Op *dst = which ? Qs : Ks;
                *reinterpret_cast<U16x8 *>(dst + t * LDK + cv * VEC) = raw;
                if constexpr (!F32IN) {
                    if (!which)
#pragma unroll
                        for (int e = 0; e < 8; ++e) KsT[(cv * 8 + e) * LDKT + t] = raw.v[e];
                }
            }
            for (int idx = tid; idx < C * BV; idx += 256) {
                const int t = idx / BV, j = idx % BV, tt = t0 + t;
                float x = 0.f;
                if (tt < T) {
                    const size_t off = (((size_t)b * T + tt) * tok_stride + h) * Dv + v0 + j;
                    if constexpr (F32IN) x = reinterpret_cast<const float *>(args.v)[off];
                    else x = bf16_to_f32(reinterpret_cast<const u16 *>(args.v)[off]);
                }
                Vs[idx] = x;
            }
            for (int idx = tid; idx < C * R; idx += 256) {
                const int t = idx / R, tt = t0 + t;
                betas[idx] = tt < T ? args.beta[(((size_t)b * T + tt) * tok_stride + h) * R + idx % R] : 0.f;
            }
        }
        // ---------------- chunk-local cumsum of the log-decay ----------------
        if (w == 0) {
            const int tt = t0 + l;
            float gsum = (l < C && tt < T) ? args.g[((size_t)b * T + tt) * tok_stride + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(gsum, off, 64);
                if (l >= off) gsum += y;
            }
            const float gl = __shfl(gsum, C - 1, 64);
            if (l < C) {
                Gs[l] = gsum;
                eG[l] = expf(gsum);
                eGLm[l] = expf(gl - gsum);
            }
            if (l == 0) gLs[0] = expf(gl);
        }
        __syncthreads();

        // ---------------- gram: A (strictly lower) and P (lower incl.) ----------------
        {
            constexpr int NTT = C / 16;
            constexpr int NLOW = NTT * (NTT + 1) / 2;
            constexpr int NTILE = 2 * R * NLOW;
            for (int it = w; it < NTILE; it += 4) {
                const int kind = it / (R * NLOW);             // 0 = A, 1 = P
                const int rem = it % (R * NLOW);
                const int bb = rem / NLOW;
                int p = rem % NLOW, ti = 0;
                while (p > ti) { p -= ti + 1; ++ti; }
                const int tj = p;
                floatx4 acc = zero4();
                const Op *arow = (kind ? Qs : Ks) + ti * 16 * LDK + bb * DK;
                const Op *brow = Ks + tj * 16 * LDK + bb * DK;
                if constexpr (F32IN) mma_f32(acc, arow, LDK, brow, LDK, DK);
                else mma_bf16(acc, arow, LDK, brow, LDK, DK);
                const int s = tj * 16 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = ti * 16 + 4 * (l >> 4) + e;
                    if (kind == 0) {
                        const float dec = s < t ? expf(Gs[t] - Gs[s]) : 0.f;
#pragma unroll
                        for (int a = 0; a < R; ++a)
                            As[(t * R + a) * LDA + s * R + bb] = betas[t * R + a] * args.mask[a * R + bb] * acc[e] * dec;
                    } else {
                        const float val = s <= t ? acc[e] * expf(Gs[t] - Gs[s]) : 0.f;
                        store_op<F32IN>(PqH, PqL, (bb * C + t) * LDPQ + s, val);
                    }
                }
            }
        }
        __syncthreads();

        // ---------------- solve: diagonal 16x16 blocks ----------------
        if (w == 0) {
            const int ib = l >> 4, col = l & 15;
            if (ib < NB) {
                const float *Ab = As + (ib * 16) * LDA + ib * 16;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
                    for (int j = 0; j < i; ++j) acc -= Ab[i * LDA + j] * x[j];
                    x[i] = acc;
                }
                float *Tbk = Ts + (ib * 16) * LDA + ib * 16 + col;
#pragma unroll
                for (int i = 0; i < 16; ++i) Tbk[i * LDA] = x[i];
            }
        }
        __syncthreads();
        // ---------------- solve: block rows, one column block per wave ----------------
#pragma unroll
        for (int st = 1; st < NB; ++st) {
            const int jb = w, ib = w + st;
            const bool act = ib < NB;
            if (act) {
                floatx4 y = zero4();
                for (int m = jb; m < ib; ++m)
                    mma_f32_bn(y, As + (ib * 16) * LDA + m * 16, LDA, Ts + (m * 16) * LDA + jb * 16, LDA, 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) Ys[(4 * (l >> 4) + e) * LDY + (l & 15)] = y[e];
            }
            __syncthreads();
            if (act) {
                floatx4 t2 = zero4();
                mma_f32_bn(t2, Ts + (ib * 16) * LDA + ib * 16, LDA, Ys, LDY, 16);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Ts[(ib * 16 + 4 * (l >> 4) + e) * LDA + jb * 16 + (l & 15)] = -t2[e];
            }
            __syncthreads();
        }
        if constexpr (!F32IN) {
            for (int idx = tid; idx < NR * NR; idx += 256) {
                const int i = idx / NR, j = idx % NR;
                if ((j >> 4) <= (i >> 4)) Tb[i * LDTB + j] = bf16_bits(Ts[i * LDA + j]);
            }
            __syncthreads();
        }

        // ---------------- chain: X_b = K_b S_b ----------------
        {
            constexpr int NX = R * (C / 16);
            for (int it = w; it < NX; it += 4) {
                const int bb = it / (C / 16), ti = it % (C / 16);
                floatx4 acc = zero4();
                if constexpr (F32IN) mma_f32(acc, Ks + ti * 16 * LDK + bb * DK, LDK, StH + bb * DK, LDST, DK);
                else mma_bf16(acc, Ks + ti * 16 * LDK + bb * DK, LDK, StH + bb * DK, LDST, DK);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Xs[(bb * C + ti * 16 + 4 * (l >> 4) + e) * BV + (l & 15)] = acc[e];
            }
        }
        __syncthreads();
        // R = diag(beta) (V - diag(e^G) sum_b M X_b), stored transposed for the next product
        for (int idx = tid; idx < NR * BV; idx += 256) {
            const int vr = idx / BV, j = idx % BV;
            const int t = vr / R, a = vr % R;
            float xs = 0.f;
#pragma unroll
            for (int bb = 0; bb < R; ++bb) xs += args.mask[a * R + bb] * Xs[(bb * C + t) * BV + j];
            const float r = betas[t * R + a] * (Vs[t * BV + j] - eG[t] * xs);
            store_op<F32IN>(RtH, RtL, j * LDRT + vr, r);
        }
        __syncthreads();
        // V_new = T R
        for (int ti = w; ti < NB; ti += 4) {
            floatx4 acc = zero4();
            if constexpr (F32IN) mma_f32(acc, Ts + ti * 16 * LDA, LDA, RtH, LDRT, NR);
            else mma_bf16_split(acc, Tb + ti * 16 * LDTB, nullptr, LDTB, RtH, RtL, LDRT, NR);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vr = ti * 16 + 4 * (l >> 4) + e;
                const int s = vr / R, bb = vr % R;
                const int o = (bb * BV + (l & 15)) * LDVT + s;
                store_op<F32IN>(VnH, VnL, o, acc[e]);
                store_op<F32IN>(VtH, VtL, o, eGLm[s] * acc[e]);
            }
        }
        __syncthreads();

        // ---------------- state update (registers) ----------------
        const float gL = gLs[0];
#pragma unroll
        for (int n = 0; n < NSTW; ++n) {
            const int ts = w + 4 * n;
            if (ts < NST) {
                const int bb = (ts * 16) / DK;
                floatx4 acc = zero4();
                if constexpr (F32IN) {
                    // A = K_b^T: element (i, s) = Ks[s][i]
                    const float *ka = Ks + ts * 16;
                    const float *vb2 = VtH + bb * BV * LDVT;
                    const float *pa = ka + (l & 15) + (l >> 4) * LDK;
                    const float *pb = vb2 + (l & 15) * LDVT + (l >> 4);
                    for (int kk = 0; kk < C; kk += 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[kk * LDK], pb[kk], acc, 0, 0, 0);
                } else {
                    mma_bf16_split(acc, KsT + ts * 16 * LDKT, nullptr, LDKT, VtH + bb * BV * LDVT,
                                   VtL + bb * BV * LDVT, LDVT, C);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[n][e] = gL * Sreg[n][e] + acc[e];
            }
        }

        // ---------------- output ----------------
        for (int ti = w; ti < C / 16; ti += 4) {
            floatx4 a1 = zero4(), a2 = zero4();
            if constexpr (F32IN) {
                mma_f32(a1, Qs + ti * 16 * LDK, LDK, StH, LDST, KD);
                const int kd = (ti + 1) * 16;
#pragma unroll
                for (int bb = 0; bb < R; ++bb)
                    mma_f32(a2, PqH + (bb * C + ti * 16) * LDPQ, LDPQ, VnH + bb * BV * LDVT, LDVT, kd);
            } else {
                mma_bf16_split(a1, Qs + ti * 16 * LDK, nullptr, LDK, StH, StL, LDST, KD);
                const int kd = (ti + 1) * 16;
#pragma unroll
                for (int bb = 0; bb < R; ++bb)
                    mma_bf16_split(a2, PqH + (bb * C + ti * 16) * LDPQ, PqL + (bb * C + ti * 16) * LDPQ, LDPQ,
                                   VnH + bb * BV * LDVT, VnL + bb * BV * LDVT, LDVT, kd);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = ti * 16 + 4 * (l >> 4) + e, tt = t0 + t;
                if (tt < T) {
                    const float ov = args.scale * (eG[t] * a1[e] + a2[e]);
                    const size_t off = (((size_t)b * T + tt) * tok_stride + h) * Dv + v0 + (l & 15);
                    if (args.out_bf16) reinterpret_cast<u16 *>(args.o)[off] = bf16_bits(ov);
                    else reinterpret_cast<float *>(args.o)[off] = ov;
                }
            }
        }
        __syncthreads();
        write_state_operand();
    }

    if (args.hT) {
#pragma unroll
        for (int n = 0; n < NSTW; ++n) {
            const int ts = w + 4 * n;
            if (ts < NST) {
                float *hp = args.hT + ((size_t)bh * KD) * Dv + v0 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) hp[(size_t)(ts * 16 + 4 * (l >> 4) + e) * Dv] = Sreg[n][e];
            }
        }
    }
}

// Launch one instantiation; returns the hipError_t of the launch.
template <bool F32IN, int KD, int C, int R>
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream) {
    const int nvb = a.Dv / 16;
    const int bhp = (a.B * a.H + 7) / 8;
    const int grid = bhp * 8 * nvb;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_fwd_kernel<F32IN, KD, C, R>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn
