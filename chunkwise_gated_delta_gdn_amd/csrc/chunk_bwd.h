// Backward of the chunkwise gated delta rule on MFMA, bf16 inputs, one step
// per token, 64-token chunks (msj19 "gated_deltaproduct" test.py names the
// chunk backward kernels of this rule: prepare_dv, dhu, dqkw and the WY
// backward; the kernels below compute the same gradients from the chunk
// form of the forward).
//
// Per chunk (G the chunk-local cumsum of g, gamma_t = e^{G_t},
// lambda_t = e^{G_L - G_t}, Lambda = e^{G_L}, Gam[t,s] = e^{G_t - G_s},
// A = strict_lower(diag(beta) (K K^T) o Gam), T = (I + A)^-1, S the state
// entering the chunk):
//   R = V - diag(gamma) K S,  Vn = T diag(beta) R,
//   O = scale (diag(gamma) Q S + Pm Vn),  Pm = lower_incl((Q K^T) o Gam),
//   S' = Lambda S + K^T diag(lambda) Vn.
// Given dO and dS' (the gradient of the state leaving the chunk):
//   dVn = scale Pm^T dO + diag(lambda) K dS',   dX = T^T dVn,
//   dS  = Lambda dS' + scale Q^T diag(gamma) dO - K^T diag(gamma beta) dX,
// a reverse recurrence over the chunks (chunk_bchain_kernel), and then, in
// parallel over chunks (chunk_bgrad_kernel), with dR = diag(beta) dX,
// M1 = lower_incl(scale (dO Vn^T) o Gam), dA = strict_lower(-dX Vn^T),
// M2 = diag(beta) dA o Gam:
//   dV = dR,
//   dQ = scale diag(gamma) dO S^T + M1 K,
//   dK = M1^T Q + M2 K + M2^T K - diag(gamma) dR S^T + diag(lambda) Vn dS'^T,
//   dbeta_t = sum_v dX R + sum_s dA (K K^T o Gam),
//   dG_t = rowsum(W) - colsum(W) + <dQ_dir_t, q_t> + <dK_R_t, k_t>
//          - <dK_S'_t, k_t>, W = M1 o (Q K^T) + dA o A,
//   dG_L += sum_t <dK_S'_t, k_t> + Lambda <dS', S>,
//   dg = reverse cumsum of dG within the chunk,
// where dQ_dir, dK_R and dK_S' are the three state terms of dQ and dK.
//
// The forward's chunk-start states S and residuals R come from the forward
// state pass (chunk_chain1_kernel<KD, 64, 3>); T, T^T and the transposed
// scores from chunk_prep2_kernel<KD, 64, true>.
//
// DPE: the first pass of the DeltaProduct backward (sub-key 0 of a 2 x 2
// lower unitriangular step mask [[1, 0], [m, 1]]).  Its errors
// e = R - A~ Vn (A~ = strict_lower((K K^T) o Gam)) feed the second pass
// through v' = (1 - m) v + m e, so the second pass's gradient of v' brings
// dE = m dv'.  Then dV0 gains -A~^T dE, the state recurrence -K^T diag(gamma)
// dE, and with dR = diag(beta) dX + dE (the total gradient of R):
//   dV = dR + (1 - m) dv' (+ m dv' through dE: dV = diag(beta) dX + dv'),
//   dB = strict_lower(-dR Vn^T) the gradient of the gram K K^T o Gam, taking
//   the place of diag(beta) dA (M2 = dB o Gam, W = M1 o (Q K^T) + dB o A~),
//   dK_R = -diag(gamma) dR S^T,  dbeta_t = sum_v dX (R - A~ Vn) = sum_v dX e,
// and dg adds the second pass's.
#pragma once

#include "chunk_chain1.h"

namespace gdn {

struct BwdChunkArgs {
    ChunkArgs a;             // q, k, v, beta, g, h0, scale; tmat, tmatT, pfrag, gtab (prep); sst, rst
    const void *dout;        // (B, T, H, Dv) bf16
    const float *dhT;        // (B, H, Dk, Dv) or null
    float *dq, *dk, *dv, *dbeta, *dg, *dh0;
    float *dsst;             // gradient of the state leaving each chunk, (B*H, NT, Dk, Dv) fp32
    float *dxst;             // dX per chunk, (B*H, NT, Dv/16, 64 lanes, 16) fp32, accumulator order
    const float *dvprev;     // DeltaProduct first pass: the second pass's gradient of v', (B, T, H, Dv)
    int nfirst;              // chunk_bgrad_kernel: workgroups in its first round (one per CU)
};

// ---------------------------------------------------------------------------
// Reverse state pass.  One workgroup per (batch, head, 16-column slice of
// the value dimension), six waves:
//   0  the chain: dS' (KD x 16, fp32) in MFMA accumulators, chunks walked
//      from the last to the first;
//   4  idle (the chain's SIMD partner; barriers only);
//   1, 2  E = scale Q^T diag(gamma) dO of the next chunk in walk order,
//      half of the state rows each (published to LDS in the chain's
//      accumulator order), and the copy of dS' the chain leaves in that
//      buffer, to the work space;
//      Wave 2 also forms dV0 = scale Pm^T dO of that chunk (Pm^T
//      fragments, hi/lo, straight from the prep into registers one step
//      ahead; published like E);
//   3, 5 staging: ring A (K rows, T^T, gate table) two steps before the
//      chain uses it, ring B (Q rows, dO slice, gate table) two steps
//      before the helpers use it, by LDS-direct loads.
// Step s = 0 .. NT: the chain processes chunk NT - s (s >= 1), the helpers
// chunk NT - 1 - s; one workgroup barrier per step.
// ---------------------------------------------------------------------------
template <int KD, bool DPE = false>
struct BChainShape {
    static constexpr int C = 64, BV = 16, NTT = 4, NCS = 2;
    static constexpr int NKS = KD / 32, NST = KD / 16, NKC = KD / 8;
    static constexpr int TSW = C / 8 - 1;
    static constexpr int NW = 6, NTHR = 64 * NW, IDLE = 4;
    static constexpr int LDK = KD, LDT = C, LDV = BV;
    static constexpr int NGATE = gate_table_len<C>();
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int SZ_KS = al(C * LDK * 2);
    static constexpr int SZ_TT = al(C * LDT * 2);
    static constexpr int SZ_GA = al(NGATE * 4);
    static constexpr int SZ_GB = al(C * 4);           // ring B holds e^G only
    static constexpr int SZ_DO = al(C * LDV * 2);
    static constexpr int SZ_EP = 64 * NST * 16;
    static constexpr int SZ_DP = 64 * NTT * 16;
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_TT = OFF_KS + 3 * SZ_KS;
    static constexpr int OFF_GA = OFF_TT + 3 * SZ_TT;
    static constexpr int OFF_QS = OFF_GA + 3 * SZ_GA;
    static constexpr int OFF_DO = OFF_QS + 3 * SZ_KS;
    // DPE: the dO slice goes to registers straight from global memory (no
    // ring), which leaves room for dE (three buffers, index chunk % 3)
    static constexpr int NDOB = DPE ? 0 : 3;
    static constexpr int OFF_GB = OFF_DO + NDOB * SZ_DO;
    static constexpr int OFF_EP = OFF_GB + 3 * SZ_GB;
    static constexpr int OFF_DP = OFF_EP + 2 * SZ_EP;
    static constexpr int OFF_DE = OFF_DP + 2 * SZ_DP;
    static constexpr int BYTES = OFF_DE + (DPE ? 3 * SZ_DP : 0);
    static_assert(KD % 32 == 0 && KD <= 128, "key width");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
    static_assert(SZ_KS % 1024 == 0 && SZ_TT % 1024 == 0 && SZ_DO % 1024 == 0, "whole 1 KiB wave loads");
};

// K^T (or Q^T) operand fragments in the chain's state-row order: tile ti of
// the state rows, 32-token step m (tokens in the permuted order), read
// transposed from swizzled rows (as the forward state pass reads them).
template <int KD>
__device__ __forceinline__ void kt_frags(const u16 *ks, bf16x8 (&ka)[KD / 16][2]) {
    using S = BChainShape<KD>;
    constexpr int NKC = S::NKC, LDK = S::LDK;
    const int l = lane_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
    for (int ti = 0; ti < KD / 16; ++ti) {
        const int pc = 4 * (ti >> 1) + (c16 & 3), hf = 4 * (ti & 1);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r0 = m * 32 + 4 * g + (c16 >> 2), r1 = r0 + 16;
            const uint2 lo = __builtin_bit_cast(uint2, ld_tr16(ks + r0 * LDK + ((pc ^ kswz<NKC>(r0)) << 3) + hf));
            const uint2 hi = __builtin_bit_cast(uint2, ld_tr16(ks + r1 * LDK + ((pc ^ kswz<NKC>(r1)) << 3) + hf));
            ka[ti][m] = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
        }
    }
}

template <int KD, bool DPE = false>
__global__ __launch_bounds__(BChainShape<KD>::NTHR) void chunk_bchain_kernel(BwdChunkArgs ba) {
    using S = BChainShape<KD, DPE>;
    constexpr int C = S::C, BV = S::BV, NTT = S::NTT, NKS = S::NKS, NST = S::NST, NCS = S::NCS, NKC = S::NKC;
    constexpr int LDK = S::LDK, LDT = S::LDT, LDV = S::LDV, TSW = S::TSW, NGATE = S::NGATE;
    constexpr int NLOW = NTT * (NTT + 1) / 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    const ChunkArgs &args = ba.a;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nvb = args.Dv / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vb = slot % nvb;
    const int bh = (slot / nvb) * 8 + xcd;      // all value slices of one head share an XCD
    if (bh >= args.B * args.H) return;
    const int T = args.T, H = args.H, Dv = args.Dv;
    const int NT = (T + C - 1) / C;
    const int nbar = NT + 3;                    // barriers every wave takes part in
    if (w == S::IDLE) {
        for (int i = 0; i < nbar; ++i) __syncthreads();
        return;
    }
    const int b = bh / H, h = bh % H;
    const int v0 = vb * BV;
    const int tlast = T - 1;

    auto Ks = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_KS + p * S::SZ_KS); };
    auto Tt = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_TT + p * S::SZ_TT); };
    auto gA = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_GA + p * S::SZ_GA); };
    auto Qs = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_QS + p * S::SZ_KS); };
    auto dOs = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_DO + p * S::SZ_DO); };
    auto gB = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_GB + p * S::SZ_GB); };
    auto Ep = [&](int p) { return reinterpret_cast<floatx4 *>(smem + S::OFF_EP + p * S::SZ_EP); };
    auto Dp = [&](int p) { return reinterpret_cast<floatx4 *>(smem + S::OFF_DP + p * S::SZ_DP); };
    auto De = [&](int p) { return reinterpret_cast<floatx4 *>(smem + S::OFF_DE + p * S::SZ_DP); };
    auto ring = [](int c) { return ((c % 3) + 3) % 3; };

    if (w == 0) {
        // ================================================================
        // chain wave: dS' rows in the forward state pass's order (tile ti,
        // accumulator row 4g + e <-> key feature feat(ti, e))
        // ================================================================
        floatx4 Sreg[NST];
        auto feat = [&](int ti, int e) { return (ti >> 1) * 32 + 8 * g + 4 * (ti & 1) + e; };
#pragma unroll
        for (int ti = 0; ti < NST; ++ti) {
            Sreg[ti] = zero4();
            if (ba.dhT) {
                const float *hp = ba.dhT + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[ti][e] = hp[(size_t)feat(ti, e) * Dv];
            }
        }
        __syncthreads();                        // prologue staging complete
        lds_barrier();                          // step 0: the helpers' first chunk
        for (int c = NT - 1; c >= 0; --c) {
            const int sq = ring(c), p = c & 1;

            const u16 *ks = Ks(sq), *tt_ = Tt(sq);
            const float *gp = gA(sq);
            bf16x8 kf[NTT][NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    const int r = tt * 16 + c16;
                    kf[tt][m] = ld8(ks + r * LDK + (((4 * m + g) ^ kswz<NKC>(r)) << 3));
                }
            // X1 = K dS' (dS' as hi + lo bf16)
            floatx4 x1[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) x1[tt] = zero4();
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                bf16x8 sh, sl;
                frag_split(Sreg[2 * m], Sreg[2 * m + 1], sh, sl);
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) x1[tt] = mfma32(kf[tt][m], sh, x1[tt]);
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) x1[tt] = mfma32(kf[tt][m], sl, x1[tt]);
            }
            bf16x8 ka[NST][NCS];
            kt_frags<KD>(ks, ka);
            // T^T fragments: row tile st, 32-token step m (t > s only: 2m + 1 >= st)
            bf16x8 tf[NTT][NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m)
#pragma unroll
                for (int st = 0; st < NTT; ++st)
                    if (2 * m + 1 >= st)
                        tf[st][m] = ld8(tt_ + (st * 16 + c16) * LDT + (((4 * m + g) ^ ((st * 16 + c16) & TSW)) << 3));
            floatx4 eg[NTT], el[NTT], bt[NTT], dv0[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                eg[tt] = *reinterpret_cast<const floatx4 *>(gp + tt * 16 + 4 * g);
                el[tt] = *reinterpret_cast<const floatx4 *>(gp + C + tt * 16 + 4 * g);
                bt[tt] = *reinterpret_cast<const floatx4 *>(gp + 2 * C + 4 + tt * 16 + 4 * g);
                dv0[tt] = Dp(p)[tt * 64 + l];
            }

            const float gL = gp[2 * C];
            // dVn = dV0 + lambda o X1; dX = dVn + T_off^T dVn (dVn rounded once)
            floatx4 dvn[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dvn[tt][e] = dv0[tt][e] + el[tt][e] * x1[tt][e];
            bf16x8 dvh[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) dvh[m] = frag_hi(dvn[2 * m], dvn[2 * m + 1]);
            floatx4 dx[NTT];
#pragma unroll
            for (int st = 0; st < NTT; ++st) dx[st] = dvn[st];
#pragma unroll
            for (int m = 0; m < NCS; ++m)
#pragma unroll
                for (int st = 0; st < NTT; ++st)
                    if (2 * m + 1 >= st) dx[st] = mfma32(tf[st][m], dvh[m], dx[st]);
            // DPE: dE = m dv' of this chunk (accumulator layout, zero past T),
            // published by wave 1 two steps earlier
            floatx4 dE[NTT];
            if constexpr (DPE) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) dE[tt] = De(sq)[tt * 64 + l];
            }
            // Z = -gamma beta dX (DPE: -gamma (beta dX + dE)), hi + lo;
            // dS = Lambda dS' + E + K^T Z
            floatx4 z[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (DPE)
                        z[tt][e] = -eg[tt][e] * (bt[tt][e] * dx[tt][e] + dE[tt][e]);
                    else
                        z[tt][e] = -(eg[tt][e] * bt[tt][e]) * dx[tt][e];
                }
            bf16x8 zh[NCS], zl[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) frag_split(z[2 * m], z[2 * m + 1], zh[m], zl[m]);
            // E initialises the update's accumulators; dS' of this chunk (the
            // gradient of the state leaving it) goes over it, and waves 1 and 2
            // write it to the work space next step
            floatx4 ds[NST];
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                ds[ti] = Ep(p)[ti * 64 + l];
                Ep(p)[ti * 64 + l] = Sreg[ti];
            }
#pragma unroll
            for (int m = 0; m < NCS; ++m) {
#pragma unroll
                for (int ti = 0; ti < NST; ++ti) ds[ti] = mfma32(ka[ti][m], zh[m], ds[ti]);
#pragma unroll
                for (int ti = 0; ti < NST; ++ti) ds[ti] = mfma32(ka[ti][m], zl[m], ds[ti]);
            }
            // dX of this chunk (rows past T zero) while the MFMAs run
            {
                floatx4 *xp = reinterpret_cast<floatx4 *>(ba.dxst) + (((size_t)bh * NT + c) * nvb + vb) * 64 * NTT + l * NTT;
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    floatx4 x = dx[tt];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c * C + tt * 16 + 4 * g + e > tlast) x[e] = 0.f;
                    xp[tt] = x;
                }
            }
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[ti][e] = gL * Sreg[ti][e] + ds[ti][e];
            lds_barrier();
        }
        __syncthreads();
        if (ba.dh0) {
            float *hp = ba.dh0 + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + c16;
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) hp[(size_t)feat(ti, e) * Dv] = Sreg[ti][e];
        }
        return;
    }

    const float scale = args.scale;
    if (w == 1 || w == 2) {
        // ================================================================
        // waves 1 and 2: E = scale Q^T diag(gamma) dO of the next chunk in
        // walk order, state row tiles [0, NST/2) and [NST/2, NST) (published
        // in the chain's accumulator order over the dS' copy the chain left
        // in that buffer one step earlier, which each wave first writes to
        // the work space for its own tiles)
        // ================================================================
        const int th0 = (w - 1) * (NST / 2);
        // the dS' copy of chunk cd, this wave's tiles, as 16-byte pieces of its
        // rows: lane l takes state row 4 (l/16) + e of tile ti ... i.e. copy
        // row rr = l/4 (accumulator row 4 g' + e' of the tile) and value
        // columns 4 (l%4) .. +3, gathered from the four lanes holding them
        auto store_ds = [&](int cd) {
            const int rr = l >> 2, q = l & 3, gq = rr >> 2, eq = rr & 3;
            const float *ep = reinterpret_cast<const float *>(Ep(cd & 1));
            float *sp = ba.dsst + ((size_t)bh * NT + cd) * KD * Dv + v0 + 4 * q;
#pragma unroll
            for (int i = 0; i < NST / 2; ++i) {
                const int ti = th0 + i;
                floatx4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = ep[(ti * 64 + gq * 16 + 4 * q + e) * 4 + eq];
                const int f = (ti >> 1) * 32 + 8 * gq + 4 * (ti & 1) + eq;
                *reinterpret_cast<floatx4 *>(sp + (size_t)f * Dv) = x;
            }
        };
        // wave 2: fragments of a chunk's transposed scores (and with DPE of
        // A~^T, the same layout), loaded one step ahead
        u32x4 pf[NLOW], af[NLOW];
        auto load_pf = [&](int c) {
            c = c < 0 ? 0 : c;                  // (past the first chunk: loaded again, unused)
            const uint4 *pc = reinterpret_cast<const uint4 *>(args.pfrag) + ((size_t)bh * NT + c) * NLOW * 64 + l;
#pragma unroll
            for (int i = 0; i < NLOW; ++i) pf[i] = __builtin_bit_cast(u32x4, pc[i * 64]);
            if constexpr (DPE) {
                const uint4 *ac = reinterpret_cast<const uint4 *>(args.atilT) + ((size_t)bh * NT + c) * NLOW * 64 + l;
#pragma unroll
                for (int i = 0; i < NLOW; ++i) af[i] = __builtin_bit_cast(u32x4, ac[i * 64]);
            }
        };
        // DPE, wave 1: dv' of a chunk, this lane's rows tt*16 + 4g + e
        // (clamped to T - 1), column v0 + c16, loaded one step before it is
        // published as dE = m dv' (rows past T zero) in De(chunk % 3), a step
        // before wave 2 and two before the chain use it (the loads are kept
        // as they are until then, so that nothing waits for them earlier)
        floatx4 dep[NTT];
        auto load_de = [&](int c) {
            c = c < 0 ? 0 : c;
            const float *dp = ba.dvprev + ((size_t)b * T * H + h) * Dv + v0 + c16;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dep[tt][e] = dp[(size_t)min(c * C + tt * 16 + 4 * g + e, tlast) * H * Dv];
        };
        // DPE: the dO slice of a chunk (rows tt*16 + 4g + e clamped to T - 1,
        // column v0 + c16), loaded one step ahead as it is (rows past T zeroed
        // where it is used), each value into a register of its own (loads into
        // halves of one register would wait for each other)
        unsigned int opre[NTT][4];
        auto load_do = [&](int c) {
            c = c < 0 ? 0 : c;
            const u16 *op = reinterpret_cast<const u16 *>(ba.dout) + ((size_t)b * T * H + h) * Dv + v0 + c16;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) opre[tt][e] = op[(size_t)min(c * C + tt * 16 + 4 * g + e, tlast) * H * Dv];
        };
        auto publish_de = [&](int c) {
            const float mc = args.mcoef;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                floatx4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = c * C + tt * 16 + 4 * g + e <= tlast ? mc * dep[tt][e] : 0.f;
                De(ring(c))[tt * 64 + l] = x;
            }
        };
        if (w == 2) load_pf(NT - 1);
        if constexpr (DPE) {
            if (w == 1) {
                load_de(NT - 1);
                publish_de(NT - 1);             // (waits for those loads: once)
                load_de(NT - 2);
            }
            load_do(NT - 1);
        }
        __syncthreads();
        for (int s = 0; s <= NT; ++s) {
            const int c = NT - 1 - s;
            if (s >= 2) store_ds(c + 2);
            if (c >= 0) {
                const int sq = ring(c), p = c & 1;
                const float *gp = gB(sq);
                shortx4 vv[NTT];
                if constexpr (DPE) {
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) {
                        unsigned int x[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = c * C + tt * 16 + 4 * g + e <= tlast ? opre[tt][e] : 0u;
                        vv[tt] = __builtin_bit_cast(shortx4, uint2{x[0] | (x[1] << 16), x[2] | (x[3] << 16)});
                    }
                    load_do(c - 1);
                } else {
                    const u16 *dos = dOs(sq);
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt)
                        vv[tt] = ld_tr16(dos + (tt * 16 + 4 * g + (c16 >> 2)) * LDV + 4 * (c16 & 3));
                }
                // E tiles of this wave: Q^T fragments (the chain's row order) times
                // gamma dO (hi + lo)
                floatx4 gd[NTT];
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    const uint2 v2 = __builtin_bit_cast(uint2, vv[tt]);
                    const floatx4 e4 = *reinterpret_cast<const floatx4 *>(gp + tt * 16 + 4 * g);
                    gd[tt] = floatx4{scale * e4[0] * __builtin_bit_cast(float, v2.x << 16),
                                     scale * e4[1] * __builtin_bit_cast(float, v2.x & 0xffff0000u),
                                     scale * e4[2] * __builtin_bit_cast(float, v2.y << 16),
                                     scale * e4[3] * __builtin_bit_cast(float, v2.y & 0xffff0000u)};
                }
                bf16x8 gh[NCS], gl[NCS];
#pragma unroll
                for (int m = 0; m < NCS; ++m) frag_split(gd[2 * m], gd[2 * m + 1], gh[m], gl[m]);
                const u16 *qs = Qs(sq);
#pragma unroll 1
                for (int i = 0; i < NST / 2; ++i) {
                    const int ti = th0 + i;
                    const int pc = 4 * (ti >> 1) + (c16 & 3), hf = 4 * (ti & 1);
                    floatx4 ev = zero4();
#pragma unroll
                    for (int m = 0; m < NCS; ++m) {
                        const int r0 = m * 32 + 4 * g + (c16 >> 2), r1 = r0 + 16;
                        const uint2 lo = __builtin_bit_cast(uint2, ld_tr16(qs + r0 * LDK + ((pc ^ kswz<NKC>(r0)) << 3) + hf));
                        const uint2 hi = __builtin_bit_cast(uint2, ld_tr16(qs + r1 * LDK + ((pc ^ kswz<NKC>(r1)) << 3) + hf));
                        const bf16x8 qa = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
                        ev = mfma32(qa, gh[m], ev);
                        ev = mfma32(qa, gl[m], ev);
                    }
                    Ep(p)[ti * 64 + l] = ev;
                }
                if (w == 2) {                   // dV0 = scale Pm^T dO (DPE: - A~^T dE, hi + lo)
                    shortx4 dh4[NTT], dl4[NTT];
                    if constexpr (DPE) {
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt) split4(De(sq)[tt * 64 + l], dh4[tt], dl4[tt]);
                    }
#pragma unroll
                    for (int st = 0; st < NTT; ++st) {
                        floatx4 acc = zero4(), acc2 = zero4();
#pragma unroll
                        for (int tt = st; tt < NTT; ++tt) {
                            const u32x4 f = pf[tt * (tt + 1) / 2 + st];
                            const shortx4 ah = __builtin_bit_cast(shortx4, uint2{f[0], f[1]});
                            const shortx4 al = __builtin_bit_cast(shortx4, uint2{f[2], f[3]});
                            acc = mfma16(ah, vv[tt], acc);
                            acc = mfma16(al, vv[tt], acc);
                            if constexpr (DPE) {
                                const u32x4 fa = af[tt * (tt + 1) / 2 + st];
                                const shortx4 bh_ = __builtin_bit_cast(shortx4, uint2{fa[0], fa[1]});
                                const shortx4 bl_ = __builtin_bit_cast(shortx4, uint2{fa[2], fa[3]});
                                acc2 = mfma16(bh_, dh4[tt], acc2);
                                acc2 = mfma16(bh_, dl4[tt], acc2);
                                acc2 = mfma16(bl_, dh4[tt], acc2);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = scale * acc[e] - acc2[e];
                        Dp(p)[st * 64 + l] = acc;
                    }
                    load_pf(c - 1);
                }
                if constexpr (DPE) {
                    if (w == 1 && c >= 1) {     // dE of the next chunk
                        publish_de(c - 1);
                        load_de(c - 2);
                    }
                }
            }
            lds_barrier();
        }
        store_ds(0);                            // published at the last step
        __syncthreads();
        return;
    }

    // ====================================================================
    // staging waves (3 and 5)
    // ====================================================================
    constexpr int NDK = S::SZ_KS / 1024, NDT = S::SZ_TT / 1024, NDO = DPE ? 0 : S::SZ_DO / 1024;
    constexpr int NGV = NGATE / 4;
    constexpr int NA = NDK + NDT + 1, NB = NDK + NDO + 1, NDMA = NA + NB;
    static_assert(NGV <= 64 && S::SZ_GA >= NGV * 16, "gate table: one partial wave load");
    const size_t tokq = (size_t)H * args.kst, tokv = (size_t)H * Dv;
    const u16 *kg = reinterpret_cast<const u16 *>(args.k) + ((size_t)b * T * H + h) * args.kst + args.koff;
    const u16 *qg = reinterpret_cast<const u16 *>(args.q) + ((size_t)b * T * H + h) * args.kst + args.koff;
    const u16 *og = reinterpret_cast<const u16 *>(ba.dout) + ((size_t)b * T * H + h) * Dv + v0;
    const u16 *tg = reinterpret_cast<const u16 *>(args.tmatT) + (size_t)bh * NT * C * C;
    const float *gtg = reinterpret_cast<const float *>(args.gtab) + (size_t)bh * NT * NGATE;
    // Each staging wave runs a copy specialised for its index LI (load k goes
    // to wave 3 + 2 (k % 2)), so its loads are straight-line code.
    auto staging_wave = [&](auto lic) {
        constexpr int LI = decltype(lic)::value;
        // ring A: chunk ca (K rows, T^T, gates); ring B: chunk cb (Q rows, dO
        // slice, gates).  A chunk before the first lands in a buffer no one
        // reads (its data clamped to chunk 0).  K rows past T are clamped (they
        // meet zero beta); Q and dO rows past T are zero.
        // Addresses: a per-call base of the chunk (scalar) plus a 32-bit
        // per-lane offset (row < 64 times a row stride below 2^24: a 24-bit
        // multiply), so that a load costs a few VALU operations rather than
        // 64-bit multiplies (these waves' issue time is a large part of a step)
        const unsigned tokq_u = (unsigned)tokq, tokv_u = (unsigned)tokv;
        auto stage = [&](int ca, int cb) {
            const int pa = ring(ca), pb = ring(cb);
            ca = ca < 0 ? 0 : ca;
            cb = cb < 0 ? 0 : cb;
            const int rla = tlast - ca * C, rlb = tlast - cb * C;   // last valid row of each chunk
            const u16 *kc = kg + (size_t)ca * C * tokq, *qc = qg + (size_t)cb * C * tokq;
            const u16 *tc = tg + (size_t)ca * C * C, *oc = og + (size_t)cb * C * tokv;
#pragma unroll
            for (int k = LI; k < NDMA; k += 2) {
                if (k < NDK) {
                    const int pos = k * 64 + l, r = pos / NKC, sc = pos % NKC;
                    const int pc = sc ^ kswz<NKC>(r);
                    dma16(kc + (__umul24(min(r, rla), tokq_u) + (unsigned)(pc << 3)), Ks(pa) + k * 512);
                } else if (k < NDK + NDT) {
                    const int kk = k - NDK, pos = kk * 64 + l, r = pos / (C / 8), sc = pos % (C / 8);
                    dma16(tc + (unsigned)(r * C + ((sc ^ (r & TSW)) << 3)), Tt(pa) + kk * 512);
                } else if (k == NDK + NDT) {
                    if (l < NGV) dma16(gtg + (size_t)ca * NGATE + l * 4, gA(pa));
                } else if (k < NA + NDK) {
                    const int kk = k - NA, pos = kk * 64 + l, r = pos / NKC, sc = pos % NKC;
                    const int pc = sc ^ kswz<NKC>(r);
                    dma16(r <= rlb ? static_cast<const void *>(qc + (__umul24(r, tokq_u) + (unsigned)(pc << 3)))
                                   : static_cast<const void *>(&kZero16),
                          Qs(pb) + kk * 512);
                } else if (k < NA + NDK + NDO) {
                    const int kk = k - NA - NDK, pos = kk * 64 + l, r = pos / 2;
                    dma16(r <= rlb ? static_cast<const void *>(oc + (__umul24(r, tokv_u) + (unsigned)((pos & 1) * 8)))
                                   : static_cast<const void *>(&kZero16),
                          dOs(pb) + kk * 512);
                } else {
                    if (l < C / 4) dma16(gtg + (size_t)cb * NGATE + l * 4, gB(pb));   // e^G
                }
            }
        };
        // loads this wave issues per step: after the barrier wait at most these
        // (this step's) are outstanding, so the previous step's are complete
        constexpr int NMINE = (NDMA - LI + 1) / 2;
        static_assert(NMINE < 64, "6-bit vmcnt");
        constexpr int WAIT_IMM = (NMINE & 15) | ((NMINE >> 4) << 14) | 0x0070;
        // prologue: ring A chunk NT-1, ring B chunks NT-1 and NT-2 (ring A's
        // chunk NT-2 is staged again, identically, at step 0; nothing reads it
        // before step 2)
        stage(NT - 1, NT - 1);
        stage(NT - 2, NT - 2);
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
        __syncthreads();
        for (int s = 0; s <= NT; ++s) {
            stage(NT - s - 2, NT - s - 3);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(WAIT_IMM);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };
    if (w == 3) staging_wave(std::integral_constant<int, 0>{});
    else staging_wave(std::integral_constant<int, 1>{});
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-chunk gradients.  One workgroup of eight waves per (batch, head,
// chunk), in phases separated by barriers:
//   0  K, Q and dO rows of the chunk staged in LDS (LDS-direct, zero past
//      T), the gates (cumsum in log2 units) and beta; every wave also issues
//      its loads of phases 1 and 3 (R, dX, T' fragments; S, dS' fragments),
//      so all of the chunk's HBM reads are in flight together;
//   1  wave w < Dv/16 owns value columns 16w..16w+15: Vn = beta R + T' R
//      (T' = T diag(beta) without its diagonal, R hi + lo), dV = beta dX,
//      dbeta's first sum; Vn and dX go to LDS as hi/lo bf16 rows;
//   2  the 10 lower 16x16 tiles of M1 (with Q K^T) and of dA, M2 (with
//      K K^T), one job per (tile, kind) over the waves; M1 and M2 go to
//      LDS as hi/lo bf16, row and column sums of W to per-tile slots;
//   3  wave w < Dk/16 owns key features 16w..16w+15: dQ and dK (products
//      taken transposed, so each lane stores 4 features of one token), and
//      their row products with q and k for the gate gradient; S and dS'
//      come straight from the work space as A operands (k = value column);
//   4  wave 0: dbeta and dg of the chunk (fixed-order sums, reverse
//      cumsum).
// ---------------------------------------------------------------------------
template <int KD>
struct BGradShape {
    static constexpr int C = 64, NTT = 4, NKS = KD / 32, NKC = KD / 8, NFS = KD / 16;
    static constexpr int DVM = 128;           // value width the LDS rows are laid out for
    static constexpr int NW = 8, NTHR = 64 * NW;
    static constexpr int SZ_KC = C * KD * 2;  // K, Q rows, bf16, swizzled pieces
    static constexpr int SZ_V = C * DVM * 2;  // Vn and dX rows (hi, lo), bf16, swizzled pieces
    static constexpr int SZ_M = C * C * 2;    // M1 and M2 (hi, lo), bf16, swizzled pieces
    static constexpr int OFF_KC = 0, OFF_QC = SZ_KC;
    static constexpr int OFF_VH = 2 * SZ_KC, OFF_VL = OFF_VH + SZ_V, OFF_XH = OFF_VL + SZ_V, OFF_XL = OFF_XH + SZ_V;
    static constexpr int OFF_M1H = OFF_XL + SZ_V, OFF_M1L = OFF_M1H + SZ_M, OFF_M2H = OFF_M1L + SZ_M,
                         OFF_M2L = OFF_M2H + SZ_M;
    static constexpr int OFF_DO = OFF_M2L + SZ_M;      // dO rows, bf16, swizzled pieces
    static constexpr int OFF_G2 = OFF_DO + SZ_V;       // G (log2 units) [C]
    static constexpr int OFF_BT = OFF_G2 + C * 4;      // beta [C]
    static constexpr int OFF_ZERO = OFF_BT + C * 4;    // cleared in phase 0:
    static constexpr int OFF_DB2 = OFF_ZERO;           //   [4][C] dbeta, second sum, by column tile
    static constexpr int OFF_GR1 = OFF_DB2 + 4 * C * 4;   // [4][C] row sums of W1 by column tile
    static constexpr int OFF_GC1 = OFF_GR1 + 4 * C * 4;   // [4][C] column sums of W1 by row tile
    static constexpr int OFF_GR2 = OFF_GC1 + 4 * C * 4;
    static constexpr int OFF_GC2 = OFF_GR2 + 4 * C * 4;
    static constexpr int OFF_ZEND = OFF_GC2 + 4 * C * 4;
    static constexpr int OFF_DB1 = OFF_ZEND;           // [8][C] dbeta, first sum, by value slice
    static constexpr int OFF_G3 = OFF_DB1 + 8 * C * 4;    // [8][C] state row products by key slice
    static constexpr int OFF_GS = OFF_G3 + 8 * C * 4;     // [8][C] <dK_S', k> by key slice
    static constexpr int OFF_SS = OFF_GS + 8 * C * 4;     // [8] <dS', S> by key slice
    static constexpr int BYTES = OFF_SS + 8 * 4;
    static_assert(KD % 32 == 0 && KD <= 128, "key width");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

// Element (r, col) of a row-major bf16 matrix with NPC 16-byte pieces per row
// whose pieces are stored at piece ^ kswz<NPC>(r).
template <int NPC>
__device__ __forceinline__ int swz_at(int r, int col) {
    return r * NPC * 8 + ((((col >> 3) ^ kswz<NPC>(r))) << 3) + (col & 7);
}
// Row fragment (A operand rows r = r0 + l%16, k = col0 + 8 (l/16) .. +7).
template <int NPC>
__device__ __forceinline__ bf16x8 row_frag(const u16 *base, int r, int col0) {
    return ld8(base + swz_at<NPC>(r, col0 + 8 * (lane_id() >> 4)));
}
// Transposed fragment: lane (g, j) gets X[r0 + e][c0 + j] for e < 8, with r0
// the caller's (per lane group) first row: the B operand X (k = rows), or the
// A operand X^T.
template <int NPC>
__device__ __forceinline__ bf16x8 tr_frag(const u16 *base, int r0, int c0) {
    const int c16 = lane_id() & 15;
    const int ra = r0 + (c16 >> 2), col = c0 + 4 * (c16 & 3);
    const uint2 lo = __builtin_bit_cast(uint2, ld_tr16(base + swz_at<NPC>(ra, col)));
    const uint2 hi = __builtin_bit_cast(uint2, ld_tr16(base + swz_at<NPC>(ra + 4, col)));
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}
// Sum over the 16 lanes of a lane group (the columns of an accumulator tile)
// by DPP moves, VALU only: pairs and quads by quad permutations, then 8 and 16
// lanes by the half-row and row mirrors (each lane of a group already holds
// the group's total, so the mirrored partner brings the other half's).
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
    v = dpp_plus<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_plus<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_plus<0x141>(v);   // row_half_mirror
    return dpp_plus<0x140>(v);  // row_mirror
}
// hi and lo bf16 of one value
__device__ __forceinline__ void split1(float x, u16 &hi, u16 &lo) { split_bf16(x, hi, lo); }

template <int KD, bool DPE = false>
__global__ __launch_bounds__(BGradShape<KD>::NTHR) void chunk_bgrad_kernel(BwdChunkArgs ba) {
    using S = BGradShape<KD>;
    constexpr int C = S::C, NTT = S::NTT, NKS = S::NKS, NKC = S::NKC, DVM = S::DVM;
    constexpr int NPV = DVM / 8, NPM = C / 8;   // pieces per row of the Vn/dX and M1/M2 arrays

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    const ChunkArgs &args = ba.a;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Every other workgroup of the first round starts ~12k cycles late.  All
    // workgroups of a round would otherwise issue their loads together and
    // then compute together, leaving HBM idle in between; the offset carries
    // over to the later rounds (the next workgroup starts where one ends).
    if ((int)blockIdx.x < ba.nfirst && (blockIdx.x & 1)) {
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(63);
    }
    const int T = args.T, H = args.H, Dv = args.Dv;
    const int NT = (T + C - 1) / C;
    const int nvs = Dv / 16, nmv = Dv / 32, nfs = KD / 16;
    const float scale = args.scale;

    u16 *Kc = reinterpret_cast<u16 *>(smem + S::OFF_KC), *Qc = reinterpret_cast<u16 *>(smem + S::OFF_QC);
    u16 *Vh = reinterpret_cast<u16 *>(smem + S::OFF_VH), *Vl = reinterpret_cast<u16 *>(smem + S::OFF_VL);
    u16 *Xh = reinterpret_cast<u16 *>(smem + S::OFF_XH), *Xl = reinterpret_cast<u16 *>(smem + S::OFF_XL);
    u16 *M1h = reinterpret_cast<u16 *>(smem + S::OFF_M1H), *M1l = reinterpret_cast<u16 *>(smem + S::OFF_M1L);
    u16 *M2h = reinterpret_cast<u16 *>(smem + S::OFF_M2H), *M2l = reinterpret_cast<u16 *>(smem + S::OFF_M2L);
    float *G2 = reinterpret_cast<float *>(smem + S::OFF_G2), *Bt = reinterpret_cast<float *>(smem + S::OFF_BT);
    float *db2 = reinterpret_cast<float *>(smem + S::OFF_DB2);
    float *gr1 = reinterpret_cast<float *>(smem + S::OFF_GR1), *gc1 = reinterpret_cast<float *>(smem + S::OFF_GC1);
    float *gr2 = reinterpret_cast<float *>(smem + S::OFF_GR2), *gc2 = reinterpret_cast<float *>(smem + S::OFF_GC2);
    float *db1 = reinterpret_cast<float *>(smem + S::OFF_DB1), *g3 = reinterpret_cast<float *>(smem + S::OFF_G3);
    float *gS = reinterpret_cast<float *>(smem + S::OFF_GS), *ss = reinterpret_cast<float *>(smem + S::OFF_SS);

    const size_t tokk = (size_t)H * args.kst, tokv = (size_t)H * Dv;
    u16 *dOc = reinterpret_cast<u16 *>(smem + S::OFF_DO);
    constexpr int NLOW = NTT * (NTT + 1) / 2;
    const int f0 = 16 * w;
    const int ws = w < nvs ? w : 0;             // a valid value slice for waves past the last

    // One chunk per workgroup (job = blockIdx.x).  Loads in three steps, each
    // behind the work that does not need it: phase 1's register operands
    // (waited for in phase 0); K, Q and dO rows into LDS (LDS-direct, issued
    // right after them, needed from phase 2); S and dS' (NP3 loads, issued
    // after phase 1, needed in phase 3).  (A persistent form, walking chunks with
    // the next chunk's operands in flight, needs more registers than two
    // waves per SIMD have: the loop keeps its lane address arithmetic live
    // and spills.)
    floatx4 rr[NTT], xr[NTT];
    bf16x8 tf[NTT][2];
    floatx4 dvr[NTT];
    u32x4 atf[NLOW];
    floatx4 sf[4][2], df[4][2];
    float graw = 0.f, braw = 0.f;               // wave NW - 1: g and beta of token t0 + l
    auto load_p1 = [&](int job) {
        const int bh = job / NT, c = job % NT, b = bh / H, h = bh % H, t0 = c * C;
        const size_t so = ((((size_t)bh * NT + c) * nvs + ws) * 64 + l) * NTT;
        const floatx4 *rp = reinterpret_cast<const floatx4 *>(args.rst) + so;
        const floatx4 *xp = reinterpret_cast<const floatx4 *>(ba.dxst) + so;
        const u16 *tg = reinterpret_cast<const u16 *>(args.tmat) + ((size_t)bh * NT + c) * C * C;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            rr[tt] = rp[tt];
            xr[tt] = xp[tt];
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                if (2 * m <= tt) tf[tt][m] = ld8(tg + (tt * 16 + c16) * C + (4 * m + g) * 8);
        if (w == S::NW - 1) {
            const int t = t0 + l;
            const bool ok = t < T;
            const size_t gi = ((size_t)b * T + (ok ? t : 0)) * H + h;
            graw = ok ? args.g[gi] : 0.f;
            braw = ok ? args.beta[gi * args.bst + args.boff] : 0.f;
        }
        if constexpr (DPE) {
            // the second pass's v' gradient of this wave's value slice (rows
            // tt*16 + 4g + e, column 16 ws + c16) and the A~ fragments
            const float *dp = ba.dvprev + ((size_t)b * T * H + h) * Dv + 16 * ws + c16;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dvr[tt][e] = dp[(size_t)min(t0 + tt * 16 + 4 * g + e, T - 1) * tokv];
            const uint4 *ap = reinterpret_cast<const uint4 *>(args.atil) + ((size_t)bh * NT + c) * NLOW * 64 + l;
#pragma unroll
            for (int i = 0; i < NLOW; ++i) atf[i] = __builtin_bit_cast(u32x4, ap[i * 64]);
        }
    };
    // S and dS' as phase 3's A operands (lane (g, j): row f0 + j, value
    // columns 32 mv + 8 g .. +7): NP3 loads
    constexpr int NP3 = 16;
    auto load_p3 = [&](int job) {
        const int bh = job / NT, c = job % NT;
        const size_t sbase = (((size_t)bh * NT + c) * KD + (w < nfs ? f0 : 0) + c16) * Dv + 8 * g;
#pragma unroll
        for (int mv = 0; mv < 4; ++mv)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const size_t o = sbase + (mv < nmv ? 32 * mv + 4 * hh : 0);
                sf[mv][hh] = *reinterpret_cast<const floatx4 *>(args.sst + o);
                df[mv][hh] = *reinterpret_cast<const floatx4 *>(ba.dsst + o);
            }
    };
    {
        const int job = blockIdx.x;
        const int bh = job / NT, c = job % NT;
        const int b = bh / H, h = bh % H, t0 = c * C;
        const size_t rowk0 = ((size_t)b * T * H + h) * args.kst + args.koff, rowv0 = ((size_t)b * T * H + h) * Dv;
        const u16 *og = reinterpret_cast<const u16 *>(ba.dout) + rowv0;
        // ---- phase 0 ----
        // phase 1's operands, waited for before the barrier
        load_p1(job);
        asm volatile("" ::: "memory");
        {
            constexpr int NDK = S::SZ_KC / 1024, NDO = S::SZ_V / 1024;
            const u16 *kg = reinterpret_cast<const u16 *>(args.k) + rowk0;
            const u16 *qg = reinterpret_cast<const u16 *>(args.q) + rowk0;
            // K, Q and dO rows (NDW LDS-direct loads per wave), in flight
            // through the rest of phase 0 and phase 1
            constexpr int NDW = (2 * NDK + NDO) / S::NW;
            static_assert((2 * NDK + NDO) % S::NW == 0, "as many LDS-direct loads on every wave");
#pragma unroll
            for (int k = w; k < 2 * NDK + NDO; k += S::NW) {
                if (k < 2 * NDK) {
                    const int kk = k % NDK, pos = kk * 64 + l, r = pos / NKC, sc = pos % NKC;
                    const int t = t0 + r, pc = sc ^ kswz<NKC>(r);
                    const u16 *src = (k < NDK ? kg : qg) + (size_t)t * tokk + (pc << 3);
                    dma16(t < T ? static_cast<const void *>(src) : static_cast<const void *>(&kZero16),
                          (k < NDK ? Kc : Qc) + kk * 512);
                } else {
                    const int kk = k - 2 * NDK, pos = kk * 64 + l, r = pos / NPV, sc = pos % NPV;
                    const int t = t0 + r, pc = sc ^ kswz<NPV>(r);
                    dma16(t < T && pc * 8 < Dv ? static_cast<const void *>(og + (size_t)t * tokv + (pc << 3))
                                               : static_cast<const void *>(&kZero16),
                          dOc + kk * 512);
                }
            }
            asm volatile("" ::: "memory");
            // M1, M2 (all four arrays, 32 KiB) and the per-tile partial slots cleared
            {
                uint4 *z = reinterpret_cast<uint4 *>(smem + S::OFF_M1H);
                for (int i = tid; i < 4 * S::SZ_M / 16; i += S::NTHR) z[i] = uint4{0u, 0u, 0u, 0u};
                float *zf = reinterpret_cast<float *>(smem + S::OFF_ZERO);
                for (int i = tid; i < (S::OFF_ZEND - S::OFF_ZERO) / 4; i += S::NTHR) zf[i] = 0.f;
            }
            if (w == S::NW - 1) {
                float gs = graw;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(gs, off, 64);
                    if (l >= off) gs += y;
                }
                G2[l] = gs * LOG2E;
                Bt[l] = braw;
            }
            // phase 1's operands (older than the LDS-direct loads) complete
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt((NDW & 15) | ((NDW >> 4) << 14) | 0x0070);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }

        // ---- phase 1: value slice w ----
        if (w < nvs) {
            const int v0 = 16 * w;
            floatx4 bt[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                bt[tt] = *reinterpret_cast<const floatx4 *>(Bt + tt * 16 + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t0 + tt * 16 + 4 * g + e >= T) rr[tt][e] = xr[tt][e] = 0.f;
            }
            if constexpr (DPE) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (t0 + tt * 16 + 4 * g + e >= T) dvr[tt][e] = 0.f;
            }
            bf16x8 rh[2], rl[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) frag_split(rr[2 * m], rr[2 * m + 1], rh[m], rl[m]);
            floatx4 vn[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vn[tt][e] = bt[tt][e] * rr[tt][e];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (2 * m <= tt) {
                        vn[tt] = mfma32(tf[tt][m], rh[m], vn[tt]);
                        vn[tt] = mfma32(tf[tt][m], rl[m], vn[tt]);
                    }
            }
            // DPE: e = R - A~ Vn for dbeta (A~ tiles as A operands, Vn tiles as B
            // operands in their accumulator layout, both hi + lo)
            floatx4 ev[NTT];
            if constexpr (DPE) {
                shortx4 nh[NTT], nl[NTT];
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) split4(vn[tt], nh[tt], nl[tt]);
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    floatx4 u = zero4();
#pragma unroll
                    for (int ss = 0; ss <= tt; ++ss) {
                        const u32x4 f = atf[tt * (tt + 1) / 2 + ss];
                        const shortx4 ah = __builtin_bit_cast(shortx4, uint2{f[0], f[1]});
                        const shortx4 al = __builtin_bit_cast(shortx4, uint2{f[2], f[3]});
                        u = mfma16(ah, nh[ss], u);
                        u = mfma16(ah, nl[ss], u);
                        u = mfma16(al, nh[ss], u);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) ev[tt][e] = rr[tt][e] - u[e];
                }
            }
            const float mc = args.mcoef;
            float *dvp = ba.dv + rowv0 + v0 + c16;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = tt * 16 + 4 * g + e, t = t0 + r;
                    const float bx = bt[tt][e] * xr[tt][e];
                    // dV = beta dX (DPE: + dv'); the X rows hold dX (DPE: dR = beta dX + m dv')
                    float xs = xr[tt][e], pb;
                    if constexpr (DPE) {
                        if (t < T) dvp[(size_t)t * tokv] = bx + dvr[tt][e];
                        xs = bx + mc * dvr[tt][e];
                        pb = sum16(xr[tt][e] * ev[tt][e]);
                    } else {
                        if (t < T) dvp[(size_t)t * tokv] = bx;
                        pb = sum16(xr[tt][e] * rr[tt][e]);
                    }
                    if (c16 == 0) db1[w * C + r] = pb;
                    u16 hi, lo;
                    const int at = swz_at<NPV>(r, v0 + c16);
                    split1(vn[tt][e], hi, lo);
                    Vh[at] = hi;
                    Vl[at] = lo;
                    split1(xs, hi, lo);
                    Xh[at] = hi;
                    Xl[at] = lo;
                }
        }
        // S and dS' in flight through phase 2; the wait (at most NP3
        // outstanding, loads complete in issue order) covers the K, Q, dO rows
        asm volatile("" ::: "memory");
        load_p3(job);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((NP3 & 15) | ((NP3 >> 4) << 14) | 0x0070);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        // ---- phase 2: lower tiles of M1 (kind 0) and of dA, M2 (kind 1) ----
        for (int job = w; job < 20; job += S::NW) {
            const int kind = job / 10, idx = job % 10;
            const int ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0, tj = idx - ti * (ti + 1) / 2;
            const int ra = ti * 16 + c16, rb = tj * 16 + c16;   // this lane's A and B operand rows
            floatx4 x = zero4(), y = zero4();
            if (kind == 0) {
                // x = dO Vn^T, y = Q K^T
#pragma unroll
                for (int mv = 0; mv < 4; ++mv)
                    if (mv < nmv) {
                        const bf16x8 oa = row_frag<NPV>(dOc, ra, 32 * mv);
                        x = mfma32(oa, row_frag<NPV>(Vh, rb, 32 * mv), x);
                        x = mfma32(oa, row_frag<NPV>(Vl, rb, 32 * mv), x);
                    }
#pragma unroll
                for (int m = 0; m < NKS; ++m) y = mfma32(row_frag<NKC>(Qc, ra, 32 * m), row_frag<NKC>(Kc, rb, 32 * m), y);
            } else {
                // x = dX Vn^T (both hi + lo), y = K K^T
#pragma unroll
                for (int mv = 0; mv < 4; ++mv)
                    if (mv < nmv) {
                        const bf16x8 ah = row_frag<NPV>(Xh, ra, 32 * mv), al = row_frag<NPV>(Xl, ra, 32 * mv);
                        const bf16x8 bh_ = row_frag<NPV>(Vh, rb, 32 * mv), bl = row_frag<NPV>(Vl, rb, 32 * mv);
                        x = mfma32(ah, bh_, x);
                        x = mfma32(ah, bl, x);
                        x = mfma32(al, bh_, x);
                    }
#pragma unroll
                for (int m = 0; m < NKS; ++m) y = mfma32(row_frag<NKC>(Kc, ra, 32 * m), row_frag<NKC>(Kc, rb, 32 * m), y);
            }
            // accumulator: lane (g, j) holds rows t = 16 ti + 4g + e, column s = 16 tj + j
            const int s = tj * 16 + c16;
            const float g2s = G2[s];
            float wv[4], csum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = ti * 16 + 4 * g + e;
                const float gam = fast_exp2(fminf(G2[t] - g2s, 0.f));
                float mval, dbv = 0.f;
                if (kind == 0) {
                    mval = s <= t ? scale * x[e] * gam : 0.f;
                    wv[e] = mval * y[e];
                } else {
                    // DPE: x = dR Vn^T, and da is dB (beta already in dR)
                    const float da = s < t ? -x[e] : 0.f, bg = s < t ? y[e] * gam : 0.f, btt = DPE ? 1.f : Bt[t];
                    wv[e] = da * btt * bg;
                    mval = btt * da * gam;
                    dbv = da * bg;
                }
                u16 hi, lo;
                split1(mval, hi, lo);
                const int at = swz_at<NPM>(t, s);
                (kind == 0 ? M1h : M2h)[at] = hi;
                (kind == 0 ? M1l : M2l)[at] = lo;
                const float rs = sum16(wv[e]);
                if (!DPE && kind == 1) {
                    const float rb2 = sum16(dbv);
                    if (c16 == 0) db2[tj * C + t] = rb2;
                }
                if (c16 == 0) (kind == 0 ? gr1 : gr2)[tj * C + t] = rs;
                csum += wv[e];
            }
            csum = add_xor32(add_xor16(csum));
            if (g == 0) (kind == 0 ? gc1 : gc2)[ti * C + s] = csum;
        }
        lds_barrier();

        // ---- phase 3: key features f0 .. f0 + 15 ----
        if (w < nfs) {
            bf16x8 sh[4], sl[4], dh[4], dl[4];
            float sdot = 0.f;
#pragma unroll
            for (int mv = 0; mv < 4; ++mv) {
                frag_split(sf[mv][0], sf[mv][1], sh[mv], sl[mv]);
                frag_split(df[mv][0], df[mv][1], dh[mv], dl[mv]);
                if (mv < nmv)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sdot += sf[mv][hh][e] * df[mv][hh][e];
            }
            sdot = add_xor32(add_xor16(sum16(sdot)));
            if (l == 0) ss[w] = sdot;
            const float g2L = G2[C - 1];
            // K and Q as B operands (k = token, n = feature f0 + j), both 32-token steps
            bf16x8 kb[2], qb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                kb[m] = tr_frag<NKC>(Kc, 32 * m + 8 * g, f0);
                qb[m] = tr_frag<NKC>(Qc, 32 * m + 8 * g, f0);
            }
            // Every product is taken transposed (operands swapped): lane (g, j) then
            // holds features f0 + 4g + e of token 16 tt + j, one 16-byte store each
            float *dqp = ba.dq + rowk0 + f0 + 4 * g;
            float *dkp = ba.dk + rowk0 + f0 + 4 * g;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int ra = tt * 16 + c16;       // this lane's token row of the row fragments
                // dQ^T: a = S dO^T, bq = K^T M1^T
                floatx4 a = zero4(), bq = zero4();
#pragma unroll
                for (int mv = 0; mv < 4; ++mv)
                    if (mv < nmv) {
                        const bf16x8 oa = row_frag<NPV>(dOc, ra, 32 * mv);
                        a = mfma32(sh[mv], oa, a);
                        a = mfma32(sl[mv], oa, a);
                    }
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (m <= tt / 2) {
                        bq = mfma32(kb[m], row_frag<NPM>(M1h, ra, 32 * m), bq);
                        bq = mfma32(kb[m], row_frag<NPM>(M1l, ra, 32 * m), bq);
                    }
                // dK^T: c1 = Q^T M1 + K^T M2 + K^T M2^T, d1 = S dX^T, d2 = dS' Vn^T
                floatx4 c1 = zero4(), d1 = zero4(), d2 = zero4();
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (m >= tt / 2) {
                        c1 = mfma32(qb[m], tr_frag<NPM>(M1h, 32 * m + 8 * g, tt * 16), c1);
                        c1 = mfma32(qb[m], tr_frag<NPM>(M1l, 32 * m + 8 * g, tt * 16), c1);
                        c1 = mfma32(kb[m], tr_frag<NPM>(M2h, 32 * m + 8 * g, tt * 16), c1);
                        c1 = mfma32(kb[m], tr_frag<NPM>(M2l, 32 * m + 8 * g, tt * 16), c1);
                    }
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (m <= tt / 2) {
                        c1 = mfma32(kb[m], row_frag<NPM>(M2h, ra, 32 * m), c1);
                        c1 = mfma32(kb[m], row_frag<NPM>(M2l, ra, 32 * m), c1);
                    }
#pragma unroll
                for (int mv = 0; mv < 4; ++mv)
                    if (mv < nmv) {
                        const bf16x8 xh = row_frag<NPV>(Xh, ra, 32 * mv), xl = row_frag<NPV>(Xl, ra, 32 * mv);
                        d1 = mfma32(sh[mv], xh, d1);
                        d1 = mfma32(sl[mv], xh, d1);
                        d1 = mfma32(sh[mv], xl, d1);
                        const bf16x8 vh = row_frag<NPV>(Vh, ra, 32 * mv), vl = row_frag<NPV>(Vl, ra, 32 * mv);
                        d2 = mfma32(dh[mv], vh, d2);
                        d2 = mfma32(dl[mv], vh, d2);
                        d2 = mfma32(dh[mv], vl, d2);
                    }
                // token r = 16 tt + j, features f0 + 4g + e
                const int r = tt * 16 + c16, t = t0 + r;
                const uint2 q2 = *reinterpret_cast<const uint2 *>(Qc + swz_at<NKC>(r, f0 + 4 * g));
                const uint2 k2 = *reinterpret_cast<const uint2 *>(Kc + swz_at<NKC>(r, f0 + 4 * g));
                const floatx4 qv{__builtin_bit_cast(float, q2.x << 16), __builtin_bit_cast(float, q2.x & 0xffff0000u),
                                 __builtin_bit_cast(float, q2.y << 16), __builtin_bit_cast(float, q2.y & 0xffff0000u)};
                const floatx4 kv{__builtin_bit_cast(float, k2.x << 16), __builtin_bit_cast(float, k2.x & 0xffff0000u),
                                 __builtin_bit_cast(float, k2.y << 16), __builtin_bit_cast(float, k2.y & 0xffff0000u)};
                const float g2 = G2[r], gam = fast_exp2(g2), lam = fast_exp2(g2L - g2), btt = Bt[r];
                floatx4 dqo, dko;
                float p3 = 0.f, ps = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float qd = scale * gam * a[e];                  // dQ_dir
                    const float kr = -gam * (DPE ? 1.f : btt) * d1[e];   // dK_R
                    const float ks_ = lam * d2[e];                        // dK_S'
                    dqo[e] = qd + bq[e];
                    dko[e] = c1[e] + kr + ks_;
                    p3 += qd * qv[e] + kr * kv[e];
                    ps += ks_ * kv[e];
                }
                if (t < T) {
                    *reinterpret_cast<floatx4 *>(dqp + (size_t)t * tokk) = dqo;
                    *reinterpret_cast<floatx4 *>(dkp + (size_t)t * tokk) = dko;
                }
                // sums over the slice's 16 features: the lane's 4, then the 4 lane groups
                p3 = add_xor32(add_xor16(p3));
                ps = add_xor32(add_xor16(ps));
                if (g == 0) {
                    g3[w * C + r] = p3;
                    gS[w * C + r] = ps;
                }
            }
        }
        lds_barrier();

        // ---- phase 4: dbeta, dg ----
        if (w == 0) {
            const int r = l, t = t0 + r;
            float db = 0.f, dG = 0.f, gsum = 0.f;
            for (int i = 0; i < nvs; ++i) db += db1[i * C + r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (!DPE) db += db2[i * C + r];
                dG += gr1[i * C + r] - gc1[i * C + r] + gr2[i * C + r] - gc2[i * C + r];
            }
            float sst = 0.f;
            for (int i = 0; i < nfs; ++i) {
                dG += g3[i * C + r];
                gsum += gS[i * C + r];
                sst += ss[i];
            }
            dG -= gsum;
            float tot = gsum;
            tot = add_xor32(add_xor16(sum16(tot)));
            if (r == C - 1) dG += tot + fast_exp2(G2[C - 1]) * sst;
            // dg_t = sum over t' >= t of dG_t'
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(dG, off, 64);
                if (r + off < 64) dG += y;
            }
            if (t < T) {
                const size_t gi = ((size_t)b * T + t) * H + h;
                ba.dbeta[gi * args.bst + args.boff] = db;
                ba.dg[gi] = DPE ? ba.dg[gi] + dG : dG;   // DPE: the second pass's share is there
            }
        }
    }
}

}  // namespace gdn
