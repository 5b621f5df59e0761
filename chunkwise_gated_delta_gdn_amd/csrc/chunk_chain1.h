// Sequential state pass + output of the chunkwise gated delta rule, for bf16
// inputs with one step per token (msj19 "gated_deltaproduct" test.py with
// r = 1: gated_chunk_delta_rule_fwd_kernel_h and
// gated_chunk_linear_attn_fwd_kernel_o; T = (I + A)^-1 comes from
// chunk_solve_kernel in the work space).
//
// One workgroup per (batch, head, 16-column slice of the value dimension),
// 1 + C/16 waves, split by role outside the chunk loop (each role keeps only
// its own registers live):
//
//   wave 0 ("chain") owns the (KD x 16) fp32 state slice in MFMA
//   accumulators and runs the dependent part of every chunk in registers:
//       X = K S;  R = beta V - (beta e^G) X;  V_new = T R;
//       S <- e^{G_L} S + K^T diag(e^{G_L - G}) V_new.
//   An MFMA accumulator tile (lane l holds rows 4*(l/16)+e, column l%16) is
//   fed back as the B operand of the next product by reading the k index of
//   a 32-wide MFMA step in the order {4g..4g+3, 16+4g..16+4g+3} (g = l/16)
//   instead of 8g..8g+7; the A operand is read from LDS in the same order,
//   so the sum over k is unchanged.  It publishes V_new and the chunk-start
//   state to LDS in fp32 for the output waves.
//
//   waves 1..C/16 ("out"), one 16-token tile each: the output, transposed,
//   O^T = S_start^T Q^T e^G + V_new^T P^T (P, the causal intra-chunk scores,
//   comes from the solve kernel as ready MFMA fragments; the transposed
//   accumulator gives each lane 4 consecutive values of one token, one
//   16-byte store), and the staging of the next chunks: a register prefetch
//   one chunk ahead, then K and K^T (8x8 blocks transposed in registers), T,
//   beta V (transposed) and the gate tables committed to LDS.
//
// One workgroup barrier per chunk.  Iteration c: the chain processes chunk c
// and publishes its start state and V_new; the out waves write the output of
// chunk c-1 and stage chunk c+1.
#pragma once

#include <type_traits>

#include "chunk_kernels.h"

namespace gdn {

template <int KD, int C>
struct Chain1Shape {
    static constexpr int BV = 16;
    static constexpr int NTT = C / 16;        // token tiles = out waves
    static constexpr int NW = 1 + NTT;        // waves per workgroup
    static constexpr int NTHR = 64 * NW;
    static constexpr int NLD = 64 * NTT;      // loader threads
    static constexpr int NKS = KD / 32;       // 32-wide steps over the key dim
    static constexpr int NST = KD / 16;       // state row tiles
    static constexpr int NCS = C / 32;        // 32-wide steps over the tokens
    static constexpr int NB8 = (C / 8) * (KD / 8);   // 8x8 blocks of K per chunk
    static constexpr int SWM = C / 8 - 1;     // K^T chunk swizzle mask
    static constexpr int LDK = KD + 8;        // Ks  [C][KD]   bf16
    static constexpr int LDKT = C + 8;        // KsT [KD][C]   bf16, 16-byte chunks swizzled
    static constexpr int LDT = C + 8;         // Tb  [C][C]    bf16
    static constexpr int LDBV = C + 4;        // BVs [BV][C]   fp32, beta V transposed
    static constexpr int LDSF = KD + 4;       // St  [BV][KD]  fp32, S_start transposed
    static constexpr int LDVF = C + 4;        // Vn  [BV][C]   fp32, V_new transposed
    // gate table: beta e^G [C], G2 [C] (log2-scaled cumsum), e^G [C], e^{G_L-G} [C], e^{G_L}
    static constexpr int NGATE = 4 * C + 4;
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int SZ_KS = al(C * LDK * 2);
    static constexpr int SZ_KST = al(KD * LDKT * 2);
    static constexpr int SZ_TB = al(C * LDT * 2);
    static constexpr int SZ_BV = al(BV * LDBV * 4);
    static constexpr int SZ_GATE = al(NGATE * 4);
    static constexpr int SZ_ST = al(BV * LDSF * 4);
    static constexpr int SZ_VN = al(BV * LDVF * 4);
    // every buffer is double: index p = chunk & 1
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_KST = OFF_KS + 2 * SZ_KS;
    static constexpr int OFF_TB = OFF_KST + 2 * SZ_KST;
    static constexpr int OFF_BV = OFF_TB + 2 * SZ_TB;
    static constexpr int OFF_GATE = OFF_BV + 2 * SZ_BV;
    static constexpr int OFF_ST = OFF_GATE + 2 * SZ_GATE;
    static constexpr int OFF_VN = OFF_ST + 2 * SZ_ST;
    static constexpr int BYTES = OFF_VN + 2 * SZ_VN;
    static_assert(C % 32 == 0 && C <= 64 && KD % 32 == 0, "32-wide MFMA steps");
    static_assert(NB8 <= NLD, "one 8x8 block of K per loader thread");
    static_assert(2 * C <= NLD, "one 16-byte vector of the V slice per loader thread");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

// 8 bf16 of a k-contiguous row at k = base + {4g..4g+3, 16+4g..16+4g+3}: the
// permuted k order of an accumulator-fed B operand.
__device__ __forceinline__ bf16x8 ld_perm(const u16 *rowp, int base, int g) {
    const uint2 lo = *reinterpret_cast<const uint2 *>(rowp + base + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2 *>(rowp + base + 16 + 4 * g);
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}

// The same read from a K^T row whose 16-byte chunks are swizzled: chunk j of
// row r is stored at chunk j ^ ((r >> 3) & SWM).  `xr` = (r >> 3) & SWM.
__device__ __forceinline__ bf16x8 ld_perm_swz(const u16 *rowp, int base, int g, int xr) {
    const int c0 = ((base + 4 * g) >> 3) ^ xr, c1 = ((base + 16 + 4 * g) >> 3) ^ xr;
    const int o = 4 * (g & 1);
    const uint2 lo = *reinterpret_cast<const uint2 *>(rowp + c0 * 8 + o);
    const uint2 hi = *reinterpret_cast<const uint2 *>(rowp + c1 * 8 + o);
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}

// bf16 fragment of two accumulator tiles, in the permuted order (hi only).
__device__ __forceinline__ bf16x8 frag_hi(const floatx4 &t0, const floatx4 &t1) {
    return __builtin_bit_cast(bf16x8, uint4{cvt2_bf16(t0[0], t0[1]), cvt2_bf16(t0[2], t0[3]),
                                            cvt2_bf16(t1[0], t1[1]), cvt2_bf16(t1[2], t1[3])});
}
// hi and lo fragments of two accumulator tiles (permuted order), or of 8
// consecutive values (natural order).
__device__ __forceinline__ void frag_split(const floatx4 &t0, const floatx4 &t1, bf16x8 &hi, bf16x8 &lo) {
    uint4 h, o;
    split2_bf16(t0[0], t0[1], h.x, o.x);
    split2_bf16(t0[2], t0[3], h.y, o.y);
    split2_bf16(t1[0], t1[1], h.z, o.z);
    split2_bf16(t1[2], t1[3], h.w, o.w);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, o);
}
__device__ __forceinline__ void split4(const floatx4 &x, shortx4 &hi, shortx4 &lo) {
    uint2 h, o;
    split2_bf16(x[0], x[1], h.x, o.x);
    split2_bf16(x[2], x[3], h.y, o.y);
    hi = __builtin_bit_cast(shortx4, h);
    lo = __builtin_bit_cast(shortx4, o);
}

__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(shortx4 a, shortx4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Column e (0..7) of an 8x8 bf16 block held as 8 rows of 4 words: the values
// rows[0..7][e], packed as 4 words (v_perm_b32 picks one half of each of two
// words).
__device__ __forceinline__ u32x4 block_col(const u32x4 (&rows)[8], int e) {
    const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const int wd = e >> 1;
    u32x4 r;
    r.x = __builtin_amdgcn_perm(rows[1][wd], rows[0][wd], sel);
    r.y = __builtin_amdgcn_perm(rows[3][wd], rows[2][wd], sel);
    r.z = __builtin_amdgcn_perm(rows[5][wd], rows[4][wd], sel);
    r.w = __builtin_amdgcn_perm(rows[7][wd], rows[6][wd], sel);
    return r;
}

template <int KD, int C>
__global__ __launch_bounds__((1 + C / 16) * 64) void chunk_chain1_kernel(ChunkArgs args) {
    using S = Chain1Shape<KD, C>;
    constexpr int BV = S::BV, NTT = S::NTT, NKS = S::NKS, NST = S::NST, NCS = S::NCS, NLD = S::NLD;
    constexpr int LDK = S::LDK, LDKT = S::LDKT, LDT = S::LDT, LDBV = S::LDBV, LDSF = S::LDSF, LDVF = S::LDVF;
    constexpr int NB8 = S::NB8, SWM = S::SWM;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];

    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nvb = args.Dv / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vb = slot % nvb;
    const int bh = (slot / nvb) * 8 + xcd;      // all value slices of one head share an XCD
    if (bh >= args.B * args.H) return;
    const int b = bh / args.H, h = bh % args.H;
    const int v0 = vb * BV;
    const int T = args.T, H = args.H, Dv = args.Dv;
    const int NT = (T + C - 1) / C;
    const int tlast = T > 0 ? T - 1 : 0;

    auto Ks = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_KS + p * S::SZ_KS); };
    auto KsT = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_KST + p * S::SZ_KST); };
    auto Tb = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_TB + p * S::SZ_TB); };
    auto BVs = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_BV + p * S::SZ_BV); };
    auto gate = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_GATE + p * S::SZ_GATE); };
    auto St = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_ST + p * S::SZ_ST); };
    auto Vn = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_VN + p * S::SZ_VN); };

    if (w == 0) {
        // =================================================================
        // chain wave
        // =================================================================
        floatx4 Sreg[NST];
        auto publish_state = [&](int p) {      // S_start, fp32 [j][i]
            float *st = St(p);
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
                *reinterpret_cast<floatx4 *>(st + c16 * LDSF + ti * 16 + 4 * g) = Sreg[ti];
        };
#pragma unroll
        for (int ti = 0; ti < NST; ++ti) {
            Sreg[ti] = zero4();
            if (args.h0) {
                const float *hp = args.h0 + ((size_t)bh * KD) * Dv + v0 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[ti][e] = hp[(size_t)(ti * 16 + 4 * g + e) * Dv];
            }
        }
        __syncthreads();
        for (int c = 0; c < NT; ++c) {
            const int p = c & 1;
            const u16 *ks = Ks(p), *kt = KsT(p), *tb = Tb(p);
            const float *bv = BVs(p), *gp = gate(p);
            bf16x8 sb[NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m) sb[m] = frag_hi(Sreg[2 * m], Sreg[2 * m + 1]);
            // X = K S, then R = beta V - (beta e^G) X, per token tile
            floatx4 r[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                floatx4 x = zero4();
                const u16 *kr = ks + (tt * 16 + c16) * LDK;
#pragma unroll
                for (int m = 0; m < NKS; ++m) x = mfma32(ld_perm(kr, m * 32, g), sb[m], x);
                if (tt == 0) publish_state(p);   // S_start of chunk c, while the MFMAs run
                const floatx4 bvt = *reinterpret_cast<const floatx4 *>(bv + c16 * LDBV + tt * 16 + 4 * g);
                const floatx4 beg = *reinterpret_cast<const floatx4 *>(gp + tt * 16 + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) r[tt][e] = bvt[e] - beg[e] * x[e];
            }
            bf16x8 rh[NCS], rl[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) frag_split(r[2 * m], r[2 * m + 1], rh[m], rl[m]);
            // V_new = T R, published fp32 [j][s]; V~ = e^{G_L - G} V_new
            float *vnp = Vn(p);
            floatx4 vt4[NTT];
#pragma unroll
            for (int vt = 0; vt < NTT; ++vt) {
                floatx4 acc = zero4();
                const u16 *trow = tb + (vt * 16 + c16) * LDT;
#pragma unroll
                for (int m = 0; m < NCS; ++m) {
                    const bf16x8 ta = ld_perm(trow, m * 32, g);
                    acc = mfma32(ta, rh[m], acc);
                    acc = mfma32(ta, rl[m], acc);
                }
                *reinterpret_cast<floatx4 *>(vnp + c16 * LDVF + vt * 16 + 4 * g) = acc;
                const floatx4 el = *reinterpret_cast<const floatx4 *>(gp + 3 * C + vt * 16 + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) vt4[vt][e] = el[e] * acc[e];
            }
            bf16x8 vh[NCS], vl[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) frag_split(vt4[2 * m], vt4[2 * m + 1], vh[m], vl[m]);
            // S <- e^{G_L} S + K^T V~
            const float gL = gp[4 * C];
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                floatx4 acc = zero4();
                const u16 *krow = kt + (ti * 16 + c16) * LDKT;
                const int xr = ((ti * 16 + c16) >> 3) & SWM;
#pragma unroll
                for (int m = 0; m < NCS; ++m) {
                    const bf16x8 ka = ld_perm_swz(krow, m * 32, g, xr);
                    acc = mfma32(ka, vh[m], acc);
                    acc = mfma32(ka, vl[m], acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[ti][e] = gL * Sreg[ti][e] + acc[e];
            }
            __syncthreads();
        }
        __syncthreads();                       // matches the out waves' drain step
        if (args.hT) {
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                float *hp = args.hT + ((size_t)bh * KD) * Dv + v0 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e) hp[(size_t)(ti * 16 + 4 * g + e) * Dv] = Sreg[ti][e];
            }
        }
        return;
    }

    // =====================================================================
    // out waves
    // =====================================================================
    // Each out wave runs a copy of the loop specialised for its token tile
    // OW (wave 1: the last tile) and its loader roles, so that its global
    // loads are straight-line code: the hardware counter of outstanding loads
    // is in order, and a load skipped on some path would make the compiler
    // wait for every load issued after the one it needs.
    //
    // Loader roles: threads [0, NB8) stage one 8x8 block of K each; wave VW
    // the V slice (C/32 16-byte vectors per lane) and the gate table; every
    // thread C/32 vectors of T.  The last wave (the lightest output tile)
    // runs slowest when C = 64 (five waves on four SIMDs: it shares one with
    // the chain wave), so it only loads T.
    constexpr int NTV = C * C / 8;              // 16-byte vectors of T
    constexpr int PT = NTV / NLD;
    constexpr int PV = C / 32;                  // V vectors per lane of wave VW
    constexpr int VW = NTT >= 3 ? 3 : NTT;
    constexpr int NLOW = NTT * (NTT + 1) / 2;
    static_assert(PT * NLD == NTV && PV * 64 == 2 * C, "loader split");
    const int ltid = tid - 64;                  // loader thread index
    const bool kload = ltid < NB8;
    const int kb8 = kload ? ltid % (KD / 8) : 0, tb8 = kload ? ltid / (KD / 8) : 0;
    const size_t tokq = (size_t)H * KD, tokv = (size_t)H * Dv;
    const u16 *kg = reinterpret_cast<const u16 *>(args.k) + ((size_t)b * T * H + h) * KD;
    const u16 *qg = reinterpret_cast<const u16 *>(args.q) + ((size_t)b * T * H + h) * KD;
    const u16 *vg = reinterpret_cast<const u16 *>(args.v) + ((size_t)b * T * H + h) * Dv + v0;
    const u16 *tg = reinterpret_cast<const u16 *>(args.tmat) + (size_t)bh * NT * C * C;
    const float *betag = args.beta + (size_t)b * T * H + h, *gg = args.g + (size_t)b * T * H + h;

    auto out_wave = [&](auto owc) {
        constexpr int OW = decltype(owc)::value;
        constexpr int WV = NTT - OW;            // this wave's index
        constexpr bool KW = (WV - 1) * 64 < NB8, VWV = WV == VW;
        // Rows past T are clamped to T-1 (and zeroed when committed); a chunk
        // index past the end is clamped to the last chunk (its staging then
        // lands in a buffer no one reads).
        u32x4 rk[8], rt[PT], rv[PV];
        float rbv[PV], rbeta = 0.f, rg = 0.f;
        auto prefetch = [&](int c) {
            c = min(c, NT - 1);
            const int t0 = c * C;
            if constexpr (KW) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = min(t0 + tb8 * 8 + j, tlast);
                    rk[j] = *reinterpret_cast<const u32x4 *>(kg + (size_t)t * tokq + kb8 * 8);
                }
            }
#pragma unroll
            for (int q = 0; q < PT; ++q)
                rt[q] = reinterpret_cast<const u32x4 *>(tg + (size_t)c * C * C)[ltid + NLD * q];
            if constexpr (VWV) {
#pragma unroll
                for (int q = 0; q < PV; ++q) {
                    const int vidx = l + 64 * q;
                    const int t = min(t0 + vidx % C, tlast);
                    rv[q] = *reinterpret_cast<const u32x4 *>(vg + (size_t)t * tokv + (vidx / C) * 8);
                    rbv[q] = betag[(size_t)t * H];
                }
                const int tt = min(t0 + l, tlast);
                rbeta = betag[(size_t)tt * H];
                rg = gg[(size_t)tt * H];
            }
        };
        auto commit = [&](int c) {
            const int p = c & 1, t0 = c * C;
            u16 *ks = Ks(p), *kt = KsT(p), *tb = Tb(p);
            float *bv = BVs(p), *gp = gate(p);
            if constexpr (KW) {
                if (kload) {
                    u32x4 rows[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        rows[j] = (t0 + tb8 * 8 + j < T) ? rk[j] : u32x4{0u, 0u, 0u, 0u};
                        *reinterpret_cast<u32x4 *>(ks + (tb8 * 8 + j) * LDK + kb8 * 8) = rows[j];
                    }
                    // row kb8*8+e of K^T: chunk tb8 stored at tb8 ^ (kb8 & SWM)
                    u16 *ktb = kt + (kb8 * 8) * LDKT + ((tb8 ^ (kb8 & SWM)) * 8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4 *>(ktb + e * LDKT) = block_col(rows, e);
                }
            }
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                const int idx = ltid + NLD * q;
                const int i = idx / (C / 8), cv = idx % (C / 8);
                *reinterpret_cast<u32x4 *>(tb + i * LDT + cv * 8) = rt[q];
            }
            if constexpr (VWV) {
#pragma unroll
                for (int q = 0; q < PV; ++q) {  // beta V, transposed to [j][t]
                    const int vidx = l + 64 * q, vtok = vidx % C, vcv = vidx / C;
                    const float bt = (t0 + vtok < T) ? rbv[q] : 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t wv = rv[q][e >> 1];
                        bv[(vcv * 8 + e) * LDBV + vtok] =
                            bt * bf16_to_f32((u16)((e & 1) ? (wv >> 16) : (wv & 0xffffu)));
                    }
                }
                // the cumsum and the gate table
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
                    const float eg = fast_exp2(g2);
                    gp[l] = (ok ? rbeta : 0.f) * eg;         // beta e^{G_t}
                    gp[C + l] = g2;                          // G2
                    gp[2 * C + l] = eg;                      // e^{G_t}
                    gp[3 * C + l] = fast_exp2(g2l - g2);     // e^{G_L - G_t}
                }
                if (l == 0) gp[4 * C] = fast_exp2(g2l);     // e^{G_L}
            }
        };

        bf16x8 qf[NKS];                         // Q fragments (B operand, token = lane%16)
        u32x4 pf[OW + 1];                       // P fragments of row tile OW: {hi01, hi23, lo01, lo23}
        float egt = 0.f;                        // e^{G_t} of this lane's token
        floatx4 ov = zero4();                   // output of the previous chunk
        const uint4 *pfg = reinterpret_cast<const uint4 *>(args.pfrag) + (size_t)bh * NT * NLOW * 64 +
                           (OW * (OW + 1) / 2) * 64 + l;
        // operands of chunk c's output, used one iteration later
        auto load_qp = [&](int c) {
            const int t = min(c * C + OW * 16 + c16, tlast);   // rows past T are never stored
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                qf[m] = *reinterpret_cast<const bf16x8 *>(qg + (size_t)t * tokq + m * 32 + 8 * g);
            const uint4 *pc = pfg + (size_t)c * NLOW * 64;
#pragma unroll
            for (int tj = 0; tj <= OW; ++tj) pf[tj] = __builtin_bit_cast(u32x4, pc[tj * 64]);
            egt = gate(c & 1)[2 * C + OW * 16 + c16];
        };
        // O^T of chunk c: a1 = S_start^T Q^T, a2 = V_new^T P^T (buffers c & 1)
        auto compute_out = [&](int c) {
            const float *st = St(c & 1), *vnp = Vn(c & 1);
            floatx4 a1 = zero4(), a2 = zero4();
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                const floatx4 s0 = *reinterpret_cast<const floatx4 *>(st + c16 * LDSF + m * 32 + 8 * g);
                const floatx4 s1 = *reinterpret_cast<const floatx4 *>(st + c16 * LDSF + m * 32 + 8 * g + 4);
                bf16x8 sh, sl;
                frag_split(s0, s1, sh, sl);
                a1 = mfma32(sh, qf[m], a1);
                a1 = mfma32(sl, qf[m], a1);
            }
#pragma unroll
            for (int tj = 0; tj <= OW; ++tj) {
                shortx4 vh4, vl4;
                split4(*reinterpret_cast<const floatx4 *>(vnp + c16 * LDVF + tj * 16 + 4 * g), vh4, vl4);
                const shortx4 ph = __builtin_bit_cast(shortx4, uint2{pf[tj][0], pf[tj][1]});
                const shortx4 pl = __builtin_bit_cast(shortx4, uint2{pf[tj][2], pf[tj][3]});
                a2 = mfma16(vh4, ph, a2);
                a2 = mfma16(vh4, pl, a2);
                a2 = mfma16(vl4, ph, a2);
            }
            const float sc = args.scale;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = sc * (egt * a1[e] + a2[e]);
        };
        auto store_out = [&](int c) {
            const int tt = c * C + OW * 16 + c16;
            if (tt < T) {
                const size_t off = (((size_t)b * T + tt) * H + h) * Dv + v0 + 4 * g;
                if (args.out_bf16)
                    *reinterpret_cast<uint2 *>(reinterpret_cast<u16 *>(args.o) + off) =
                        uint2{cvt2_bf16(ov[0], ov[1]), cvt2_bf16(ov[2], ov[3])};
                else
                    *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(args.o) + off) = ov;
            }
        };

        // Iteration c (one barrier each): output of chunk c-1, operands of
        // chunk c, commit of chunk c+1, prefetch of chunk c+2.
        prefetch(0);
        commit(0);
        prefetch(1);
        __syncthreads();
        load_qp(0);
        commit(1);
        prefetch(2);
        __syncthreads();
        for (int c = 1; c < NT; ++c) {
            compute_out(c - 1);
            load_qp(c);
            commit(c + 1);
            prefetch(c + 2);
            store_out(c - 1);
            __syncthreads();
        }
        compute_out(NT - 1);
        store_out(NT - 1);
        __syncthreads();
    };
    if (NT == 0) {                              // no chunks: match the chain wave's two barriers
        __syncthreads();
        __syncthreads();
        return;
    }
    const int ow = NTT - w;                     // token tile of this wave (wave 1: the last)
    if (ow == 0) out_wave(std::integral_constant<int, 0>{});
    if (ow == 1) out_wave(std::integral_constant<int, 1>{});
    if constexpr (NTT == 4) {
        if (ow == 2) out_wave(std::integral_constant<int, 2>{});
        if (ow == 3) out_wave(std::integral_constant<int, 3>{});
    }
}

}  // namespace gdn
