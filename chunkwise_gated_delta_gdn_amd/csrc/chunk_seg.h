// Segment-parallel state pass + output of the chunkwise gated delta rule,
// for bf16 inputs, one step per token, 64-token chunks (msj19
// "gated_deltaproduct" test.py with r = 1: gated_chunk_delta_rule_fwd_kernel_h
// and gated_chunk_linear_attn_fwd_kernel_o; T diag(beta), the P tiles and
// the gate tables come from chunk_prep2_kernel in the work space).
//
// The chunks of one (batch, head) are cut into P segments of LS chunks.  The
// state after a segment is affine in the state before it (Sana
// "fused_gdn_cp.py", module docstring: the per-step transitions compose), so
//   S_{p+1} = A_p S_p + B_p,
// with A_p the segment's transition (Dk x Dk: the chunk steps run on the
// identity with zero values) and B_p its state from zero (from h0 for p = 0).
// Three launches after the prep:
//   summaries  (parallel over segments) B_0 from h0, and A_p, B_p for
//              p = 1 .. P-2;
//   compose    (sequential over segments, parallel over heads and 32-column
//              slices) S_1 = B_0, S_{p+1} = A_p S_p + B_p, written over B_p;
//   output     (parallel over segments) every segment again from its true
//              start state, with the output of each chunk; the last one
//              writes hT.
// With P = 1 only the output launch runs.
//
// One workgroup per (batch, head, segment, 128-column group): eight waves,
// two per SIMD (so each SIMD interleaves two independent chains), wave w
// owning the 16-column slice w of the state (of V's columns, or of A's
// columns for the transition).  The waves share one staging of each chunk's
// K rows, T diag(beta), gate table and V columns (LDS-direct loads).  The state slice lives in MFMA
// accumulators, as in chunk_chain1_kernel (same algebra: V_new = T diag(beta)
// (V - e^G K S), S <- e^{G_L} S + K^T (e^{G_L-G} V_new)).  The output of a
// chunk, O^T = S_start^T Q^T e^G + V_new^T P^T, is computed by the same wave
// from its registers: the bf16 fragments of S_start that feed K S are the A
// operand of S_start^T Q^T, and V_new's accumulator tiles are the A operand
// of V_new^T P^T, so nothing is published through LDS; Q rows and the P
// fragments are staged with the chunk.  Two staging buffers: iteration c
// stores the output of chunk c-1 (kept in registers), issues chunk c+1's
// loads, computes chunk c, waits for its loads (vmcnt(0): the stores went
// out an iteration earlier) and meets the other waves at one barrier.
#pragma once

#include "chunk_chain1.h"

namespace gdn {

struct SegArgs {
    ChunkArgs a;
    float *amat;     // [B*H][P][KD][KD]   transition of segment p (p = 1 .. P-2)
    float *bmat;     // [B*H][P][KD][Dv]   state after segment p from zero (from h0 for p = 0);
                     //                    compose overwrites entry p with the start state of p + 1
    int P, LS;       // segments per (b, h), chunks per segment (the last may be shorter)
    int nseg_units;  // summary launch: units (b*h, segment) in the grid
};

template <int KD>
struct SegShape {
    static constexpr int C = 64, BV = 16, NS = 1, NW = 8, NTHR = 64 * NW;
    static constexpr int CG = NW * NS * BV;   // 128 columns per workgroup
    static constexpr int NTT = C / 16, NKS = KD / 32, NST = KD / 16, NCS = C / 32;
    static constexpr int NKC = KD / 8;        // 16-byte pieces of a K (or Q) row
    static constexpr int NVC = CG / 8;        // 16-byte pieces of a staged V row
    static constexpr int TSW = C / 8 - 1;     // T diag(beta) swizzle mask
    static constexpr int NGATE = gate_table_len<C>();
    static constexpr int NLOW = NTT * (NTT + 1) / 2;
    static constexpr int al1k(int x) { return (x + 1023) & ~1023; }
    static constexpr int SZ_K = C * KD * 2;
    static constexpr int SZ_T = C * C * 2;
    static constexpr int SZ_G = al1k(NGATE * 4);
    static constexpr int SZ_V = C * CG * 2;
    static constexpr int SZ_Q = C * KD * 2;
    static constexpr int SZ_P = NLOW * 1024;
    // staging buffer b (of 2): K, T diag(beta), gates, V (and Q, P for the output)
    static constexpr int OFF_K = 0, OFF_T = SZ_K, OFF_G = OFF_T + SZ_T, OFF_V = OFF_G + SZ_G;
    static constexpr int OFF_Q = OFF_V + SZ_V, OFF_P = OFF_Q + SZ_Q;
    static constexpr int SZ_STAGE_SUM = OFF_Q, SZ_STAGE_OUT = OFF_P + SZ_P;
    static constexpr int BYTES_OUT = 2 * SZ_STAGE_OUT;
    static constexpr int BYTES_SUM = 2 * SZ_STAGE_SUM;
    // 1 KiB wave loads per staged chunk
    static constexpr int NDK = SZ_K / 1024, NDT = SZ_T / 1024, NDV = SZ_V / 1024;
    static constexpr int NDS = NDK + NDT + 1 + NDV;   // + one (partial) gate-table load
    static constexpr int NDQ = SZ_Q / 1024, NDP = SZ_P / 1024, NDQP = NDQ + NDP;
    static_assert(KD % 32 == 0 && KD <= 128, "key width of the segment pass");
    static_assert(SZ_K % 1024 == 0 && SZ_V % 1024 == 0, "whole 1 KiB wave loads");
    static_assert(BYTES_OUT <= 160 * 1024, "LDS budget");
    static_assert(NGATE * 4 <= 1024, "gate table: one partial wave load");
};

// Stored position of 16-byte piece j of staged V row r (XOR by 2*(r%8): the
// 8-byte transposed reads of 32 lanes, rows r0..r0+7 at one pair of pieces,
// then touch 16 distinct pieces, all 64 banks once).
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 7); }

// mode: 0 output (true start state; o, and hT for the last segment);
//       1 summaries (B_p: V from the input, start from h0 (p = 0) or zero;
//         A_p: zero values, start from the identity columns)
template <int KD, bool OUT>
__global__ __launch_bounds__(512) void chunk_seg_kernel(SegArgs sa) {
    using S = SegShape<KD>;
    constexpr int C = S::C, BV = S::BV, NS = S::NS, NW = S::NW, CG = S::CG;
    constexpr int NTT = S::NTT, NKS = S::NKS, NST = S::NST, NCS = S::NCS, NKC = S::NKC;
    constexpr int TSW = S::TSW, NLOW = S::NLOW;
    constexpr int NDK = S::NDK, NDT = S::NDT, NDS = S::NDS, NDQ = S::NDQ, NDQP = S::NDQP;
    __shared__ __attribute__((aligned(16))) unsigned char smem[OUT ? S::BYTES_OUT : S::BYTES_SUM];

    const ChunkArgs &a = sa.a;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, H = a.H, Dv = a.Dv, kw = a.kw, P = sa.P;
    const int NT = (T + C - 1) / C;

    // ---- which (b, h, segment, part, column group) ----
    int bh, seg, isA = 0, cg;
    if constexpr (OUT) {
        const int ncg = (Dv + CG - 1) / CG;
        cg = blockIdx.x % ncg;
        const int u = blockIdx.x / ncg;
        bh = u / P;
        seg = u % P;
    } else {
        // block = (slot, xcd) with xcd = block % 8; unit u = (slot / ncg) * 8 +
        // xcd and part/column group j = slot % ncg, so every workgroup of a
        // unit runs on one XCD (its K, T diag(beta) and gates in one L2)
        const int ncgv = (Dv + CG - 1) / CG, ncga = (KD + CG - 1) / CG, ncg = ncgv + ncga;
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int u = (slot / ncg) * 8 + xcd, j = slot % ncg;
        if (u >= sa.nseg_units) return;
        // unit 0 .. BH-1: segment 0 (B only); then (bh, p) for p = 1 .. P-2
        if (u < a.B * H) {
            bh = u;
            seg = 0;
        } else {
            bh = (u - a.B * H) / (P - 2);
            seg = 1 + (u - a.B * H) % (P - 2);
        }
        isA = j >= ncgv;
        cg = isA ? j - ncgv : j;
        if (seg == 0 && isA) return;
    }
    const int b = bh / H, h = bh % H;
    const int c0 = seg * sa.LS, c1 = min(NT, c0 + sa.LS);
    int vcol[NS];                                 // first column of each slice (>= ncols: idle)
#pragma unroll
    for (int s = 0; s < NS; ++s) vcol[s] = cg * CG + (w * NS + s) * BV;
    const int tlast = T > 0 ? T - 1 : 0;

    constexpr int SZB = OUT ? S::SZ_STAGE_OUT : S::SZ_STAGE_SUM;
    auto Ks = [&](int p) { return reinterpret_cast<u16 *>(smem + p * SZB + S::OFF_K); };
    auto Tb = [&](int p) { return reinterpret_cast<u16 *>(smem + p * SZB + S::OFF_T); };
    auto Gt = [&](int p) { return reinterpret_cast<float *>(smem + p * SZB + S::OFF_G); };
    auto Vs = [&](int p) { return reinterpret_cast<u16 *>(smem + p * SZB + S::OFF_V); };
    auto Qs = [&](int p) { return reinterpret_cast<u16 *>(smem + p * SZB + S::OFF_Q); };
    auto Ps = [&](int p) { return reinterpret_cast<uint4 *>(smem + p * SZB + S::OFF_P); };

    const int tokq = H * kw, tokv = H * Dv;       // element strides of one token row
    const u16 *kg = reinterpret_cast<const u16 *>(a.k) + ((size_t)b * T * H + h) * kw;
    const u16 *qg = reinterpret_cast<const u16 *>(a.q) + ((size_t)b * T * H + h) * kw;
    const u16 *vg = reinterpret_cast<const u16 *>(a.v) + ((size_t)b * T * H + h) * Dv;
    const u16 *tg = reinterpret_cast<const u16 *>(a.tmat) + (size_t)bh * NT * C * C;
    const float *gtg = reinterpret_cast<const float *>(a.gtab) + (size_t)bh * NT * S::NGATE;
    const uint4 *pg = reinterpret_cast<const uint4 *>(a.pfrag) + (size_t)bh * NT * NLOW * 64;
    const int vbase = cg * CG;                    // first V column staged by this workgroup

    // ---- staging of chunk c (clamped to the segment) into buffer p.  Load k
    //      of the list runs on wave k % 4; slot kk = k - k0 of a kind that
    //      starts at list index k0 then has kk % 4 = (w - k0) % 4 on every
    //      load of the wave.  K and Q rows are 4 kk + l/16 (16 pieces of 16
    //      bytes a row, swizzle kswz(r) = 4 (r % 4) + (r / 4) % 4 =
    //      4 (l/16) + kk % 4), V rows alike (vswz(r) = 2 (r % 8) =
    //      2 (4 (kk % 2) + l/16)), T diag(beta) rows 8 kk + l/8 (swizzle
    //      l/8): each lane's offset is a per-wave constant plus a multiple of
    //      the row stride common to the wave.
    //      Token rows past T (the last chunk only) are clamped (they meet
    //      zero columns of T diag(beta) and zero gates); K and Q pieces past
    //      kw and V pieces past Dv come from a 16-byte zero ----
    const int la = l >> 4, lsc = l & 15;
    constexpr int K0_V = NDK + NDT + 1;
    const int kpc = NKC == 16 ? (lsc ^ ((la << 2) | (w & 3))) : 0;           // K piece (KD = 128)
    const int qpc = NKC == 16 ? (lsc ^ ((la << 2) | ((w - NDS) & 3))) : 0;   // Q piece
    const int vpc = lsc ^ (2 * (4 * ((w - K0_V) & 1) + la));                  // V piece
    const bool kpad = kpc * 8 >= kw, qpad = qpc * 8 >= kw;
    const int koff = kpad ? 0 : kpc * 8, qoff = qpad ? 0 : qpc * 8;         // in-row offsets
    const int vcol0 = vbase + vpc * 8;
    const bool vpad = isA || vcol0 >= Dv;
    const int tpc = (l & 7) ^ (l >> 3);                                      // T diag(beta) piece
    auto stage = [&](int c, int p) __attribute__((always_inline)) {
        c = min(c, c1 - 1);
        const bool tail = c * C + C - 1 > tlast;  // rows past T: clamp them
        const int rmax = tlast - c * C;
        const u16 *kc = kg + (size_t)c * C * tokq, *qc = qg + (size_t)c * C * tokq;
        const u16 *vc = vg + (size_t)c * C * tokv;
        const u16 *tc = tg + (size_t)c * C * C;
        const float *gc = gtg + (size_t)c * S::NGATE;
        const uint4 *pc_ = pg + (size_t)c * NLOW * 64;
        constexpr int NQ = OUT ? NDQP : 0;
        constexpr int NTOT = NDS + NQ;
#pragma unroll
        for (int k = 0; k < NTOT; ++k) {
            if (k % NW != w) continue;
            if (k < NDK || (k >= NDS && k < NDS + NDQ)) {          // K or Q row pieces
                const bool isq = k >= NDS;
                const int kk = isq ? k - NDS : k;
                int r, off;
                bool pad;
                if constexpr (NKC == 16) {
                    r = 4 * kk + la;
                    off = isq ? qoff : koff;
                    pad = isq ? qpad : kpad;
                } else {
                    const int pos = kk * 64 + l, sc = pos % NKC;
                    r = pos / NKC;
                    const int pc = sc ^ kswz<NKC>(r);
                    pad = pc * 8 >= kw;
                    off = pad ? 0 : pc * 8;
                }
                if (tail) r = min(r, rmax);
                const u16 *src = (isq ? qc : kc) + (r * tokq + off);
                dma16(pad ? static_cast<const void *>(&kZero16) : static_cast<const void *>(src),
                      (isq ? Qs(p) : Ks(p)) + kk * 512);
            } else if (k < NDK + NDT) {
                const int kk = k - NDK;
                dma16(tc + ((8 * kk + (l >> 3)) * C + (tpc << 3)), Tb(p) + kk * 512);
            } else if (k == NDK + NDT) {
                if (l < S::NGATE / 4) dma16(gc + l * 4, Gt(p));
            } else if (k < NDS) {
                if (!isA) {                                        // V columns (the transition has none)
                    const int kk = k - NDK - NDT - 1;
                    int r = 4 * kk + la;
                    if (tail) r = min(r, rmax);
                    dma16(vpad ? static_cast<const void *>(&kZero16) : static_cast<const void *>(vc + (r * tokv + vcol0)),
                          Vs(p) + kk * 512);
                }
            } else {                                               // P fragments
                const int kk = k - NDS - NDQ;
                dma16(pc_ + (kk * 64 + l), Ps(p) + kk * 64);
            }
        }
    };

    // ---- state slices in MFMA accumulators: tile ti = 2 mk + hh, row 4 g + e
    //      holds key feature 32 mk + 8 g + 4 hh + e (as in chunk_chain1_kernel) ----
    auto feat = [&](int ti, int e) { return (ti >> 1) * 32 + 8 * g + 4 * (ti & 1) + e; };
    floatx4 Sreg[NS][NST];
    {
        const float *src = nullptr;
        size_t rs = 0;                            // row stride of src
        int rows = 0;                             // rows of src (past them: zero)
        if (isA) {
            // identity columns
        } else if (seg == 0) {
            src = a.h0 ? a.h0 + (size_t)bh * kw * Dv : nullptr;
            rs = Dv;
            rows = kw;
        } else if (OUT) {
            src = sa.bmat + ((size_t)bh * P + seg - 1) * KD * Dv;
            rs = Dv;
            rows = KD;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                Sreg[s][ti] = zero4();
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = feat(ti, e), col = vcol[s] + c16;
                    if (isA) Sreg[s][ti][e] = f == col && f < kw ? 1.f : 0.f;
                    else if (src && f < rows && col < Dv) Sreg[s][ti][e] = src[(size_t)f * rs + col];
                }
            }
    }

    const int nc = c1 - c0;
    if (nc > 0) stage(c0, 0);
    __builtin_amdgcn_s_waitcnt(0x3F70);          // vmcnt(0)
    __syncthreads();

    floatx4 ov[NS][NTT];                          // output of the previous chunk, stored one iteration later
    auto store_out = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int ti = 0; ti < NTT; ++ti) {
            const int t = c * C + ti * 16 + c16;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (t < T && vcol[s] < Dv) {
                    const size_t off = (((size_t)b * T + t) * H + h) * Dv + vcol[s] + 4 * g;
                    if (a.out_bf16)
                        *reinterpret_cast<uint2 *>(reinterpret_cast<u16 *>(a.o) + off) =
                            uint2{cvt2_bf16(ov[s][ti][0], ov[s][ti][1]), cvt2_bf16(ov[s][ti][2], ov[s][ti][3])};
                    else
                        *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(a.o) + off) = ov[s][ti];
                }
        }
    };

    for (int i = 0; i < nc; ++i) {
        const int c = c0 + i, pb = i & 1;
        if constexpr (OUT)
            if (i > 0) store_out(c - 1);
        stage(c + 1, pb ^ 1);

        const u16 *ks = Ks(pb), *tb = Tb(pb), *bvs = Vs(pb);
        const float *gp = Gt(pb);
        // S_start fragments (hi; lo for the output)
        bf16x8 sb[NS][NKS], sl[NS][NKS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                if constexpr (OUT) frag_split(Sreg[s][2 * m], Sreg[s][2 * m + 1], sb[s][m], sl[s][m]);
                else sb[s][m] = frag_hi(Sreg[s][2 * m], Sreg[s][2 * m + 1]);
            }
        // ---- Y = K S, K row fragments per 32-wide key step ----
        floatx4 y[NS][NTT];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) y[s][tt] = zero4();
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
            bf16x8 kf[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int r = tt * 16 + c16;
                kf[tt] = ld8(ks + r * KD + (((4 * m + g) ^ kswz<NKC>(r)) << 3));
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int s = 0; s < NS; ++s) y[s][tt] = mfma32(kf[tt], sb[s][m], y[s][tt]);
        }
        // ---- R = V - e^G Y;  V_new = beta R + T' R ----
        floatx4 rr[NS][NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const floatx4 eg = *reinterpret_cast<const floatx4 *>(gp + tt * 16 + 4 * g);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float vx[4] = {0.f, 0.f, 0.f, 0.f};
                if (!isA) {
                    const int vcl = vcol[s] - vbase + 4 * (c16 & 3);   // column inside the staged rows
                    const int r = tt * 16 + 4 * g + (c16 >> 2);
                    const uint2 v2 = __builtin_bit_cast(uint2, ld_tr16(bvs + r * CG + (((vcl >> 3) ^ vswz(r)) << 3) + (vcl & 7)));
                    vx[0] = __builtin_bit_cast(float, v2.x << 16);
                    vx[1] = __builtin_bit_cast(float, v2.x & 0xffff0000u);
                    vx[2] = __builtin_bit_cast(float, v2.y << 16);
                    vx[3] = __builtin_bit_cast(float, v2.y & 0xffff0000u);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) rr[s][tt][e] = vx[e] - eg[e] * y[s][tt][e];
            }
        }
        bf16x8 rh[NS][NCS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int m = 0; m < NCS; ++m) rh[s][m] = frag_hi(rr[s][2 * m], rr[s][2 * m + 1]);
        floatx4 vn[NS][NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const floatx4 bt = *reinterpret_cast<const floatx4 *>(gp + 2 * C + 4 + tt * 16 + 4 * g);
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) vn[s][tt][e] = bt[e] * rr[s][tt][e];
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int m = 0; m < NCS; ++m)
                if (2 * m <= tt) {
                    const bf16x8 tf = ld8(tb + (tt * 16 + c16) * C + (((4 * m + g) ^ ((tt * 16 + c16) & TSW)) << 3));
#pragma unroll
                    for (int s = 0; s < NS; ++s) vn[s][tt] = mfma32(tf, rh[s][m], vn[s][tt]);
                }

        if constexpr (OUT) {
            // ---- output of chunk c: O^T = S_start^T Q^T e^G + V_new^T P^T ----
            const u16 *qs = Qs(pb);
            const uint4 *ps = Ps(pb);
            const float sc = a.scale;
            shortx4 nh[NS][NTT], nl[NS][NTT];   // V_new as the A operand of V_new^T P^T
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) split4(vn[s][tt], nh[s][tt], nl[s][tt]);
            // accumulators of every (tile, slice) interleaved: consecutive
            // MFMAs are independent
            floatx4 a1[NTT][NS], a2[NTT][NS];
#pragma unroll
            for (int ti = 0; ti < NTT; ++ti)
#pragma unroll
                for (int s = 0; s < NS; ++s) a1[ti][s] = a2[ti][s] = zero4();
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                bf16x8 qf[NTT];
#pragma unroll
                for (int ti = 0; ti < NTT; ++ti) {
                    const int r = ti * 16 + c16;
                    qf[ti] = ld8(qs + r * KD + (((4 * m + g) ^ kswz<NKC>(r)) << 3));
                }
#pragma unroll
                for (int ti = 0; ti < NTT; ++ti)
#pragma unroll
                    for (int s = 0; s < NS; ++s) a1[ti][s] = mfma32(sb[s][m], qf[ti], a1[ti][s]);
#pragma unroll
                for (int ti = 0; ti < NTT; ++ti)
#pragma unroll
                    for (int s = 0; s < NS; ++s) a1[ti][s] = mfma32(sl[s][m], qf[ti], a1[ti][s]);
            }
#pragma unroll
            for (int tj = 0; tj < NTT; ++tj) {
                shortx4 ph[NTT], pl[NTT];
#pragma unroll
                for (int ti = tj; ti < NTT; ++ti) {
                    const u32x4 pf = __builtin_bit_cast(u32x4, ps[(ti * (ti + 1) / 2 + tj) * 64 + l]);
                    ph[ti] = __builtin_bit_cast(shortx4, uint2{pf[0], pf[1]});
                    pl[ti] = __builtin_bit_cast(shortx4, uint2{pf[2], pf[3]});
                }
#pragma unroll
                for (int ti = tj; ti < NTT; ++ti)
#pragma unroll
                    for (int s = 0; s < NS; ++s) a2[ti][s] = mfma16(nh[s][tj], ph[ti], a2[ti][s]);
#pragma unroll
                for (int ti = tj; ti < NTT; ++ti)
#pragma unroll
                    for (int s = 0; s < NS; ++s) a2[ti][s] = mfma16(nh[s][tj], pl[ti], a2[ti][s]);
#pragma unroll
                for (int ti = tj; ti < NTT; ++ti)
#pragma unroll
                    for (int s = 0; s < NS; ++s) a2[ti][s] = mfma16(nl[s][tj], ph[ti], a2[ti][s]);
            }
#pragma unroll
            for (int ti = 0; ti < NTT; ++ti) {
                const float egt = gp[ti * 16 + c16];
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[s][ti][e] = sc * (egt * a1[ti][s][e] + a2[ti][s][e]);
            }
        }
        // ---- V~ = e^{G_L - G} V_new (hi + lo);  S <- e^{G_L} S + K^T V~ ----
        bf16x8 vh[NS][NCS], vl[NS][NCS];
#pragma unroll
        for (int m = 0; m < NCS; ++m) {
            const floatx4 e0 = *reinterpret_cast<const floatx4 *>(gp + C + 32 * m + 4 * g);
            const floatx4 e1 = *reinterpret_cast<const floatx4 *>(gp + C + 32 * m + 16 + 4 * g);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                floatx4 t0, t1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t0[e] = e0[e] * vn[s][2 * m][e];
                    t1[e] = e1[e] * vn[s][2 * m + 1][e];
                }
                frag_split(t0, t1, vh[s][m], vl[s][m]);
            }
        }
        const float gL = gp[2 * C];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[s][ti][e] *= gL;
        // K^T fragments (transposed reads of the K rows), per 32-token step;
        // the hi products of every state tile, then the lo products
#pragma unroll
        for (int m = 0; m < NCS; ++m) {
            bf16x8 ka[NST];
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                const int pc = 4 * (ti >> 1) + (c16 & 3), hf = 4 * (ti & 1);
                const int r0 = m * 32 + 4 * g + (c16 >> 2), r1 = r0 + 16;
                const uint2 lo = __builtin_bit_cast(uint2, ld_tr16(ks + r0 * KD + ((pc ^ kswz<NKC>(r0)) << 3) + hf));
                const uint2 hi = __builtin_bit_cast(uint2, ld_tr16(ks + r1 * KD + ((pc ^ kswz<NKC>(r1)) << 3) + hf));
                ka[ti] = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
            }
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int s = 0; s < NS; ++s) Sreg[s][ti] = mfma32(ka[ti], vh[s][m], Sreg[s][ti]);
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int s = 0; s < NS; ++s) Sreg[s][ti] = mfma32(ka[ti], vl[s][m], Sreg[s][ti]);
        }
        // the next chunk's loads (and the previous chunk's stores) are done;
        // every wave's, and every wave is done with buffer pb
        __builtin_amdgcn_s_waitcnt(0x3F70);      // vmcnt(0)
        lds_barrier();
    }
    if constexpr (OUT)
        if (nc > 0) store_out(c1 - 1);

    // ---- the state after the segment ----
    float *dst = nullptr;
    size_t rs = 0;
    int rows = 0, cols = 0;
    if constexpr (OUT) {
        if (seg == P - 1 && a.hT) {
            dst = a.hT + (size_t)bh * kw * Dv;
            rs = Dv;
            rows = kw;
            cols = Dv;
        }
    } else if (isA) {
        dst = sa.amat + ((size_t)bh * P + seg) * KD * KD;
        rs = KD;
        rows = KD;
        cols = KD;
    } else {
        dst = sa.bmat + ((size_t)bh * P + seg) * KD * Dv;
        rs = Dv;
        rows = KD;
        cols = Dv;
    }
    if (dst) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = feat(ti, e), col = vcol[s] + c16;
                    if (f < rows && col < cols) dst[(size_t)f * rs + col] = Sreg[s][ti][e];
                }
    }
}

// ---------------------------------------------------------------------------
// Compose: S_1 = B_0 (already in place), S_{p+1} = A_p S_p + B_p for
// p = 1 .. P-2, each written over B_p.  One workgroup per (b, h, 32-column
// slice); wave w owns row tiles 2w, 2w+1 .. (KD/16 tiles over 4 waves) of
// both 16-column tiles.  Products on bf16 MFMA with hi + lo operands (three
// MFMAs per step: the lo x lo term is below fp32 rounding); S_p is kept in
// LDS transposed ([column][row], fp32) between steps.
// ---------------------------------------------------------------------------
template <int KD>
__global__ __launch_bounds__(256) void seg_compose_kernel(SegArgs sa) {
    constexpr int NRT = KD / 16, RPW = (NRT + 3) / 4, NKS = KD / 32, LDS_ = KD + 4;
    __shared__ __attribute__((aligned(16))) float St[32 * LDS_];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Dv = sa.a.Dv, P = sa.P;
    const int nsl = (Dv + 31) / 32;
    const int bh = blockIdx.x / nsl, j0 = (blockIdx.x % nsl) * 32;
    float *bm = sa.bmat + (size_t)bh * P * KD * Dv;
    const float *am = sa.amat + (size_t)bh * P * KD * KD;
    // S_1 = B_0 into LDS, transposed
    for (int idx = tid; idx < 32 * KD; idx += 256) {
        const int r = idx / 32, cc = idx % 32;
        St[cc * LDS_ + r] = j0 + cc < Dv ? bm[(size_t)r * Dv + j0 + cc] : 0.f;
    }
    __syncthreads();
    // A_p rows and B_p values of the next step are loaded while the current
    // product runs
    floatx4 an[RPW][NKS][2], bn[RPW][2];
    auto load_step = [&](int p) __attribute__((always_inline)) {
        const float *A = am + (size_t)p * KD * KD;
        const float *Bp = bm + (size_t)p * KD * Dv;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int ti = min(w + 4 * i, NRT - 1);
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                const float *ar = A + (size_t)(ti * 16 + c16) * KD + 32 * m + 8 * g;
                an[i][m][0] = *reinterpret_cast<const floatx4 *>(ar);
                an[i][m][1] = *reinterpret_cast<const floatx4 *>(ar + 4);
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = min(j0 + ct * 16 + c16, Dv - 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) bn[i][ct][e] = Bp[(size_t)(ti * 16 + 4 * g + e) * Dv + col];
            }
        }
    };
    if (P > 2) load_step(1);
    for (int p = 1; p <= P - 2; ++p) {
        float *Bp = bm + (size_t)p * KD * Dv;
        floatx4 acc[RPW][2];
        bf16x8 ahi[RPW][NKS], alo[RPW][NKS];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[i][ct] = bn[i][ct];
#pragma unroll
            for (int m = 0; m < NKS; ++m) frag_split(an[i][m][0], an[i][m][1], ahi[i][m], alo[i][m]);
        }
        if (p + 1 <= P - 2) load_step(p + 1);
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
            // B operand: S_p[32m + 8g + e][col c16 of tile ct]
            bf16x8 bhi[2], blo[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                frag_split(*reinterpret_cast<const floatx4 *>(St + (ct * 16 + c16) * LDS_ + 32 * m + 8 * g),
                           *reinterpret_cast<const floatx4 *>(St + (ct * 16 + c16) * LDS_ + 32 * m + 8 * g + 4),
                           bhi[ct], blo[ct]);
#pragma unroll
            for (int i = 0; i < RPW; ++i)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    acc[i][ct] = mfma32(ahi[i][m], bhi[ct], acc[i][ct]);
                    acc[i][ct] = mfma32(ahi[i][m], blo[ct], acc[i][ct]);
                    acc[i][ct] = mfma32(alo[i][m], bhi[ct], acc[i][ct]);
                }
        }
        lds_barrier();                            // every wave has read S_p
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int ti = w + 4 * i;
            if (ti >= NRT) continue;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = j0 + ct * 16 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = ti * 16 + 4 * g + e;
                    St[(ct * 16 + c16) * LDS_ + r] = acc[i][ct][e];
                    if (col < Dv) Bp[(size_t)r * Dv + col] = acc[i][ct][e];
                }
            }
        }
        lds_barrier();
    }
}

// Work space of the segment pass after the prep's: A_p and B_p of every
// segment.
template <int KD>
size_t seg_workspace_bytes(int B, int H, int Dv, int P) {
    if (P <= 1) return 0;
    return (size_t)B * H * P * KD * (KD + Dv) * 4;
}

}  // namespace gdn
