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
// Two kernels.
//
// 1. chunk_solve_kernel - fully parallel, one workgroup per chunk of one
//    (batch, head):
//      cumsum  G_t = sum_{t'<=t} g_t'
//      gram    A[(t,a),(s,b)] = [s<t] beta_{t,a} M[a][b] (k_{t,b}.k_{s,b}) e^{G_t-G_s}
//              (bf16 MFMA on the exact inputs, fp32 accumulation)
//      solve   T = (I + A)^-1: 16x16 diagonal blocks by forward substitution
//              (one lane per column), then block rows T_ij = -T_ii sum A_im T_mj
//              (fp32 MFMA)
//    and writes T (bf16 for bf16 inputs, fp32 for fp32 inputs) to the
//    work space.
//
// 2. chunk_chain_kernel - one 512-thread workgroup per (batch, head,
//    16-column slice of the value dimension), walking the chunks in order.
//    Waves 0-3 ("chain") hold the (Dk x 16) fp32 state slice in MFMA
//    accumulators and run the dependent part of each chunk:
//      X_b = K_b S_b;  R = diag(beta) (V - diag(e^G) sum_b M X_b)
//      V_new = T R;    S_b <- e^{G_L} S_b + K_b^T diag(e^{G_L-G}) V_new_b
//    Waves 4-7 ("out") run everything else, overlapped with the chain:
//      P_b[t][s] = [s<=t] (q_{t,b}.k_{s,b}) e^{G_t-G_s}
//      O = scale (diag(e^G) Q S_start + sum_b P_b V_new_b)  -> HBM
//      the global loads of the next chunks (register prefetch, LDS commit)
//      and the chunk-local cumsum of the next chunk.
//    Three workgroup barriers per chunk separate the phases.  They hand over
//    LDS only (no wave reads global memory that another wave writes), so
//    they wait for LDS operations alone and leave the output stores and the
//    prefetch loads in flight.
//
// V_new = T diag(beta) (V - diag(e^G) E S) is the page's u - w h with
// w = T diag(beta e^G) E and u = T diag(beta) V, regrouped so that W is never
// formed: the state only enters through the product K S.
//
// Virtual rows j = t*R + a (token-major) carry the R steps of each token.
//
// Precision (bf16 inputs): products of exact bf16 inputs use one bf16 MFMA;
// fp32 operands derived inside the kernels are split into hi + lo bf16 pairs
// (2 or 3 MFMAs) except T and the state in K S, which are rounded to bf16
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
    void *tmat;      // work space: T per chunk, [B*H][NT][NR][NR]
    void *pfrag;     // work space: intra-chunk P tiles as MFMA fragments (PFRAG shapes)
    void *gtab;      // work space: e^{G_t} [C], e^{G_L - G_t} [C], e^{G_L}, 0, 0, 0 per chunk, fp32 (PFRAG shapes)
    int B, T, H, Dv;
    int kw;          // key width (q, k, h0, hT rows); KD >= kw, features past kw are zero
    int kst, koff;   // q, k: elements per (token, head) row and first column of this key (kst = kw, koff = 0
                     // except for a DeltaProduct sub-key pass)
    int bst, boff;   // beta[((b T + t) H + h) bst + boff] (1, 0 except for a DeltaProduct sub-key pass)
    int hrows, hoff; // h0, hT: (B, H, hrows, Dv), this key's rows start at row hoff (kw, 0 ...)
    // DeltaProduct sub-key passes of the single-chain kernels:
    void *atil;      // prep: [s<t] (k_t . k_s) e^{G_t - G_s} as hi/lo fragments (P's layout), or null
    float *vout;     // first pass: v' = (1 - m) v + m e written here, fp32 (B, T, H, Dv)
    const float *vin;    // second pass: the values v' (fp32), in place of v
    const float *oprev;  // second pass: the first pass's output (fp32), added to this pass's
    float mcoef;     // m = step_mask[1][0]
    int nsub;        // prep: sub-keys prepared in one launch (1, or 2 for a DeltaProduct call:
                     // sub-key 1 at column koff + kw, beta offset boff + 1, its work space after
                     // sub-key 0's (subws bytes on), no A~)
    size_t subws;
    int out_bf16;
    float scale;
    float mask[4];   // R x R step mask, row-major
    // backward of the single-step bf16 path (64-token chunks):
    void *tmatT;     // prep: T^T without its diagonal (unscaled), rows s, columns t in the permuted k order
    void *atilT;     // prep (backward, sub-key 0 with atil): A~ as hi/lo fragments in the transposed-score layout
    float *sst;      // state pass: chunk-start state per chunk, (B*H, NT, Dk, Dv) fp32
    float *rst;      // state pass: R = V - e^G K S per chunk, (B*H, NT, Dv/16, 64 lanes, 16) fp32
};

constexpr float LOG2E = 1.4426950408889634f;

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The "permuted order" of a k-contiguous MFMA operand row: within each block
// of 32, the 4-element groups are stored as 0, 4, 1, 5, 2, 6, 3, 7, so that
// lane group g (= lane/16) finds its k = {4g..4g+3, 16+4g..16+4g+3} in one
// 16-byte piece at 8g.  Stored position of element k (k % 4 == 0 keeps the
// group together).
__device__ __forceinline__ int perm4_pos(int k) {
    const int grp = (k >> 2) & 7;                 // group within the 32-block
    return (k & ~31) + (((grp & 3) * 2 + (grp >> 2)) << 2) + (k & 3);
}

template <bool F32IN, int KD, int C, int R>
struct ChunkShape {
    static constexpr int BV = 16;
    static constexpr int DK = KD / R;
    static constexpr int NR = C * R;           // virtual rows per chunk
    static constexpr int NB = NR / 16;         // 16-row blocks of the solve
    static constexpr int ESZ = F32IN ? 4 : 2;  // operand element size
    static constexpr int PAD = F32IN ? 4 : 8;  // row padding (elements)
    static constexpr int NLO = F32IN ? 0 : 1;  // number of "lo" copies
    static constexpr int VEC = 16 / ESZ;       // elements per 16-byte vector
    static constexpr int NTT = C / 16;         // token tiles per chunk
    static constexpr int NLOW = NTT * (NTT + 1) / 2;
    static constexpr int LDK = KD + PAD;       // Ks, Qs:  [C][KD]
    static constexpr int LDA = NR + 4;         // As, Ts:  [NR][NR] fp32
    static constexpr int LDTB = NR + PAD;      // Tb:      [NR][NR]
    static constexpr int LDPQ = C + PAD;       // Pq:      [R][C][C]
    static constexpr int LDST = KD + PAD;      // St:      [BV][KD]
    static constexpr int LDRT = NR + PAD;      // RT:      [BV][NR]
    static constexpr int LDVT = C + PAD;       // Vn/Vt:   [R][BV][C]
    static constexpr int LDY = 17;             // merge scratch [16][17] fp32
    // bf16 inputs, one step per token, 32-multiple widths: these shapes run
    // chunk_prep2_kernel + chunk_chain1_kernel, whose work space also holds
    // the P fragments and gate tables of every chunk.
    static constexpr bool PFRAG = !F32IN && R == 1 && C % 32 == 0 && KD % 32 == 0;
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static_assert(KD % R == 0, "key width must split into R sub-keys");
    static_assert(DK % 16 == 0 && C % 16 == 0, "sizes must be multiples of 16");
    static_assert(NR <= 64, "the solve handles at most 64 virtual rows per chunk");
};

// ===========================================================================
// Kernel 1: per-chunk T = (I + A)^-1
// ===========================================================================
template <bool F32IN, int KD, int C, int R>
struct SolveLds {
    using S = ChunkShape<F32IN, KD, C, R>;
    static constexpr int SZ_KS = C * S::LDK * S::ESZ;
    static constexpr int SZ_GATE = (C * R + C) * 4;
    static constexpr int SZ_A = S::NR * S::LDA * 4;
    static constexpr int SZ_Y = 4 * 16 * S::LDY * 4;
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_GATE = OFF_KS + S::al(SZ_KS);
    static constexpr int OFF_AS = OFF_GATE + S::al(SZ_GATE);
    static constexpr int OFF_TS = OFF_AS + S::al(SZ_A);
    static constexpr int OFF_Y = OFF_TS + S::al(SZ_A);
    static constexpr int BYTES = OFF_Y + S::al(SZ_Y);
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

template <bool F32IN, int KD, int C, int R>
__global__ __launch_bounds__(256) void chunk_solve_kernel(ChunkArgs args) {
    using S = ChunkShape<F32IN, KD, C, R>;
    using L = SolveLds<F32IN, KD, C, R>;
    using Op = typename OpType<F32IN>::type;
    constexpr int DK = S::DK, NR = S::NR, NB = S::NB, LDK = S::LDK, LDA = S::LDA, LDY = S::LDY;
    constexpr int VEC = S::VEC, NV = KD / VEC;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    Op *Ks = reinterpret_cast<Op *>(smem + L::OFF_KS);
    float *betas = reinterpret_cast<float *>(smem + L::OFF_GATE);
    float *G2 = betas + C * R;
    float *As = reinterpret_cast<float *>(smem + L::OFF_AS);
    float *Ts = reinterpret_cast<float *>(smem + L::OFF_TS);

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    float *Ys = reinterpret_cast<float *>(smem + L::OFF_Y) + w * 16 * LDY;
    const int T = args.T, H = args.H;
    const int NT = (T + C - 1) / C;
    const int bh = blockIdx.x / NT, c = blockIdx.x % NT;
    const int b = bh / H, h = bh % H;
    const int t0 = c * C;

    // ---- load the chunk's keys and gates ----
    for (int idx = tid; idx < C * NV; idx += 256) {
        const int t = idx / NV, cv = idx % NV, tt = t0 + t;
        U16x8 raw;
        if (tt < T && cv * VEC < args.kw) {
            const size_t row = ((size_t)b * T + tt) * H + h;
            raw = *reinterpret_cast<const U16x8 *>(reinterpret_cast<const unsigned char *>(args.k) +
                                                   (row * args.kst + args.koff + cv * VEC) * S::ESZ);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) raw.v[e] = 0;
        }
        *reinterpret_cast<U16x8 *>(Ks + t * LDK + cv * VEC) = raw;
    }
    for (int idx = tid; idx < C * R; idx += 256) {
        const int tt = t0 + idx / R;
        betas[idx] = tt < T ? args.beta[(((size_t)b * T + tt) * H + h) * R + idx % R] : 0.f;
    }
    if (w == 0) {
        float gs = (l < C && t0 + l < T) ? args.g[((size_t)b * T + t0 + l) * H + h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gs, off, 64);
            if (l >= off) gs += y;
        }
        if (l < C) G2[l] = gs * LOG2E;
    }
    __syncthreads();

    // ---- gram: strictly-lower A over tokens, with beta, mask and decay ----
    for (int it = w; it < R * S::NLOW; it += 4) {
        const int bb = it / S::NLOW;
        int p = it % S::NLOW, ti = 0;
        while (p > ti) { p -= ti + 1; ++ti; }
        const int tj = p;
        floatx4 acc = zero4();
        if constexpr (F32IN) mma_f32(acc, Ks + ti * 16 * LDK + bb * DK, LDK, Ks + tj * 16 * LDK + bb * DK, LDK, DK);
        else mma_bf16(acc, Ks + ti * 16 * LDK + bb * DK, LDK, Ks + tj * 16 * LDK + bb * DK, LDK, DK);
        const int s = tj * 16 + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = ti * 16 + 4 * (l >> 4) + e;
            const float dec = s < t ? fast_exp2(fminf(G2[t] - G2[s], 0.f)) : 0.f;
#pragma unroll
            for (int a = 0; a < R; ++a)
                As[(t * R + a) * LDA + s * R + bb] = betas[t * R + a] * args.mask[a * R + bb] * acc[e] * dec;
        }
    }
    __syncthreads();

    // ---- diagonal 16x16 blocks: forward substitution, one lane per column ----
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
            float *Tc = Ts + (ib * 16) * LDA + ib * 16 + col;
#pragma unroll
            for (int i = 0; i < 16; ++i) Tc[i * LDA] = x[i];
        }
    }
    __syncthreads();

    // ---- block rows: T_ij = -T_ii sum_{j<=m<i} A_im T_mj, one column block per wave ----
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
            for (int e = 0; e < 4; ++e) Ts[(ib * 16 + 4 * (l >> 4) + e) * LDA + jb * 16 + (l & 15)] = -t2[e];
        }
        __syncthreads();
    }

    // ---- write T (zero above the block diagonal) ----
    Op *out = reinterpret_cast<Op *>(args.tmat) + ((size_t)bh * NT + c) * NR * NR;
    for (int idx = tid; idx < NR * NR / 8; idx += 256) {       // 8 consecutive entries of a row
        const int i = idx / (NR / 8), j0 = (idx % (NR / 8)) * 8;
        floatx4 x0 = *reinterpret_cast<const floatx4 *>(Ts + i * LDA + j0);
        floatx4 x1 = *reinterpret_cast<const floatx4 *>(Ts + i * LDA + j0 + 4);
        if ((j0 >> 4) > (i >> 4)) x0 = x1 = zero4();
        if constexpr (F32IN) {
            *reinterpret_cast<floatx4 *>(out + (size_t)i * NR + j0) = x0;
            *reinterpret_cast<floatx4 *>(out + (size_t)i * NR + j0 + 4) = x1;
        } else {
            *reinterpret_cast<uint4 *>(out + (size_t)i * NR + j0) =
                uint4{cvt2_bf16(x0[0], x0[1]), cvt2_bf16(x0[2], x0[3]), cvt2_bf16(x1[0], x1[1]), cvt2_bf16(x1[2], x1[3])};
        }
    }
}

// ===========================================================================
// Kernel 2: sequential state pass + output
// ===========================================================================
template <bool F32IN, int KD, int C, int R>
struct ChainLds {
    using S = ChunkShape<F32IN, KD, C, R>;
    static constexpr int SZ_KS = C * S::LDK * S::ESZ;            // x2 (double buffer)
    static constexpr int SZ_QS = C * S::LDK * S::ESZ;
    static constexpr int SZ_VS = C * S::BV * 4;
    static constexpr int NGATE = C * R + 3 * C + 4;                // beta, G2, eG, eGLm, gL
    static constexpr int SZ_GATE = NGATE * 4;                      // x2
    static constexpr int SZ_TB = S::NR * S::LDTB * S::ESZ;
    static constexpr int SZ_PQ = R * C * S::LDPQ * S::ESZ;         // x(1+NLO)
    static constexpr int SZ_ST = S::BV * S::LDST * S::ESZ;         // x(1+NLO)
    static constexpr int SZ_VT = R * S::BV * S::LDVT * S::ESZ;     // x(1+NLO), Vn and Vt
    static constexpr int SZ_RT = S::BV * S::LDRT * S::ESZ;         // x(1+NLO)
    static constexpr int NP = 1 + S::NLO;
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_QS = OFF_KS + 2 * S::al(SZ_KS);
    static constexpr int OFF_VS = OFF_QS + S::al(SZ_QS);
    static constexpr int OFF_GATE = OFF_VS + S::al(SZ_VS);
    static constexpr int OFF_TB = OFF_GATE + 2 * S::al(SZ_GATE);
    static constexpr int OFF_PQ = OFF_TB + S::al(SZ_TB);
    static constexpr int OFF_ST = OFF_PQ + NP * S::al(SZ_PQ);
    static constexpr int OFF_VN = OFF_ST + NP * S::al(SZ_ST);
    static constexpr int OFF_VT = OFF_VN + NP * S::al(SZ_VT);
    static constexpr int OFF_RT = OFF_VT + NP * S::al(SZ_VT);
    static constexpr int BYTES = OFF_RT + NP * S::al(SZ_RT);
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

template <bool F32IN, int KD, int C, int R>
__global__ __launch_bounds__(512) void chunk_chain_kernel(ChunkArgs args) {
    using S = ChunkShape<F32IN, KD, C, R>;
    using L = ChainLds<F32IN, KD, C, R>;
    using Op = typename OpType<F32IN>::type;
    constexpr int BV = S::BV, DK = S::DK, NR = S::NR, NB = S::NB, NTT = S::NTT;
    constexpr int LDK = S::LDK, LDTB = S::LDTB, LDPQ = S::LDPQ, LDST = S::LDST, LDRT = S::LDRT,
                  LDVT = S::LDVT;
    constexpr int NST = KD / 16;                 // state row tiles
    constexpr int NSTW = (NST + 3) / 4;          // state tiles per chain wave (max)
    constexpr int VEC = S::VEC;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const bool chain = w < 4;
    const int ow = w - 4, otid = tid - 256;     // output-group wave / thread index
    const int nvb = args.Dv / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vb = slot % nvb;
    const int bh = (slot / nvb) * 8 + xcd;      // all value slices of one head share an XCD
    if (bh >= args.B * args.H) return;
    const int b = bh / args.H, h = bh % args.H;
    const int v0 = vb * BV;
    const int T = args.T, H = args.H, Dv = args.Dv;
    const int NT = (T + C - 1) / C;

    Op *KsBuf = reinterpret_cast<Op *>(smem + L::OFF_KS);
    Op *Qs = reinterpret_cast<Op *>(smem + L::OFF_QS);
    float *Vs = reinterpret_cast<float *>(smem + L::OFF_VS);
    float *GateBuf = reinterpret_cast<float *>(smem + L::OFF_GATE);
    Op *Tb = reinterpret_cast<Op *>(smem + L::OFF_TB);
    Op *PqH = reinterpret_cast<Op *>(smem + L::OFF_PQ);
    Op *PqL = reinterpret_cast<Op *>(smem + L::OFF_PQ + S::al(L::SZ_PQ));
    Op *StH = reinterpret_cast<Op *>(smem + L::OFF_ST);
    Op *StL = reinterpret_cast<Op *>(smem + L::OFF_ST + S::al(L::SZ_ST));
    Op *VnH = reinterpret_cast<Op *>(smem + L::OFF_VN);
    Op *VnL = reinterpret_cast<Op *>(smem + L::OFF_VN + S::al(L::SZ_VT));
    Op *VtH = reinterpret_cast<Op *>(smem + L::OFF_VT);
    Op *VtL = reinterpret_cast<Op *>(smem + L::OFF_VT + S::al(L::SZ_VT));
    Op *RtH = reinterpret_cast<Op *>(smem + L::OFF_RT);
    Op *RtL = reinterpret_cast<Op *>(smem + L::OFF_RT + S::al(L::SZ_RT));
    auto Ks = [&](int p) { return KsBuf + p * (S::al(L::SZ_KS) / S::ESZ); };
    // gate block p: beta [C*R], G2 [C] (log2-scaled cumsum), eG [C], eGLm [C], gL [1]
    auto gate = [&](int p) { return GateBuf + p * (S::al(L::SZ_GATE) / 4); };

    // ---- output group: register prefetch of one chunk, LDS commit ----
    constexpr int NV = KD / VEC;
    constexpr int NKQ = 2 * C * NV;               // k and q vectors per chunk
    constexpr int PKQ = (NKQ + 255) / 256;
    constexpr int VV = BV / VEC;                  // vectors per v row slice
    constexpr int NVV = C * VV;
    constexpr int PV = (NVV + 255) / 256;
    constexpr int NTV = NR * NR / VEC;            // T vectors per chunk
    constexpr int PT = (NTV + 255) / 256;
    constexpr int TROW = NR / VEC;                // T vectors per row
    U16x8 rkq[PKQ], rv[PV], rt[PT];
    float rbeta = 0.f, rg = 0.f;
    // Per-slot source offsets (bytes) at chunk 0; chunk c adds c*C token rows.
    const int kw = args.kw;
    const size_t tok_bytes_qk = (size_t)H * args.kst * S::ESZ, tok_bytes_v = (size_t)H * Dv * S::ESZ;
    size_t kq_off[PKQ], v_off[PV];
    int kq_t[PKQ], v_t[PV];
    bool kq_pad[PKQ];                             // a feature vector past kw: zero
#pragma unroll
    for (int p = 0; p < PKQ; ++p) {
        const int idx = otid + 256 * p;
        const int rem = idx % (C * NV);
        kq_t[p] = rem / NV;
        kq_pad[p] = (rem % NV) * VEC >= kw;
        kq_off[p] = ((((size_t)b * T + kq_t[p]) * H + h) * args.kst + args.koff) * S::ESZ +
                    (kq_pad[p] ? 0 : (size_t)(rem % NV) * 16);
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int idx = otid + 256 * p;
        v_t[p] = idx / VV;
        v_off[p] = ((((size_t)b * T + v_t[p]) * H + h) * Dv + v0) * S::ESZ + (size_t)(idx % VV) * 16;
    }
    const unsigned char *kbase = reinterpret_cast<const unsigned char *>(args.k);
    const unsigned char *qbase = reinterpret_cast<const unsigned char *>(args.q);
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(args.v);
    auto prefetch = [&](int c) {
        const int t0 = c * C;
        const bool full = t0 + C <= T;
#pragma unroll
        for (int p = 0; p < PKQ; ++p) {
            const int idx = otid + 256 * p;
            if (idx < NKQ) {
                const unsigned char *src = (idx < C * NV ? kbase : qbase) + kq_off[p] + (size_t)t0 * tok_bytes_qk;
                if ((full || t0 + kq_t[p] < T) && !kq_pad[p]) {
                    rkq[p] = *reinterpret_cast<const U16x8 *>(src);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) rkq[p].v[e] = 0;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int idx = otid + 256 * p;
            if (idx < NVV) {
                if (full || t0 + v_t[p] < T) {
                    rv[p] = *reinterpret_cast<const U16x8 *>(vbase + v_off[p] + (size_t)t0 * tok_bytes_v);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) rv[p].v[e] = 0;
                }
            }
        }
        const U16x8 *tsrc = reinterpret_cast<const U16x8 *>(args.tmat) + ((size_t)bh * NT + c) * NTV;
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int idx = otid + 256 * p;
            if (idx < NTV) rt[p] = tsrc[idx];
        }
        if (otid < C * R) {
            const int tt = t0 + otid / R;
            rbeta = tt < T ? args.beta[(((size_t)b * T + tt) * H + h) * R + otid % R] : 0.f;
        }
        if (otid < C) {
            const int tt = t0 + otid;
            rg = tt < T ? args.g[((size_t)b * T + tt) * H + h] : 0.f;
        }
    };
    // commit the prefetched chunk into LDS buffer p and build its gate tables
    auto commit = [&](int p) {
        Op *ks = Ks(p);
#pragma unroll
        for (int q = 0; q < PKQ; ++q) {
            const int idx = otid + 256 * q;
            if (idx < NKQ) {
                const int which = idx / (C * NV), rem = idx % (C * NV);
                const int t = rem / NV, cv = rem % NV;
                *reinterpret_cast<U16x8 *>((which ? Qs : ks) + t * LDK + cv * VEC) = rkq[q];
            }
        }
#pragma unroll
        for (int q = 0; q < PV; ++q) {
            const int idx = otid + 256 * q;
            if (idx < NVV) {
                const int t = idx / VV, cv = idx % VV;
                float *dst = Vs + t * BV + cv * VEC;
                if constexpr (F32IN) {
                    const float4 f = __builtin_bit_cast(float4, rv[q]);
                    dst[0] = f.x; dst[1] = f.y; dst[2] = f.z; dst[3] = f.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) dst[e] = bf16_to_f32(rv[q].v[e]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int idx = otid + 256 * q;
            if (idx < NTV) {
                const int i = idx / TROW, cv = idx % TROW;
                *reinterpret_cast<U16x8 *>(Tb + i * LDTB + cv * VEC) = rt[q];
            }
        }
        float *gp = gate(p);
        if (otid < C * R) gp[otid] = rbeta;
        if (ow == 0) {
            float gs = rg;       // zero for lanes >= C and for tokens past T
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(gs, off, 64);
                if (l >= off) gs += y;
            }
            const float g2 = gs * LOG2E;
            const float g2l = __shfl(g2, C - 1, 64);
            if (l < C) {
                gp[C * R + l] = g2;                          // G2
                gp[C * R + C + l] = fast_exp2(g2);           // e^{G_t}
                gp[C * R + 2 * C + l] = fast_exp2(g2l - g2); // e^{G_L - G_t}
            }
            if (l == 0) gp[C * R + 3 * C] = fast_exp2(g2l); // e^{G_L}
        }
    };

    // ---- chain group: state slice in accumulators ----
    floatx4 Sreg[NSTW];
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

    // ---- prologue ----
    if (chain) {
#pragma unroll
        for (int n = 0; n < NSTW; ++n) {
            Sreg[n] = zero4();
            const int ts = w + 4 * n;
            if (ts < NST && args.h0) {
                const float *hp = args.h0 + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = ts * 16 + 4 * (l >> 4) + e;
                    Sreg[n][e] = row < args.kw ? hp[(size_t)row * Dv] : 0.f;
                }
            }
        }
        write_state_operand();
    } else if (NT > 0) {
        prefetch(0);
        commit(0);
        if (NT > 1) prefetch(1);
    }
    __syncthreads();

    floatx4 a1[1];                                // output group: Q S_start of its tile
    for (int c = 0; c < NT; ++c) {
        const int p = c & 1;
        const Op *ks = Ks(p);
        const float *gp = gate(p);
        const float *betas = gp, *G2 = gp + C * R, *eG = gp + C * R + C, *eGLm = gp + C * R + 2 * C;
        // ================= phase 1 =================
        if (chain) {
            // X_b = K_b S_b for token tile w, all b; then R rows (t, a) of that tile
            if (w < NTT) {
                floatx4 xa[R];
#pragma unroll
                for (int bb = 0; bb < R; ++bb) {
                    xa[bb] = zero4();
                    if constexpr (F32IN) mma_f32(xa[bb], ks + w * 16 * LDK + bb * DK, LDK, StH + bb * DK, LDST, DK);
                    else mma_bf16(xa[bb], ks + w * 16 * LDK + bb * DK, LDK, StH + bb * DK, LDST, DK);
                }
                const int j = l & 15;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = w * 16 + 4 * (l >> 4) + e;
#pragma unroll
                    for (int a = 0; a < R; ++a) {
                        float xs = 0.f;
#pragma unroll
                        for (int bb = 0; bb < R; ++bb) xs += args.mask[a * R + bb] * xa[bb][e];
                        const float r = betas[t * R + a] * (Vs[t * BV + j] - eG[t] * xs);
                        store_op<F32IN>(RtH, RtL, j * LDRT + t * R + a, r);
                    }
                }
            }
        } else {
            // P_b = [s<=t] (q_t,b . k_s,b) e^{G_t - G_s}, lower tiles
            for (int it = ow; it < R * S::NLOW; it += 4) {
                const int bb = it / S::NLOW;
                int pp = it % S::NLOW, ti = 0;
                while (pp > ti) { pp -= ti + 1; ++ti; }
                const int tj = pp;
                floatx4 acc = zero4();
                if constexpr (F32IN)
                    mma_f32(acc, Qs + ti * 16 * LDK + bb * DK, LDK, ks + tj * 16 * LDK + bb * DK, LDK, DK);
                else
                    mma_bf16(acc, Qs + ti * 16 * LDK + bb * DK, LDK, ks + tj * 16 * LDK + bb * DK, LDK, DK);
                const int s = tj * 16 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = ti * 16 + 4 * (l >> 4) + e;
                    const float dec = fast_exp2(fminf(G2[t] - G2[s], 0.f));
                    const float val = s <= t ? acc[e] * dec : 0.f;
                    store_op<F32IN>(PqH, PqL, (bb * C + t) * LDPQ + s, val);
                }
            }
        }
        lds_barrier();
        // ================= phase 2 =================
        if (!chain) {
            // Q S_start for the output tile of this wave (the output group is
            // otherwise idle while the chain forms V_new)
            if (ow < NTT) {
                a1[0] = zero4();
                if constexpr (F32IN) mma_f32(a1[0], Qs + ow * 16 * LDK, LDK, StH, LDST, KD);
                else mma_bf16_split(a1[0], Qs + ow * 16 * LDK, nullptr, LDK, StH, StL, LDST, KD);
            }
        }
        if (chain) {
            // V_new = T R, rows of virtual tile w
            if (w < NB) {
                floatx4 acc = zero4();
                if constexpr (F32IN) mma_f32(acc, Tb + w * 16 * LDTB, LDTB, RtH, LDRT, NR);
                else mma_bf16_split(acc, Tb + w * 16 * LDTB, nullptr, LDTB, RtH, RtL, LDRT, NR);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int vr = w * 16 + 4 * (l >> 4) + e;
                    const int s = vr / R, bb = vr % R;
                    const int o = (bb * BV + (l & 15)) * LDVT + s;
                    store_op<F32IN>(VnH, VnL, o, acc[e]);
                    store_op<F32IN>(VtH, VtL, o, eGLm[s] * acc[e]);
                }
            }
        }
        lds_barrier();
        // ================= phase 3 =================
        if (chain) {
            const float gL = gp[C * R + 3 * C];
#pragma unroll
            for (int n = 0; n < NSTW; ++n) {
                const int ts = w + 4 * n;
                if (ts < NST) {
                    const int bb = (ts * 16) / DK;
                    floatx4 acc = zero4();
                    if constexpr (F32IN) {
                        // A = K_b^T: element (i, s) = Ks[s][i]
                        const float *pa = ks + ts * 16 + (l & 15) + (l >> 4) * LDK;
                        const float *pb = VtH + bb * BV * LDVT + (l & 15) * LDVT + (l >> 4);
                        for (int kk = 0; kk < C; kk += 4)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[kk * LDK], pb[kk], acc, 0, 0, 0);
                    } else {
                        if constexpr (C % 32 == 0) {
                            // A = K_b^T: lane (g, j) takes column ts*16 + j of token rows
                            // kk + 8g .. +7 with two transposed LDS reads
                            const int l = lane_id(), g = l >> 4, c16 = l & 15;
                            const u16 *bh = VtH + bb * BV * LDVT + c16 * LDVT, *bl = VtL + bb * BV * LDVT + c16 * LDVT;
#pragma unroll
                            for (int kk = 0; kk < C; kk += 32) {
                                const u16 *pa = ks + (kk + 8 * g + (c16 >> 2)) * LDK + ts * 16 + 4 * (c16 & 3);
                                const uint2 x0 = __builtin_bit_cast(uint2, ld_tr16(pa));
                                const uint2 x1 = __builtin_bit_cast(uint2, ld_tr16(pa + 4 * LDK));
                                const bf16x8 ah = __builtin_bit_cast(bf16x8, uint4{x0.x, x0.y, x1.x, x1.y});
                                acc = mfma32(ah, ld8(bh + kk + 8 * g), acc);
                                acc = mfma32(ah, ld8(bl + kk + 8 * g), acc);
                            }
                        } else {
                            mma_bf16_at_split(acc, ks + ts * 16, LDK, VtH + bb * BV * LDVT, VtL + bb * BV * LDVT,
                                              LDVT, C);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sreg[n][e] = gL * Sreg[n][e] + acc[e];
                }
            }
            write_state_operand();
        } else {
            // stage the next chunk first, so that its wait for the prefetched
            // loads does not also wait for this chunk's output stores (the
            // commit writes the other Ks/gate buffer and Qs, Vs, Tb, none of
            // which the output below reads)
            if (c + 1 < NT) commit(p ^ 1);
            // finish the output of chunk c
            if (ow < NTT) {
                floatx4 a2 = zero4();
                const int kd = (ow + 1) * 16;
#pragma unroll
                for (int bb = 0; bb < R; ++bb) {
                    if constexpr (F32IN)
                        mma_f32(a2, PqH + (bb * C + ow * 16) * LDPQ, LDPQ, VnH + bb * BV * LDVT, LDVT, kd);
                    else
                        mma_bf16_split(a2, PqH + (bb * C + ow * 16) * LDPQ, PqL + (bb * C + ow * 16) * LDPQ, LDPQ,
                                       VnH + bb * BV * LDVT, VnL + bb * BV * LDVT, LDVT, kd);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = ow * 16 + 4 * (l >> 4) + e, tt = c * C + t;
                    if (tt < T) {
                        const float ov = args.scale * (eG[t] * a1[0][e] + a2[e]);
                        const size_t off = (((size_t)b * T + tt) * H + h) * Dv + v0 + (l & 15);
                        if (args.out_bf16) reinterpret_cast<u16 *>(args.o)[off] = bf16_bits(ov);
                        else reinterpret_cast<float *>(args.o)[off] = ov;
                    }
                }
            }
            // start loading the chunk after the next
            if (c + 2 < NT) prefetch(c + 2);
        }
        lds_barrier();
    }

    if (chain && args.hT) {
#pragma unroll
        for (int n = 0; n < NSTW; ++n) {
            const int ts = w + 4 * n;
            if (ts < NST) {
                float *hp = args.hT + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = ts * 16 + 4 * (l >> 4) + e;
                    if (row < args.kw) hp[(size_t)row * Dv] = Sreg[n][e];
                }
            }
        }
    }
}

// Per-chunk gate table of the PFRAG shapes (fp32): e^{G_t} [C], e^{G_L - G_t}
// [C], e^{G_L}, 0, 0, 0, beta_t [C] (zero past the end of the sequence).
template <int C>
constexpr int gate_table_len() { return 3 * C + 4; }

// Work space: T of every chunk, then (PFRAG shapes) the P fragments and the
// gate tables of every chunk.
template <bool F32IN, int KD, int C, int R>
size_t chunk_tmat_bytes(int B, int T, int H) {
    using S = ChunkShape<F32IN, KD, C, R>;
    const size_t NT = (size_t)(T + C - 1) / C;
    return ((size_t)B * H * NT * S::NR * S::NR * S::ESZ + 255) & ~(size_t)255;
}
template <bool F32IN, int KD, int C, int R>
size_t chunk_pfrag_bytes(int B, int T, int H) {
    using S = ChunkShape<F32IN, KD, C, R>;
    const size_t NT = (size_t)(T + C - 1) / C;
    return S::PFRAG ? (size_t)B * H * NT * S::NLOW * 64 * 16 : 0;
}
template <bool F32IN, int KD, int C, int R>
size_t chunk_workspace_bytes(int B, int T, int H) {
    using S = ChunkShape<F32IN, KD, C, R>;
    const size_t NT = (size_t)(T + C - 1) / C;
    const size_t gbytes = S::PFRAG ? (size_t)B * H * NT * gate_table_len<C>() * 4 : 0;  // gate tables
    return chunk_tmat_bytes<F32IN, KD, C, R>(B, T, H) + chunk_pfrag_bytes<F32IN, KD, C, R>(B, T, H) + gbytes;
}

}  // namespace gdn
