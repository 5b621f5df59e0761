// Sequential state pass + output of the chunkwise gated delta rule, for bf16
// inputs with one step per token (msj19 "gated_deltaproduct" test.py with
// r = 1: gated_chunk_delta_rule_fwd_kernel_h and
// gated_chunk_linear_attn_fwd_kernel_o; T diag(beta), the P tiles and the
// gate tables come from chunk_prep2_kernel in the work space).
//
// One workgroup per (batch, head, 16-column slice of the value dimension),
// 1 + C/16 waves, split by role outside the chunk loop (each role keeps only
// its own registers live):
//
//   wave 0 ("chain") owns the (KD x 16) fp32 state slice in MFMA
//   accumulators and runs the dependent part of every chunk in registers.
//   The WY form's u - w h (U = T diag(beta) V, W = T diag(beta e^G) K) is
//   taken as one product with T diag(beta) on the left:
//       V_new = T diag(beta) (V - e^G K S),
//       S <- e^{G_L} S + K^T diag(e^{G_L - G}) V_new,
//   so only K itself is staged (no W), and the residual V - e^G K S, not
//   two large terms, meets the rounding of T diag(beta).
//   An MFMA accumulator tile (lane l holds rows 4*(l/16)+e, column l%16) is
//   fed back as the B operand of the next product by reading the k index of
//   a 32-wide MFMA step in the order {4g..4g+3, 16+4g..16+4g+3} (g = l/16)
//   instead of 8g..8g+7; T diag(beta) is stored with its columns in that
//   permuted order, and K^T fragments are read transposed from the K rows
//   (ds_read_b64_tr_b16) with the token rows and key columns each lane
//   needs.  It publishes V_new (fp32) and the chunk-start state (hi + lo
//   bf16) to LDS for the output waves.
//
//   waves 1..C/16 ("out"), one 16-token tile each: the output, transposed,
//   O^T = S_start^T Q^T e^G + V_new^T P^T (P, the causal intra-chunk scores,
//   comes from the prep kernel as ready MFMA fragments; the transposed
//   accumulator gives each lane 4 consecutive values of one token, one
//   16-byte store); staging waves copy a later chunk's K rows and V slice
//   (from the inputs) and T diag(beta) and gate table (from the prep kernel)
//   straight into LDS with LDS-direct loads.
//
// One workgroup barrier per chunk.  Iteration c: the chain processes chunk c
// and publishes its start state and V_new; the other waves write the output
// of chunk c-1 and stage chunk c+2.
//
// DPM selects a pass of the gated DeltaProduct with a lower unitriangular
// 2 x 2 step mask [[1, 0], [m, 1]] (two sub-keys): the first row block of the
// state is then a gated delta rule on (k_0, v, beta_0) and the second one on
// (k_1, v', beta_1) with v'_t = v_t - m p_t, p_t the first block's prediction
// at token t (the product of the page's erase key with the gated state).
//   DPM = 1: the pass on sub-key 0; also forms the per-token errors
//            e = R - A~ V_new (A~ the decay-masked gram without beta, from the
//            prep; V_new = beta e) and writes v' = (1 - m) v + m e (fp32);
//            its output goes to an fp32 buffer.  The chain wave publishes
//            W = (1 - m) v + m R next to V_new, and the output waves form
//            v' = W - m A~ V_new for their token tiles a step later, with
//            the A~ fragments loaded from global memory like P's;
//   DPM = 2: the pass on sub-key 1 with v' (fp32, read by the chain wave) as
//            the values; its output adds the first pass's.
//
// DPM = 3 is the state pass of the backward: no output; every chunk's start
// state S goes out row-major (fp32; waves 1 and 2 copy the published state,
// half of the key rows each) and the chain wave writes the residual
// R = V - e^G K S (this lane's 16 values, accumulator order).  The
// DeltaProduct backward has two more such passes: DPM = 5 on sub-key 0,
// which also writes v' as DPM = 1 does, and DPM = 4 on sub-key 1, which
// reads v' as DPM = 2 does.
#pragma once

#include <type_traits>

#include "chunk_kernels.h"

namespace gdn {

// DUAL (C = 64, the forward only): the configuration for more chains than
// compute units, two workgroups per CU -- four waves, two staging buffers
// (about 78.5 KB of LDS at KD = 128).
template <int KD, int C, bool DUAL = false>
struct Chain1Shape {
    static constexpr int BV = 16;
    static constexpr int NTT = C / 16;        // token tiles
    static_assert(!DUAL || NTT == 4, "the two-workgroup configuration runs 64-token chunks");
    // Waves (they go to the four SIMDs of a CU in turn):
    //   C = 64: 0 the chain; 4 idle (it only takes part in the barriers, so
    //           the chain has its SIMD to itself); 1, 2 the output of token
    //           tiles {3, 0} and {2, 1} (equal score work; each reads the
    //           start state once for its two tiles); 3, 5 the staging.
    //   C = 64, DUAL: 0 the chain; 1, 2 the output as above; 3 the staging.
    //   C = 32: 0 the chain; 1, 2 the output of tiles 1, 0 and the staging.
    static constexpr int IDLE = NTT == 4 && !DUAL ? 4 : -1;
    static constexpr int NW = NTT == 4 ? (DUAL ? 4 : 6) : 1 + NTT;
    static constexpr int NTHR = 64 * NW;
    static constexpr int NLW = DUAL ? 1 : 2;  // staging ("loader") waves
    static constexpr int NB = DUAL ? 2 : 3;   // staging buffers
    static constexpr int NLOW = NTT * (NTT + 1) / 2;
    static constexpr int NKS = KD / 32;       // 32-wide steps over the key dim
    static constexpr int NST = KD / 16;       // state row tiles
    static constexpr int NCS = C / 32;        // 32-wide steps over the tokens
    // Staging buffers are filled by LDS-direct loads (global_load_lds_dwordx4:
    // lane i of a wave writes 16 bytes at base + 16 i), so their rows are
    // unpadded; the 16-byte piece j of row r sits at piece j ^ swizzle(r) to
    // spread the state pass's reads over the banks.
    static constexpr int NKC = KD / 8;        // 16-byte pieces of a K row
    static constexpr int TSW = C / 8 - 1;     // Tb swizzle mask
    static constexpr int LDK = KD;            // Ks  [C][KD]   bf16, K rows (natural order)
    static constexpr int LDT = C;             // Tb  [C][C]    bf16, T diag(beta) (permuted k order)
    static constexpr int LDV = BV;            // Vs  [C][BV]   bf16, the V slice (row-major)
    static constexpr int LDSF = KD + 4;       // St  [BV][KD]  fp32, S_start transposed
    static constexpr int LDVF = C + 4;        // Vn  [BV][C]   fp32, V_new transposed
    // gate table: e^G [C], e^{G_L-G} [C], e^{G_L} (+3), beta [C]
    static constexpr int NGATE = gate_table_len<C>();
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int SZ_KS = al(C * LDK * 2);
    static constexpr int SZ_TB = al(C * LDT * 2);
    static constexpr int SZ_BV = al(C * LDV * 2);
    static constexpr int SZ_GATE = al(NGATE * 4);
    static constexpr int SZ_ST = al(BV * LDSF * 4);
    static constexpr int SZ_VN = al(BV * LDVF * 4);
    // staging buffers are triple (index chunk % 3: staged two iterations
    // ahead), St and Vn double (index chunk & 1)
    static constexpr int OFF_KS = 0;
    static constexpr int OFF_TB = OFF_KS + NB * SZ_KS;
    static constexpr int OFF_BV = OFF_TB + NB * SZ_TB;
    static constexpr int OFF_GATE = OFF_BV + NB * SZ_BV;
    static constexpr int OFF_ST = OFF_GATE + NB * SZ_GATE;
    static constexpr int OFF_VN = OFF_ST + 2 * SZ_ST;
    static constexpr int OFF_WT = OFF_VN + 2 * SZ_VN;             // W = (1 - m) v + m R (DeltaProduct first pass)
    static constexpr int BYTES = OFF_WT + 2 * SZ_VN;
    static constexpr int BYTES_PLAIN = OFF_WT;
    static_assert(C % 32 == 0 && C <= 64 && KD % 32 == 0, "32-wide MFMA steps");
    static_assert(BYTES <= 160 * 1024 || KD > 128, "LDS budget of one workgroup exceeded");
    static_assert(BYTES_PLAIN <= 160 * 1024, "LDS budget of one workgroup exceeded");
    static_assert(SZ_KS % 1024 == 0 && SZ_TB % 1024 == 0 && SZ_BV % 1024 == 0,
                  "staging buffers are whole 1 KiB wave loads");
};

// Swizzle of K row r (token): the piece index is XORed with a permutation of
// r's low four bits that keeps both read patterns free of bank conflicts (16
// rows at one piece; 4 rows x 4 pieces for the transposed reads).
template <int NKC>
__device__ __forceinline__ int kswz(int r) {
    if constexpr (NKC >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (NKC == 8) return ((r & 3) << 1) | ((r >> 2) & 1);
    else return r & 3;
}

// Sixteen zero bytes in global memory: the source of the LDS-direct loads of
// K pieces past the key width (every lane of such a load writes its piece).
static __device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

// LDS-direct 16-byte load: lane i writes at lds_base + 16 i (lds_base uniform).
__device__ __forceinline__ void dma16(const void *src, void *lds_base) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 16, 0, 0);
}

// Which LDS-direct loads of an iteration staging wave LI issues.  With two
// staging waves at C = 64, wave 3 (alone on its SIMD) takes two of every three
// and wave 5 (beside output wave 1) the third; otherwise they alternate.
template <int NTT, int NLW, int LI>
__host__ __device__ constexpr bool dma_mine(int k) {
    return NLW == 1 || (NTT == 4 ? (LI == 0 ? k % 3 != 2 : k % 3 == 2) : k % NLW == LI);
}
template <int NTT, int NLW, int LI, int NDMA>
__host__ __device__ constexpr int dma_count() {
    int n = 0;
    for (int k = 0; k < NDMA; ++k) n += dma_mine<NTT, NLW, LI>(k) ? 1 : 0;
    return n;
}

template <int KD, int C, int DPM = 0, bool DUAL = false>
__global__ __launch_bounds__((Chain1Shape<KD, C, DUAL>::NTHR)) __attribute__((amdgpu_waves_per_eu(DUAL ? 2 : 1)))
void chunk_chain1_kernel(ChunkArgs args) {
    using S = Chain1Shape<KD, C, DUAL>;
    static_assert(DPM == 0 || C == 64, "DeltaProduct and backward passes run 64-token chunks");
    static_assert(!DUAL || DPM == 0, "the two-workgroup configuration is the forward's");
    static_assert(!DUAL || S::BYTES_PLAIN <= 80 * 1024, "two workgroups per CU");
    constexpr bool VIN = DPM == 2 || DPM == 4;  // values v' (fp32, read by the chain wave)
    constexpr bool ERR = DPM == 1 || DPM == 5;  // per-token errors and v' out
    constexpr bool BST = DPM >= 3;              // backward state pass: states and R out, no output
    constexpr int BV = S::BV, NTT = S::NTT, NKS = S::NKS, NST = S::NST, NCS = S::NCS, NKC = S::NKC;
    constexpr int LDK = S::LDK, LDT = S::LDT, LDV = S::LDV, LDSF = S::LDSF, LDVF = S::LDVF;
    constexpr int TSW = S::TSW;

    __shared__ __attribute__((aligned(16))) unsigned char smem[ERR ? S::BYTES : S::BYTES_PLAIN];

    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nvb = args.Dv / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vb = slot % nvb;
    const int bh = (slot / nvb) * 8 + xcd;      // all value slices of one head share an XCD
    if (bh >= args.B * args.H) return;
    if (w == S::IDLE) {                         // the chain wave's SIMD partner: barriers only
        const int nb = (args.T + C - 1) / C + 2;
        for (int i = 0; i < nb; ++i) __syncthreads();
        return;
    }
    const int b = bh / args.H, h = bh % args.H;
    const int v0 = vb * BV;
    const int T = args.T, H = args.H, Dv = args.Dv;
    const int NT = (T + C - 1) / C;
    const int tlast = T > 0 ? T - 1 : 0;

    auto Ks = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_KS + p * S::SZ_KS); };
    auto Tb = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_TB + p * S::SZ_TB); };
    auto BVs = [&](int p) { return reinterpret_cast<u16 *>(smem + S::OFF_BV + p * S::SZ_BV); };
    auto gate = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_GATE + p * S::SZ_GATE); };
    auto St = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_ST + p * S::SZ_ST); };
    auto Vn = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_VN + p * S::SZ_VN); };
    auto Wt = [&](int p) { return reinterpret_cast<float *>(smem + S::OFF_WT + p * S::SZ_VN); };
    // DeltaProduct hand-offs between passes in the work space (v' from
    // DPM 1 / 5 to DPM 2 / 4, the first output from DPM 1 to DPM 2), in tile
    // order: per (chunk, value slice, token tile) a 1 KiB block whose 16
    // bytes at 16 l are output lane l's four values (token 16 tile + l%16,
    // columns 4 (l/16) .. +3 of the slice).  Blocks cover whole chunks.
    auto tile_base = [&](int c, int tile) { return ((((size_t)bh * NT + c) * nvb + vb) * NTT + tile) * 256; };

    if (w == 0) {
        // =================================================================
        // chain wave
        // =================================================================
        // State row tile ti = 2 mk + h, accumulator row 4 g + e holds key
        // feature 32 mk + 8 g + 4 h + e: the bf16 fragment of tiles 2 mk and
        // 2 mk + 1 is then features 32 mk + 8 g + {0..7} in natural order
        // (the B operand of K S), and K^T fragments pick their rows to match.
        floatx4 Sreg[NST];
        auto feat = [&](int ti, int e) { return (ti >> 1) * 32 + 8 * g + 4 * (ti & 1) + e; };
        // S_start (fp32, transposed to [j][i]) for the output waves, which
        // split their fragments into hi + lo bf16 themselves: the four rows
        // of a tile are consecutive key features
        auto publish_state = [&](int p) {
            float *sf = St(p) + c16 * LDSF;
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) *reinterpret_cast<floatx4 *>(sf + feat(ti, 0)) = Sreg[ti];
        };
#pragma unroll
        for (int ti = 0; ti < NST; ++ti) {
            Sreg[ti] = zero4();
            if (args.h0) {
                const float *hp = args.h0 + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (feat(ti, e) < args.kw) Sreg[ti][e] = hp[(size_t)feat(ti, e) * Dv];
            }
        }
        // VIN: this lane's values v' (rows tt*16 + 4g + e, column c16) of
        // the next chunk, loaded one iteration ahead
        floatx4 vpre[NTT];
        // (row 4g + e of token tile tt, column c16: the writer's lane
        // 16 (c16 / 4) + 4g + e, its value c16 % 4; rows past T hold finite
        // values that meet zero columns of T diag(beta) only)
        auto load_vin = [&](int c) {
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const float *vp = args.vin + tile_base(c, tt) + (c16 >> 2) * 64 + (c16 & 3);
#pragma unroll
                for (int e = 0; e < 4; ++e) vpre[tt][e] = vp[(4 * g + e) * 4];
            }
        };
        if constexpr (VIN) load_vin(0);
        __syncthreads();
        for (int c = 0, sq = 0; c < NT; ++c, sq = sq == S::NB - 1 ? 0 : sq + 1) {
            const int p = c & 1;                 // St, Vn; staging buffers: sq = c % NB
            const u16 *ks = Ks(sq), *tb = Tb(sq), *bv = BVs(sq);
            const float *gp = gate(sq);
            // LDS operands of K S first (nothing here depends on the state), so
            // their latency overlaps; the MFMAs run over the token tiles
            // innermost, so consecutive MFMAs are independent.
            bf16x8 kf[NTT][NKS], tf[NTT][NCS];
#pragma unroll
            for (int m = 0; m < NKS; ++m)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    const int r = tt * 16 + c16;
                    kf[tt][m] = ld8(ks + r * LDK + (((4 * m + g) ^ kswz<NKC>(r)) << 3));
                }
            shortx4 vv[NTT];                     // V rows tt*16 + 4g + e, column c16
            floatx4 vcur[NTT];                   // VIN: v' of this chunk
            if constexpr (VIN) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) vcur[tt] = vpre[tt];
                if (c + 1 < NT) load_vin(c + 1);
            } else {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) vv[tt] = ld_tr16(bv + (tt * 16 + 4 * g + (c16 >> 2)) * LDV + 4 * (c16 & 3));
            }
#pragma unroll
            for (int m = 0; m < NCS; ++m)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
                    if (2 * m <= tt)
                        tf[tt][m] = ld8(tb + (tt * 16 + c16) * LDT + (((4 * m + g) ^ ((tt * 16 + c16) & TSW)) << 3));
            bf16x8 sb[NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m) sb[m] = frag_hi(Sreg[2 * m], Sreg[2 * m + 1]);
            // Y = K S
            floatx4 y[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) y[tt] = zero4();
#pragma unroll
            for (int m = 0; m < NKS; ++m)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) y[tt] = mfma32(kf[tt][m], sb[m], y[tt]);
            // K^T fragments of the state update, read while the MFMAs run: lane
            // (g, j) of tile ti gets feature feat(ti, j%4 .. ) from the pointers
            // of lanes 4a + b (token row 32m + 4g + a, piece 4 mk + b, half h)
            bf16x8 ka[NST][NCS];
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                const int pc = 4 * (ti >> 1) + (c16 & 3), hf = 4 * (ti & 1);
#pragma unroll
                for (int m = 0; m < NCS; ++m) {
                    const int r0 = m * 32 + 4 * g + (c16 >> 2), r1 = r0 + 16;
                    const uint2 lo = __builtin_bit_cast(uint2, ld_tr16(ks + r0 * LDK + ((pc ^ kswz<NKC>(r0)) << 3) + hf));
                    const uint2 hi = __builtin_bit_cast(uint2, ld_tr16(ks + r1 * LDK + ((pc ^ kswz<NKC>(r1)) << 3) + hf));
                    ka[ti][m] = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
                }
            }
            floatx4 eg[NTT], el[NTT], bt[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                eg[tt] = *reinterpret_cast<const floatx4 *>(gp + tt * 16 + 4 * g);
                el[tt] = *reinterpret_cast<const floatx4 *>(gp + C + tt * 16 + 4 * g);
                bt[tt] = *reinterpret_cast<const floatx4 *>(gp + 2 * C + 4 + tt * 16 + 4 * g);
            }
            const float gL = gp[2 * C];
            // R = V - e^G Y; V_new = (T diag(beta)) R: its diagonal, beta, in fp32
            // on R, the rest (block lower triangular, entries well below beta)
            // by MFMA on R rounded to bf16
            floatx4 rr[NTT], vin4[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                if constexpr (VIN) {
                    vin4[tt] = vcur[tt];
                } else {
                    const uint2 v2 = __builtin_bit_cast(uint2, vv[tt]);
                    vin4[tt] = floatx4{__builtin_bit_cast(float, v2.x << 16), __builtin_bit_cast(float, v2.x & 0xffff0000u),
                                       __builtin_bit_cast(float, v2.y << 16), __builtin_bit_cast(float, v2.y & 0xffff0000u)};
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) rr[tt][e] = vin4[tt][e] - eg[tt][e] * y[tt][e];
            }
            if constexpr (BST) {
                floatx4 *rp = reinterpret_cast<floatx4 *>(args.rst) + (((size_t)bh * NT + c) * nvb + vb) * 64 * NTT + l * NTT;
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) rp[tt] = rr[tt];
            }
            bf16x8 rh[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) rh[m] = frag_hi(rr[2 * m], rr[2 * m + 1]);
            floatx4 vn[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) vn[tt][e] = bt[tt][e] * rr[tt][e];
#pragma unroll
            for (int m = 0; m < NCS; ++m)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
                    if (2 * m <= tt) vn[tt] = mfma32(tf[tt][m], rh[m], vn[tt]);
            // V_new published fp32 [j][s]; V~ = e^{G_L - G} V_new
            float *vnp = Vn(p);
            floatx4 vt4[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                if constexpr (!BST || ERR) *reinterpret_cast<floatx4 *>(vnp + c16 * LDVF + tt * 16 + 4 * g) = vn[tt];
#pragma unroll
                for (int e = 0; e < 4; ++e) vt4[tt][e] = el[tt][e] * vn[tt][e];
            }
            bf16x8 vh[NCS], vl[NCS];
#pragma unroll
            for (int m = 0; m < NCS; ++m) frag_split(vt4[2 * m], vt4[2 * m + 1], vh[m], vl[m]);
            // S <- e^{G_L} S + K^T V~
            floatx4 ds[NST];
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) ds[ti] = zero4();
#pragma unroll
            for (int m = 0; m < NCS; ++m) {
#pragma unroll
                for (int ti = 0; ti < NST; ++ti) ds[ti] = mfma32(ka[ti][m], vh[m], ds[ti]);
#pragma unroll
                for (int ti = 0; ti < NST; ++ti) ds[ti] = mfma32(ka[ti][m], vl[m], ds[ti]);
            }
            // S_start of chunk c goes out while the state MFMAs run (its LDS
            // writes then do not queue ahead of this chunk's operand reads)
            publish_state(p);
            if constexpr (ERR) {
                // W = (1 - m) v + m R, published like V_new ([j][s]); the waves
                // that read V_new a step later form v' = W - m A~ V_new
                const float mc = args.mcoef;
                float *wp = Wt(p) + c16 * LDVF + 4 * g;
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    floatx4 w4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w4[e] = (1.f - mc) * vin4[tt][e] + mc * rr[tt][e];
                    *reinterpret_cast<floatx4 *>(wp + tt * 16) = w4;
                }
            }
#pragma unroll
            for (int ti = 0; ti < NST; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[ti][e] = gL * Sreg[ti][e] + ds[ti][e];
            // LDS operations only: the chain wave's own global loads (v' of the
            // next chunk) stay in flight across the barrier
            lds_barrier();
        }
        __syncthreads();                       // matches the out waves' drain step
        if (args.hT) {
#pragma unroll
            for (int ti = 0; ti < NST; ++ti) {
                float *hp = args.hT + ((size_t)bh * args.hrows + args.hoff) * Dv + v0 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (feat(ti, e) < args.kw) hp[(size_t)feat(ti, e) * Dv] = Sreg[ti][e];
            }
        }
        return;
    }

    // =====================================================================
    // out waves
    // =====================================================================
    // Each out wave runs a copy of the loop specialised for its roles, so
    // that its global loads are straight-line code: the hardware counter of
    // outstanding loads is in order, and a load skipped on some path would
    // make the compiler wait for every load issued after the one it needs.
    //
    // Roles: OA, OB = token tiles of the output (-1: none); LI = staging
    // index (-1: none).  Staging of chunk c+2 in iteration c: NDMA LDS-direct wave
    // loads of 1 KiB (K, T diag(beta), the V slice, the gate table),
    // load k on the staging wave dma_mine picks, waited for before the barrier.
    constexpr int NLW = S::NLW;
    constexpr int NLOW = NTT * (NTT + 1) / 2;
    constexpr int NGV = S::NGATE / 4;           // 16-byte vectors of a gate table
    constexpr int NDK = S::SZ_KS / 1024, NDT = S::SZ_TB / 1024, NDV = VIN ? 0 : S::SZ_BV / 1024;
    constexpr int NDMA = NDK + NDT + NDV + 1;
    static_assert(NGV <= 64 && S::SZ_GATE >= NGV * 16, "gate table: one partial wave load");
    const int kw = args.kw;                     // key width; pieces past it are zero
    const size_t tokq = (size_t)H * args.kst, tokv = (size_t)H * Dv;
    const u16 *kg = reinterpret_cast<const u16 *>(args.k) + ((size_t)b * T * H + h) * args.kst + args.koff;
    const u16 *qg = reinterpret_cast<const u16 *>(args.q) + ((size_t)b * T * H + h) * args.kst + args.koff;
    const u16 *vg = reinterpret_cast<const u16 *>(args.v) + ((size_t)b * T * H + h) * Dv + v0;
    const u16 *tg = reinterpret_cast<const u16 *>(args.tmat) + (size_t)bh * NT * C * C;
    const float *gtg = reinterpret_cast<const float *>(args.gtab) + (size_t)bh * NT * S::NGATE;

    auto out_wave = [&](auto owa, auto owb, auto lic) {
        constexpr int OA = decltype(owa)::value, OB = decltype(owb)::value, LI = decltype(lic)::value;
        constexpr bool TILE = OA >= 0, LOAD = LI >= 0;
        // Stage chunk c (clamped to the last chunk; a past-the-end chunk lands in
        // a buffer no one reads) into buffers c % NB.  Rows of the prep's
        // outputs past T are zero; K and V rows past T are clamped to T-1:
        // they only meet zero columns of T diag(beta), and V_new is zero there.
        // Addresses: the chunk's base (scalar) plus a 32-bit per-lane offset,
        // a row below 64 times a token-row stride below 2^24 elements (the
        // entry points refuse longer rows): a 24-bit multiply per load
        // instead of 64-bit products (these waves' issue time counts).
        auto stage = [&](int c) {
            const int p = c % S::NB;
            c = min(c, NT - 1);
            const int rl = tlast - c * C;       // last valid row of the chunk
            const unsigned tokq_u = (unsigned)tokq, tokv_u = (unsigned)tokv;
            const u16 *kc = kg + (size_t)c * C * tokq, *vc = vg + (size_t)c * C * tokv;
            const u16 *tc = tg + (size_t)c * C * C;
#pragma unroll
            for (int k = 0; k < NDMA; ++k) {
                if (!dma_mine<NTT, NLW, LI>(k)) continue;
                if (k < NDK) {                  // K: row r (token), stored piece j holds piece j ^ kswz(r)
                    const int pos = k * 64 + l, r = pos / NKC, sc = pos % NKC;
                    const int pc = sc ^ kswz<NKC>(r);
                    dma16(pc * 8 < kw ? static_cast<const void *>(kc + (__umul24(min(r, rl), tokq_u) + (unsigned)(pc << 3)))
                                      : static_cast<const void *>(&kZero16),
                          Ks(p) + k * 512);
                } else if (k < NDK + NDT) {     // T diag(beta): row r (token)
                    const int kk = k - NDK, pos = kk * 64 + l, r = pos / (C / 8), sc = pos % (C / 8);
                    dma16(tc + (unsigned)(r * C + ((sc ^ (r & TSW)) << 3)), Tb(p) + kk * 512);
                } else if (k < NDK + NDT + NDV) {   // V slice: token pos / 2, half pos % 2
                    const int kk = k - NDK - NDT, pos = kk * 64 + l;
                    dma16(vc + (__umul24(min(pos / 2, rl), tokv_u) + (unsigned)((pos & 1) * 8)), BVs(p) + kk * 512);
                } else {                            // gate table
                    if (l < NGV) dma16(gtg + (size_t)c * S::NGATE + l * 4, gate(p));
                }
            }
        };
        // token tiles of this wave: OA, and OB if any
        constexpr int NTW = OB >= 0 ? 2 : 1;
        constexpr int TW0 = OA >= 0 ? OA : 0, TW1 = OB >= 0 ? OB : 0;
        constexpr int TWMAX = TW0 > TW1 ? TW0 : TW1;
        auto tw = [](int i) { return i == 0 ? TW0 : TW1; };
        bf16x8 qf[NTW][NKS];                    // Q fragments (B operand, token = lane%16)
        u32x4 pf[NTW][NTT];                     // P fragments of each tile: {hi01, hi23, lo01, lo23}
        float egt[NTW];                         // e^{G_t} of this lane's tokens
        floatx4 ov[NTW];                        // outputs of the previous chunk
        floatx4 op[NTW];                        // DPM 2: the first pass's output of those tokens
        u32x4 af[NTW][NTT];                     // ERR: A~ fragments of each tile (P's layout)
        floatx4 vq[NTW];                        // ERR: v' of the previous chunk (4 columns of one token)
        // DPM 1 -> 2 hand-offs in tile order (whole-line accesses per wave
        // instead of 64-byte pieces of 16 token rows)
        auto tile_off = [&](int c, int tile) { return tile_base(c, tile) + 4 * l; };
        // operands of chunk c's output, used one iteration later
        auto load_qp = [&](int c) {
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int t = min(c * C + tw(i) * 16 + c16, tlast);   // rows past T are never stored
                if (kw == KD) {                 // (wave-uniform) no padded key features
#pragma unroll
                    for (int m = 0; m < NKS; ++m)
                        qf[i][m] = *reinterpret_cast<const bf16x8 *>(qg + (size_t)t * tokq + m * 32 + 8 * g);
                } else {
#pragma unroll
                    for (int m = 0; m < NKS; ++m) {
                        const bool pad = m * 32 + 8 * g >= kw;   // loaded anyway (counted loads), then zeroed
                        qf[i][m] = *reinterpret_cast<const bf16x8 *>(qg + (size_t)t * tokq + (pad ? 0 : m * 32 + 8 * g));
                        if (pad) qf[i][m] = bf16x8{};
                    }
                }
                const uint4 *pc = reinterpret_cast<const uint4 *>(args.pfrag) + ((size_t)bh * NT + c) * NLOW * 64 +
                                  (tw(i) * (tw(i) + 1) / 2) * 64 + l;
#pragma unroll
                for (int tj = 0; tj <= tw(i); ++tj) pf[i][tj] = __builtin_bit_cast(u32x4, pc[tj * 64]);
                egt[i] = gate(c % S::NB)[tw(i) * 16 + c16];
                if constexpr (ERR) {
                    const uint4 *ac = reinterpret_cast<const uint4 *>(args.atil) + ((size_t)bh * NT + c) * NLOW * 64 +
                                      (tw(i) * (tw(i) + 1) / 2) * 64 + l;
#pragma unroll
                    for (int tj = 0; tj <= tw(i); ++tj) af[i][tj] = __builtin_bit_cast(u32x4, ac[tj * 64]);
                }
                if constexpr (DPM == 2)
                    op[i] = *reinterpret_cast<const floatx4 *>(args.oprev + tile_off(c, tw(i)));
            }
        };
        // O^T of chunk c: a1 = S_start^T Q^T, a2 = V_new^T P^T (buffers c & 1);
        // the start state and V_new fragments are split once for both tiles
        auto compute_out = [&](int c) {
            const float *sf = St(c & 1) + c16 * LDSF;
            const float *vnp = Vn(c & 1);
            bf16x8 sh[NKS], sl[NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                frag_split(*reinterpret_cast<const floatx4 *>(sf + m * 32 + 8 * g),
                           *reinterpret_cast<const floatx4 *>(sf + m * 32 + 8 * g + 4), sh[m], sl[m]);
            shortx4 vh4[TWMAX + 1], vl4[TWMAX + 1];
#pragma unroll
            for (int tj = 0; tj <= TWMAX; ++tj)
                split4(*reinterpret_cast<const floatx4 *>(vnp + c16 * LDVF + tj * 16 + 4 * g), vh4[tj], vl4[tj]);
            const float sc = args.scale;
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                floatx4 a1 = zero4(), a2 = zero4();
#pragma unroll
                for (int m = 0; m < NKS; ++m) {
                    a1 = mfma32(sh[m], qf[i][m], a1);
                    a1 = mfma32(sl[m], qf[i][m], a1);
                }
#pragma unroll
                for (int tj = 0; tj <= tw(i); ++tj) {
                    const shortx4 ph = __builtin_bit_cast(shortx4, uint2{pf[i][tj][0], pf[i][tj][1]});
                    const shortx4 pl = __builtin_bit_cast(shortx4, uint2{pf[i][tj][2], pf[i][tj][3]});
                    a2 = mfma16(vh4[tj], ph, a2);
                    a2 = mfma16(vh4[tj], pl, a2);
                    a2 = mfma16(vl4[tj], ph, a2);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[i][e] = sc * (egt[i] * a1[e] + a2[e]) + (DPM == 2 ? op[i][e] : 0.f);
                if constexpr (ERR) {
                    // v'^T = W^T - m V_new^T A~^T (A~ in P's layout, hi + lo)
                    floatx4 a3 = zero4();
#pragma unroll
                    for (int tj = 0; tj <= tw(i); ++tj) {
                        const shortx4 ah = __builtin_bit_cast(shortx4, uint2{af[i][tj][0], af[i][tj][1]});
                        const shortx4 al = __builtin_bit_cast(shortx4, uint2{af[i][tj][2], af[i][tj][3]});
                        a3 = mfma16(vh4[tj], ah, a3);
                        a3 = mfma16(vh4[tj], al, a3);
                        a3 = mfma16(vl4[tj], ah, a3);
                    }
                    const float *wt = Wt(c & 1) + tw(i) * 16 + c16;
                    const float mc = args.mcoef;
#pragma unroll
                    for (int e = 0; e < 4; ++e) vq[i][e] = wt[(4 * g + e) * LDVF] - mc * a3[e];
                }
            }
        };
        auto store_out = [&](int c) {
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int tt = c * C + tw(i) * 16 + c16;
                if (tt < T) {
                    const size_t off = (((size_t)b * T + tt) * H + h) * Dv + v0 + 4 * g;
                    if constexpr (DPM == 1)     // the first pass's output, in tile order
                        *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(args.o) + tile_off(c, tw(i))) = ov[i];
                    else if (args.out_bf16)
                        *reinterpret_cast<uint2 *>(reinterpret_cast<u16 *>(args.o) + off) =
                            uint2{cvt2_bf16(ov[i][0], ov[i][1]), cvt2_bf16(ov[i][2], ov[i][3])};
                    else
                        *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(args.o) + off) = ov[i];
                }
                // v' of every row (rows past T finite: read as the next pass's values)
                if constexpr (ERR) *reinterpret_cast<floatx4 *>(args.vout + tile_off(c, tw(i))) = vq[i];
            }
        };

        // The workgroup barrier of an output or staging wave: its LDS
        // operations done (the buffers it reads are rewritten next), but its
        // newest global operations left in flight -- this iteration's staging
        // (waited for at the next barrier), Q and P loads (used next
        // iteration) and output stores.  __syncthreads() would wait for all of
        // them.  The hardware counter of outstanding global operations is in
        // order, so "at most N outstanding" completes everything older than
        // the newest N; a staging wave's N counts only the operations it
        // issues unconditionally after the previous staging (its Q and P
        // loads, then this staging), so that staging is always complete.  An
        // output-only wave stages nothing and waits for none of its own.
        constexpr int NMINE = LOAD ? dma_count<NTT, NLW, (LI < 0 ? 0 : LI), NDMA>() : 0;
        constexpr int NPF = (TW0 + 1) + (NTW > 1 ? TW1 + 1 : 0);   // P (and A~) fragment loads
        constexpr int NQP = TILE ? NTW * NKS + NPF * (ERR ? 2 : 1) : 0;
        // (two staging buffers: the staging of this iteration completes at its barrier)
        constexpr int NOWN = LOAD ? (S::NB == 2 ? 0 : NMINE + NQP) : 63;
        static_assert(NOWN < 64, "6-bit vmcnt");
        // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, lgkmcnt(0), expcnt at its maximum
        constexpr int WAIT_IMM = (NOWN & 15) | ((NOWN >> 4) << 14) | 0x0070;
        auto wave_barrier = [&]() {
            asm volatile("" ::: "memory");      // keep memory operations on their side
            __builtin_amdgcn_s_waitcnt(WAIT_IMM);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };

        // Iteration c (one barrier each): output of chunk c-1, operands of
        // chunk c, staging of chunk c+NB-1 (waited for NB-2 iterations later:
        // one with three buffers, at its own barrier with two).
        if constexpr (LOAD) {
            for (int j = 0; j < S::NB - 1; ++j) stage(j);
            __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0)
        }
        __syncthreads();
        if constexpr (TILE) load_qp(0);
        if constexpr (LOAD) stage(S::NB - 1);
        wave_barrier();
        for (int c = 1; c < NT; ++c) {
            if constexpr (TILE) {
                compute_out(c - 1);
                load_qp(c);
                store_out(c - 1);
            }
            if constexpr (LOAD) stage(c + S::NB - 1);
            wave_barrier();
        }
        if constexpr (TILE) {
            compute_out(NT - 1);
            store_out(NT - 1);
        }
        __syncthreads();
    };
    if (NT == 0) {                              // no chunks: match the chain wave's two barriers
        __syncthreads();
        __syncthreads();
        return;
    }
    using std::integral_constant;
    using none = integral_constant<int, -1>;
    if constexpr (BST) {
        // no output: waves 1 and 2 write the published chunk-start states of
        // the previous iteration to the work space, row-major, key rows
        // [0, KD/2) and [KD/2, KD): lane l takes row 16 i + l/4, value columns
        // 4 (l%4) .. +3 (one 16-byte store)
        if (w == 1 || w == 2) {
            const int f0 = (w - 1) * (KD / 2);
            auto store_state = [&](int c) {
                const float *sf = St(c & 1);
#pragma unroll
                for (int i = 0; i < KD / 32; ++i) {
                    const int f = f0 + 16 * i + (l >> 2), v4 = 4 * (l & 3);
                    floatx4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = sf[(v4 + e) * LDSF + f];
                    if (f < kw)
                        *reinterpret_cast<floatx4 *>(args.sst + (((size_t)bh * NT + c) * kw + f) * args.Dv + v0 + v4) = x;
                }
            };
            // DPM 5: v' of the previous chunk for token tiles {3, 0} (wave 1)
            // or {2, 1} (wave 2), as the output waves of DPM 1 form it
            auto err_wave = [&](auto owa, auto owb) {
                constexpr int TA = decltype(owa)::value, TB = decltype(owb)::value;
                constexpr int TM = TA > TB ? TA : TB;
                auto twi = [](int i) { return i == 0 ? TA : TB; };
                u32x4 af[2][NTT];
                auto load_af = [&](int c) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const uint4 *ac = reinterpret_cast<const uint4 *>(args.atil) + ((size_t)bh * NT + c) * NLOW * 64 +
                                          (twi(i) * (twi(i) + 1) / 2) * 64 + l;
#pragma unroll
                        for (int tj = 0; tj <= twi(i); ++tj) af[i][tj] = __builtin_bit_cast(u32x4, ac[tj * 64]);
                    }
                };
                auto err = [&](int c) {
                    const float *vnp = Vn(c & 1);
                    shortx4 vh4[TM + 1], vl4[TM + 1];
#pragma unroll
                    for (int tj = 0; tj <= TM; ++tj)
                        split4(*reinterpret_cast<const floatx4 *>(vnp + c16 * LDVF + tj * 16 + 4 * g), vh4[tj], vl4[tj]);
                    const float mc = args.mcoef;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        floatx4 a3 = zero4();
#pragma unroll
                        for (int tj = 0; tj <= twi(i); ++tj) {
                            const shortx4 ah = __builtin_bit_cast(shortx4, uint2{af[i][tj][0], af[i][tj][1]});
                            const shortx4 al = __builtin_bit_cast(shortx4, uint2{af[i][tj][2], af[i][tj][3]});
                            a3 = mfma16(vh4[tj], ah, a3);
                            a3 = mfma16(vh4[tj], al, a3);
                            a3 = mfma16(vl4[tj], ah, a3);
                        }
                        const float *wt = Wt(c & 1) + twi(i) * 16 + c16;
                        floatx4 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = wt[(4 * g + e) * LDVF] - mc * a3[e];
                        // v' of every row, in tile order (read as the next pass's values)
                        *reinterpret_cast<floatx4 *>(args.vout + tile_base(c, twi(i)) + 4 * l) = x;
                    }
                };
                load_af(0);
                __syncthreads();
                lds_barrier();
                for (int c = 1; c < NT; ++c) {
                    store_state(c - 1);
                    err(c - 1);
                    load_af(c);
                    lds_barrier();
                }
                store_state(NT - 1);
                err(NT - 1);
                __syncthreads();
            };
            if constexpr (ERR) {
                if (w == 1) err_wave(integral_constant<int, 3>{}, integral_constant<int, 0>{});
                else err_wave(integral_constant<int, 2>{}, integral_constant<int, 1>{});
            } else {
                __syncthreads();
                lds_barrier();
                for (int c = 1; c < NT; ++c) {
                    store_state(c - 1);
                    lds_barrier();
                }
                store_state(NT - 1);
                __syncthreads();
            }
        }
        if (w == 3) out_wave(none{}, none{}, integral_constant<int, 0>{});
        if (w == 5) out_wave(none{}, none{}, integral_constant<int, 1>{});
    } else if constexpr (NTT == 4) {
        if (w == 1) out_wave(integral_constant<int, 3>{}, integral_constant<int, 0>{}, none{});
        if (w == 2) out_wave(integral_constant<int, 2>{}, integral_constant<int, 1>{}, none{});
        if (w == 3) out_wave(none{}, none{}, integral_constant<int, 0>{});
        if constexpr (!DUAL)
            if (w == 5) out_wave(none{}, none{}, integral_constant<int, 1>{});
    } else {
        static_assert(NTT == 2, "chunk of 32 or 64 tokens");
        if (w == 1) out_wave(integral_constant<int, 1>{}, none{}, integral_constant<int, 0>{});
        if (w == 2) out_wave(integral_constant<int, 0>{}, none{}, integral_constant<int, 1>{});
    }
}

}  // namespace gdn
