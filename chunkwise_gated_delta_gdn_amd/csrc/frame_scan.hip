// Camera-branch numerator-only scan, frame-synchronous: Sana
// "fused_cam_gdn.py" _cam_scan_kernel (forward direction) and cam_scan_func.
//
// Every token of frame f predicts from the same gated state P = e^{g_f} S,
// so the frame update is affine in S:
//   S_f = P + sum_s beta_s k_s (v_s - P^T k_s)^T = (I - G_f) P + H_f,
//   G_f = sum_{s in f} beta_s k_s k_s^T,   H_f = sum_{s in f} beta_s k_s v_s^T
// (the matrix form of the page's _torch_cam_scan_single_chunk).  Kernels:
//   frame_gram_bf16_kernel / frame_gram_kernel (fp32 inputs)
//                       parallel over (b, h, f, token range): partial G_f and
//                       H_f from K^T diag(beta) K and K^T diag(beta) V (MFMA);
//   frame_reduce_kernel sums the partials of more than two token ranges (the
//                       state pass adds two itself);
//   frame_state_kernel  per (b, h, 16-column slice of S), sequential over
//                       frames: S_f = e^{g_f} (S - G_f S) + H_f in fp32 (fp32
//                       MFMA), stores S_f and the final state;
//   frame_out_bf16_kernel / frame_out_kernel (fp32 inputs, D = 16)
//                       parallel over (b, h, f, token tile):
//                       out_s = scale * S_f^T q_s.
// Inputs q, k, v (B, H, N, D) as written by gdn_prep; out (B, H, N, D) fp32.
#include <math.h>

#include "api_common.h"
#include "gdn_common.h"

namespace gdn {
namespace {

struct FrameArgs {
    const void *q, *k, *v;
    const float *beta, *g, *h0;
    float *hT, *out;
    float *part;     // [B*H*F][nsplit][2][D][D] partial G_f, H_f (= gh when nsplit is 1)
    float *gh;       // [B*H*F][2][D][D] G_f, H_f
    float *sf;       // [B*H][F][D][D] state after each frame, transposed ([column][row])
    int B, H, F, S, nsplit, spl;
    int dd;          // head width in HBM (q, k, v, out rows; h0, hT); the kernels' D >= dd,
                     // features past dd read as zero and are never stored
    int reverse;     // anti-causal scan: frame f reads the state built from frames f+1 .. F-1
    int den;         // normaliser stream: unit values (v = 1), vector state z (h0/hT are z0/zT,
                     // (B, H, D)), out is den (B, H, N)
    float scale;
};

constexpr int TS = 32;   // tokens per step of the fp32 gram kernel

template <bool F32IN>
struct OpT { typedef u16 type; };
template <>
struct OpT<true> { typedef float type; };

template <bool F32IN>
__device__ __forceinline__ void put_op(typename OpT<F32IN>::type *hi, typename OpT<F32IN>::type *lo, int i,
                                       float x) {
    if constexpr (F32IN) {
        hi[i] = x;
    } else {
        u16 a, b;
        split_bf16(x, a, b);
        hi[i] = a;
        lo[i] = b;
    }
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of a group receives the group total.
template <int W>
__device__ __forceinline__ float lane_group_sum(float x) {
#pragma unroll
    for (int off = 1; off < W; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <bool F32IN>
__device__ __forceinline__ void load8(const void *base, size_t elem, float (&x)[8]) {
    if constexpr (F32IN) {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + elem);
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const U16x8 r = *reinterpret_cast<const U16x8 *>(reinterpret_cast<const u16 *>(base) + elem);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(r.v[e]);
    }
}

// ---------------------------------------------------------------------------
// partial G_f = K^T diag(beta) K and H_f = K^T diag(beta) V over one token range
// ---------------------------------------------------------------------------
template <bool F32IN, int D, bool VONES>
__global__ __launch_bounds__(256) void frame_gram_kernel(FrameArgs a) {
    using Op = typename OpT<F32IN>::type;
    constexpr int PAD = F32IN ? 4 : 8, LD = TS + PAD;
    constexpr int NT1 = D / 16, NTILE = 2 * NT1 * NT1, PERW = (NTILE + 3) / 4;
    constexpr int SEGS = D / 8;                      // 8-element segments per token row
    __shared__ __attribute__((aligned(16))) Op KT[D * LD], BKh[D * LD], BKl[F32IN ? 1 : D * LD],
        BVh[D * LD], BVl[F32IN ? 1 : D * LD];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = blockIdx.x / a.nsplit, sp = blockIdx.x % a.nsplit;
    const int bh = unit / a.F, f = unit % a.F;
    const size_t N = (size_t)a.F * a.S;
    const int s_lo = sp * a.spl, s_hi = min(a.S, (sp + 1) * a.spl);
    const size_t row0 = (size_t)bh * N + (size_t)f * a.S;   // token row of frame start

    floatx4 acc[PERW];
#pragma unroll
    for (int i = 0; i < PERW; ++i) acc[i] = zero4();

    for (int s0 = s_lo; s0 < s_hi; s0 += TS) {
        for (int idx = tid; idx < TS * SEGS; idx += 256) {
            const int s = idx / SEGS, i0 = (idx % SEGS) * 8;
            float kx[8], vx[8];
            float bt = 0.f;
            if (s0 + s < s_hi && i0 < a.dd) {
                const size_t row = row0 + s0 + s;
                load8<F32IN>(a.k, row * a.dd + i0, kx);
                if constexpr (VONES) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vx[e] = 1.f;
                } else {
                    load8<F32IN>(a.v, row * a.dd + i0, vx);
                }
                bt = a.beta[row];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kx[e] = vx[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int o = (i0 + e) * LD + s;
                if constexpr (F32IN) KT[o] = kx[e];
                else KT[o] = bf16_bits(kx[e]);       // exact: k is bf16
                put_op<F32IN>(BKh, BKl, o, bt * kx[e]);
                put_op<F32IN>(BVh, BVl, o, bt * vx[e]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int tile = w + 4 * n;
            if (tile < NTILE) {
                const int kind = tile / (NT1 * NT1), ti = (tile / NT1) % NT1, tj = tile % NT1;
                const Op *bh_ = kind ? BVh : BKh;
                if constexpr (F32IN) {
                    mma_f32(acc[n], KT + ti * 16 * LD, LD, bh_ + tj * 16 * LD, LD, TS);
                } else {
                    const Op *bl_ = kind ? BVl : BKl;
                    mma_bf16_split(acc[n], KT + ti * 16 * LD, nullptr, LD, bh_ + tj * 16 * LD, bl_ + tj * 16 * LD,
                                   LD, TS);
                }
            }
        }
        __syncthreads();
    }
    float *dst = a.part + ((size_t)unit * a.nsplit + sp) * 2 * D * D;
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        const int tile = w + 4 * n;
        if (tile < NTILE) {
            const int kind = tile / (NT1 * NT1), ti = (tile / NT1) % NT1, tj = tile % NT1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(size_t)kind * D * D + (ti * 16 + 4 * (l >> 4) + e) * D + tj * 16 + (l & 15)] = acc[n][e];
        }
    }
}

// ---------------------------------------------------------------------------
// partial G_f and H_f for bf16 inputs.  G = K^T diag(beta) K and
// H = K^T diag(beta) V contract over tokens, so both MFMA operands need 8
// consecutive tokens of one feature per lane: the token rows are staged
// row-major in LDS (64 tokens a step, two buffers, 16-byte pieces
// XOR-swizzled per row) and read back transposed with ds_read_b64_tr_b16.  A = K^T (exact bf16); B = beta (.) K or
// beta (.) V, scaled in fp32 after the transposed read and split hi + lo.
// Wave w owns whole column tiles ("jobs": matrix G or H, column tile tj;
// eight waves at D >= 32, one job each at D = 64); every wave reads the A
// fragments of all row tiles.
//
// Loads run one round (SPW steps) ahead in two register sets.  Every load is
// unconditional (rows past the range end read the range's last row, whose
// beta is replaced by 0, so they add nothing) so that the wait before
// staging a set counts only that set's loads.
// ---------------------------------------------------------------------------
constexpr int TSG = 64;      // tokens per staged step of the bf16 gram kernel
// steps per round (register budget of the two sets)
template <int D>
constexpr int gram_steps() { return D == 128 ? 1 : 2; }
constexpr int gram_round(int D) { return (D == 128 ? 1 : 2) * TSG; }

template <int D>
constexpr int gram_waves() { return D >= 32 ? 8 : 4; }

// CROSS (the scan's backward): only the second product, with the constant
// weight `scale` for beta: K^T V * scale (called with q for k and dout for v:
// A_f = scale Q_f^T dO_f), one D x D matrix per partial.
template <int D, bool VONES, bool CROSS = false>
__global__ __launch_bounds__(512) void frame_gram_bf16_kernel(FrameArgs a) {
    constexpr int NW = gram_waves<D>(), NTH = 64 * NW;   // waves, threads
    constexpr int NT1 = D / 16;                 // row tiles = column tiles of one matrix
    constexpr int NJOB = (CROSS ? 1 : 2) * NT1, JPW = (NJOB + NW - 1) / NW;
    // Rows are unpadded; the 16-byte piece p of row r sits at p ^ swz(r), so
    // that the 8 rows x 32 bytes that 32 lanes of a transposed read take
    // (rows 8g + {0..3} of two lane groups) cover all 64 banks once.
    constexpr int LDR = D;
    auto swz = [](int r) __attribute__((always_inline)) {
        if constexpr (D == 128) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
        else if constexpr (D == 64) return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
        else if constexpr (D == 32) return 2 * ((r >> 3) & 1);
        else return 0;
    };
    // element offset of (row r, column c) in a staged buffer
    auto at = [&](int r, int c) __attribute__((always_inline)) {
        return r * LDR + ((((c >> 3) ^ swz(r))) << 3) + (c & 7);
    };
    constexpr int SEGS = D / 8;                 // 16-byte pieces per token row
    constexpr int PPT = 2 * TSG * SEGS / NTH;   // pieces of k and v per thread per step
    constexpr int SPW = gram_steps<D>(), RND = SPW * TSG;
    static_assert(PPT * NTH == 2 * TSG * SEGS, "whole pieces per thread");
    __shared__ __attribute__((aligned(16))) u16 Ks[2][TSG * LDR], Vs[2][TSG * LDR];
    __shared__ __attribute__((aligned(16))) float Bs[2][TSG];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = blockIdx.x / a.nsplit, sp = blockIdx.x % a.nsplit;
    const size_t N = (size_t)a.F * a.S;
    const int s_lo = sp * a.spl, s_hi = min(a.S, (sp + 1) * a.spl);
    const int nrnd = (s_hi - s_lo + RND - 1) / RND;
    const size_t row0 = (size_t)(unit / a.F) * N + (size_t)(unit % a.F) * a.S;   // frame start
    const u16 *kin = reinterpret_cast<const u16 *>(a.k), *vin = reinterpret_cast<const u16 *>(a.v);

    floatx4 acc[JPW][NT1];
#pragma unroll
    for (int jb = 0; jb < JPW; ++jb)
#pragma unroll
        for (int ti = 0; ti < NT1; ++ti) acc[jb][ti] = zero4();

    struct Set {                                // native vectors keep the sets in registers
        u32x4 x[SPW][PPT];
        float b[SPW];
    };
    Set sa, sb;
    auto gload = [&](Set &st, int rnd) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int s0 = s_lo + rnd * RND + u * TSG;
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int p = tid + NTH * i;
                const int mat = p / (TSG * SEGS), rem = p % (TSG * SEGS), r = rem / SEGS, sg = rem % SEGS;
                const int s = min(s0 + r, s_hi - 1);
                if (!VONES || !mat) {          // unit values: no V rows
                    // pieces past dd: loaded from the row start (the loads stay
                    // unconditional), then zeroed
                    const bool pad = sg * 8 >= a.dd;
                    st.x[u][i] = *reinterpret_cast<const u32x4 *>((mat ? vin : kin) + (row0 + s) * a.dd +
                                                                  (pad ? 0 : sg * 8));
                    if (pad) st.x[u][i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            const int s = s0 + (tid & (TSG - 1));
            const float bt = CROSS ? a.scale : a.beta[row0 + min(s, s_hi - 1)];
            st.b[u] = s < s_hi ? bt : 0.f;
        }
    };
    auto lstore = [&](const Set &st, int u, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + NTH * i;
            const int mat = p / (TSG * SEGS), rem = p % (TSG * SEGS), r = rem / SEGS, sg = rem % SEGS;
            if (!VONES || !mat) *reinterpret_cast<u32x4 *>((mat ? Vs[buf] : Ks[buf]) + at(r, sg * 8)) = st.x[u][i];
        }
        if (tid < TSG) Bs[buf][tid] = st.b[u];
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const u16 *ks = Ks[buf], *vs = Vs[buf];
#pragma unroll
        for (int kk = 0; kk < TSG / 32; ++kk) {
            // lane (g, c16) receives tokens kk*32 + 8g + e (e < 8) of one column
            const int ra = kk * 32 + 8 * g + (c16 >> 2), cq = 4 * (c16 & 3);
            bf16x8 af[NT1];
#pragma unroll
            for (int ti = 0; ti < NT1; ++ti) {
                const uint2 x0 = __builtin_bit_cast(uint2, ld_tr16(ks + at(ra, ti * 16 + cq)));
                const uint2 x1 = __builtin_bit_cast(uint2, ld_tr16(ks + at(ra + 4, ti * 16 + cq)));
                af[ti] = __builtin_bit_cast(bf16x8, uint4{x0.x, x0.y, x1.x, x1.y});
            }
            const float4 b0 = *reinterpret_cast<const float4 *>(&Bs[buf][kk * 32 + 8 * g]);
            const float4 b1 = *reinterpret_cast<const float4 *>(&Bs[buf][kk * 32 + 8 * g + 4]);
            const float bt[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int jb = 0; jb < JPW; ++jb) {
                const int job = w + NW * jb;
                if (job < NJOB) {
                    const int tj = job % NT1;
                    const u16 *src = job < NT1 && !CROSS ? ks : vs;
                    uint2 x0, x1;
                    if (VONES && job >= NT1) {
                        x0 = x1 = uint2{0x3F803F80u, 0x3F803F80u};      // bf16 ones
                    } else {
                        x0 = __builtin_bit_cast(uint2, ld_tr16(src + at(ra, tj * 16 + cq)));
                        x1 = __builtin_bit_cast(uint2, ld_tr16(src + at(ra + 4, tj * 16 + cq)));
                    }
                    const unsigned u[4] = {x0.x, x0.y, x1.x, x1.y};
                    uint4 hi, lo;
                    unsigned *ph = &hi.x, *pl = &lo.x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float y0 = __uint_as_float(u[e] << 16) * bt[2 * e];
                        const float y1 = __uint_as_float(u[e] & 0xffff0000u) * bt[2 * e + 1];
                        split2_bf16(y0, y1, ph[e], pl[e]);
                    }
                    const bf16x8 bh = __builtin_bit_cast(bf16x8, hi), bl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
                    for (int ti = 0; ti < NT1; ++ti) {
                        acc[jb][ti] = mfma32(af[ti], bh, acc[jb][ti]);
                        acc[jb][ti] = mfma32(af[ti], bl, acc[jb][ti]);
                    }
                }
            }
        }
    };
    // Step n is staged into buffer n & 1 and multiplied after one barrier;
    // the barrier of step n also ends every read of the buffer that step n+1
    // overwrites (read by step n-1).  Rounds come in pairs (set a, then set
    // b at step offset SPW), so buffer parities are fixed at compile time.
    // Round conditions are uniform over the workgroup.
    auto consume = [&](const Set &st, int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            lstore(st, u, (base + u) & 1);
            lds_barrier();
            compute((base + u) & 1);
        }
    };
    gload(sa, 0);
    for (int rnd = 0; rnd < nrnd; rnd += 2) {
        gload(sb, min(rnd + 1, nrnd - 1));
        consume(sa, 0);
        gload(sa, min(rnd + 2, nrnd - 1));
        if (rnd + 1 < nrnd) consume(sb, SPW);
    }
    lds_barrier();
    float *dst = a.part + ((size_t)unit * a.nsplit + sp) * (CROSS ? 1 : 2) * D * D;
#pragma unroll
    for (int jb = 0; jb < JPW; ++jb) {
        const int job = w + NW * jb;
        if (job < NJOB) {
            const int kind = CROSS ? 0 : job / NT1, tj = job % NT1;
#pragma unroll
            for (int ti = 0; ti < NT1; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(size_t)kind * D * D + (ti * 16 + 4 * g + e) * D + tj * 16 + c16] = acc[jb][ti][e];
        }
    }
}

// ---------------------------------------------------------------------------
// G_f, H_f = sum of the partials over token ranges (one float4 per thread)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void frame_reduce_kernel(FrameArgs a) {
    constexpr size_t PU4 = 2 * D * D / 4;       // float4 per unit
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t units = (size_t)a.B * a.H * a.F;
    if (idx >= units * PU4) return;
    const size_t unit = idx / PU4, e = idx % PU4;
    const float4 *p = reinterpret_cast<const float4 *>(a.part) + unit * a.nsplit * PU4 + e;
    float4 s = p[0];
    for (int sp = 1; sp < a.nsplit; ++sp) {
        const float4 x = p[sp * PU4];
        s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
    }
    reinterpret_cast<float4 *>(a.gh)[idx] = s;
}

// G_f (all of it) and the H_f slice of columns j0 .. j0+15 as float4 per
// thread (row idx / 4 of H, columns j0 + 4 (idx % 4) ..).
// The loads of one frame's operands: the gate, then G_f and the H_f slice
// of columns j0 .. j0+15 as float4 per thread (H row idx / 4, columns
// j0 + 4 (idx % 4) ..) from one or two token-range partials.  With two
// ranges the state pass adds them itself (no reduction kernel) when it
// stores them to LDS; both are loaded unconditionally (the second pointer
// repeats the first with one range).  The gate goes out first: waiting for
// it later does not wait for the operand loads behind it.
template <int NG4, int NH4>
struct FrameOps {
    floatx4 g0[NG4], g1[NG4], h0[NH4], h1[NH4];
    float gate;
};
template <int D, int NG4, int NH4>
__device__ __forceinline__ void state_fetch(const float *gate, const float *p0, const float *p1, int j0, int tid,
                                            FrameOps<NG4, NH4> &o) {
    o.gate = *gate;
    const floatx4 *q0 = reinterpret_cast<const floatx4 *>(p0), *q1 = reinterpret_cast<const floatx4 *>(p1);
#pragma unroll
    for (int i = 0; i < NG4; ++i) {
        const int idx = tid + 256 * i;
        if (NG4 * 256 == D * D / 4 || idx < D * D / 4) {
            o.g0[i] = q0[idx];
            o.g1[i] = q1[idx];
        }
    }
#pragma unroll
    for (int i = 0; i < NH4; ++i) {
        const int idx = tid + 256 * i;
        if (NH4 * 256 == D * 4 || idx < D * 4) {
            const int off = (D * D + (idx >> 2) * D + j0) / 4 + (idx & 3);
            o.h0[i] = q0[off];
            o.h1[i] = q1[off];
        }
    }
}

// ---------------------------------------------------------------------------
// sequential frame pass on a 16-column slice of the state.  G_{f+1} and the
// H_{f+1} slice are loaded into registers while frame f is computed.  S_f is
// stored transposed ([column][row]) for the output kernels.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void frame_state_kernel(FrameArgs a) {
    constexpr int LDG = D + 4, LDS_ = 16 + 4;
    constexpr int NRT = D / 16, PERW = (NRT + 3) / 4;
    constexpr int NG4 = (D * D / 4 + 255) / 256, NH4 = (D * 4 + 255) / 256;   // float4 per thread
    __shared__ __attribute__((aligned(16))) float Gs[D * LDG], Sl[D * LDS_], Hs[D * LDS_];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // normaliser stream: one slice, whose 16 columns all carry z (the unit
    // values make every column of H_f equal to b_f)
    const int ncb = a.den ? 1 : D / 16;
    // workgroups go round-robin over the 8 XCDs: block b runs on XCD b % 8,
    // so the slices of one head, which all read its G_f, share an L2
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int bh = (slot / ncb) * 8 + xcd, cb = slot % ncb, j0 = cb * 16;
    if (bh >= a.B * a.H) return;               // padding of the head count to 8

    floatx4 S[PERW];
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        S[n] = zero4();
        const int ti = w + 4 * n;
        if (ti < NRT && a.h0)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = ti * 16 + 4 * (l >> 4) + e, col = j0 + (l & 15);
                if (row < a.dd && (a.den || col < a.dd))
                    S[n][e] = a.den ? a.h0[(size_t)bh * a.dd + row] : a.h0[((size_t)bh * a.dd + row) * a.dd + col];
            }
    }
    // the initial state is complete before the frame loop: otherwise the
    // compiler treats the state registers as possibly pending in every
    // iteration and waits for the operand prefetch before each update
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    FrameOps<NG4, NH4> ops;      // native vectors: arrays of HIP float4 structs end up in scratch
    // Step i folds in the keys and values of frame kf and stores the state
    // that frame of reads.  Forward: kf = of = i.  Reverse (the page's
    // flip-and-shift: q flipped; k, v, beta flipped and shifted by one frame
    // with zeros; the gates flipped and shifted with a gate of 1): step 0
    // only stores the zero state for the last frame, step i >= 1 folds in
    // frame F - i with its own gate and stores the state of frame F - 1 - i.
    const bool rev = a.reverse != 0;
    // G_f and the H_f slice of frame f: the reduced sums, or (two ranges, no
    // reduction kernel) the two partials added here
    const bool two = a.nsplit == 2;
    const float *src = two ? a.part : a.gh;
    const int nsrc = two ? 2 : 1;
    const float w1 = two ? 1.f : 0.f;
    auto fetch = [&](int f) __attribute__((always_inline)) {
        const float *p0 = src + ((size_t)bh * a.F + f) * nsrc * 2 * D * D;
        state_fetch<D, NG4, NH4>(a.g + (size_t)bh * a.F + f, p0, p0 + (two ? 2 * D * D : 0), j0, tid, ops);
    };
    if ((rev ? 1 : 0) < a.F)
        fetch(rev ? a.F - 1 : 0);
    for (int i = 0; i < a.F; ++i) {
        const bool upd = !rev || i > 0;          // uniform over the workgroup
        const int of = rev ? a.F - 1 - i : i;    // (operands: frame rev ? F - i : i, fetched ahead)
        if (upd) {
#pragma unroll
            for (int j = 0; j < NG4; ++j) {
                const int idx = tid + 256 * j;
                if (idx < D * D / 4) {
                    const int r = (idx * 4) / D, c = (idx * 4) % D;
                    *reinterpret_cast<floatx4 *>(Gs + r * LDG + c) = ops.g0[j] + w1 * ops.g1[j];
                }
            }
#pragma unroll
            for (int j = 0; j < NH4; ++j) {
                const int idx = tid + 256 * j;
                if (idx < D * 4)
                    *reinterpret_cast<floatx4 *>(Hs + (idx >> 2) * LDS_ + 4 * (idx & 3)) = ops.h0[j] + w1 * ops.h1[j];
            }
        }
        // current state slice into LDS as the B operand ([k][col])
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sl[(ti * 16 + 4 * (l >> 4) + e) * LDS_ + (l & 15)] = S[n][e];
        }
        const float dec = upd ? expf(ops.gate) : 1.f;   // this frame's gate, loaded with its operands
        lds_barrier();                  // the prefetch below stays in flight across barriers
        if (upd && i + 1 < a.F)
            fetch(rev ? a.F - 1 - i : i + 1);
        const size_t unit = (size_t)bh * a.F + of;
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT) {
                if (upd) {
                    floatx4 gs = zero4();
                    mma_f32_bn(gs, Gs + ti * 16 * LDG, LDG, Sl, LDS_, D);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[n][e] = dec * (S[n][e] - gs[e]) + Hs[(ti * 16 + 4 * (l >> 4) + e) * LDS_ + (l & 15)];
                }
                *reinterpret_cast<float4 *>(a.sf + (unit * D + j0 + (l & 15)) * D + ti * 16 + 4 * (l >> 4)) =
                    float4{S[n][0], S[n][1], S[n][2], S[n][3]};
            }
        }
        lds_barrier();
    }
    if (a.hT) {
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = ti * 16 + 4 * (l >> 4) + e, col = j0 + (l & 15);
                    if (row >= a.dd) continue;
                    if (!a.den) {
                        if (col < a.dd) a.hT[((size_t)bh * a.dd + row) * a.dd + col] = S[n][e];
                    } else if ((l & 15) == 0) {
                        a.hT[(size_t)bh * a.dd + row] = S[n][e];
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// out_s = scale * S_f^T q_s for a tile of up to 64 tokens of one frame
// (general path: fp32 inputs, D = 16)
// ---------------------------------------------------------------------------
template <bool F32IN, int D>
__global__ __launch_bounds__(256) void frame_out_kernel(FrameArgs a) {
    using Op = typename OpT<F32IN>::type;
    constexpr int TT = 64;
    constexpr int PAD = F32IN ? 4 : 8, LDQ = D + PAD, LDT = D + PAD;
    constexpr int NTILE = (TT / 16) * (D / 16), PERW = (NTILE + 3) / 4;
    __shared__ __attribute__((aligned(16))) Op Qs[TT * LDQ], SH[D * LDT], SL[F32IN ? 1 : D * LDT];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntt = (a.S + TT - 1) / TT;
    const int unit = blockIdx.x / ntt, tt = blockIdx.x % ntt;
    const int bh = unit / a.F, f = unit % a.F;
    const size_t N = (size_t)a.F * a.S;
    const size_t row0 = (size_t)bh * N + (size_t)f * a.S + (size_t)tt * TT;
    const int nrows = min(TT, a.S - tt * TT);

    // S_f transposed ([j][i], as stored) as the B operand
    const float *sf = a.sf + (size_t)unit * D * D;
    for (int idx = tid; idx < D * D; idx += 256) put_op<F32IN>(SH, SL, (idx / D) * LDT + idx % D, sf[idx]);
    constexpr int SEGS = D / 8;
    for (int idx = tid; idx < TT * SEGS; idx += 256) {
        const int r = idx / SEGS, i0 = (idx % SEGS) * 8;
        U16x8 raw[F32IN ? 2 : 1];
        if (r < nrows && i0 < a.dd) {
            const unsigned char *src = reinterpret_cast<const unsigned char *>(a.q) +
                                       ((row0 + r) * a.dd + i0) * (F32IN ? 4 : 2);
            raw[0] = reinterpret_cast<const U16x8 *>(src)[0];
            if constexpr (F32IN) raw[1] = reinterpret_cast<const U16x8 *>(src)[1];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                raw[0].v[e] = 0;
                if constexpr (F32IN) raw[1].v[e] = 0;
            }
        }
        U16x8 *dst = reinterpret_cast<U16x8 *>(Qs + r * LDQ + i0);
        dst[0] = raw[0];
        if constexpr (F32IN) dst[1] = raw[1];
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        const int tile = w + 4 * n;
        if (tile < NTILE) {
            const int ti = tile / (D / 16), tj = tile % (D / 16);
            floatx4 acc = zero4();
            if constexpr (F32IN) mma_f32(acc, Qs + ti * 16 * LDQ, LDQ, SH + tj * 16 * LDT, LDT, D);
            else mma_bf16_split(acc, Qs + ti * 16 * LDQ, nullptr, LDQ, SH + tj * 16 * LDT, SL + tj * 16 * LDT, LDT, D);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = ti * 16 + 4 * (l >> 4) + e;
                if (r < nrows && tj * 16 < a.dd) a.out[(row0 + r) * a.dd + tj * 16 + (l & 15)] = a.scale * acc[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// out for bf16 inputs and D >= 32, computed transposed: out^T = S_f^T Q^T.
// A = S_f^T (hi + lo bf16, staged once per workgroup in LDS from the stored
// transpose), B = Q^T: lane (g, c16) needs 8 consecutive features of token
// c16, one 16-byte load straight from the (token, D) rows.  The accumulator
// gives each lane 4 consecutive outputs of one token: one 16-byte store.
// A workgroup (eight waves) covers 512 tokens of one frame, each wave 64 of
// them, so S_f is staged once per 512 tokens.
// ---------------------------------------------------------------------------
constexpr int OUT_WAVES = 8, OUT_TOK = OUT_WAVES * 64;   // 64 tokens per wave

template <int D>
__global__ __launch_bounds__(64 * OUT_WAVES) void frame_out_bf16_kernel(FrameArgs a) {
    constexpr int NT1 = D / 16, NK = D / 32, LDT = D + 8, SUB = 4;   // SUB tiles of 16 tokens per wave
    static_assert(D >= 32, "32-deep k steps");
    __shared__ __attribute__((aligned(16))) u16 SH[D * LDT], SL[D * LDT];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntt = (a.S + OUT_TOK - 1) / OUT_TOK;
    // the token tiles of one (head, frame) read the same S_f: keep them on
    // one XCD (block b runs on XCD b % 8) so that it is fetched into one L2
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int unit = (slot / ntt) * 8 + xcd, tb = slot % ntt;
    if (unit >= a.B * a.H * a.F) return;        // padding of the unit count to 8
    const size_t N = (size_t)a.F * a.S;
    const size_t row0 = (size_t)(unit / a.F) * N + (size_t)(unit % a.F) * a.S;
    const int t0 = tb * OUT_TOK + w * (SUB * 16);          // this wave's first token in the frame
    const u16 *qin = reinterpret_cast<const u16 *>(a.q);

    // Q^T fragments of this wave's tokens go out first
    bf16x8 bq[SUB][NK];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
        const int t = t0 + u * 16 + c16;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            uint4 x = uint4{0u, 0u, 0u, 0u};
            if (t < a.S && kk * 32 + 8 * g < a.dd)
                x = *reinterpret_cast<const uint4 *>(qin + (row0 + t) * a.dd + kk * 32 + 8 * g);
            bq[u][kk] = __builtin_bit_cast(bf16x8, x);
        }
    }
    // S_f^T rows (output feature i, input features contiguous) split into LDS
    const float4 *sf = reinterpret_cast<const float4 *>(a.sf + (size_t)unit * D * D);
    for (int idx = tid; idx < D * D / 4; idx += 64 * OUT_WAVES) {
        const float4 x = sf[idx];
        const int r = (idx * 4) / D, c = (idx * 4) % D;
        uint2 hi, lo;
        split2_bf16(x.x, x.y, hi.x, lo.x);
        split2_bf16(x.z, x.w, hi.y, lo.y);
        *reinterpret_cast<uint2 *>(SH + r * LDT + c) = hi;
        *reinterpret_cast<uint2 *>(SL + r * LDT + c) = lo;
    }
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < NT1; ++ti) {
        bf16x8 ah[NK], al[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int o = (ti * 16 + c16) * LDT + kk * 32 + 8 * g;
            ah[kk] = ld8(SH + o);
            al[kk] = ld8(SL + o);
        }
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            floatx4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                acc = mfma32(ah[kk], bq[u][kk], acc);
                acc = mfma32(al[kk], bq[u][kk], acc);
            }
            const int t = t0 + u * 16 + c16;
            if (t < a.S && ti * 16 < a.dd)
                *reinterpret_cast<float4 *>(a.out + (row0 + t) * a.dd + ti * 16 + 4 * g) =
                    float4{a.scale * acc[0], a.scale * acc[1], a.scale * acc[2], a.scale * acc[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// normaliser stream read-out: den_s = z_f . q_s, z_f = column 0 of S_f (the
// first row of the stored transpose).  Each token's row is split over L
// consecutive lanes (16-byte pieces, coalesced), partial dot products summed
// over the L lanes by DPP; 256-thread workgroups walk 64/L tokens per wave
// per step over one frame.
// ---------------------------------------------------------------------------
template <bool F32IN, int D>
__global__ __launch_bounds__(256) void frame_den_kernel(FrameArgs a) {
    constexpr int EPP = F32IN ? 4 : 8;            // elements per 16-byte piece
    constexpr int L = D / EPP;                    // lanes per token
    constexpr int TPW = 64 / L;                   // tokens per wave and step
    static_assert(L >= 2 && L <= 64 && 64 % L == 0, "lanes per token");
    __shared__ __attribute__((aligned(16))) float zs[D];
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int ntb = (a.S + 255) / 256;
    const int unit = blockIdx.x / ntb, tb = blockIdx.x % ntb;
    const size_t N = (size_t)a.F * a.S;
    const size_t row0 = (size_t)(unit / a.F) * N + (size_t)(unit % a.F) * a.S;
    if (tid < D) zs[tid] = a.sf[(size_t)unit * D * D + tid];
    __syncthreads();
    const int pc = l % L;                          // this lane's piece of the row
    float z[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) z[e] = zs[pc * EPP + e];
    for (int t = tb * 256 + w * TPW + l / L; t < min(a.S, tb * 256 + 256); t += 4 * TPW) {
        float x[EPP];
        const bool pad = pc * EPP >= a.dd;       // loaded from the row start, then zeroed
        const size_t off = (row0 + t) * a.dd + (pad ? 0 : pc * EPP);
        if constexpr (F32IN) {
            const float4 p0 = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + off);
            x[0] = p0.x; x[1] = p0.y; x[2] = p0.z; x[3] = p0.w;
        } else {
            const U16x8 r = *reinterpret_cast<const U16x8 *>(reinterpret_cast<const u16 *>(a.q) + off);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(r.v[e]);
        }
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc += x[e] * z[e];
        if (pad) acc = 0.f;
        acc = lane_group_sum<L>(acc);
        if (pc == 0) a.out[row0 + t] = a.scale * acc;
    }
}

// Token ranges of the gram kernels: about one eight-wave workgroup per
// compute unit, whole rounds of staged steps per range.
int frame_nsplit(int B, int H, int F, int S, int D, int *spl_out) {
    const long units = (long)B * H * F;
    const int RND = gram_round(D);
    const int maxsp = (S + RND - 1) / RND;
    long want = units > 0 ? (256 + units - 1) / units : 1;
    if (want > maxsp) want = maxsp;
    if (want < 1) want = 1;
    const int per = (int)((S + want - 1) / want);
    const int spl = (per + RND - 1) / RND * RND;
    if (spl_out) *spl_out = spl;
    return (S + spl - 1) / spl;
}

size_t frame_workspace(int B, int H, int F, int S, int D) {
    const int ns = frame_nsplit(B, H, F, S, D, nullptr);
    const size_t units = (size_t)B * H * F;
    // partials (only with more than one range), G_f and H_f, S_f
    return (ns > 1 ? units * ns * 2 * D * D : 0) * sizeof(float) + units * 2 * D * D * sizeof(float) +
           units * D * D * sizeof(float);
}

template <bool F32IN, int D, bool VONES>
hipError_t launch_gram(const FrameArgs &a, hipStream_t s) {
    const int units = a.B * a.H * a.F;
    if constexpr (F32IN)
        hipLaunchKernelGGL((frame_gram_kernel<true, D, VONES>), dim3(units * a.nsplit), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((frame_gram_bf16_kernel<D, VONES>), dim3(units * a.nsplit), dim3(64 * gram_waves<D>()),
                           0, s, a);
    return hipGetLastError();
}

template <bool F32IN, int D>
hipError_t launch_frame(FrameArgs a, hipStream_t s) {
    const int units = a.B * a.H * a.F;
    hipError_t e = a.den ? launch_gram<F32IN, D, true>(a, s) : launch_gram<F32IN, D, false>(a, s);
    if (e != hipSuccess) return e;
    if (a.nsplit > 2) {                        // two ranges: the state pass adds them
        const size_t n4 = (size_t)units * 2 * D * D / 4;
        hipLaunchKernelGGL((frame_reduce_kernel<D>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((frame_state_kernel<D>), dim3((a.B * a.H + 7) / 8 * 8 * (a.den ? 1 : D / 16)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.den) {
        hipLaunchKernelGGL((frame_den_kernel<F32IN, D>), dim3(units * ((a.S + 255) / 256)), dim3(256), 0, s, a);
    } else if constexpr (!F32IN && D >= 32) {
        const int ntt = (a.S + OUT_TOK - 1) / OUT_TOK;
        hipLaunchKernelGGL((frame_out_bf16_kernel<D>), dim3((units + 7) / 8 * 8 * ntt), dim3(64 * OUT_WAVES), 0, s, a);
    } else {
        const int ntt = (a.S + 63) / 64;
        hipLaunchKernelGGL((frame_out_kernel<F32IN, D>), dim3(units * ntt), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// hT = h0 (or 0 without h0): the final state of a scan over no frames.
__global__ __launch_bounds__(256) void state_copy_kernel(const float *h0, float *hT, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

// Kernel head width that runs heads of width dd: the next power of two
// (16 ... 128; the kernels read the features past dd as zero and never store
// them), or 0 when dd is not a multiple of 16 up to 128.
int padded_head_width(int dd) {
    if (dd <= 0 || dd % 16 || dd > 128) return 0;
    int D = 16;
    while (D < dd) D *= 2;
    return D;
}

// Shared body of the two scan entry points (checks, work space carving, launch).
int frame_entry(const char *name, const void *q, const void *k, const void *v, const float *beta,
                const float *log_decay, float scale, const float *h0, float *hT, float *out, int B, int H, int F,
                int S, int dd, int dtype, int reverse, int den, void *workspace, size_t workspace_bytes,
                void *stream) {
    GDN_REQUIRE(B >= 0 && H >= 0 && F >= 0, GDN_EINVAL, "%s: negative size (B=%d H=%d F=%d)", name, B, H, F);
    GDN_REQUIRE(S >= 1, GDN_EINVAL, "%s: S=%d (at least one token per frame)", name, S);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    const int D = padded_head_width(dd);
    GDN_REQUIRE(D > 0, GDN_EUNSUPPORTED, "%s: D=%d (supported: multiples of 16 up to 128)", name, dd);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    GDN_REQUIRE(reverse == 0 || reverse == 1, GDN_EINVAL, "%s: reverse=%d (0 or 1)", name, reverse);
    GDN_REQUIRE(!reverse || (!h0 && !hT), GDN_EUNSUPPORTED,
                "%s: the reverse scan takes no initial state and returns no final state", name);
    if ((long)B * H == 0) return GDN_OK;
    const bool work = (long)F > 0;
    if (work) {
        GDN_REQUIRE(q && k && (den || v) && beta && log_decay && out, GDN_EINVAL, "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && (den || gdn::aligned(v, 16)) &&
                        gdn::aligned(out, den ? 4 : 16),
                    GDN_EINVAL, "%s: q, k, v must be 16-byte aligned, out %d-byte aligned", name, den ? 4 : 16);
        GDN_REQUIRE(gdn::aligned(beta, 4) && gdn::aligned(log_decay, 4), GDN_EINVAL,
                    "%s: beta and log_decay must be 4-byte aligned", name);
    }
    GDN_REQUIRE(!h0 || gdn::aligned(h0, 4), GDN_EINVAL, "%s: initial state misaligned", name);
    GDN_REQUIRE(!hT || gdn::aligned(hT, 4), GDN_EINVAL, "%s: final state misaligned", name);
    const size_t need = frame_workspace(B, H, F, S, D);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!work) {
        // no frames: the final state is the initial one
        if (!hT) return GDN_OK;
        // (a kernel rather than a memset or copy node, so that a captured
        // graph holds kernels only)
        const size_t n = (size_t)B * H * dd * (den ? 1 : dd);
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h0, hT, n);
        return check_hip(hipGetLastError(), name);
    }
    FrameArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = log_decay;
    a.h0 = h0;
    a.hT = hT;
    a.out = out;
    a.B = B;
    a.H = H;
    a.F = F;
    a.S = S;
    a.nsplit = frame_nsplit(B, H, F, S, D, &a.spl);
    a.dd = dd;
    a.scale = scale;
    a.reverse = reverse;
    a.den = den;
    const size_t units = (size_t)B * H * F;
    float *ws = reinterpret_cast<float *>(workspace);
    a.gh = ws;
    a.sf = a.gh + units * 2 * D * D;
    a.part = a.nsplit > 1 ? a.sf + units * D * D : a.gh;
    const bool f32 = dtype == GDN_DTYPE_F32;
    hipError_t e;
    switch (D) {
        case 16: e = f32 ? launch_frame<true, 16>(a, s) : launch_frame<false, 16>(a, s); break;
        case 32: e = f32 ? launch_frame<true, 32>(a, s) : launch_frame<false, 32>(a, s); break;
        case 64: e = f32 ? launch_frame<true, 64>(a, s) : launch_frame<false, 64>(a, s); break;
        default: e = f32 ? launch_frame<true, 128>(a, s) : launch_frame<false, 128>(a, s); break;
    }
    return check_hip(e, name);
}

// ===========================================================================
// Backward of the frame-synchronous scan (reverse mode through the frame
// steps).  With S_f = (I - G_f) P_f + H_f, P_f = e^{g_f} S_{f-1} and
// out_s = scale S_f^T q_s (s in frame f), let X_f = dL/dS_f including the
// read-out of frame f: X_f = dS_f + A_f with A_f = scale Q_f^T dO_f and dS_f
// the gradient carried back from frame f + 1 (dhT after the last frame).
// Every token of frame f predicts from P_f, so the prediction terms of the
// frame sum to G_f X_f, and
//   X_{f-1} = e^{g_f} (I - G_f) X_f + A_{f-1},   dh0 = e^{g_0} (I - G_0) X_0,
//   dg_f = <(I - G_f) X_f, P_f>,
// and per token s of frame f, with u_s = X_f^T k_s and r_s = v_s - P_f^T k_s:
//   dq_s = scale S_f do_s,  dv_s = beta_s u_s,  dbeta_s = u_s . r_s,
//   dk_s = beta_s (X_f r_s - P_f u_s).
// Kernels: the forward's gram and state passes (G_f, S_f), the gram kernel
// in CROSS mode (A_f), frame_bstate_kernel (X_f, dg partials, dh0) and
// frame_bgrad_kernel (token gradients, dg).
// ===========================================================================
struct FrameBwdArgs {
    FrameArgs a;             // q, k, v, beta, g, h0, scale; gh (G_f), sf (S_f), nsplit, spl
    const void *dout;        // (B, H, N, D) as q
    const float *dhT;        // (B, H, D, D) or null
    const float *apart;      // [B*H*F][nsplit][D][D] partial A_f
    float *xf;               // [B*H][F][D][D] X_f, transposed ([column][row])
    float *dgp;              // [B*H][F][D/16] gate gradient by state column slice
    float *dq, *dk, *dv, *dbeta, *dg, *dh0;
};

// X_f backwards over the frames, per (b, h, 16-column slice of X), fp32 MFMA
// (the frame state pass's form).  Stores every X_f (transposed, as the
// forward stores S_f), the slice's share of dg_f, and dh0.
template <int D>
__global__ __launch_bounds__(256) void frame_bstate_kernel(FrameBwdArgs ba) {
    constexpr int LDG = D + 4, LDS_ = 16 + 4;
    constexpr int NRT = D / 16, PERW = (NRT + 3) / 4;
    __shared__ __attribute__((aligned(16))) float Gs[D * LDG], Xl[D * LDS_];
    __shared__ float red[4];
    const FrameArgs &a = ba.a;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int ncb = D / 16;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int bh = (slot / ncb) * 8 + xcd, cb = slot % ncb, j0 = cb * 16;
    if (bh >= a.B * a.H) return;
    const int col = j0 + (l & 15);
    auto row_of = [&](int ti, int e) { return ti * 16 + 4 * (l >> 4) + e; };

    floatx4 X[PERW];
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        X[n] = zero4();
        const int ti = w + 4 * n;
        if (ti < NRT && ba.dhT)
#pragma unroll
            for (int e = 0; e < 4; ++e) X[n][e] = ba.dhT[((size_t)bh * D + row_of(ti, e)) * D + col];
    }
    for (int f = a.F - 1; f >= 0; --f) {
        const size_t unit = (size_t)bh * a.F + f;
        // G_f into LDS; X += A_f (sum of the token-range partials)
        const floatx4 *gsrc = reinterpret_cast<const floatx4 *>(a.gh + unit * 2 * D * D);
        for (int idx = tid; idx < D * D / 4; idx += 256) {
            const int r = (idx * 4) / D, c = (idx * 4) % D;
            *reinterpret_cast<floatx4 *>(Gs + r * LDG + c) = gsrc[idx];
        }
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
                for (int sp = 0; sp < a.nsplit; ++sp) {
                    const float *ap = ba.apart + (unit * a.nsplit + sp) * D * D;
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[n][e] += ap[row_of(ti, e) * D + col];
                }
        }
        // X_f out (transposed) and into LDS as the B operand
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT) {
                *reinterpret_cast<float4 *>(ba.xf + (unit * D + col) * D + ti * 16 + 4 * (l >> 4)) =
                    float4{X[n][0], X[n][1], X[n][2], X[n][3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) Xl[row_of(ti, e) * LDS_ + (l & 15)] = X[n][e];
            }
        }
        __syncthreads();
        const float dec = expf(a.g[unit]);
        // P_f = e^{g_f} S_{f-1}: the stored S_{f-1} (transposed), or h0 for f = 0
        float part = 0.f;
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT) {
                floatx4 gx = zero4();
                mma_f32_bn(gx, Gs + ti * 16 * LDG, LDG, Xl, LDS_, D);
                floatx4 pv = zero4();
                if (f > 0) {
                    const float4 x = *reinterpret_cast<const float4 *>(a.sf + ((unit - 1) * D + col) * D + ti * 16 +
                                                                       4 * (l >> 4));
                    pv = floatx4{x.x, x.y, x.z, x.w};
                } else if (a.h0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv[e] = a.h0[((size_t)bh * D + row_of(ti, e)) * D + col];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = X[n][e] - gx[e];
                    part += y * pv[e];
                    X[n][e] = dec * y;
                }
            }
        }
        // dg_f share of this slice: dec * sum (I - G_f) X_f o S_{f-1}
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off, 64);
        if (l == 0) red[w] = part;
        __syncthreads();
        if (tid == 0) ba.dgp[unit * ncb + cb] = dec * (((red[0] + red[1]) + red[2]) + red[3]);
    }
    if (ba.dh0) {
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
#pragma unroll
                for (int e = 0; e < 4; ++e) ba.dh0[((size_t)bh * D + row_of(ti, e)) * D + col] = X[n][e];
        }
    }
}

// Token gradients of one frame, 512 tokens per workgroup (8 waves x 4 tiles
// of 16), bf16 inputs, D >= 32.  Products are taken transposed so each lane
// holds 4 consecutive features of one token (16-byte stores):
//   u^T = X_f^T K^T,  r^T = V^T - P_f^T K^T           (A: X^T, P^T rows)
//   dk^T = beta (X_f r^T - P_f u^T)                    (A: X, P rows, read
//                                                      transposed; B: r^T, u^T
//                                                      from the accumulators,
//                                                      permuted k order)
//   dq^T = scale S_f dO^T                              (A: S rows, read transposed)
// X^T, P^T (then S^T) are staged in LDS as hi/lo bf16 from the stored
// transposes.  The workgroup of each frame's first block also adds the dg
// shares of the state slices.
constexpr int BG_WAVES = 8, BG_TOK = BG_WAVES * 64;

template <int D>
__global__ __launch_bounds__(64 * BG_WAVES) void frame_bgrad_kernel(FrameBwdArgs ba) {
    constexpr int NT1 = D / 16, NK = D / 32, LDT = D + 8, SUB = 4;
    static_assert(D >= 32, "32-deep k steps");
    __shared__ __attribute__((aligned(16))) u16 AH[D * LDT], AL[D * LDT], BH[D * LDT], BL[D * LDT];
    const FrameArgs &a = ba.a;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntt = (a.S + BG_TOK - 1) / BG_TOK;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int unit = (slot / ntt) * 8 + xcd, tb = slot % ntt;
    if (unit >= a.B * a.H * a.F) return;
    const int bh = unit / a.F, f = unit % a.F;
    const size_t N = (size_t)a.F * a.S;
    const size_t row0 = (size_t)bh * N + (size_t)f * a.S;
    const int t0 = tb * BG_TOK + w * (SUB * 16);
    const u16 *kin = reinterpret_cast<const u16 *>(a.k), *vin = reinterpret_cast<const u16 *>(a.v);
    const u16 *oin = reinterpret_cast<const u16 *>(ba.dout);
    const float dec = expf(a.g[unit]);
    if (tb == 0 && tid == 0) {
        float s = 0.f;
        for (int cb = 0; cb < NT1; ++cb) s += ba.dgp[(size_t)unit * NT1 + cb];
        ba.dg[unit] = s;
    }
    // stage a transposed D x D matrix (src[r][c], r = column of the state)
    // times `mul` as hi/lo bf16 rows
    auto stage = [&](u16 *hi, u16 *lo, const float *src, float mul) {
        const float4 *p = reinterpret_cast<const float4 *>(src);
        for (int idx = tid; idx < D * D / 4; idx += 64 * BG_WAVES) {
            const float4 x = p[idx];
            const int r = (idx * 4) / D, c = (idx * 4) % D;
            uint2 h, o;
            split2_bf16(mul * x.x, mul * x.y, h.x, o.x);
            split2_bf16(mul * x.z, mul * x.w, h.y, o.y);
            *reinterpret_cast<uint2 *>(hi + r * LDT + c) = h;
            *reinterpret_cast<uint2 *>(lo + r * LDT + c) = o;
        }
    };
    stage(AH, AL, ba.xf + (size_t)unit * D * D, 1.f);            // X_f^T
    if (f > 0) {
        stage(BH, BL, a.sf + (size_t)(unit - 1) * D * D, dec);   // P_f^T = e^{g_f} S_{f-1}^T
    } else {
        for (int idx = tid; idx < D * D; idx += 64 * BG_WAVES) {
            const int r = idx / D, c = idx % D;                  // P^T[r][c] = e^{g} h0[c][r]
            const float x = a.h0 ? dec * a.h0[((size_t)bh * D + c) * D + r] : 0.f;
            u16 h, o;
            split_bf16(x, h, o);
            BH[r * LDT + c] = h;
            BL[r * LDT + c] = o;
        }
    }
    // B operand fragments of this wave's tokens (lane (g, c16): token c16 of
    // tile u, features 32 kk + 8 g .. +7): k, and dO in the dq phase
    auto row_frag8 = [&](const u16 *in, int t, int kk) {
        uint4 x = uint4{0u, 0u, 0u, 0u};
        if (t < a.S) x = *reinterpret_cast<const uint4 *>(in + (row0 + t) * D + kk * 32 + 8 * g);
        return __builtin_bit_cast(bf16x8, x);
    };
    __syncthreads();
    // A operand of rows i of a matrix M whose transpose is staged (M^T[j][i]):
    // lane (g, c16) gets M[i0 + c16][j] for j = r0 .. r0+3 and r1 .. r1+3
    auto tr_a = [&](const u16 *mt, int r0, int r1, int i0) {
        const uint2 x0 = __builtin_bit_cast(uint2, ld_tr16(mt + (r0 + (c16 >> 2)) * LDT + i0 + 4 * (c16 & 3)));
        const uint2 x1 = __builtin_bit_cast(uint2, ld_tr16(mt + (r1 + (c16 >> 2)) * LDT + i0 + 4 * (c16 & 3)));
        return __builtin_bit_cast(bf16x8, uint4{x0.x, x0.y, x1.x, x1.y});
    };
#pragma unroll 1
    for (int u = 0; u < SUB; ++u) {
        // (the staged operands are read again for every tile: a compiler fence
        // keeps their loads from being hoisted out of the loop into registers)
        asm volatile("" ::: "memory");
        const int t = t0 + u * 16 + c16;        // this lane's token (B operand column)
        bf16x8 bk[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) bk[kk] = row_frag8(kin, t, kk);
        const float bt = t < a.S ? a.beta[row0 + t] : 0.f;
        // u^T and r^T tiles (rows j = jt*16 + 4g + e, column token c16)
        floatx4 ut[NT1], rt[NT1];
#pragma unroll
        for (int jt = 0; jt < NT1; ++jt) {
            floatx4 ua = zero4(), pa = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int o = (jt * 16 + c16) * LDT + kk * 32 + 8 * g;
                ua = mfma32(ld8(AH + o), bk[kk], ua);
                ua = mfma32(ld8(AL + o), bk[kk], ua);
                pa = mfma32(ld8(BH + o), bk[kk], pa);
                pa = mfma32(ld8(BL + o), bk[kk], pa);
            }
            uint2 vr = uint2{0u, 0u};
            if (t < a.S) vr = *reinterpret_cast<const uint2 *>(vin + (row0 + t) * D + jt * 16 + 4 * g);
            const floatx4 vv = floatx4{__builtin_bit_cast(float, vr.x << 16), __builtin_bit_cast(float, vr.x & 0xffff0000u),
                                       __builtin_bit_cast(float, vr.y << 16), __builtin_bit_cast(float, vr.y & 0xffff0000u)};
            ut[jt] = ua;
#pragma unroll
            for (int e = 0; e < 4; ++e) rt[jt][e] = vv[e] - pa[e];
        }
        // dv = beta u, dbeta = u . r
        float db = 0.f;
#pragma unroll
        for (int jt = 0; jt < NT1; ++jt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) db += ut[jt][e] * rt[jt][e];
            if (t < a.S)
                *reinterpret_cast<float4 *>(ba.dv + (row0 + t) * D + jt * 16 + 4 * g) =
                    float4{bt * ut[jt][0], bt * ut[jt][1], bt * ut[jt][2], bt * ut[jt][3]};
        }
        db += __shfl_xor(db, 16, 64);
        db += __shfl_xor(db, 32, 64);
        if (g == 0 && t < a.S) ba.dbeta[row0 + t] = db;
        // dk^T = beta (X r^T - P u^T): r^T, u^T as B operands (hi + lo), k = j in
        // the permuted order of two accumulator tiles
        bf16x8 rh[NK], rl[NK], uh[NK], ul[NK];
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            frag_split(rt[2 * m], rt[2 * m + 1], rh[m], rl[m]);
            frag_split(ut[2 * m], ut[2 * m + 1], uh[m], ul[m]);
        }
#pragma unroll
        for (int it = 0; it < NT1; ++it) {
            floatx4 acc = zero4();
#pragma unroll
            for (int m = 0; m < NK; ++m) {
                const int r0 = m * 32 + 4 * g, r1 = r0 + 16;
                const bf16x8 xh = tr_a(AH, r0, r1, it * 16), xl = tr_a(AL, r0, r1, it * 16);
                acc = mfma32(xh, rh[m], acc);
                acc = mfma32(xh, rl[m], acc);
                acc = mfma32(xl, rh[m], acc);
                const bf16x8 ph = tr_a(BH, r0, r1, it * 16), pl = tr_a(BL, r0, r1, it * 16);
                floatx4 nacc = zero4();
                nacc = mfma32(ph, uh[m], nacc);
                nacc = mfma32(ph, ul[m], nacc);
                nacc = mfma32(pl, uh[m], nacc);
                acc -= nacc;
            }
            if (t < a.S)
                *reinterpret_cast<float4 *>(ba.dk + (row0 + t) * D + it * 16 + 4 * g) =
                    float4{bt * acc[0], bt * acc[1], bt * acc[2], bt * acc[3]};
        }
    }
    // dq^T = scale S_f dO^T: S_f^T staged over X^T
    __syncthreads();
    stage(AH, AL, a.sf + (size_t)unit * D * D, 1.f);
    __syncthreads();
#pragma unroll 1
    for (int u = 0; u < SUB; ++u) {
        asm volatile("" ::: "memory");
        const int t = t0 + u * 16 + c16;
        bf16x8 bo[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) bo[kk] = row_frag8(oin, t, kk);
#pragma unroll
        for (int it = 0; it < NT1; ++it) {
            floatx4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int r0 = kk * 32 + 8 * g;
                acc = mfma32(tr_a(AH, r0, r0 + 4, it * 16), bo[kk], acc);
                acc = mfma32(tr_a(AL, r0, r0 + 4, it * 16), bo[kk], acc);
            }
            if (t < a.S)
                *reinterpret_cast<float4 *>(ba.dq + (row0 + t) * D + it * 16 + 4 * g) =
                    float4{a.scale * acc[0], a.scale * acc[1], a.scale * acc[2], a.scale * acc[3]};
        }
    }
}

// Work space of the backward: the forward's (partials, G_f and H_f, S_f),
// then the partial A_f, X_f, and the dg shares.
size_t frame_bwd_workspace(int B, int H, int F, int S, int D) {
    const int ns = frame_nsplit(B, H, F, S, D, nullptr);
    const size_t units = (size_t)B * H * F;
    return (units * ns * 2 * D * D + units * 2 * D * D + units * D * D + units * ns * D * D + units * D * D +
            units * (D / 16)) * sizeof(float);
}

template <int D>
hipError_t launch_frame_bwd(FrameBwdArgs ba, hipStream_t s) {
    FrameArgs &a = ba.a;
    const int units = a.B * a.H * a.F;
    // forward: G_f, H_f (summed over the token ranges) and S_f
    hipError_t e = launch_gram<false, D, false>(a, s);
    if (e != hipSuccess) return e;
    if (a.nsplit > 1) {
        const size_t n4 = (size_t)units * 2 * D * D / 4;
        hipLaunchKernelGGL((frame_reduce_kernel<D>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    FrameArgs fa = a;
    fa.nsplit = 1;                              // G_f, H_f reduced
    fa.part = fa.gh;
    hipLaunchKernelGGL((frame_state_kernel<D>), dim3((a.B * a.H + 7) / 8 * 8 * (D / 16)), dim3(256), 0, s, fa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // A_f = scale Q_f^T dO_f (partials)
    FrameArgs ca = a;
    ca.k = a.q;
    ca.v = ba.dout;
    ca.part = const_cast<float *>(ba.apart);
    hipLaunchKernelGGL((frame_gram_bf16_kernel<D, false, true>), dim3(units * a.nsplit), dim3(64 * gram_waves<D>()),
                       0, s, ca);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((frame_bstate_kernel<D>), dim3((a.B * a.H + 7) / 8 * 8 * (D / 16)), dim3(256), 0, s, ba);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ntt = (a.S + BG_TOK - 1) / BG_TOK;
    hipLaunchKernelGGL((frame_bgrad_kernel<D>), dim3((units + 7) / 8 * 8 * ntt), dim3(64 * BG_WAVES), 0, s, ba);
    return hipGetLastError();
}

int frame_bwd_entry(const void *q, const void *k, const void *v, const float *beta, const float *log_decay,
                    float scale, const float *h0, const void *dout, const float *dhT, float *dq, float *dk, float *dv,
                    float *dbeta, float *dlog_decay, float *dh0, int B, int H, int F, int S, int D, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream) {
    const char *name = "gdn_recurrent_bwd";
    GDN_REQUIRE(B >= 0 && H >= 0 && F >= 0, GDN_EINVAL, "%s: negative size (B=%d H=%d F=%d)", name, B, H, F);
    GDN_REQUIRE(S >= 1, GDN_EINVAL, "%s: S=%d (at least one token per frame)", name, S);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(dtype == GDN_DTYPE_BF16, GDN_EUNSUPPORTED, "%s: bf16 inputs only", name);
    GDN_REQUIRE(D == 32 || D == 64 || D == 128, GDN_EUNSUPPORTED, "%s: D=%d (supported: 32, 64, 128)", name, D);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    if ((long)B * H == 0) return GDN_OK;
    const bool work = F > 0;
    if (work) {
        GDN_REQUIRE(q && k && v && beta && log_decay && dout && dq && dk && dv && dbeta && dlog_decay, GDN_EINVAL,
                    "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && gdn::aligned(v, 16) && gdn::aligned(dout, 16) &&
                        gdn::aligned(dq, 16) && gdn::aligned(dk, 16) && gdn::aligned(dv, 16),
                    GDN_EINVAL, "%s: q, k, v, dout, dq, dk, dv must be 16-byte aligned", name);
        GDN_REQUIRE(gdn::aligned(beta, 4) && gdn::aligned(log_decay, 4) && gdn::aligned(dbeta, 4) &&
                        gdn::aligned(dlog_decay, 4),
                    GDN_EINVAL, "%s: misaligned gate pointer", name);
    }
    GDN_REQUIRE((!h0 || gdn::aligned(h0, 4)) && (!dhT || gdn::aligned(dhT, 4)) && (!dh0 || gdn::aligned(dh0, 4)),
                GDN_EINVAL, "%s: misaligned state pointer", name);
    const size_t need = frame_bwd_workspace(B, H, F, S, D);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!work) {                                // no frames: dh0 = dhT (or 0)
        if (!dh0) return GDN_OK;
        const size_t n = (size_t)B * H * D * D;
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dhT, dh0, n);
        return check_hip(hipGetLastError(), name);
    }
    FrameBwdArgs ba;
    FrameArgs &a = ba.a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = log_decay;
    a.h0 = h0;
    a.hT = nullptr;
    a.out = nullptr;
    a.B = B;
    a.H = H;
    a.F = F;
    a.S = S;
    a.nsplit = frame_nsplit(B, H, F, S, D, &a.spl);
    a.dd = D;
    a.scale = scale;
    a.reverse = 0;
    a.den = 0;
    const size_t units = (size_t)B * H * F;
    float *ws = reinterpret_cast<float *>(workspace);
    a.part = ws;
    a.gh = a.part + units * a.nsplit * 2 * D * D;
    a.sf = a.gh + units * 2 * D * D;
    float *ap = a.sf + units * D * D;
    ba.apart = ap;
    ba.xf = ap + units * a.nsplit * D * D;
    ba.dgp = ba.xf + units * D * D;
    if (a.nsplit == 1) a.part = a.gh;            // one range: the gram kernel writes G_f, H_f directly
    ba.dout = dout;
    ba.dhT = dhT;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dbeta = dbeta;
    ba.dg = dlog_decay;
    ba.dh0 = dh0;
    hipError_t e;
    switch (D) {
        case 32: e = launch_frame_bwd<32>(ba, s); break;
        case 64: e = launch_frame_bwd<64>(ba, s); break;
        default: e = launch_frame_bwd<128>(ba, s); break;
    }
    return check_hip(e, name);
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_recurrent_fwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype) {
    (void)dtype;
    const int KD = gdn::padded_head_width(D);
    if (B < 0 || H < 0 || F < 0 || S <= 0 || KD == 0) return 0;
    return gdn::frame_workspace(B, H, F, S, KD);
}

extern "C" int gdn_recurrent_fwd(const void *q, const void *k, const void *v, const float *beta,
                                 const float *log_decay, float scale, const float *h0, float *hT, float *out,
                                 int B, int H, int F, int S, int D, int dtype, int reverse, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return gdn::frame_entry("gdn_recurrent_fwd", q, k, v, beta, log_decay, scale, h0, hT, out, B, H, F, S, D,
                            dtype, reverse, 0, workspace, workspace_bytes, stream);
}

extern "C" size_t gdn_recurrent_den_fwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype) {
    return gdn_recurrent_fwd_workspace_bytes(B, H, F, S, D, dtype);
}

extern "C" int gdn_recurrent_den_fwd(const void *q_den, const void *k_z, const float *beta, const float *log_decay,
                                     float scale, const float *z0, float *zT, float *den, int B, int H, int F, int S,
                                     int D, int dtype, int reverse, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    return gdn::frame_entry("gdn_recurrent_den_fwd", q_den, k_z, nullptr, beta, log_decay, scale, z0, zT, den, B, H,
                            F, S, D, dtype, reverse, 1, workspace, workspace_bytes, stream);
}

extern "C" size_t gdn_recurrent_bwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype) {
    (void)dtype;
    if (B < 0 || H < 0 || F < 0 || S <= 0 || (D != 32 && D != 64 && D != 128)) return 0;
    return gdn::frame_bwd_workspace(B, H, F, S, D);
}

extern "C" int gdn_recurrent_bwd(const void *q, const void *k, const void *v, const float *beta,
                                 const float *log_decay, float scale, const float *h0, const void *dout,
                                 const float *dhT, float *dq, float *dk, float *dv, float *dbeta, float *dlog_decay,
                                 float *dh0, int B, int H, int F, int S, int D, int dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return gdn::frame_bwd_entry(q, k, v, beta, log_decay, scale, h0, dout, dhT, dq, dk, dv, dbeta, dlog_decay, dh0,
                                B, H, F, S, D, dtype, workspace, workspace_bytes, stream);
}
