// Gradients of the gated delta rule (the backward of gdn_chunk_fwd), taken on
// the token recurrence.  msj19 "gated_deltaproduct" test.py lists the chunk
// backward kernels of this rule (prepare_dv, dhu, dqkw, WY backward); this is
// the gradient they compute, in reverse mode through the steps of one token:
//   gate      P = e^{g_t} S_{t-1}
//   predict   p = P^T k_t
//   correct   S_t = P + beta_t k_t (v_t - p)^T
//   read out  o_t = scale S_t^T q_t
// walked from the last token back with dS = dL/dS_t:
//   dS += scale q do^T,   dq = scale S_t do,   r = v - p,   u = dS^T k,
//   dv = beta u,   dbeta = u . r,   dp = -beta u,
//   dk = beta dS r + P dp,   dP = dS + k dp^T,   dg = <dP, P>,   dS <- e^{g} dP,
// and dh0 = dS after the first token.
//
// Kernels:
//   bwd_scan_kernel    one workgroup per (b, h, 16-column group of the
//                      state), one wave per 4-column slice.  Lane (row group
//                      rg = l / 4, column c = l % 4) holds rows rg*Dk/16 ..
//                      of column c in registers.  Tokens go in 12-token
//                      segments whose k, q rows, v, dout columns and gates
//                      are staged in LDS once for the four waves (the next
//                      segment's are loaded into registers while one is
//                      computed).  A forward sweep keeps the state entering
//                      every segment in the work space; the reverse sweep
//                      recomputes each segment's states into LDS and walks
//                      its tokens backwards.  The columns of a slice are
//                      summed in registers (reduce-scatter over the 4 column
//                      lanes), the four slices' rows in LDS at the end of a
//                      segment; dv and dh0 belong to one column and are
//                      written directly, dq, dk, dbeta and dg are
//                      per-group partial sums.
//   bwd_reduce_kernel  sums the partials over the groups.
#include <math.h>

#include "api_common.h"
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int BWD_SEG = 12;     // tokens between kept states (one LDS-staged segment)
constexpr int BWD_CW = 4;       // state columns per wave
constexpr int BWD_WAVES = 4;    // waves per workgroup (their partials are added in LDS)

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *beta, *g, *h0, *dhT;
    float *dq, *dk, *dv, *dbeta, *dg, *dh0;
    float *ck, *part;           // work space: kept states, partials
    size_t pstride;             // floats per slice of partials (a multiple of 4)
    int B, T, H, Dv, nvs;       // nvs: 16-column groups (one workgroup, one partial each)
    float scale;
};

// N consecutive elements at element offset `off` (16-byte pieces; 8, 4 or
// 2 bytes for fewer elements).
template <bool F32, int N>
__device__ __forceinline__ void load_rows(const void *p, size_t off, float (&x)[N]) {
    if constexpr (N == 1) {
        x[0] = F32 ? reinterpret_cast<const float *>(p)[off] : bf16_to_f32(reinterpret_cast<const u16 *>(p)[off]);
    } else if constexpr (N == 2) {
        if constexpr (F32) {
            const floatx2 t = *reinterpret_cast<const floatx2 *>(reinterpret_cast<const float *>(p) + off);
            x[0] = t[0];
            x[1] = t[1];
        } else {
            const uint32_t t = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const u16 *>(p) + off);
            x[0] = __builtin_bit_cast(float, t << 16);
            x[1] = __builtin_bit_cast(float, t & 0xffff0000u);
        }
    } else if constexpr (F32) {
        const floatx4 *s = reinterpret_cast<const floatx4 *>(reinterpret_cast<const float *>(p) + off);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const floatx4 t = s[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * i + e] = t[e];
        }
    } else if constexpr (N >= 8) {
        const u32x4 *s = reinterpret_cast<const u32x4 *>(reinterpret_cast<const u16 *>(p) + off);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            const u32x4 t = s[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * i + 2 * e] = __builtin_bit_cast(float, t[e] << 16);
                x[8 * i + 2 * e + 1] = __builtin_bit_cast(float, t[e] & 0xffff0000u);
            }
        }
    } else {
        static_assert(N == 4, "row count");
        const u32x2 t = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const u16 *>(p) + off);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            x[2 * e] = __builtin_bit_cast(float, t[e] << 16);
            x[2 * e + 1] = __builtin_bit_cast(float, t[e] & 0xffff0000u);
        }
    }
}

template <bool F32>
__device__ __forceinline__ float load1(const void *p, size_t off) {
    if constexpr (F32) return reinterpret_cast<const float *>(p)[off];
    else return bf16_to_f32(reinterpret_cast<const u16 *>(p)[off]);
}

// Cross-lane moves inside a 16-lane row by DPP (VALU latency, no LDS
// round trip): quad permutations [1,0,3,2] and [2,3,0,1] are the lane XORs
// 1 and 2; row rotations by 4 and 8 keep a lane's index mod 4 (mod 8).
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// x from lane l ^ O
template <int O>
__device__ __forceinline__ float xor_lane(float x) {
    if constexpr (O == 1) return dpp<DPP_XOR1>(x);
    else if constexpr (O == 2) return dpp<DPP_XOR2>(x);
    else return __shfl_xor(x, O, 64);
}

// Sum of x over the column lanes of a row group, scattered: at each
// exchange (lane distance O = BWD_CW/2, ..., 2, 1) a lane keeps one half of its
// window of rows and adds its partner's copy of that half.  At the end
// x[0 .. max(N/BWD_CW, 1) - 1] holds the sums of rows base + j of the window;
// with N < BWD_CW the last exchanges add single values, and lanes that differ
// only in those bits (`dup`) hold the same sums.
template <int N, int O>
__device__ __forceinline__ void col_reduce_scatter(float *x, int c, int &base, int &dup) {
    if constexpr (O >= 1) {
        if constexpr (N > 1) {
            constexpr int HALF = N / 2;
            const bool hi = (c & O) != 0;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const float send = hi ? x[j] : x[HALF + j];
                const float keep = hi ? x[HALF + j] : x[j];
                x[j] = keep + xor_lane<O>(send);
            }
            base += hi ? HALF : 0;
            col_reduce_scatter<HALF, O / 2>(x, c, base, dup);
        } else {
            x[0] += xor_lane<O>(x[0]);
            dup |= O;
            col_reduce_scatter<1, O / 2>(x, c, base, dup);
        }
    }
}

// sum over the row groups (lanes c, c + BWD_CW, c + 2 BWD_CW, ...): by row
// rotations inside each 16-lane row, then across the four rows
__device__ __forceinline__ float row_sum(float x) {
    static_assert(BWD_CW == 4 || BWD_CW == 8 || BWD_CW == 16, "column lanes");
    if constexpr (BWD_CW == 4) x += dpp<DPP_ROR4>(x);
    if constexpr (BWD_CW <= 8) x += dpp<DPP_ROR8>(x);
    return add_xor32(add_xor16(x));
}
// sum over all 64 lanes
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    x += dpp<DPP_ROR4>(x);
    x += dpp<DPP_ROR8>(x);
    return add_xor32(add_xor16(x));
}

template <bool F32, int DK>
struct BwdShape {
    static constexpr int NW = BWD_WAVES, GC = BWD_WAVES * BWD_CW;   // waves and columns per workgroup
    static constexpr int NT = 64 * NW;                      // threads
    static constexpr int ES = F32 ? 4 : 2;                  // input element bytes
    static constexpr int RPG = DK * BWD_CW / 64;            // state rows per lane
    static constexpr int PW = 2 * DK + 2;                   // partial row: dq, dk, dbeta, dg
    static constexpr int PPR = DK * ES / 16;                // 16-byte pieces of a k (or q) row
    static constexpr int KP = BWD_SEG * PPR;                // ... of a segment's k rows
    static constexpr int KPT = (KP + NT - 1) / NT;          // ... per thread
    static constexpr int VPR = GC * ES / 16;                // pieces of a token's v (or dout) columns
    static constexpr int VP = BWD_SEG * VPR;
    // LDS (bytes): per wave, the states entering each token of the segment,
    // fp32 [token][row i][lane] (lane-contiguous: conflict-free); the
    // segment's k and q rows, v and dout columns (input type), beta and g,
    // shared by the waves; the waves' partial rows [token][wave][PW]
    static constexpr int ST_W = BWD_SEG * DK * BWD_CW * 4;  // one wave's states
    static constexpr int OFF_ST = 0;
    static constexpr int OFF_K = OFF_ST + NW * ST_W;
    static constexpr int OFF_Q = OFF_K + BWD_SEG * DK * ES;
    static constexpr int OFF_V = OFF_Q + BWD_SEG * DK * ES;
    static constexpr int OFF_O = OFF_V + BWD_SEG * GC * ES;
    static constexpr int OFF_B = OFF_O + BWD_SEG * GC * ES;
    static constexpr int OFF_G = OFF_B + BWD_SEG * 4;
    static constexpr int OFF_P = OFF_G + BWD_SEG * 4;
    static constexpr int BYTES = OFF_P + BWD_SEG * NW * PW * 4;
    static_assert(VP <= NT && BWD_SEG <= NT && VPR >= 1 && RPG >= 1, "staging pieces");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <bool F32, int DK>
__global__ __launch_bounds__(64 * BWD_WAVES) void bwd_scan_kernel(BwdArgs a) {
    using SH = BwdShape<F32, DK>;
    constexpr int RPG = SH::RPG, KPT = SH::KPT, ES = SH::ES, NW = SH::NW, GC = SH::GC, NT = SH::NT;
    constexpr int NOUT = RPG >= BWD_CW ? RPG / BWD_CW : 1;   // summed rows per lane
    constexpr int PW = SH::PW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SH::BYTES];
    const unsigned char *ks = smem + SH::OFF_K, *qs = smem + SH::OFF_Q;
    const unsigned char *vsl = smem + SH::OFF_V, *os = smem + SH::OFF_O;
    const float *bs = reinterpret_cast<const float *>(smem + SH::OFF_B);
    const float *gs = reinterpret_cast<const float *>(smem + SH::OFF_G);
    float *pbuf = reinterpret_cast<float *>(smem + SH::OFF_P);

    const int tid = threadIdx.x, l = tid & 63, c = l % BWD_CW, rg = l / BWD_CW;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = blockIdx.x;                         // (b H + h) ngrp + vg
    const int vg = grp % a.nvs, bh = grp / a.nvs, b = bh / a.H, h = bh % a.H;
    const int wcol = w * BWD_CW + c;                    // column within the group
    const int col = vg * GC + wcol, r0 = rg * RPG;
    const int T = a.T, H = a.H, Dv = a.Dv;
    const int nseg = (T + BWD_SEG - 1) / BWD_SEG;
    float *sst = reinterpret_cast<float *>(smem + SH::OFF_ST + w * SH::ST_W);
    float *ck = a.ck + ((size_t)grp * NW + w) * nseg * DK * BWD_CW;   // [nseg][RPG][64]
    auto row_of = [&](int t) { return ((size_t)b * T + t) * H + h; };
    auto state_at = [&](size_t i) { return ((size_t)bh * DK + r0 + i) * Dv + col; };

    // the next segment's inputs (and this wave's kept state), loaded into
    // registers while the current one is computed
    struct Pre {
        u32x4 k[KPT], q[KPT], v, o;
        float b, g;
        float x[RPG];
    } pre;
    auto prefetch = [&](int s, bool bwd) __attribute__((always_inline)) {
        const int t0 = s * BWD_SEG;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int idx = tid + NT * j, tt = idx / SH::PPR, t = t0 + tt;
            pre.k[j] = pre.q[j] = u32x4{0u, 0u, 0u, 0u};
            if (idx < SH::KP && t < T) {
                const size_t off = row_of(t) * DK * ES + (idx % SH::PPR) * 16;
                pre.k[j] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const unsigned char *>(a.k) + off);
                if (bwd) pre.q[j] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const unsigned char *>(a.q) + off);
            }
        }
        {
            const int tt = tid / SH::VPR, t = t0 + tt;
            pre.v = pre.o = u32x4{0u, 0u, 0u, 0u};
            if (tid < SH::VP && t < T) {
                const size_t off = (row_of(t) * Dv + vg * GC) * ES + (tid % SH::VPR) * 16;
                pre.v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const unsigned char *>(a.v) + off);
                if (bwd) pre.o = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const unsigned char *>(a.dout) + off);
            }
        }
        pre.b = pre.g = 0.f;
        if (tid < BWD_SEG && t0 + tid < T) {
            pre.b = a.beta[row_of(t0 + tid)];
            pre.g = a.g[row_of(t0 + tid)];
        }
        if (bwd)
#pragma unroll
            for (int i = 0; i < RPG; ++i) pre.x[i] = ck[((size_t)s * RPG + i) * 64 + l];
    };
    auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int idx = tid + NT * j;
            if (idx < SH::KP) {
                *reinterpret_cast<u32x4 *>(smem + SH::OFF_K + idx * 16) = pre.k[j];
                *reinterpret_cast<u32x4 *>(smem + SH::OFF_Q + idx * 16) = pre.q[j];
            }
        }
        if (tid < SH::VP) {
            *reinterpret_cast<u32x4 *>(smem + SH::OFF_V + tid * 16) = pre.v;
            *reinterpret_cast<u32x4 *>(smem + SH::OFF_O + tid * 16) = pre.o;
        }
        if (tid < BWD_SEG) {
            reinterpret_cast<float *>(smem + SH::OFF_B)[tid] = pre.b;
            reinterpret_cast<float *>(smem + SH::OFF_G)[tid] = pre.g;
        }
    };

    // one forward token step (token tt of the staged segment) on this lane's
    // rows of its column
    auto fwd_step = [&](float (&X)[RPG], int tt) __attribute__((always_inline)) {
        float kr[RPG];
        load_rows<F32, RPG>(ks, tt * DK + r0, kr);
        const float vc = load1<F32>(vsl, tt * GC + wcol);
        const float dec = expf(gs[tt]), bt = bs[tt];
        float pl = 0.f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) pl += kr[i] * X[i];
        const float e = bt * (vc - dec * row_sum(pl));
#pragma unroll
        for (int i = 0; i < RPG; ++i) X[i] = dec * X[i] + kr[i] * e;
    };

    float S[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) S[i] = a.h0 ? a.h0[state_at(i)] : 0.f;
    // forward sweep: the state entering every segment is kept.  The segment
    // loops run the same trip counts in every wave, so every barrier below
    // is reached by the whole workgroup.
    if (nseg > 0) prefetch(0, false);
    for (int s = 0; s < nseg; ++s) {
        commit();
        if (s + 1 < nseg) prefetch(s + 1, false);
        lds_barrier();                                  // the segment is staged
#pragma unroll
        for (int i = 0; i < RPG; ++i) ck[((size_t)s * RPG + i) * 64 + l] = S[i];
        const int len = min(BWD_SEG, T - s * BWD_SEG);
        for (int tt = 0; tt < len; ++tt) fwd_step(S, tt);
        lds_barrier();                                  // staging may be overwritten
    }

    float dS[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) dS[i] = a.dhT ? a.dhT[state_at(i)] : 0.f;
    // reverse sweep; S holds S_t of the token being walked back (S_T first)
    if (nseg > 0) prefetch(nseg - 1, true);
    for (int s = nseg - 1; s >= 0; --s) {
        commit();
        float X[RPG];
#pragma unroll
        for (int i = 0; i < RPG; ++i) X[i] = pre.x[i];
        if (s > 0) prefetch(s - 1, true);
        lds_barrier();                                  // the segment is staged
        const int t0 = s * BWD_SEG, len = min(BWD_SEG, T - t0);
        for (int tt = 0; tt < len; ++tt) {
#pragma unroll
            for (int i = 0; i < RPG; ++i) sst[(tt * RPG + i) * 64 + l] = X[i];
            fwd_step(X, tt);
        }
        for (int tt = len - 1; tt >= 0; --tt) {
            float Sp[RPG], kr[RPG], qr[RPG], x[RPG];
#pragma unroll
            for (int i = 0; i < RPG; ++i) Sp[i] = sst[(tt * RPG + i) * 64 + l];
            load_rows<F32, RPG>(ks, tt * DK + r0, kr);
            load_rows<F32, RPG>(qs, tt * DK + r0, qr);
            const float vc = load1<F32>(vsl, tt * GC + wcol), doc = load1<F32>(os, tt * GC + wcol);
            const float dec = expf(gs[tt]), bt = bs[tt];
            float *pp = pbuf + (tt * NW + w) * PW;
            // read-out
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                dS[i] += a.scale * qr[i] * doc;
                x[i] = a.scale * S[i] * doc;
            }
            {
                int base = 0, dup = 0;
                col_reduce_scatter<RPG, BWD_CW / 2>(x, c, base, dup);
                if ((c & dup) == 0)
#pragma unroll
                    for (int j = 0; j < NOUT; ++j) pp[r0 + base + j] = x[j];
            }
            // correct and predict
            float pl = 0.f, ul = 0.f;
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                pl += kr[i] * Sp[i];
                ul += kr[i] * dS[i];
            }
            const float r = vc - dec * row_sum(pl), u = row_sum(ul), dp = -bt * u;
            if (rg == 0) a.dv[row_of(t0 + tt) * Dv + col] = bt * u;
            float db = u * r;
#pragma unroll
            for (int o = BWD_CW / 2; o >= 4; o >>= 1) db += __shfl_xor(db, o, 64);
            db += dpp<DPP_XOR2>(db);
            db += dpp<DPP_XOR1>(db);
            // dk, dg and the gate's adjoint
            float dgl = 0.f;
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                const float P = dec * Sp[i];
                const float dP = dS[i] + kr[i] * dp;
                x[i] = bt * dS[i] * r + P * dp;
                dgl += dP * P;
                dS[i] = dec * dP;
            }
            {
                int base = 0, dup = 0;
                col_reduce_scatter<RPG, BWD_CW / 2>(x, c, base, dup);
                if ((c & dup) == 0)
#pragma unroll
                    for (int j = 0; j < NOUT; ++j) pp[DK + r0 + base + j] = x[j];
            }
            dgl = wave_sum(dgl);
            if (l == 0) {
                pp[2 * DK] = db;
                pp[2 * DK + 1] = dgl;
            }
#pragma unroll
            for (int i = 0; i < RPG; ++i) S[i] = Sp[i];
        }
        lds_barrier();                                  // every wave's partial rows are in LDS
        // the group's partial: the waves' rows added in wave order
        float *gp = a.part + (size_t)vg * a.pstride;
        for (int e = tid; e < len * PW; e += NT) {
            const int tt = e / PW, j = e % PW;
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) sum += pbuf[(tt * NW + v) * PW + j];
            gp[row_of(t0 + tt) * PW + j] = sum;
        }
        lds_barrier();                                  // staging and partial rows may be overwritten
    }
    if (a.dh0)
#pragma unroll
        for (int i = 0; i < RPG; ++i) a.dh0[state_at(i)] = dS[i];
}

// dq, dk, dbeta, dg: the per-slice partials summed in slice order, four
// consecutive entries of the flat partial array per thread (16-byte loads;
// the last thread takes a tail of fewer)
template <int DK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
    constexpr int PW = 2 * DK + 2;
    const size_t NROW = (size_t)a.B * a.T * a.H, n = NROW * PW;
    const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i0 >= n) return;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if (i0 + 4 <= n) {
        for (int vs = 0; vs < a.nvs; ++vs) {
            const floatx4 x = *reinterpret_cast<const floatx4 *>(a.part + (size_t)vs * a.pstride + i0);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += x[e];
        }
    } else {
        for (int vs = 0; vs < a.nvs; ++vs)
            for (size_t i = i0; i < n; ++i) s[i - i0] += a.part[(size_t)vs * a.pstride + i];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const size_t i = i0 + e;
        if (i >= n) break;
        const size_t row = i / PW;
        const int c = (int)(i % PW);
        if (c < DK) a.dq[row * DK + c] = s[e];
        else if (c < 2 * DK) a.dk[row * DK + c - DK] = s[e];
        else if (c == 2 * DK) a.dbeta[row] = s[e];
        else a.dg[row] = s[e];
    }
}

size_t bwd_workspace(int B, int T, int H, int Dk, int Dv) {
    const size_t ngrp = (size_t)Dv / (BWD_WAVES * BWD_CW), nw = (size_t)B * H * ngrp * BWD_WAVES;
    const size_t nseg = ((size_t)T + BWD_SEG - 1) / BWD_SEG;
    const size_t pstride = ((size_t)B * T * H * (2 * Dk + 2) + 3) & ~(size_t)3;
    const size_t fl = nw * nseg * Dk * BWD_CW + ngrp * pstride;
    return fl * sizeof(float);
}

template <bool F32, int DK>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    const unsigned ngrp = (unsigned)((size_t)a.B * a.H * a.nvs);
    hipLaunchKernelGGL((bwd_scan_kernel<F32, DK>), dim3(ngrp), dim3(64 * BWD_WAVES), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)a.B * a.T * a.H * (2 * DK + 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_reduce_kernel<DK>), dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace gdn

namespace gdn {
// chunk_bwd.hip: the chunkwise MFMA path
bool chunk_bwd_eligible(int T, int H, int Dk, int Dv, int dtype);
size_t chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv);
hipError_t chunk_bwd_launch(const void *q, const void *k, const void *v, const float *beta, const float *g,
                            float scale, const float *h0, const void *dout, const float *dhT, float *dq, float *dk,
                            float *dv, float *dbeta, float *dg, float *dh0, int B, int T, int H, int Dk, int Dv,
                            void *workspace, hipStream_t s);
}  // namespace gdn

extern "C" size_t gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int dtype) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 0;
    if (gdn::chunk_bwd_eligible(T, H, Dk, Dv, dtype)) return gdn::chunk_bwd_workspace(B, T, H, Dk, Dv);
    return gdn::bwd_workspace(B, T, H, Dk, Dv);
}

extern "C" int gdn_bwd(const void *q, const void *k, const void *v, const float *beta, const float *log_decay,
                       float scale, const float *h0, const void *dout, const float *dhT, float *dq, float *dk,
                       float *dv, float *dbeta, float *dlog_decay, float *dh0, int B, int T, int H, int Dk, int Dv,
                       int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    const char *name = "gdn_bwd";
    GDN_REQUIRE(B >= 0 && T >= 0 && H >= 0, GDN_EINVAL, "%s: negative size (B=%d T=%d H=%d)", name, B, T, H);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(Dk == 16 || Dk == 32 || Dk == 64 || Dk == 128, GDN_EUNSUPPORTED,
                "%s: Dk=%d (supported: 16, 32, 64, 128)", name, Dk);
    GDN_REQUIRE(Dv >= 16 && Dv % 16 == 0 && Dv <= 4096, GDN_EUNSUPPORTED,
                "%s: Dv=%d (a multiple of 16 up to 4096)", name, Dv);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    if ((long)B * H == 0) return GDN_OK;
    if (T > 0) {
        GDN_REQUIRE(q && k && v && beta && log_decay && dout && dq && dk && dv && dbeta && dlog_decay, GDN_EINVAL,
                    "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && gdn::aligned(v, 16) && gdn::aligned(dout, 16) &&
                        gdn::aligned(dq, 16) && gdn::aligned(dk, 16),
                    GDN_EINVAL, "%s: q, k, v, dout, dq and dk must be 16-byte aligned", name);
        GDN_REQUIRE(gdn::aligned(v, 4) && gdn::aligned(dout, 4) && gdn::aligned(beta, 4) &&
                        gdn::aligned(log_decay, 4) && gdn::aligned(dq, 4) && gdn::aligned(dk, 4) &&
                        gdn::aligned(dv, 4) && gdn::aligned(dbeta, 4) && gdn::aligned(dlog_decay, 4),
                    GDN_EINVAL, "%s: misaligned tensor pointer", name);
        GDN_REQUIRE(dtype == GDN_DTYPE_F32 || (gdn::aligned(v, 2) && gdn::aligned(dout, 2)), GDN_EINVAL,
                    "%s: misaligned tensor pointer", name);
    }
    GDN_REQUIRE((!h0 || gdn::aligned(h0, 4)) && (!dhT || gdn::aligned(dhT, 4)) && (!dh0 || gdn::aligned(dh0, 4)),
                GDN_EINVAL, "%s: misaligned state pointer", name);
    const bool chunked = gdn::chunk_bwd_eligible(T, H, Dk, Dv, dtype);
    const size_t need = chunked ? gdn::chunk_bwd_workspace(B, T, H, Dk, Dv) : gdn::bwd_workspace(B, T, H, Dk, Dv);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    GDN_REQUIRE((size_t)B * H * (Dv / 16) < (1u << 31), GDN_EUNSUPPORTED, "%s: too many (b, h, column group) units",
                name);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (chunked) {
        GDN_REQUIRE((size_t)B * H * ((T + 63) / 64) < (1u << 31), GDN_EUNSUPPORTED, "%s: too many chunks", name);
        return gdn::check_hip(gdn::chunk_bwd_launch(q, k, v, beta, log_decay, scale, h0, dout, dhT, dq, dk, dv,
                                                    dbeta, dlog_decay, dh0, B, T, H, Dk, Dv, workspace, s),
                              name);
    }
    gdn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.beta = beta;
    a.g = log_decay;
    a.h0 = h0;
    a.dhT = dhT;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dbeta = dbeta;
    a.dg = dlog_decay;
    a.dh0 = dh0;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dv = Dv;
    a.nvs = Dv / (gdn::BWD_WAVES * gdn::BWD_CW);       // 16-column groups
    a.scale = scale;
    const size_t nw = (size_t)B * H * a.nvs * gdn::BWD_WAVES, nseg = ((size_t)T + gdn::BWD_SEG - 1) / gdn::BWD_SEG;
    float *ws = reinterpret_cast<float *>(workspace);
    a.ck = ws;
    a.part = a.ck + nw * nseg * Dk * gdn::BWD_CW;
    a.pstride = ((size_t)B * T * H * (2 * Dk + 2) + 3) & ~(size_t)3;
    if (!dh0 && T == 0) return GDN_OK;
    const bool f32 = dtype == GDN_DTYPE_F32;
    hipError_t e;
    switch (Dk) {
        case 16: e = f32 ? gdn::launch_bwd<true, 16>(a, s) : gdn::launch_bwd<false, 16>(a, s); break;
        case 32: e = f32 ? gdn::launch_bwd<true, 32>(a, s) : gdn::launch_bwd<false, 32>(a, s); break;
        case 64: e = f32 ? gdn::launch_bwd<true, 64>(a, s) : gdn::launch_bwd<false, 64>(a, s); break;
        default: e = f32 ? gdn::launch_bwd<true, 128>(a, s) : gdn::launch_bwd<false, 128>(a, s); break;
    }
    return gdn::check_hip(e, name);
}
