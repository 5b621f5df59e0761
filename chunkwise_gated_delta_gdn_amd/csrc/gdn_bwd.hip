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
//   bwd_scan_kernel    one wave per (b, h, 16-column slice of the state).
//                      Lane (row group rg = l / 16, column c = l % 16) holds
//                      rows rg*Dk/4 .. of column c in registers.  A forward
//                      sweep keeps the state entering every 32-token segment
//                      in the work space; the reverse sweep recomputes each
//                      segment's states into the work space and walks its
//                      tokens backwards.  The columns of a slice are summed
//                      in registers (reduce-scatter over the 16 column
//                      lanes); dv and dh0 belong to one slice and are
//                      written directly, dq, dk, dbeta and dg are per-slice
//                      partial sums.
//   bwd_reduce_kernel  sums the partials over the slices.
#include <math.h>

#include "api_common.h"
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int BWD_SEG = 32;     // tokens between kept states

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *beta, *g, *h0, *dhT;
    float *dq, *dk, *dv, *dbeta, *dg, *dh0;
    float *ck, *st, *part;      // work space: kept states, segment states, partials
    int B, T, H, Dv, nvs;
    float scale;
};

// N consecutive elements at element offset `off` (16-byte pieces; 8 bytes
// for four bf16).
template <bool F32, int N>
__device__ __forceinline__ void load_rows(const void *p, size_t off, float (&x)[N]) {
    if constexpr (F32) {
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

// Sum of x over the 16 column lanes of a row group, scattered: at each
// exchange (lane distance O = 8, 4, 2, 1) a lane keeps one half of its
// window of rows and adds its partner's copy of that half.  At the end
// x[0 .. max(N/16, 1) - 1] holds the sums of rows base + j of the window;
// with N < 16 the last exchanges add single values, and lanes that differ
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
                x[j] = keep + __shfl_xor(send, O, 64);
            }
            base += hi ? HALF : 0;
            col_reduce_scatter<HALF, O / 2>(x, c, base, dup);
        } else {
            x[0] += __shfl_xor(x[0], O, 64);
            dup |= O;
            col_reduce_scatter<1, O / 2>(x, c, base, dup);
        }
    }
}

// sum over the four row groups (lanes c, c + 16, c + 32, c + 48)
__device__ __forceinline__ float row_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <bool F32, int DK>
__global__ __launch_bounds__(64) void bwd_scan_kernel(BwdArgs a) {
    constexpr int RPG = DK / 4;                        // rows per lane
    constexpr int NOUT = RPG >= 16 ? RPG / 16 : 1;     // summed rows per lane
    constexpr int PW = 2 * DK + 2;                     // partial row: dq, dk, dbeta, dg
    const int l = threadIdx.x, c = l & 15, rg = l >> 4;
    const int wv = blockIdx.x;                          // (b H + h) nvs + vs
    const int vs = wv % a.nvs, bh = wv / a.nvs, b = bh / a.H, h = bh % a.H;
    const int col = vs * 16 + c, r0 = rg * RPG;
    const int T = a.T, H = a.H, Dv = a.Dv;
    const int nseg = (T + BWD_SEG - 1) / BWD_SEG;
    const size_t NROW = (size_t)a.B * T * H;
    float *ck = a.ck + (size_t)wv * nseg * DK * 16;     // [nseg][DK][16]
    float *st = a.st + (size_t)wv * BWD_SEG * DK * 16;  // [BWD_SEG][DK][16]
    auto row_of = [&](int t) { return ((size_t)b * T + t) * H + h; };
    auto state_at = [&](size_t i) { return ((size_t)bh * DK + r0 + i) * Dv + col; };

    // one forward token step on this lane's rows of column c
    auto fwd_step = [&](float (&X)[RPG], int t) __attribute__((always_inline)) {
        const size_t row = row_of(t);
        float kr[RPG];
        load_rows<F32, RPG>(a.k, row * DK + r0, kr);
        const float vc = load1<F32>(a.v, row * Dv + col);
        const float dec = expf(a.g[row]), bt = a.beta[row];
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
    for (int t = 0; t < T; ++t) {
        if (t % BWD_SEG == 0) {
            float *cp = ck + (size_t)(t / BWD_SEG) * DK * 16;
#pragma unroll
            for (int i = 0; i < RPG; ++i) cp[(r0 + i) * 16 + c] = S[i];
        }
        fwd_step(S, t);
    }

    float dS[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) dS[i] = a.dhT ? a.dhT[state_at(i)] : 0.f;
    // S holds S_t of the token being walked back (S_T first)
    for (int s = nseg - 1; s >= 0; --s) {
        const int t0 = s * BWD_SEG, t1 = min(T, t0 + BWD_SEG);
        float X[RPG];
        const float *cp = ck + (size_t)s * DK * 16;
#pragma unroll
        for (int i = 0; i < RPG; ++i) X[i] = cp[(r0 + i) * 16 + c];
        for (int t = t0; t < t1; ++t) {
            float *sp = st + (size_t)(t - t0) * DK * 16;
#pragma unroll
            for (int i = 0; i < RPG; ++i) sp[(r0 + i) * 16 + c] = X[i];
            fwd_step(X, t);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t row = row_of(t);
            float Sp[RPG], kr[RPG], qr[RPG], x[RPG];
            const float *sp = st + (size_t)(t - t0) * DK * 16;
#pragma unroll
            for (int i = 0; i < RPG; ++i) Sp[i] = sp[(r0 + i) * 16 + c];
            load_rows<F32, RPG>(a.k, row * DK + r0, kr);
            load_rows<F32, RPG>(a.q, row * DK + r0, qr);
            const float vc = load1<F32>(a.v, row * Dv + col), doc = load1<F32>(a.dout, row * Dv + col);
            const float dec = expf(a.g[row]), bt = a.beta[row];
            float *pp = a.part + ((size_t)vs * NROW + row) * PW;
            // read-out
#pragma unroll
            for (int i = 0; i < RPG; ++i) {
                dS[i] += a.scale * qr[i] * doc;
                x[i] = a.scale * S[i] * doc;
            }
            {
                int base = 0, dup = 0;
                col_reduce_scatter<RPG, 8>(x, c, base, dup);
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
            if (rg == 0) a.dv[row * Dv + col] = bt * u;
            float db = u * r;
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) db += __shfl_xor(db, o, 64);
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
                col_reduce_scatter<RPG, 8>(x, c, base, dup);
                if ((c & dup) == 0)
#pragma unroll
                    for (int j = 0; j < NOUT; ++j) pp[DK + r0 + base + j] = x[j];
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) dgl += __shfl_xor(dgl, o, 64);
            if (l == 0) {
                pp[2 * DK] = db;
                pp[2 * DK + 1] = dgl;
            }
#pragma unroll
            for (int i = 0; i < RPG; ++i) S[i] = Sp[i];
        }
    }
    if (a.dh0)
#pragma unroll
        for (int i = 0; i < RPG; ++i) a.dh0[state_at(i)] = dS[i];
}

// dq, dk, dbeta, dg: the per-slice partials summed in slice order
template <int DK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
    constexpr int PW = 2 * DK + 2;
    const size_t NROW = (size_t)a.B * a.T * a.H;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= NROW * PW) return;
    const size_t row = i / PW;
    const int e = (int)(i % PW);
    float s = 0.f;
    for (int vs = 0; vs < a.nvs; ++vs) s += a.part[(size_t)vs * NROW * PW + i];
    if (e < DK) a.dq[row * DK + e] = s;
    else if (e < 2 * DK) a.dk[row * DK + e - DK] = s;
    else if (e == 2 * DK) a.dbeta[row] = s;
    else a.dg[row] = s;
}

size_t bwd_workspace(int B, int T, int H, int Dk, int Dv) {
    const size_t nvs = (size_t)Dv / 16, nw = (size_t)B * H * nvs;
    const size_t nseg = ((size_t)T + BWD_SEG - 1) / BWD_SEG;
    const size_t fl = nw * nseg * Dk * 16 + nw * BWD_SEG * Dk * 16 + nvs * (size_t)B * T * H * (2 * Dk + 2);
    return fl * sizeof(float);
}

template <bool F32, int DK>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    const unsigned nw = (unsigned)((size_t)a.B * a.H * a.nvs);
    hipLaunchKernelGGL((bwd_scan_kernel<F32, DK>), dim3(nw), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)a.B * a.T * a.H * (2 * DK + 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_reduce_kernel<DK>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 0;
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
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16), GDN_EINVAL, "%s: q and k must be 16-byte aligned",
                    name);
        GDN_REQUIRE(gdn::aligned(v, 4) && gdn::aligned(dout, 4) && gdn::aligned(beta, 4) &&
                        gdn::aligned(log_decay, 4) && gdn::aligned(dq, 4) && gdn::aligned(dk, 4) &&
                        gdn::aligned(dv, 4) && gdn::aligned(dbeta, 4) && gdn::aligned(dlog_decay, 4),
                    GDN_EINVAL, "%s: misaligned tensor pointer", name);
        GDN_REQUIRE(dtype == GDN_DTYPE_F32 || (gdn::aligned(v, 2) && gdn::aligned(dout, 2)), GDN_EINVAL,
                    "%s: misaligned tensor pointer", name);
    }
    GDN_REQUIRE((!h0 || gdn::aligned(h0, 4)) && (!dhT || gdn::aligned(dhT, 4)) && (!dh0 || gdn::aligned(dh0, 4)),
                GDN_EINVAL, "%s: misaligned state pointer", name);
    const size_t need = gdn::bwd_workspace(B, T, H, Dk, Dv);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    GDN_REQUIRE((size_t)B * H * (Dv / 16) < (1u << 31), GDN_EUNSUPPORTED, "%s: too many (b, h, slice) units", name);
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
    a.nvs = Dv / 16;
    a.scale = scale;
    const size_t nw = (size_t)B * H * a.nvs, nseg = ((size_t)T + gdn::BWD_SEG - 1) / gdn::BWD_SEG;
    float *ws = reinterpret_cast<float *>(workspace);
    a.ck = ws;
    a.st = a.ck + nw * nseg * Dk * 16;
    a.part = a.st + nw * gdn::BWD_SEG * Dk * 16;
    if (!dh0 && T == 0) return GDN_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
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
