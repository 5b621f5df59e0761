// Camera-branch numerator-only scan, frame-synchronous: Sana
// "fused_cam_gdn.py" _cam_scan_kernel (forward direction) and cam_scan_func.
//
// Every token of frame f predicts from the same gated state P = e^{g_f} S,
// so the frame update is affine in S:
//   S_f = P + sum_s beta_s k_s (v_s - P^T k_s)^T = (I - G_f) P + H_f,
//   G_f = sum_{s in f} beta_s k_s k_s^T,   H_f = sum_{s in f} beta_s k_s v_s^T
// (the matrix form of the page's _torch_cam_scan_single_chunk).  Three
// kernels:
//   frame_gram_kernel   parallel over (b, h, f, token range): partial G_f and
//                       H_f from K^T diag(beta) K and K^T diag(beta) V (MFMA);
//   frame_state_kernel  per (b, h, 16-column slice of S), sequential over
//                       frames: S_f = e^{g_f} (S - G_f S) + H_f in fp32 (fp32
//                       MFMA), stores S_f and the final state;
//   frame_out_kernel    parallel over (b, h, f, 64-token tile):
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
    float *part;     // [B*H*F][NSPLIT][2][D][D] partial G_f, H_f
    float *sf;       // [B*H][F][D][D] state after each frame
    int B, H, F, S, nsplit, spl;
    float scale;
};

constexpr int TS = 32;   // tokens per gram step

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
template <bool F32IN, int D>
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
            if (s0 + s < s_hi) {
                const size_t row = row0 + s0 + s;
                load8<F32IN>(a.k, row * D + i0, kx);
                load8<F32IN>(a.v, row * D + i0, vx);
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
// sequential frame pass on a 16-column slice of the state
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void frame_state_kernel(FrameArgs a) {
    constexpr int LDG = D + 4, LDS_ = 16 + 4;
    constexpr int NRT = D / 16, PERW = (NRT + 3) / 4;
    __shared__ __attribute__((aligned(16))) float Gs[D * LDG], Sl[D * LDS_];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncb = D / 16;
    const int bh = blockIdx.x / ncb, cb = blockIdx.x % ncb, j0 = cb * 16;

    floatx4 S[PERW];
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        S[n] = zero4();
        const int ti = w + 4 * n;
        if (ti < NRT && a.h0)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[n][e] = a.h0[((size_t)bh * D + ti * 16 + 4 * (l >> 4) + e) * D + j0 + (l & 15)];
    }
    for (int f = 0; f < a.F; ++f) {
        const size_t unit = (size_t)bh * a.F + f;
        const float *pp = a.part + unit * a.nsplit * 2 * D * D;
        // G_f (all of it) into LDS, summed over the token ranges
        for (int idx = tid; idx < D * D / 4; idx += 256) {
            float4 sum = {0.f, 0.f, 0.f, 0.f};
            for (int sp = 0; sp < a.nsplit; ++sp) {
                const float4 x = reinterpret_cast<const float4 *>(pp + (size_t)sp * 2 * D * D)[idx];
                sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
            }
            const int i = (idx * 4) / D, c = (idx * 4) % D;
            float *gd = Gs + i * LDG + c;
            gd[0] = sum.x; gd[1] = sum.y; gd[2] = sum.z; gd[3] = sum.w;
        }
        // current state slice into LDS as the B operand ([k][col])
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sl[(ti * 16 + 4 * (l >> 4) + e) * LDS_ + (l & 15)] = S[n][e];
        }
        __syncthreads();
        const float dec = expf(a.g[unit]);
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT) {
                floatx4 gs = zero4();
                mma_f32_bn(gs, Gs + ti * 16 * LDG, LDG, Sl, LDS_, D);
                float hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = ti * 16 + 4 * (l >> 4) + e;
                    float hsum = 0.f;
                    for (int sp = 0; sp < a.nsplit; ++sp)
                        hsum += pp[(size_t)sp * 2 * D * D + (size_t)D * D + i * D + j0 + (l & 15)];
                    hv[e] = hsum;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[n][e] = dec * (S[n][e] - gs[e]) + hv[e];
                    a.sf[(unit * D + ti * 16 + 4 * (l >> 4) + e) * D + j0 + (l & 15)] = S[n][e];
                }
            }
        }
        __syncthreads();
    }
    if (a.hT) {
#pragma unroll
        for (int n = 0; n < PERW; ++n) {
            const int ti = w + 4 * n;
            if (ti < NRT)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.hT[((size_t)bh * D + ti * 16 + 4 * (l >> 4) + e) * D + j0 + (l & 15)] = S[n][e];
        }
    }
}

// ---------------------------------------------------------------------------
// out_s = scale * S_f^T q_s for a tile of up to 64 tokens of one frame
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

    // S_f transposed ([j][i]) as the B operand
    const float *sf = a.sf + (size_t)unit * D * D;
    for (int idx = tid; idx < D * D; idx += 256) {
        const int i = idx / D, j = idx % D;
        put_op<F32IN>(SH, SL, j * LDT + i, sf[idx]);
    }
    constexpr int SEGS = D / 8;
    for (int idx = tid; idx < TT * SEGS; idx += 256) {
        const int r = idx / SEGS, i0 = (idx % SEGS) * 8;
        U16x8 raw[F32IN ? 2 : 1];
        if (r < nrows) {
            const unsigned char *src = reinterpret_cast<const unsigned char *>(a.q) +
                                       ((row0 + r) * D + i0) * (F32IN ? 4 : 2);
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
                if (r < nrows) a.out[(row0 + r) * D + tj * 16 + (l & 15)] = a.scale * acc[e];
            }
        }
    }
}

int frame_nsplit(int B, int H, int F, int S) {
    const long units = (long)B * H * F;
    const int maxsp = (S + TS - 1) / TS;
    long want = units > 0 ? (512 + units - 1) / units : 1;
    if (want > maxsp) want = maxsp;
    if (want < 1) want = 1;
    return (int)want;
}

size_t frame_workspace(int B, int H, int F, int S, int D) {
    const int ns = frame_nsplit(B, H, F, S);
    const size_t units = (size_t)B * H * F;
    return units * ns * 2 * D * D * sizeof(float) + units * D * D * sizeof(float);
}

template <bool F32IN, int D>
hipError_t launch_frame(FrameArgs a, hipStream_t s) {
    const int units = a.B * a.H * a.F;
    hipLaunchKernelGGL((frame_gram_kernel<F32IN, D>), dim3(units * a.nsplit), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((frame_state_kernel<D>), dim3(a.B * a.H * (D / 16)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntt = (a.S + 63) / 64;
    hipLaunchKernelGGL((frame_out_kernel<F32IN, D>), dim3(units * ntt), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_recurrent_fwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype) {
    (void)dtype;
    if (B < 0 || H < 0 || F < 0 || S <= 0 || D <= 0) return 0;
    return gdn::frame_workspace(B, H, F, S, D);
}

extern "C" int gdn_recurrent_fwd(const void *q, const void *k, const void *v, const float *beta,
                                 const float *log_decay, float scale, const float *h0, float *hT, float *out,
                                 int B, int H, int F, int S, int D, int dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    const char *name = "gdn_recurrent_fwd";
    GDN_REQUIRE(B >= 0 && H >= 0 && F >= 0, GDN_EINVAL, "%s: negative size (B=%d H=%d F=%d)", name, B, H, F);
    GDN_REQUIRE(S >= 1, GDN_EINVAL, "%s: S=%d (at least one token per frame)", name, S);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(D == 16 || D == 32 || D == 64 || D == 128, GDN_EUNSUPPORTED,
                "%s: D=%d (supported: 16, 32, 64, 128)", name, D);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    if ((long)B * H == 0) return GDN_OK;
    const bool work = (long)F > 0;
    if (work) {
        GDN_REQUIRE(q && k && v && beta && log_decay && out, GDN_EINVAL, "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && gdn::aligned(v, 16) && gdn::aligned(out, 16),
                    GDN_EINVAL, "%s: q, k, v and out must be 16-byte aligned", name);
        GDN_REQUIRE(gdn::aligned(beta, 4) && gdn::aligned(log_decay, 4), GDN_EINVAL,
                    "%s: beta and log_decay must be 4-byte aligned", name);
    }
    GDN_REQUIRE(!h0 || gdn::aligned(h0, 4), GDN_EINVAL, "%s: h0 misaligned", name);
    GDN_REQUIRE(!hT || gdn::aligned(hT, 4), GDN_EINVAL, "%s: hT misaligned", name);
    const size_t need = gdn::frame_workspace(B, H, F, S, D);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!work) {
        // no frames: the final state is the initial one
        if (!hT) return GDN_OK;
        const size_t bytes = (size_t)B * H * D * D * sizeof(float);
        hipError_t e = h0 ? hipMemcpyAsync(hT, h0, bytes, hipMemcpyDeviceToDevice, s) : hipMemsetAsync(hT, 0, bytes, s);
        return gdn::check_hip(e, name);
    }
    gdn::FrameArgs a;
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
    a.nsplit = gdn::frame_nsplit(B, H, F, S);
    a.spl = ((S + a.nsplit - 1) / a.nsplit + gdn::TS - 1) / gdn::TS * gdn::TS;
    a.scale = scale;
    const size_t units = (size_t)B * H * F;
    a.part = reinterpret_cast<float *>(workspace);
    a.sf = a.part + units * a.nsplit * 2 * D * D;
    const bool f32 = dtype == GDN_DTYPE_F32;
    hipError_t e;
    switch (D) {
        case 16: e = f32 ? gdn::launch_frame<true, 16>(a, s) : gdn::launch_frame<false, 16>(a, s); break;
        case 32: e = f32 ? gdn::launch_frame<true, 32>(a, s) : gdn::launch_frame<false, 32>(a, s); break;
        case 64: e = f32 ? gdn::launch_frame<true, 64>(a, s) : gdn::launch_frame<false, 64>(a, s); break;
        default: e = f32 ? gdn::launch_frame<true, 128>(a, s) : gdn::launch_frame<false, 128>(a, s); break;
    }
    return gdn::check_hip(e, name);
}
