// Camera-branch prep, one HBM pass: Sana "fused_cam_gdn.py" _cam_prep_kernel
// and cam_prep_func, with the inverse RMS of _precompute_cam_inv_rms fused
// in (the page computes it in separate torch reductions that re-read q and k).
//
// One wave per token at a time (workgroups walk blocks of consecutive
// tokens with a stride of the grid).  The C = H*D channels of q, k and v are cut into 8-element
// segments; lane l owns segments l, l+64, ... .  A segment lies in
// one head and in one half of it (D/2 is a multiple of 8), so each lane works
// either on two UCPE groups of 4 or on four RoPE pairs, in registers:
//   1. load q, k, v segments (16-byte vector loads), sum q^2 and k^2, reduce
//      over the wave -> inv_rms_q, inv_rms_k;
//   2. q~ = relu(q inv_rms_q w_q), k~ = relu(k inv_rms_k w_k) k_scale, v~ = v;
//   3. first half: y = P x per group of 4 (P = proj_q for q, proj_kv for k, v);
//      second half: y[d] = x[d] cos[n][d] + x[d^1] sin[n][d];
//   4. ||k~||^2 and ||k_out||^2 per head: reduction over the D/8 lanes of the
//      head; inflation = max(post, 1e-12) / max(pre, 1e-12);
//   5. store q, k, v to (B, H, N, D) (16-byte stores, each head row of a
//      token is D contiguous values; bf16 or fp32) and the per-head scalars
//      to (B, H, N).
#include <math.h>

#include "api_common.h"
#include "gdn_common.h"

namespace gdn {
namespace {

struct PrepArgs {
    const void *qkv;
    const float *qw, *kw, *proj_q, *proj_kv, *cosv, *sinv;
    float k_scale, eps;
    void *qo, *ko, *vo;
    float *pre, *post, *infl;
    int B, N, H, D;
};

// 16-byte streaming (nontemporal) store of a q, k or v output piece: the
// outputs are not read again by this kernel
__device__ __forceinline__ void st16(void *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
template <bool F32OUT>
__device__ __forceinline__ void store8(void *base, size_t elem, const float (&x)[8]) {
    if constexpr (F32OUT) {
        float *p = reinterpret_cast<float *>(base) + elem;
        st16(p, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
        st16(p + 4, u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
    } else {
        st16(reinterpret_cast<u16 *>(base) + elem,
             u32x4{cvt2_bf16(x[0], x[1]), cvt2_bf16(x[2], x[3]), cvt2_bf16(x[4], x[5]), cvt2_bf16(x[6], x[7])});
    }
}

// Sums over lane groups by DPP moves (VALU, no LDS round trip): within a
// quad by quad permutations, within 8 and 16 lanes by the half-row and row
// mirrors (after the smaller sums every lane of a group holds the group
// total, so a mirrored partner from the other half gives the wider total).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int W>                                // W in {1, 2, 4, 8, 16}: consecutive lanes
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x = dpp_add<0xB1>(x);     // quad_perm [1,0,3,2]
    if constexpr (W >= 4) x = dpp_add<0x4E>(x);     // quad_perm [2,3,0,1]
    if constexpr (W >= 8) x = dpp_add<0x141>(x);    // row_half_mirror
    if constexpr (W >= 16) x = dpp_add<0x140>(x);   // row_mirror
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    x = group_sum<16>(x);
    const int xi = __builtin_bit_cast(int, x);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48)));
}

// A token's raw q, k or v segment (8 values) as loaded: bf16 in one 16-byte
// vector, fp32 in two.
template <bool F32IN>
struct Raw8 {
    uint4 w[F32IN ? 2 : 1];
};
template <bool F32IN>
__device__ __forceinline__ Raw8<F32IN> load_raw8(const void *base, size_t elem) {
    Raw8<F32IN> r;
    if constexpr (F32IN) {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(base) + elem);
        r.w[0] = p[0];
        r.w[1] = p[1];
    } else {
        r.w[0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const u16 *>(base) + elem);
    }
    return r;
}
template <bool F32IN>
__device__ __forceinline__ void unpack8(const Raw8<F32IN> &r, float (&x)[8]) {
    if constexpr (F32IN) {
        x[0] = __uint_as_float(r.w[0].x); x[1] = __uint_as_float(r.w[0].y);
        x[2] = __uint_as_float(r.w[0].z); x[3] = __uint_as_float(r.w[0].w);
        x[4] = __uint_as_float(r.w[1].x); x[5] = __uint_as_float(r.w[1].y);
        x[6] = __uint_as_float(r.w[1].z); x[7] = __uint_as_float(r.w[1].w);
    } else {
        const unsigned u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(u[e] << 16);
            x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
    }
}
__device__ __forceinline__ void load_f8(const float *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// tokens per block of consecutive tokens a workgroup takes
constexpr int PREP_TPB = 32;
// Lanes per head: LPH = D/8 rounded up to a power of two (the lanes past D/8
// of each head idle), 64/LPH heads per wave step, NSEG = ceil(H / (64/LPH))
// heads per lane.  Lane l holds the 8-channel segment at offset 8 (l % LPH)
// of heads (l / LPH) + i (64/LPH), so its segments share one offset in the
// head (one RoPE table row piece) and a head's lanes are LPH consecutive
// lanes (sums over a head by DPP).  Workgroups take blocks of TPB
// consecutive tokens with a stride of the grid, wave w tokens w, w+4, ...
// of each block, so one workgroup writes TPB consecutive entries of every
// per-head output row (whole 128-byte lines of the per-head scalars).  The
// RMSNorm weights of a wave's channels stay in registers, and its next
// token's q, k, v (and RoPE table row) are loaded while the current one is
// processed.
template <bool F32IN, bool F32OUT, int LPH, int NSEG>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    constexpr int TPB = PREP_TPB, TPW = TPB / 4, HPS = 64 / LPH;
    static_assert(TPB % 4 == 0, "whole tokens per wave");
    static_assert(LPH >= 2 && LPH <= 16 && (LPH & (LPH - 1)) == 0, "lanes per head");
    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long ntok = (long)a.B * a.N;
    long blk = blockIdx.x;
    int jw = 0;                                  // this wave's token index inside the block
    long tok = blk * TPB + w;
    if (tok >= ntok) return;
    const int H = a.H, D = a.D, C = H * D;
    const int HALF = D / 2;
    const int d0 = 8 * (l % LPH);                // this lane's offset in each of its heads
    const bool lane_ok = d0 < D;

    // this lane's segments: head hseg[i], channel c0 = hseg[i] * D + d0 (a
    // segment never straddles a half of a head: D/2 is a multiple of 8);
    // inactive segments point at channel 0 and store nothing
    int hseg[NSEG];
    bool act[NSEG];
    float wq[NSEG][8], wk[NSEG][8];
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
        hseg[i] = i * HPS + l / LPH;
        act[i] = lane_ok && hseg[i] < H;
        const int c0 = act[i] ? hseg[i] * D + d0 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[i][e] = wk[i][e] = 1.f;
        if (a.qw) load_f8(a.qw + c0, wq[i]);
        if (a.kw) load_f8(a.kw + c0, wk[i]);
    }
    // RoPE lanes read 8 cos and 8 sin values of their token; UCPE lanes read
    // the same row at offset 0 and ignore it
    const int dr = lane_ok && d0 >= HALF ? d0 - HALF : 0;

    Raw8<F32IN> rq[NSEG], rk[NSEG], rv[NSEG];
    float cv[8], sv[8];
    auto load_token = [&](long t) {
        const size_t tbase = (size_t)t * 3 * C;
#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            const int c0 = act[i] ? hseg[i] * D + d0 : 0;
            rq[i] = load_raw8<F32IN>(a.qkv, tbase + c0);
            rk[i] = load_raw8<F32IN>(a.qkv, tbase + C + c0);
            rv[i] = load_raw8<F32IN>(a.qkv, tbase + 2 * C + c0);
        }
        const int n = (int)(t % a.N);
        load_f8(a.cosv + (size_t)n * HALF + dr, cv);
        load_f8(a.sinv + (size_t)n * HALF + dr, sv);
    };
    load_token(tok);
    while (tok < ntok) {
        float xq[NSEG][8], xk[NSEG][8], xv[NSEG][8], cs[8], sn[8];
#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            unpack8<F32IN>(rq[i], xq[i]);
            unpack8<F32IN>(rk[i], xk[i]);
            unpack8<F32IN>(rv[i], xv[i]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            cs[e] = cv[e];
            sn[e] = sv[e];
        }
        const int b = (int)(tok / a.N), n = (int)(tok % a.N);
        // per-token projections (wave-uniform addresses: scalar loads)
        float Pq[16], Pkv[16];
        const float *pq = a.proj_q + tok * 16, *pkv = a.proj_kv + tok * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Pq[i] = pq[i];
            Pkv[i] = pkv[i];
        }
        // the next token's loads go out now (past the end: the last token again)
        long nblk = blk;
        int njw = jw + 1;
        if (njw == TPW) {
            njw = 0;
            nblk += gridDim.x;
        }
        const long next = nblk * TPB + w + 4 * njw;
        load_token(next < ntok ? next : ntok - 1);

        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NSEG; ++i)
            if (act[i]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq += xq[i][e] * xq[i][e];
                    sk += xk[i][e] * xk[i][e];
                }
            }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float inv_q = 1.f / sqrtf(sq / C + a.eps);
        const float inv_k = 1.f / sqrtf(sk / C + a.eps);

#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            const int h = hseg[i];
            float kpre = 0.f, kpost = 0.f;
            float qn[8], kn[8], yq[8], yk[8], yv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float vq = xq[i][e] * inv_q * wq[i][e];
                const float vk = xk[i][e] * inv_k * wk[i][e];
                qn[e] = vq > 0.f ? vq : 0.f;
                kn[e] = (vk > 0.f ? vk : 0.f) * a.k_scale;
                kpre += kn[e] * kn[e];
            }
            if (d0 < HALF) {
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float aq = 0.f, ak = 0.f, av = 0.f;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            aq += Pq[r * 4 + c] * qn[g * 4 + c];
                            ak += Pkv[r * 4 + c] * kn[g * 4 + c];
                            av += Pkv[r * 4 + c] * xv[i][g * 4 + c];
                        }
                        yq[g * 4 + r] = aq;
                        yk[g * 4 + r] = ak;
                        yv[g * 4 + r] = av;
                    }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    yq[e] = qn[e] * cs[e] + qn[e ^ 1] * sn[e];
                    yk[e] = kn[e] * cs[e] + kn[e ^ 1] * sn[e];
                    yv[e] = xv[i][e] * cs[e] + xv[i][e ^ 1] * sn[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) kpost += yk[e] * yk[e];
            if (act[i]) {
                const size_t o = (((size_t)b * H + h) * a.N + n) * D + d0;
                store8<F32OUT>(a.qo, o, yq);
                store8<F32OUT>(a.ko, o, yk);
                store8<F32OUT>(a.vo, o, yv);
            }
            // every lane takes part in the head reductions
            kpre = group_sum<LPH>(act[i] ? kpre : 0.f);
            kpost = group_sum<LPH>(act[i] ? kpost : 0.f);
            if (act[i] && d0 == 0) {
                const size_t so = ((size_t)b * H + h) * a.N + n;
                a.pre[so] = kpre;
                a.post[so] = kpost;
                if (a.infl) a.infl[so] = fmaxf(kpost, 1e-12f) / fmaxf(kpre, 1e-12f);
            }
        }
        blk = nblk;
        jw = njw;
        tok = next;
    }
}

template <bool F32IN, bool F32OUT, int LPH>
hipError_t launch_prep(const PrepArgs &a, hipStream_t s) {
    const long ntok = (long)a.B * a.N;
    const int nseg = (a.H + 64 / LPH - 1) / (64 / LPH);      // heads per lane
    // blocks of PREP_TPB tokens, eight per wave: weights stay resident, loads overlap
    long blocks = (ntok + PREP_TPB - 1) / PREP_TPB;
    if (blocks < 1) blocks = 1;
    if (blocks > 65535) blocks = 65535;
    const dim3 grid((unsigned)blocks);
    if (nseg <= 1) hipLaunchKernelGGL((prep_kernel<F32IN, F32OUT, LPH, 1>), grid, dim3(256), 0, s, a);
    else if (nseg <= 2) hipLaunchKernelGGL((prep_kernel<F32IN, F32OUT, LPH, 2>), grid, dim3(256), 0, s, a);
    else if (nseg <= 4) hipLaunchKernelGGL((prep_kernel<F32IN, F32OUT, LPH, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((prep_kernel<F32IN, F32OUT, LPH, 8>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// ===========================================================================
// Backward of the prep ([cam] _cam_prep_bwd_kernel and
// _cam_prep_bwd_dispatch): reverse mode through the steps above, with the
// forward's values recomputed per token (same lane layout and token walk as
// prep_kernel).  Per token:
//   1. the forward again: inv_rms_q, inv_rms_k (wave sums), q~, k~, v and, on
//      k, the outputs and their norms (sums over a head's lanes);
//   2. the norm outputs' gradients: inflation = max(post, 1e-12) /
//      max(pre, 1e-12) sends ginf / max(pre, 1e-12) to post (post > 1e-12)
//      and -ginf max(post, 1e-12) / pre^2 to pre (pre > 1e-12); post sends
//      2 k_out gpost to k_out, pre sends 2 k~ gpre to k~;
//   3. RoPE^T on the second half, gx[d] = gy[d] cos[d] + gy[d^1] sin[d^1];
//      UCPE^T on the first half, gx_g = P^T gy_g, and dP += gy_g x_g^T;
//   4. the ReLU mask (and K-scale on k) gives ga; the RMSNorm backward over
//      all C channels, gx_c = inv w_c ga_c - inv^3 / C x_c sum_c' ga_c' w_c' x_c'
//      (one more wave sum per stream); dw_c += ga_c x_c inv in registers;
//   5. dqkv (fp32) out; the projection gradients summed over the wave;
// every wave writes its dw partial sums at the end, and prep_bwd_reduce_kernel
// adds them in a fixed order.
// ===========================================================================
struct PrepBwdArgs {
    PrepArgs a;                   // forward inputs (qkv, weights, proj, tables, k_scale, eps, sizes)
    const void *gq, *gk, *gv;     // upstream gradients of q, k, v (B, H, N, D), gdtype
    const float *gpre, *gpost, *ginf;   // of k_pre_sq, k_post_sq, inflation_sq (B, H, N), nullable
    float *dqkv;                  // (B, N, 3, H, D)
    float *dpq, *dpkv;            // (B, N, 4, 4), nullable
    float *wpart;                 // [waves][2][C] partial weight gradients, or null
    float *dqw, *dkw;             // (C), nullable
    int nwaves;
};

template <bool F32IN, bool F32G, int LPH, int NSEG>
__global__ __launch_bounds__(256) void prep_bwd_kernel(PrepBwdArgs ba) {
    const PrepArgs &a = ba.a;
    constexpr int TPB = PREP_TPB, TPW = TPB / 4, HPS = 64 / LPH;
    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long ntok = (long)a.B * a.N;
    long blk = blockIdx.x;
    int jw = 0;
    long tok = blk * TPB + w;
    const int H = a.H, D = a.D, C = H * D;
    const int HALF = D / 2;
    const int d0 = 8 * (l % LPH);
    const bool lane_ok = d0 < D;
    int hseg[NSEG];
    bool act[NSEG];
    float wq[NSEG][8], wk[NSEG][8], dwq[NSEG][8], dwk[NSEG][8];
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
        hseg[i] = i * HPS + l / LPH;
        act[i] = lane_ok && hseg[i] < H;
        const int c0 = act[i] ? hseg[i] * D + d0 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wq[i][e] = wk[i][e] = 1.f;
            dwq[i][e] = dwk[i][e] = 0.f;
        }
        if (a.qw) load_f8(a.qw + c0, wq[i]);
        if (a.kw) load_f8(a.kw + c0, wk[i]);
    }
    const int dr = lane_ok && d0 >= HALF ? d0 - HALF : 0;
    const bool rope = d0 >= HALF;
    const float ks = a.k_scale;
    while (tok < ntok) {
        const int b = (int)(tok / a.N), n = (int)(tok % a.N);
        const size_t tbase = (size_t)tok * 3 * C;
        float xq[NSEG][8], xk[NSEG][8], xv[NSEG][8], cs[8], sn[8];
#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            const int c0 = act[i] ? hseg[i] * D + d0 : 0;
            unpack8<F32IN>(load_raw8<F32IN>(a.qkv, tbase + c0), xq[i]);
            unpack8<F32IN>(load_raw8<F32IN>(a.qkv, tbase + C + c0), xk[i]);
            unpack8<F32IN>(load_raw8<F32IN>(a.qkv, tbase + 2 * C + c0), xv[i]);
        }
        load_f8(a.cosv + (size_t)n * HALF + dr, cs);
        load_f8(a.sinv + (size_t)n * HALF + dr, sn);
        float Pq[16], Pkv[16];
        const float *pq = a.proj_q + tok * 16, *pkv = a.proj_kv + tok * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Pq[i] = pq[i];
            Pkv[i] = pkv[i];
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NSEG; ++i)
            if (act[i])
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq += xq[i][e] * xq[i][e];
                    sk += xk[i][e] * xk[i][e];
                }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float inv_q = 1.f / sqrtf(sq / C + a.eps);
        const float inv_k = 1.f / sqrtf(sk / C + a.eps);
        float gaq[NSEG][8], gak[NSEG][8];
        float dPq[16], dPkv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) dPq[i] = dPkv[i] = 0.f;
        float rq = 0.f, rk = 0.f;                // sums of ga w x for the RMSNorm backward
#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            const int h = hseg[i];
            // (an inactive segment reads the head row's start: lanes past D/8 of a
            // head would read past the end of the last row)
            const size_t o = (((size_t)b * H + (act[i] ? h : 0)) * a.N + n) * D + (act[i] ? d0 : 0);
            float gyq[8], gyk[8], gyv[8];
            unpack8<F32G>(load_raw8<F32G>(ba.gq, o), gyq);
            unpack8<F32G>(load_raw8<F32G>(ba.gk, o), gyk);
            unpack8<F32G>(load_raw8<F32G>(ba.gv, o), gyv);
            const size_t so = ((size_t)b * H + (act[i] ? h : 0)) * a.N + n;
            float qa[8], qn[8], ka[8], kn[8], yk[8];
            float kpre = 0.f, kpost = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qa[e] = xq[i][e] * inv_q * wq[i][e];
                qn[e] = qa[e] > 0.f ? qa[e] : 0.f;
                ka[e] = xk[i][e] * inv_k * wk[i][e];
                kn[e] = (ka[e] > 0.f ? ka[e] : 0.f) * ks;
                kpre += kn[e] * kn[e];
            }
            if (!rope) {
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float acc = 0.f;
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc += Pkv[r * 4 + c] * kn[g * 4 + c];
                        yk[g * 4 + r] = acc;
                    }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) yk[e] = kn[e] * cs[e] + kn[e ^ 1] * sn[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) kpost += yk[e] * yk[e];
            kpre = group_sum<LPH>(act[i] ? kpre : 0.f);
            kpost = group_sum<LPH>(act[i] ? kpost : 0.f);
            float gpo = ba.gpost ? ba.gpost[so] : 0.f, gpr = ba.gpre ? ba.gpre[so] : 0.f;
            if (ba.ginf) {
                const float gi = ba.ginf[so];
                if (kpost > 1e-12f) gpo += gi / fmaxf(kpre, 1e-12f);
                if (kpre > 1e-12f) gpr -= gi * fmaxf(kpost, 1e-12f) / (kpre * kpre);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) gyk[e] += 2.f * yk[e] * gpo;
            // RoPE^T or UCPE^T (with the projection gradients)
            float gxq[8], gxk[8], gxv[8];
            if (!rope) {
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float aq = 0.f, ak = 0.f, av = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            aq += Pq[r * 4 + c] * gyq[g * 4 + r];
                            ak += Pkv[r * 4 + c] * gyk[g * 4 + r];
                            av += Pkv[r * 4 + c] * gyv[g * 4 + r];
                            if (act[i]) {
                                dPq[r * 4 + c] += gyq[g * 4 + r] * qn[g * 4 + c];
                                dPkv[r * 4 + c] += gyk[g * 4 + r] * kn[g * 4 + c] + gyv[g * 4 + r] * xv[i][g * 4 + c];
                            }
                        }
                        gxq[g * 4 + c] = aq;
                        gxk[g * 4 + c] = ak;
                        gxv[g * 4 + c] = av;
                    }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    gxq[e] = gyq[e] * cs[e] + gyq[e ^ 1] * sn[e ^ 1];
                    gxk[e] = gyk[e] * cs[e] + gyk[e ^ 1] * sn[e ^ 1];
                    gxv[e] = gyv[e] * cs[e] + gyv[e ^ 1] * sn[e ^ 1];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gxk[e] += 2.f * kn[e] * gpr;
                gaq[i][e] = qa[e] > 0.f ? gxq[e] : 0.f;
                gak[i][e] = ka[e] > 0.f ? gxk[e] * ks : 0.f;
            }
            if (act[i]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rq += gaq[i][e] * wq[i][e] * xq[i][e];
                    rk += gak[i][e] * wk[i][e] * xk[i][e];
                    dwq[i][e] += gaq[i][e] * xq[i][e] * inv_q;
                    dwk[i][e] += gak[i][e] * xk[i][e] * inv_k;
                }
                float *dv = ba.dqkv + tbase + 2 * C + hseg[i] * D + d0;
                *reinterpret_cast<float4 *>(dv) = float4{gxv[0], gxv[1], gxv[2], gxv[3]};
                *reinterpret_cast<float4 *>(dv + 4) = float4{gxv[4], gxv[5], gxv[6], gxv[7]};
            }
        }
        rq = wave_sum(rq);
        rk = wave_sum(rk);
        const float cq = inv_q * inv_q * inv_q / C * rq, ck = inv_k * inv_k * inv_k / C * rk;
#pragma unroll
        for (int i = 0; i < NSEG; ++i)
            if (act[i]) {
                float gq8[8], gk8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    gq8[e] = inv_q * wq[i][e] * gaq[i][e] - cq * xq[i][e];
                    gk8[e] = inv_k * wk[i][e] * gak[i][e] - ck * xk[i][e];
                }
                float *dq = ba.dqkv + tbase + hseg[i] * D + d0, *dk = dq + C;
                *reinterpret_cast<float4 *>(dq) = float4{gq8[0], gq8[1], gq8[2], gq8[3]};
                *reinterpret_cast<float4 *>(dq + 4) = float4{gq8[4], gq8[5], gq8[6], gq8[7]};
                *reinterpret_cast<float4 *>(dk) = float4{gk8[0], gk8[1], gk8[2], gk8[3]};
                *reinterpret_cast<float4 *>(dk + 4) = float4{gk8[4], gk8[5], gk8[6], gk8[7]};
            }
        if (ba.dpq) {
            // projection gradients: sums over the wave, lane i < 16 writes entry i
            // of proj_q's, lanes 16..31 of proj_kv's
            float mine = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float sq_ = wave_sum(dPq[i]), skv = wave_sum(dPkv[i]);
                if (l == i) mine = sq_;
                if (l == 16 + i) mine = skv;
            }
            if (l < 16) ba.dpq[tok * 16 + l] = mine;
            else if (l < 32) ba.dpkv[tok * 16 + l - 16] = mine;
        }
        // the next token of this wave
        int njw = jw + 1;
        if (njw == TPW) {
            njw = 0;
            blk += gridDim.x;
        }
        jw = njw;
        tok = blk * TPB + w + 4 * jw;
    }
    if (ba.wpart) {
        float *wp = ba.wpart + (size_t)(blockIdx.x * 4 + w) * 2 * C;
#pragma unroll
        for (int i = 0; i < NSEG; ++i)
            if (act[i]) {
                const int c0 = hseg[i] * D + d0;
                *reinterpret_cast<float4 *>(wp + c0) = float4{dwq[i][0], dwq[i][1], dwq[i][2], dwq[i][3]};
                *reinterpret_cast<float4 *>(wp + c0 + 4) = float4{dwq[i][4], dwq[i][5], dwq[i][6], dwq[i][7]};
                *reinterpret_cast<float4 *>(wp + C + c0) = float4{dwk[i][0], dwk[i][1], dwk[i][2], dwk[i][3]};
                *reinterpret_cast<float4 *>(wp + C + c0 + 4) = float4{dwk[i][4], dwk[i][5], dwk[i][6], dwk[i][7]};
            }
    }
}

// dq_norm_w, dk_norm_w: the waves' partial sums, 64 channels per workgroup
// of 16 waves; wave j adds partials j, j + 16, ... (four interleaved
// accumulators), then the 16 wave totals are added in wave order.
constexpr int PRB_WAVES = 16;
__global__ __launch_bounds__(64 * PRB_WAVES) void prep_bwd_reduce_kernel(PrepBwdArgs ba) {
    __shared__ float tot[PRB_WAVES][64];
    const int C = ba.a.H * ba.a.D;
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + l;
    const bool ok = c < 2 * C;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int wv = w;
    if (ok) {
        const float *p = ba.wpart + c;
        const size_t st = (size_t)2 * C * PRB_WAVES;
        for (; wv + 3 * PRB_WAVES < ba.nwaves; wv += 4 * PRB_WAVES) {
            s0 += p[(size_t)wv * 2 * C];
            s1 += p[(size_t)wv * 2 * C + st];
            s2 += p[(size_t)wv * 2 * C + 2 * st];
            s3 += p[(size_t)wv * 2 * C + 3 * st];
        }
        for (; wv < ba.nwaves; wv += PRB_WAVES) s0 += p[(size_t)wv * 2 * C];
    }
    tot[w][l] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    if (w == 0 && ok) {
        float s = 0.f;
        for (int i = 0; i < PRB_WAVES; ++i) s += tot[i][l];
        if (c < C) {
            if (ba.dqw) ba.dqw[c] = s;
        } else if (ba.dkw) {
            ba.dkw[c - C] = s;
        }
    }
}

long prep_bwd_grid(long ntok) {
    long blocks = (ntok + PREP_TPB - 1) / PREP_TPB;
    if (blocks < 1) blocks = 1;
    if (blocks > 65535) blocks = 65535;
    return blocks;
}

template <bool F32IN, bool F32G, int LPH>
hipError_t launch_prep_bwd(const PrepBwdArgs &ba, hipStream_t s) {
    const PrepArgs &a = ba.a;
    const long ntok = (long)a.B * a.N;
    const int nseg = (a.H + 64 / LPH - 1) / (64 / LPH);
    const dim3 grid((unsigned)prep_bwd_grid(ntok));
    if (nseg <= 1) hipLaunchKernelGGL((prep_bwd_kernel<F32IN, F32G, LPH, 1>), grid, dim3(256), 0, s, ba);
    else if (nseg <= 2) hipLaunchKernelGGL((prep_bwd_kernel<F32IN, F32G, LPH, 2>), grid, dim3(256), 0, s, ba);
    else if (nseg <= 4) hipLaunchKernelGGL((prep_bwd_kernel<F32IN, F32G, LPH, 4>), grid, dim3(256), 0, s, ba);
    else hipLaunchKernelGGL((prep_bwd_kernel<F32IN, F32G, LPH, 8>), grid, dim3(256), 0, s, ba);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !ba.wpart) return e;
    const int C = a.H * a.D;
    hipLaunchKernelGGL(prep_bwd_reduce_kernel, dim3((2 * C + 63) / 64), dim3(64 * PRB_WAVES), 0, s, ba);
    return hipGetLastError();
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_prep(const void *qkv, const float *q_norm_w, const float *k_norm_w, const float *proj_q,
                        const float *proj_kv, const float *rope_cos, const float *rope_sin, float k_scale,
                        float norm_eps, void *q_out, void *k_out, void *v_out, float *k_pre_sq,
                        float *k_post_sq, float *inflation_sq, int B, int N, int H, int D, int dtype,
                        int out_dtype, void *stream) {
    const char *name = "gdn_prep";
    GDN_REQUIRE(B >= 0 && N >= 0 && H >= 0, GDN_EINVAL, "%s: negative size (B=%d N=%d H=%d)", name, B, N, H);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(out_dtype == GDN_DTYPE_F32 || out_dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown out_dtype %d",
                name, out_dtype);
    GDN_REQUIRE(D > 0 && D % 16 == 0 && D <= 128, GDN_EUNSUPPORTED,
                "%s: D=%d (supported: multiples of 16 up to 128)", name, D);
    int lph = 2;                                 // lanes per head: D/8 rounded up to a power of two
    while (lph < D / 8) lph *= 2;
    GDN_REQUIRE((long)H * 8 * lph <= 4096, GDN_EUNSUPPORTED,
                "%s: H=%d heads of D=%d (at most 4096 / %d heads)", name, H, D, 8 * lph);
    GDN_REQUIRE(isfinite(k_scale) && isfinite(norm_eps) && norm_eps >= 0.f, GDN_EINVAL,
                "%s: k_scale and norm_eps must be finite, norm_eps >= 0", name);
    if ((long)B * N * H == 0) return GDN_OK;
    GDN_REQUIRE(qkv && proj_q && proj_kv && rope_cos && rope_sin && q_out && k_out && v_out && k_pre_sq &&
                    k_post_sq,
                GDN_EINVAL, "%s: null tensor pointer", name);
    GDN_REQUIRE(gdn::aligned(qkv, 16) && gdn::aligned(q_out, 16) && gdn::aligned(k_out, 16) &&
                    gdn::aligned(v_out, 16) && gdn::aligned(rope_cos, 16) && gdn::aligned(rope_sin, 16) &&
                    (!q_norm_w || gdn::aligned(q_norm_w, 16)) && (!k_norm_w || gdn::aligned(k_norm_w, 16)),
                GDN_EINVAL, "%s: qkv, the q/k/v outputs, the norm weights and the RoPE tables must be 16-byte aligned",
                name);
    GDN_REQUIRE(gdn::aligned(proj_q, 4) && gdn::aligned(proj_kv, 4) && gdn::aligned(k_pre_sq, 4) &&
                    gdn::aligned(k_post_sq, 4) && (!inflation_sq || gdn::aligned(inflation_sq, 4)),
                GDN_EINVAL, "%s: float tensors must be 4-byte aligned", name);
    gdn::PrepArgs a;
    a.qkv = qkv;
    a.qw = q_norm_w;
    a.kw = k_norm_w;
    a.proj_q = proj_q;
    a.proj_kv = proj_kv;
    a.cosv = rope_cos;
    a.sinv = rope_sin;
    a.k_scale = k_scale;
    a.eps = norm_eps;
    a.qo = q_out;
    a.ko = k_out;
    a.vo = v_out;
    a.pre = k_pre_sq;
    a.post = k_post_sq;
    a.infl = inflation_sq;
    a.B = B;
    a.N = N;
    a.H = H;
    a.D = D;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    const int sel = (dtype == GDN_DTYPE_F32 ? 2 : 0) + (out_dtype == GDN_DTYPE_F32 ? 1 : 0);
#define GDN_PREP_D(DD)                                                             \
    switch (sel) {                                                                 \
        case 0: e = gdn::launch_prep<false, false, DD>(a, s); break;               \
        case 1: e = gdn::launch_prep<false, true, DD>(a, s); break;                \
        case 2: e = gdn::launch_prep<true, false, DD>(a, s); break;                \
        default: e = gdn::launch_prep<true, true, DD>(a, s); break;                \
    }
    switch (lph) {
        case 2: GDN_PREP_D(2) break;
        case 4: GDN_PREP_D(4) break;
        case 8: GDN_PREP_D(8) break;
        default: GDN_PREP_D(16) break;
    }
#undef GDN_PREP_D
    return gdn::check_hip(e, name);
}

extern "C" size_t gdn_prep_bwd_workspace_bytes(int B, int N, int H, int D) {
    if (B < 0 || N < 0 || H <= 0 || D <= 0) return 0;
    return (size_t)gdn::prep_bwd_grid((long)B * N) * 4 * 2 * H * D * sizeof(float);
}

extern "C" int gdn_prep_bwd(const void *qkv, const float *q_norm_w, const float *k_norm_w, const float *proj_q,
                            const float *proj_kv, const float *rope_cos, const float *rope_sin, float k_scale,
                            float norm_eps, const void *dq_out, const void *dk_out, const void *dv_out,
                            const float *dk_pre_sq, const float *dk_post_sq, const float *dinflation_sq,
                            float *dqkv, float *dq_norm_w, float *dk_norm_w, float *dproj_q, float *dproj_kv,
                            int B, int N, int H, int D, int dtype, int grad_dtype, void *workspace,
                            size_t workspace_bytes, void *stream) {
    const char *name = "gdn_prep_bwd";
    GDN_REQUIRE(B >= 0 && N >= 0 && H >= 0, GDN_EINVAL, "%s: negative size (B=%d N=%d H=%d)", name, B, N, H);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(grad_dtype == GDN_DTYPE_F32 || grad_dtype == GDN_DTYPE_BF16, GDN_EINVAL,
                "%s: unknown grad_dtype %d", name, grad_dtype);
    GDN_REQUIRE(D > 0 && D % 16 == 0 && D <= 128, GDN_EUNSUPPORTED,
                "%s: D=%d (supported: multiples of 16 up to 128)", name, D);
    int lph = 2;
    while (lph < D / 8) lph *= 2;
    GDN_REQUIRE((long)H * 8 * lph <= 4096, GDN_EUNSUPPORTED,
                "%s: H=%d heads of D=%d (at most 4096 / %d heads)", name, H, D, 8 * lph);
    GDN_REQUIRE(isfinite(k_scale) && isfinite(norm_eps) && norm_eps >= 0.f, GDN_EINVAL,
                "%s: k_scale and norm_eps must be finite, norm_eps >= 0", name);
    GDN_REQUIRE(!dproj_q == !dproj_kv, GDN_EINVAL, "%s: dproj_q and dproj_kv are both given or both NULL", name);
    const bool wgrad = dq_norm_w || dk_norm_w;
    const size_t need = wgrad ? gdn_prep_bwd_workspace_bytes(B, N, H, D) : 0;
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);
    if ((long)H == 0) return GDN_OK;
    const bool any = (long)B * N > 0;
    if (any) {
        GDN_REQUIRE(qkv && proj_q && proj_kv && rope_cos && rope_sin && dq_out && dk_out && dv_out && dqkv,
                    GDN_EINVAL, "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(qkv, 16) && gdn::aligned(dq_out, 16) && gdn::aligned(dk_out, 16) &&
                        gdn::aligned(dv_out, 16) && gdn::aligned(dqkv, 16) && gdn::aligned(rope_cos, 16) &&
                        gdn::aligned(rope_sin, 16) && (!q_norm_w || gdn::aligned(q_norm_w, 16)) &&
                        (!k_norm_w || gdn::aligned(k_norm_w, 16)),
                    GDN_EINVAL, "%s: qkv, the gradients, dqkv, the weights and the RoPE tables must be 16-byte aligned",
                    name);
    }
    GDN_REQUIRE(gdn::aligned(proj_q, 4) && gdn::aligned(proj_kv, 4) && (!dk_pre_sq || gdn::aligned(dk_pre_sq, 4)) &&
                    (!dk_post_sq || gdn::aligned(dk_post_sq, 4)) && (!dinflation_sq || gdn::aligned(dinflation_sq, 4)) &&
                    (!dproj_q || (gdn::aligned(dproj_q, 4) && gdn::aligned(dproj_kv, 4))) &&
                    (!dq_norm_w || gdn::aligned(dq_norm_w, 4)) && (!dk_norm_w || gdn::aligned(dk_norm_w, 4)),
                GDN_EINVAL, "%s: float tensors must be 4-byte aligned", name);
    gdn::PrepBwdArgs ba;
    gdn::PrepArgs &a = ba.a;
    a.qkv = qkv;
    a.qw = q_norm_w;
    a.kw = k_norm_w;
    a.proj_q = proj_q;
    a.proj_kv = proj_kv;
    a.cosv = rope_cos;
    a.sinv = rope_sin;
    a.k_scale = k_scale;
    a.eps = norm_eps;
    a.qo = a.ko = a.vo = nullptr;
    a.pre = a.post = a.infl = nullptr;
    a.B = B;
    a.N = N;
    a.H = H;
    a.D = D;
    ba.gq = dq_out;
    ba.gk = dk_out;
    ba.gv = dv_out;
    ba.gpre = dk_pre_sq;
    ba.gpost = dk_post_sq;
    ba.ginf = dinflation_sq;
    ba.dqkv = dqkv;
    ba.dpq = dproj_q;
    ba.dpkv = dproj_kv;
    ba.wpart = wgrad ? reinterpret_cast<float *>(workspace) : nullptr;
    ba.dqw = dq_norm_w;
    ba.dkw = dk_norm_w;
    ba.nwaves = (int)gdn::prep_bwd_grid((long)B * N) * 4;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    const int sel = (dtype == GDN_DTYPE_F32 ? 2 : 0) + (grad_dtype == GDN_DTYPE_F32 ? 1 : 0);
#define GDN_PREPB_D(DD)                                                            \
    switch (sel) {                                                                 \
        case 0: e = gdn::launch_prep_bwd<false, false, DD>(ba, s); break;          \
        case 1: e = gdn::launch_prep_bwd<false, true, DD>(ba, s); break;           \
        case 2: e = gdn::launch_prep_bwd<true, false, DD>(ba, s); break;           \
        default: e = gdn::launch_prep_bwd<true, true, DD>(ba, s); break;           \
    }
    switch (lph) {
        case 2: GDN_PREPB_D(2) break;
        case 4: GDN_PREPB_D(4) break;
        case 8: GDN_PREPB_D(8) break;
        default: GDN_PREPB_D(16) break;
    }
#undef GDN_PREPB_D
    return gdn::check_hip(e, name);
}
