// Chunkwise backward of the gated delta rule (bf16 inputs, one step per
// token, 64-token chunks): work-space layout and the four launches (prep,
// forward state pass, reverse state pass, per-chunk gradients); and the
// backward of the two-step gated DeltaProduct with a lower unitriangular
// step mask as two chained passes of the same kernels (C ABI
// deltaproduct_bwd).
#include <math.h>

#include "api_common.h"
#include "chunk_bwd.h"
#include "chunk_dispatch.h"
#include "gdn.h"

namespace gdn {

namespace {

constexpr int BC = 64;                          // chunk length of the backward

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work-space regions, per (batch*head, chunk): T diag(beta) and T^T (bf16,
// C x C), the transposed scores (hi/lo fragments), the gate table, the
// forward's chunk-start state and residual R, the backward's dS' and dX.
struct BwdLayout {
    size_t tmat, tmatT, pfrag, gtab, sst, rst, dsst, dxst, total;
};

BwdLayout bwd_layout(int B, int T, int H, int Dk, int Dv) {
    const size_t n = (size_t)B * H * ((T + BC - 1) / BC);
    constexpr int NLOW = (BC / 16) * (BC / 16 + 1) / 2;
    BwdLayout L;
    size_t o = 0;
    L.tmat = o;  o += al256(n * BC * BC * 2);
    L.tmatT = o; o += al256(n * BC * BC * 2);
    L.pfrag = o; o += al256(n * NLOW * 64 * 16);
    L.gtab = o;  o += al256(n * gate_table_len<BC>() * 4);
    L.sst = o;   o += al256(n * Dk * Dv * 4);
    L.rst = o;   o += al256(n * BC * Dv * 4);
    L.dsst = o;  o += al256(n * Dk * Dv * 4);
    L.dxst = o;  o += al256(n * BC * Dv * 4);
    L.total = o;
    return L;
}

template <int KD>
hipError_t launch(BwdChunkArgs ba, char *ws, hipStream_t s) {
    ChunkArgs &a = ba.a;
    const BwdLayout L = bwd_layout(a.B, a.T, a.H, KD, a.Dv);
    a.tmat = ws + L.tmat;
    a.tmatT = ws + L.tmatT;
    a.pfrag = ws + L.pfrag;
    a.gtab = ws + L.gtab;
    a.sst = reinterpret_cast<float *>(ws + L.sst);
    a.rst = reinterpret_cast<float *>(ws + L.rst);
    ba.dsst = reinterpret_cast<float *>(ws + L.dsst);
    ba.dxst = reinterpret_cast<float *>(ws + L.dxst);
    const int NT = (a.T + BC - 1) / BC, nbh = a.B * a.H;
    const int nwg = (nbh * NT + 3) / 4;
    const int pgrid = nwg < 2 * num_cus() ? nwg : 2 * num_cus();
    hipLaunchKernelGGL((chunk_prep2_kernel<KD, BC, true>), dim3(pgrid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int cgrid = ((nbh + 7) / 8) * 8 * (a.Dv / 16);
    hipLaunchKernelGGL((chunk_chain1_kernel<KD, BC, 3>), dim3(cgrid), dim3(Chain1Shape<KD, BC>::NTHR), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_bchain_kernel<KD>), dim3(cgrid), dim3(BChainShape<KD>::NTHR), 0, s, ba);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ba.nfirst = num_cus();
    hipLaunchKernelGGL((chunk_bgrad_kernel<KD>), dim3(nbh * NT), dim3(BGradShape<KD>::NTHR), 0, s, ba);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// DeltaProduct, r = 2, step mask [[1, 0], [m, 1]]: the state's row block 0 is
// a gated delta rule on (q_0, k_0, v, beta_0) and row block 1 one on
// (q_1, k_1, v', beta_1), v' = (1 - m) v + m e with e block 0's per-token
// errors.  Backward: block 1's backward (its dv is the gradient of v'), then
// block 0's with dE = m dv' (DPE kernels), which also adds dv' to dv and
// block 1's dg to dg.  Work space: per sub-key the prep's outputs and the
// forward states and residuals (subws bytes each), then dS' and dX (shared
// by the passes), A~ in both fragment layouts (sub-key 0) and v'.
// ---------------------------------------------------------------------------
struct DpBwdLayout {
    BwdLayout L;            // regions of one sub-key (tmat .. rst), then dsst, dxst
    size_t subws, dsst, dxst, atil, atilT, vprime, total;
};

DpBwdLayout dp_bwd_layout(int B, int T, int H, int dk, int Dv) {
    DpBwdLayout D;
    D.L = bwd_layout(B, T, H, dk, Dv);
    const size_t n = (size_t)B * H * ((T + BC - 1) / BC);
    constexpr int NLOW = (BC / 16) * (BC / 16 + 1) / 2;
    D.subws = D.L.dsst;     // tmat, tmatT, pfrag, gtab, sst, rst
    size_t o = 2 * D.subws;
    D.dsst = o;   o += al256(n * dk * Dv * 4);
    D.dxst = o;   o += al256(n * BC * Dv * 4);
    D.atil = o;   o += al256(n * NLOW * 64 * 16);
    D.atilT = o;  o += al256(n * NLOW * 64 * 16);
    D.vprime = o; o += al256(n * BC * Dv * 4);      // v' in tile order (whole chunks)
    D.total = o;
    return D;
}

template <int KD>
hipError_t launch_dp(BwdChunkArgs ba, char *ws, hipStream_t s) {
    const DpBwdLayout D = dp_bwd_layout(ba.a.B, ba.a.T, ba.a.H, KD, ba.a.Dv);
    const BwdLayout &L = D.L;
    const int NT = (ba.a.T + BC - 1) / BC, nbh = ba.a.B * ba.a.H;
    ba.dsst = reinterpret_cast<float *>(ws + D.dsst);
    ba.dxst = reinterpret_cast<float *>(ws + D.dxst);
    // the arguments of sub-key `sub`: its work-space block, key columns,
    // beta column and state rows
    auto sub_args = [&](int sub) {
        BwdChunkArgs x = ba;
        ChunkArgs &a = x.a;
        char *blk = ws + sub * D.subws;
        a.tmat = blk + L.tmat;
        a.tmatT = blk + L.tmatT;
        a.pfrag = blk + L.pfrag;
        a.gtab = blk + L.gtab;
        a.sst = reinterpret_cast<float *>(blk + L.sst);
        a.rst = reinterpret_cast<float *>(blk + L.rst);
        a.koff = sub * KD;
        a.boff = sub;
        a.hoff = sub * KD;
        return x;
    };
    float *vprime = reinterpret_cast<float *>(ws + D.vprime);
    // prep of both sub-keys in one launch (sub-key 1's outputs subws bytes on);
    // A~ of sub-key 0 in both layouts
    BwdChunkArgs b0 = sub_args(0), b1 = sub_args(1);
    ChunkArgs pp = b0.a;
    pp.nsub = 2;
    pp.subws = D.subws;
    pp.atil = ws + D.atil;
    pp.atilT = ws + D.atilT;
    const int nwg = (2 * nbh * NT + 3) / 4;
    const int pgrid = nwg < 2 * num_cus() ? nwg : 2 * num_cus();
    hipLaunchKernelGGL((chunk_prep2_kernel<KD, BC, true>), dim3(pgrid), dim3(256), 0, s, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int cgrid = ((nbh + 7) / 8) * 8 * (ba.a.Dv / 16);
    // forward state passes: sub-key 0 (also writing v'), then sub-key 1 on v'
    ChunkArgs f0 = b0.a;
    f0.atil = ws + D.atil;
    f0.vout = vprime;
    hipLaunchKernelGGL((chunk_chain1_kernel<KD, BC, 5>), dim3(cgrid), dim3(Chain1Shape<KD, BC>::NTHR), 0, s, f0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ChunkArgs f1 = b1.a;
    f1.vin = vprime;
    hipLaunchKernelGGL((chunk_chain1_kernel<KD, BC, 4>), dim3(cgrid), dim3(Chain1Shape<KD, BC>::NTHR), 0, s, f1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the backward of sub-key 1 (dv gets the gradient of v')
    hipLaunchKernelGGL((chunk_bchain_kernel<KD, false>), dim3(cgrid), dim3(BChainShape<KD>::NTHR), 0, s, b1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    b1.nfirst = num_cus();
    hipLaunchKernelGGL((chunk_bgrad_kernel<KD, false>), dim3(nbh * NT), dim3(BGradShape<KD>::NTHR), 0, s, b1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the backward of sub-key 0 with dE = m dv'
    b0.a.atil = ws + D.atil;
    b0.a.atilT = ws + D.atilT;
    b0.dvprev = ba.dv;
    hipLaunchKernelGGL((chunk_bchain_kernel<KD, true>), dim3(cgrid), dim3(BChainShape<KD>::NTHR), 0, s, b0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    b0.nfirst = num_cus();
    hipLaunchKernelGGL((chunk_bgrad_kernel<KD, true>), dim3(nbh * NT), dim3(BGradShape<KD>::NTHR), 0, s, b0);
    return hipGetLastError();
}

// dh0 of an empty sequence: dhT, or zero
__global__ void dp_pass_state_kernel(const float *dhT, float *dh0, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dh0[i] = dhT ? dhT[i] : 0.f;
}

}  // namespace

bool dp_bwd_eligible(int dk, int Dv) {
    return (dk == 32 || dk == 64 || dk == 128) && Dv % 32 == 0 && Dv >= 32 && Dv <= 128;
}

size_t dp_bwd_workspace(int B, int T, int H, int dk, int Dv) {
    return T > 0 ? dp_bwd_layout(B, T, H, dk, Dv).total : 0;
}

hipError_t dp_bwd_launch(const BwdChunkArgs &ba, int dk, void *workspace, hipStream_t s) {
    char *ws = static_cast<char *>(workspace);
    switch (dk) {
        case 32: return launch_dp<32>(ba, ws, s);
        case 64: return launch_dp<64>(ba, ws, s);
        default: return launch_dp<128>(ba, ws, s);
    }
}

// The chunkwise path takes bf16 inputs with Dk in {32, 64, 128} and Dv a
// multiple of 32 up to 128, and token rows (H Dk and H Dv elements) below
// 2^24 elements: its staging forms row offsets with 24-bit multiplies.
bool chunk_bwd_strides_ok(int H, int K, int Dv) {
    return (size_t)H * K < (1u << 24) && (size_t)H * Dv < (1u << 24);
}
bool chunk_bwd_eligible(int T, int H, int Dk, int Dv, int dtype) {
    return dtype == GDN_DTYPE_BF16 && T > 0 && (Dk == 32 || Dk == 64 || Dk == 128) && Dv % 32 == 0 && Dv >= 32 &&
           Dv <= 128 && chunk_bwd_strides_ok(H, Dk, Dv);
}

size_t chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv) { return bwd_layout(B, T, H, Dk, Dv).total; }

hipError_t chunk_bwd_launch(const void *q, const void *k, const void *v, const float *beta, const float *g,
                            float scale, const float *h0, const void *dout, const float *dhT, float *dq, float *dk,
                            float *dv, float *dbeta, float *dg, float *dh0, int B, int T, int H, int Dk, int Dv,
                            void *workspace, hipStream_t s) {
    BwdChunkArgs ba = {};
    ChunkArgs &a = ba.a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.h0 = h0;
    a.hT = nullptr;
    a.o = nullptr;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dv = Dv;
    a.kw = Dk;
    a.kst = Dk;
    a.koff = 0;
    a.bst = 1;
    a.boff = 0;
    a.hrows = Dk;
    a.hoff = 0;
    a.atil = nullptr;
    a.vout = nullptr;
    a.vin = nullptr;
    a.oprev = nullptr;
    a.mcoef = 0.f;
    a.nsub = 1;
    a.subws = 0;
    a.out_bf16 = 0;
    a.scale = scale;
    ba.dout = dout;
    ba.dhT = dhT;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dbeta = dbeta;
    ba.dg = dg;
    ba.dh0 = dh0;
    char *ws = static_cast<char *>(workspace);
    switch (Dk) {
        case 32: return launch<32>(ba, ws, s);
        case 64: return launch<64>(ba, ws, s);
        default: return launch<128>(ba, ws, s);
    }
}

}  // namespace gdn

extern "C" size_t deltaproduct_bwd_workspace_bytes(int B, int T, int H, int r, int dk, int Dv, int dtype) {
    if (B < 0 || T < 0 || H < 0 || r != 2 || dtype != GDN_DTYPE_BF16 || !gdn::dp_bwd_eligible(dk, Dv) ||
        !gdn::chunk_bwd_strides_ok(H, 2 * dk, Dv))
        return 0;
    return gdn::dp_bwd_workspace(B, T, H, dk, Dv);
}

extern "C" int deltaproduct_bwd(const void *q, const void *k, const void *v, const float *beta,
                                const float *log_decay, const float *step_mask, int r, float scale,
                                const float *h0, const void *dout, const float *dhT, float *dq, float *dk,
                                float *dv, float *dbeta, float *dlog_decay, float *dh0, int B, int T, int H,
                                int sub_dk, int Dv, int dtype, void *workspace, size_t workspace_bytes,
                                void *stream) {
    const char *name = "deltaproduct_bwd";
    GDN_REQUIRE(B >= 0 && T >= 0 && H >= 0, GDN_EINVAL, "%s: negative size (B=%d T=%d H=%d)", name, B, T, H);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(dtype == GDN_DTYPE_BF16, GDN_EUNSUPPORTED, "%s: bf16 inputs only", name);
    GDN_REQUIRE(r == 2, GDN_EUNSUPPORTED, "%s: r=%d (supported: 2; r=1 is gdn_bwd)", name, r);
    GDN_REQUIRE(step_mask, GDN_EINVAL, "%s: step_mask is required", name);
    for (int i = 0; i < 4; ++i)
        GDN_REQUIRE(isfinite(step_mask[i]), GDN_EINVAL, "%s: step_mask[%d] is not finite", name, i);
    GDN_REQUIRE(step_mask[0] == 1.f && step_mask[1] == 0.f && step_mask[3] == 1.f, GDN_EUNSUPPORTED,
                "%s: step mask must be lower unitriangular [[1, 0], [m, 1]]", name);
    GDN_REQUIRE(sub_dk == 32 || sub_dk == 64 || sub_dk == 128, GDN_EUNSUPPORTED,
                "%s: sub-key width %d (supported: 32, 64, 128)", name, sub_dk);
    GDN_REQUIRE(gdn::dp_bwd_eligible(sub_dk, Dv), GDN_EUNSUPPORTED, "%s: Dv=%d (a multiple of 32 from 32 to 128)",
                name, Dv);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    if ((size_t)B * H == 0) return GDN_OK;
    const size_t nst = (size_t)B * H * 2 * sub_dk * Dv;
    GDN_REQUIRE((!h0 || gdn::aligned(h0, 16)) && (!dhT || gdn::aligned(dhT, 16)) && (!dh0 || gdn::aligned(dh0, 16)),
                GDN_EINVAL, "%s: misaligned state pointer", name);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T == 0) {           // no tokens: dh0 = dhT
        if (!dh0) return GDN_OK;
        hipLaunchKernelGGL(gdn::dp_pass_state_kernel, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, s, dhT, dh0,
                           nst);
        return gdn::check_hip(hipGetLastError(), name);
    }
    GDN_REQUIRE(q && k && v && beta && log_decay && dout && dq && dk && dv && dbeta && dlog_decay, GDN_EINVAL,
                "%s: null tensor pointer", name);
    GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && gdn::aligned(v, 16) && gdn::aligned(dout, 16) &&
                    gdn::aligned(dq, 16) && gdn::aligned(dk, 16) && gdn::aligned(dv, 16),
                GDN_EINVAL, "%s: q, k, v, dout, dq, dk and dv must be 16-byte aligned", name);
    GDN_REQUIRE(gdn::aligned(beta, 4) && gdn::aligned(log_decay, 4) && gdn::aligned(dbeta, 4) &&
                    gdn::aligned(dlog_decay, 4),
                GDN_EINVAL, "%s: misaligned tensor pointer", name);
    const size_t need = gdn::dp_bwd_workspace(B, T, H, sub_dk, Dv);
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(workspace && gdn::aligned(workspace, 256), GDN_EINVAL,
                "%s: workspace must be a 256-byte aligned device pointer", name);
    GDN_REQUIRE((size_t)B * H * ((T + 63) / 64) < (1u << 31), GDN_EUNSUPPORTED, "%s: too many chunks", name);
    GDN_REQUIRE(gdn::chunk_bwd_strides_ok(H, 2 * sub_dk, Dv), GDN_EUNSUPPORTED,
                "%s: token rows of H * K or H * Dv elements must be below 2^24", name);
    gdn::BwdChunkArgs ba = {};
    gdn::ChunkArgs &a = ba.a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = log_decay;
    a.h0 = h0;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dv = Dv;
    a.kw = sub_dk;
    a.kst = 2 * sub_dk;
    a.bst = 2;
    a.hrows = 2 * sub_dk;
    a.mcoef = step_mask[2];
    a.nsub = 1;
    a.scale = scale;
    ba.dout = dout;
    ba.dhT = dhT;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dbeta = dbeta;
    ba.dg = dlog_decay;
    ba.dh0 = dh0;
    return gdn::check_hip(gdn::dp_bwd_launch(ba, sub_dk, workspace, s), name);
}
