// Chunkwise backward of the gated delta rule (bf16 inputs, one step per
// token, 64-token chunks): work-space layout and the four launches (prep,
// forward state pass, reverse state pass, per-chunk gradients).
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
    hipLaunchKernelGGL((chunk_bgrad_kernel<KD>), dim3(nbh * NT), dim3(BGradShape<KD>::NTHR), 0, s, ba);
    return hipGetLastError();
}

}  // namespace

// The chunkwise path takes bf16 inputs with Dk in {32, 64, 128} and Dv a
// multiple of 32 up to 128.
bool chunk_bwd_eligible(int T, int Dk, int Dv, int dtype) {
    return dtype == GDN_DTYPE_BF16 && T > 0 && (Dk == 32 || Dk == 64 || Dk == 128) && Dv % 32 == 0 && Dv >= 32 &&
           Dv <= 128;
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
