// C ABI: gdn_chunk_fwd and deltaproduct_chunk_fwd (argument checks and
// dispatch to the chunk kernel instantiations).
#include <math.h>

#include <mutex>

#include "api_common.h"
#include "chunk_dispatch.h"

// Scratch of gdn_chunk_fwd_noalloc: the work space of that entry point, one
// copy per device, held from the library's first use on a device until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): it passes the device address
// hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_dev[64];        // per device ordinal: device address of `scratch`

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void **out, const char *name) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return gdn::check_hip(e, name);
    GDN_REQUIRE(dev >= 0 && dev < 64, GDN_EUNSUPPORTED, "%s: device ordinal %d (at most 63)", name, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return gdn::check_hip(e, name);
        GDN_REQUIRE(p != nullptr, GDN_EHIP, "%s: no device address for the scratch array", name);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

// Instantiated key width that runs a key of width r*dk: the width itself
// for r = 2, else the next power of two (16 ... 256; the kernels read the
// features past r*dk as zero and never store them).
int padded_key_width(int r, int dk) {
    if (r != 1) return r * dk;
    int kd = 16;
    while (kd < dk) kd *= 2;
    return kd;
}

// Work space of a DeltaProduct call: enough for the general path and for
// the two-pass one (the query does not see the step mask).
size_t dp2_workspace(int dk, int B, int T, int H, int Dv, const gdn::ChunkImpl &general) {
    gdn::ChunkImpl dp2;
    const size_t g = general.workspace(B, T, H, Dv);
    if (!gdn::find_dp2(dk, &dp2)) return g;
    const size_t f = dp2.workspace(B, T, H, Dv);
    return f > g ? f : g;
}

// Token rows (H*K or H*Dv elements) below 2^24: the state passes form
// row offsets with 24-bit multiplies.
bool rows_ok(int H, int K, int Dv) { return (size_t)H * K < (1u << 24) && (size_t)H * Dv < (1u << 24); }

bool find_impl(int dtype, int r, int KD, int chunk, gdn::ChunkImpl *impl) {
    if (dtype == GDN_DTYPE_F32) return gdn::find_chunk_f32(KD, chunk, r, impl);
    if (r == 1) return gdn::find_chunk_bf16_r1(KD, chunk, impl);
    if (r == 2) return gdn::find_chunk_bf16_r2(KD, chunk, impl);
    return false;
}

int chunk_common(const void *q, const void *k, const void *v, const float *beta,
                 const float *log_decay, const float *step_mask, int r, float scale,
                 const float *h0, float *hT, void *o, int B, int T, int H, int dk, int Dv,
                 int chunk, int dtype, int out_dtype, void *workspace, size_t workspace_bytes,
                 void *stream, const char *name, bool noalloc = false) {
    GDN_REQUIRE(B >= 0 && T >= 0 && H >= 0, GDN_EINVAL, "%s: negative size (B=%d T=%d H=%d)", name, B, T, H);
    GDN_REQUIRE(dtype == GDN_DTYPE_F32 || dtype == GDN_DTYPE_BF16, GDN_EINVAL, "%s: unknown dtype %d", name, dtype);
    GDN_REQUIRE(out_dtype == GDN_DTYPE_F32 || out_dtype == GDN_DTYPE_BF16, GDN_EINVAL,
                "%s: unknown out_dtype %d", name, out_dtype);
    GDN_REQUIRE(r == 1 || r == 2, GDN_EUNSUPPORTED, "%s: r=%d (supported: 1, 2)", name, r);
    if (r == 1)
        GDN_REQUIRE(dk > 0 && dk % 16 == 0 && dk <= 256, GDN_EUNSUPPORTED,
                    "%s: key width %d (supported: multiples of 16 up to 256)", name, dk);
    else
        GDN_REQUIRE(dk == 16 || dk == 32 || dk == 64 || dk == 128, GDN_EUNSUPPORTED,
                    "%s: sub-key width %d (supported: 16, 32, 64, 128)", name, dk);
    GDN_REQUIRE(r * dk <= 256, GDN_EUNSUPPORTED, "%s: total key width r*dk=%d exceeds 256", name, r * dk);
    GDN_REQUIRE(Dv > 0 && Dv % 16 == 0 && Dv <= 256, GDN_EUNSUPPORTED,
                "%s: Dv=%d (must be a multiple of 16, at most 256)", name, Dv);
    GDN_REQUIRE(chunk == 16 || chunk == 32 || chunk == 64, GDN_EUNSUPPORTED,
                "%s: chunk=%d (supported: 16, 32, 64)", name, chunk);
    GDN_REQUIRE(chunk * r <= 64, GDN_EUNSUPPORTED, "%s: chunk*r=%d exceeds 64", name, chunk * r);
    GDN_REQUIRE(rows_ok(H, r * dk, Dv), GDN_EUNSUPPORTED,
                "%s: token rows of H*K=%zu or H*Dv=%zu elements (at most 2^24 - 1)", name, (size_t)H * r * dk,
                (size_t)H * Dv);
    GDN_REQUIRE(isfinite(scale), GDN_EINVAL, "%s: scale is not finite", name);
    const size_t ntok = (size_t)B * T * H;
    if (ntok > 0) {
        GDN_REQUIRE(q && k && v && beta && log_decay && o, GDN_EINVAL, "%s: null tensor pointer", name);
        GDN_REQUIRE(gdn::aligned(q, 16) && gdn::aligned(k, 16) && gdn::aligned(v, 16) && gdn::aligned(o, 16),
                    GDN_EINVAL, "%s: q, k, v and o must be 16-byte aligned", name);
        GDN_REQUIRE(gdn::aligned(beta, 4) && gdn::aligned(log_decay, 4), GDN_EINVAL,
                    "%s: beta and log_decay must be 4-byte aligned", name);
    }
    GDN_REQUIRE(!h0 || gdn::aligned(h0, 4), GDN_EINVAL, "%s: h0 misaligned", name);
    GDN_REQUIRE(!hT || gdn::aligned(hT, 4), GDN_EINVAL, "%s: hT misaligned", name);
    GDN_REQUIRE(r == 1 || step_mask, GDN_EINVAL, "%s: step_mask is required for r=%d", name, r);
    if (step_mask)
        for (int i = 0; i < r * r; ++i)
            GDN_REQUIRE(isfinite(step_mask[i]), GDN_EINVAL, "%s: step_mask[%d] is not finite", name, i);
    const int KD = padded_key_width(r, dk);
    gdn::ChunkImpl impl;
    GDN_REQUIRE(find_impl(dtype, r, KD, chunk, &impl), GDN_EUNSUPPORTED,
                "%s: no kernel for dtype=%s r=%d key width=%d chunk=%d", name,
                dtype == GDN_DTYPE_F32 ? "f32" : "bf16", r, r * dk, chunk);
    // two steps with a lower unitriangular mask (bf16): two passes of the
    // single-chain kernels (the work-space query covers both paths)
    gdn::ChunkImpl dp2;
    const bool use_dp2 = r == 2 && T > 0 && dtype == GDN_DTYPE_BF16 && step_mask[0] == 1.f &&
                         step_mask[1] == 0.f && step_mask[3] == 1.f && gdn::find_dp2(dk, &dp2);
    if ((size_t)B * H == 0) return GDN_OK;
    const size_t need = use_dp2 ? dp2_workspace(dk, B, T, H, Dv, impl) : impl.workspace(B, T, H, Dv);
    if (noalloc) {
        GDN_REQUIRE(need <= GDN_NOALLOC_SCRATCH_BYTES, GDN_EWORKSPACE,
                    "%s: this shape needs %zu bytes of scratch, the no-allocation entry point holds at most "
                    "%zu (call gdn_chunk_fwd with a work space)", name, need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        if (need > 0) {
            const int rc = scratch_address(&workspace, name);
            if (rc != GDN_OK) return rc;
        }
        workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
    }
    GDN_REQUIRE(workspace_bytes >= need, GDN_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", name,
                workspace_bytes, need);
    GDN_REQUIRE(need == 0 || (workspace && gdn::aligned(workspace, 16)), GDN_EINVAL,
                "%s: workspace must be a 16-byte aligned device pointer", name);

    gdn::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = log_decay;
    a.h0 = h0;
    a.hT = hT;
    a.o = o;
    a.tmat = workspace;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dv = Dv;
    a.kw = r * dk;
    a.kst = r * dk;
    a.koff = 0;
    a.bst = 1;
    a.boff = 0;
    a.hrows = r * dk;
    a.hoff = 0;
    a.atil = nullptr;
    a.vout = nullptr;
    a.vin = nullptr;
    a.oprev = nullptr;
    a.mcoef = r == 2 ? step_mask[2] : 0.f;
    a.nsub = 1;
    a.subws = 0;
    a.out_bf16 = out_dtype == GDN_DTYPE_BF16;
    a.scale = scale;
    a.tmatT = nullptr;
    a.atilT = nullptr;
    a.sst = a.rst = nullptr;
    for (int i = 0; i < 4; ++i) a.mask[i] = 0.f;
    if (r == 1) {
        a.mask[0] = step_mask ? step_mask[0] : 1.f;
    } else {
        for (int i = 0; i < r * r; ++i) a.mask[i] = step_mask[i];
    }
    return gdn::check_hip((use_dp2 ? dp2 : impl).launch(a, reinterpret_cast<hipStream_t>(stream)), name);
}

}  // namespace

extern "C" int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *beta,
                             const float *log_decay, float scale, const float *h0, float *hT, void *o,
                             int B, int T, int H, int Dk, int Dv, int chunk, int dtype, int out_dtype,
                             void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_common(q, k, v, beta, log_decay, nullptr, 1, scale, h0, hT, o, B, T, H, Dk, Dv, chunk,
                        dtype, out_dtype, workspace, workspace_bytes, stream, "gdn_chunk_fwd");
}

extern "C" int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *beta,
                                     const float *log_decay, float scale, const float *h0, float *hT, void *o,
                                     int B, int T, int H, int Dk, int Dv, int chunk, int dtype, int out_dtype,
                                     void *stream) {
    return chunk_common(q, k, v, beta, log_decay, nullptr, 1, scale, h0, hT, o, B, T, H, Dk, Dv, chunk,
                        dtype, out_dtype, nullptr, 0, stream, "gdn_chunk_fwd_noalloc", true);
}

extern "C" size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, int dtype) {
    gdn::ChunkImpl impl;
    if (B < 0 || T < 0 || H < 0 || Dv <= 0 || Dk <= 0 || Dk % 16 || Dk > 256 || !rows_ok(H, Dk, Dv) ||
        !find_impl(dtype, 1, padded_key_width(1, Dk), chunk, &impl))
        return 0;
    return impl.workspace(B, T, H, Dv);
}

extern "C" int deltaproduct_chunk_fwd(const void *q, const void *k, const void *v, const float *beta,
                                      const float *log_decay, const float *step_mask, int r, float scale,
                                      const float *h0, float *hT, void *o, int B, int T, int H, int dk,
                                      int Dv, int chunk, int dtype, int out_dtype, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    return chunk_common(q, k, v, beta, log_decay, step_mask, r, scale, h0, hT, o, B, T, H, dk, Dv, chunk,
                        dtype, out_dtype, workspace, workspace_bytes, stream, "deltaproduct_chunk_fwd");
}

extern "C" size_t deltaproduct_chunk_fwd_workspace_bytes(int B, int T, int H, int r, int dk, int Dv,
                                                         int chunk, int dtype) {
    gdn::ChunkImpl impl;
    if (B < 0 || T < 0 || H < 0 || Dv <= 0 || dk <= 0 || dk % 16 || r * dk > 256 || !rows_ok(H, r * dk, Dv) ||
        !find_impl(dtype, r, padded_key_width(r, dk), chunk, &impl))
        return 0;
    if (r == 2 && dtype == GDN_DTYPE_BF16) return dp2_workspace(dk, B, T, H, Dv, impl);
    return impl.workspace(B, T, H, Dv);
}
