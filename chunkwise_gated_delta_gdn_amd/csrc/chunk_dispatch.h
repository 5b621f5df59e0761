// Lookup of the chunk kernel instantiations (one source file per input type
// and step count, so they compile in parallel).
#pragma once

#include <atomic>

#include "chunk_chain1.h"
#include "chunk_kernels.h"
#include "chunk_prep2.h"
#include "chunk_seg.h"

namespace gdn {

// The single-chain-wave state pass covers bf16 inputs, one step per token,
// and chunk / key widths that are multiples of 32; everything else runs the
// general 8-wave state pass.
template <bool F32IN, int KD, int C, int R>
constexpr bool use_chain1() {
    return ChunkShape<F32IN, KD, C, R>::PFRAG;
}

// Compute units of the current device.  Cached per device ordinal in an
// atomic (relaxed): concurrent first calls on one device each query the
// attribute and store the same value, so the cache needs no lock.
inline int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// bf16 inputs, one step per token, 64-token chunks and key widths up to 128
// run the segment pass (chunk_seg.h) after the prep.
template <bool F32IN, int KD, int C, int R>
constexpr bool use_seg() {
    return !F32IN && R == 1 && C == 64 && KD % 32 == 0 && KD <= 128;
}

// Choice between the two state passes for the segment-pass shapes, and the
// segment count: a model of a 256-CU device with per-chunk-step times
// measured on MI355X (B=2 H=16 T=4096 and B=1 H=16 T=65536, Dk = Dv = 128):
//   chunk_chain1_kernel   one workgroup per (b, h, 16 columns), one per CU,
//                         1.3 us per chunk step;
//   segment pass          summaries 3.3 us per chunk step (one workgroup per
//                         CU), compose 4 us per segment, output 6.7 us per
//                         chunk step (one workgroup per CU), each workgroup
//                         covering 128 columns.
// Returns 0 for chunk_chain1_kernel, else the segment count P (1 = the
// output pass over all chunks).  A fixed model (not the queried device), so
// the work space does not depend on the device it is queried on.
inline int seg_count(int nbh, int NT, int Dv, int KD) {
    constexpr int SLOTS = 256, MIN_LS = 4;
    constexpr double T_CHAIN = 1.3, T_SUM = 3.3, T_COMP = 4.0, T_OUT = 6.7;
    const int ncgv = (Dv + 127) / 128, ncga = (KD + 127) / 128;
    auto rounds = [&](long wgs) { return (double)((wgs + SLOTS - 1) / SLOTS); };
    double best = rounds((long)nbh * (Dv / 16)) * NT * T_CHAIN;
    int bestP = 0;
    const double t1 = rounds((long)nbh * ncgv) * NT * T_OUT;
    if (t1 < best) {
        best = t1;
        bestP = 1;
    }
    for (int P = 3; P <= NT / MIN_LS && P <= 256; ++P) {
        const int LS = (NT + P - 1) / P, Pe = (NT + LS - 1) / LS;
        if (Pe < 3) continue;
        const long sum_wgs = (long)nbh * ncgv + (long)nbh * (Pe - 2) * (ncgv + ncga);
        const double t = rounds(sum_wgs) * LS * T_SUM + (Pe - 2) * T_COMP + rounds((long)nbh * Pe * ncgv) * LS * T_OUT;
        if (t < best) {
            best = t;
            bestP = Pe;
        }
    }
    return bestP;
}

template <int KD>
hipError_t launch_seg(const ChunkArgs &a, char *seg_ws, hipStream_t stream) {
    const int NT = (a.T + 63) / 64, nbh = a.B * a.H;
    SegArgs sa;
    sa.a = a;
    sa.P = seg_count(nbh, NT, a.Dv, KD);
    sa.LS = (NT + sa.P - 1) / sa.P;
    sa.P = (NT + sa.LS - 1) / sa.LS;
    sa.amat = reinterpret_cast<float *>(seg_ws);
    sa.bmat = sa.amat + (size_t)nbh * sa.P * KD * KD;
    const int ncgv = (a.Dv + 127) / 128, ncga = (KD + 127) / 128;
    if (sa.P > 1) {
        sa.nseg_units = nbh + nbh * (sa.P - 2);
        const int grid = (sa.nseg_units + 7) / 8 * 8 * (ncgv + ncga);
        hipLaunchKernelGGL((chunk_seg_kernel<KD, false>), dim3(grid), dim3(SegShape<KD>::NTHR), 0, stream, sa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (sa.P > 2) {
            hipLaunchKernelGGL((seg_compose_kernel<KD>), dim3(nbh * ((a.Dv + 31) / 32)), dim3(256), 0, stream, sa);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    sa.nseg_units = 0;
    hipLaunchKernelGGL((chunk_seg_kernel<KD, true>), dim3(nbh * sa.P * ncgv), dim3(SegShape<KD>::NTHR), 0, stream, sa);
    return hipGetLastError();
}

// Launch the kernels of one instantiation on `stream`.
template <bool F32IN, int KD, int C, int R>
hipError_t launch_chunk_fwd(const ChunkArgs &args, hipStream_t stream) {
    ChunkArgs a = args;
    a.pfrag = a.gtab = nullptr;
    if (use_chain1<F32IN, KD, C, R>()) {
        char *ws = static_cast<char *>(a.tmat) + chunk_tmat_bytes<F32IN, KD, C, R>(a.B, a.T, a.H);
        a.pfrag = ws;
        a.gtab = ws + chunk_pfrag_bytes<F32IN, KD, C, R>(a.B, a.T, a.H);
    }
    const int NT = (a.T + C - 1) / C;
    const int nbh = a.B * a.H;
    if (nbh == 0) return hipSuccess;
    if (NT > 0) {
        if constexpr (use_chain1<F32IN, KD, C, R>()) {
            // one wave per chunk, four per workgroup, at most two workgroups per
            // CU resident; waves walk the chunks with the grid stride
            const int nchunks = nbh * NT;
            const int nwg = (nchunks + 3) / 4;
            const int grid = nwg < 2 * num_cus() ? nwg : 2 * num_cus();
            hipLaunchKernelGGL((chunk_prep2_kernel<KD, C>), dim3(grid), dim3(256), 0, stream, a);
        } else {
            hipLaunchKernelGGL((chunk_solve_kernel<F32IN, KD, C, R>), dim3(nbh * NT), dim3(256), 0, stream, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (use_seg<F32IN, KD, C, R>()) {
        if (NT > 0 && seg_count(nbh, NT, a.Dv, KD) > 0) {
            char *seg_ws = static_cast<char *>(a.tmat) + chunk_workspace_bytes<F32IN, KD, C, R>(a.B, a.T, a.H);
            return launch_seg<KD>(a, seg_ws, stream);
        }
    }
    const int nvb = a.Dv / 16;
    const int grid = ((nbh + 7) / 8) * 8 * nvb;
    if constexpr (use_chain1<F32IN, KD, C, R>()) {
        // more chains than compute units: the two-workgroups-per-CU
        // configuration runs them in one round instead of two or more
        if constexpr (C == 64) {
            if (grid > num_cus()) {
                hipLaunchKernelGGL((chunk_chain1_kernel<KD, C, 0, true>), dim3(grid), dim3(Chain1Shape<KD, C, true>::NTHR),
                                   0, stream, a);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((chunk_chain1_kernel<KD, C>), dim3(grid), dim3(Chain1Shape<KD, C>::NTHR), 0, stream, a);
    } else {
        hipLaunchKernelGGL((chunk_chain_kernel<F32IN, KD, C, R>), dim3(grid), dim3(512), 0, stream, a);
    }
    return hipGetLastError();
}

// Work space of one instantiation: the prep's, and the segment pass's.
template <bool F32IN, int KD, int C, int R>
size_t chunk_fwd_workspace_bytes(int B, int T, int H, int Dv) {
    size_t n = chunk_workspace_bytes<F32IN, KD, C, R>(B, T, H);
    if constexpr (use_seg<F32IN, KD, C, R>()) {
        const int NT = (T + C - 1) / C;
        int P = NT > 0 ? seg_count(B * H, NT, Dv, KD) : 0;
        if (P > 0) {
            const int LS = (NT + P - 1) / P;
            P = (NT + LS - 1) / LS;
            n += seg_workspace_bytes<KD>(B, H, Dv, P);
        }
    }
    return n;
}

// Gated DeltaProduct, two sub-keys of width KD, lower unitriangular step
// mask [[1, 0], [m, 1]], bf16: two passes of the single-chain kernels with
// 64-token chunks (chunk_chain1.h, DPM), the first on sub-key 0 (also
// writing v' and its output in fp32), the second on sub-key 1 with v' as
// the values.  Work space: the prep's (shared by the passes), the A~
// fragments, v' and the first output.
template <int KD>
size_t dp2_workspace_bytes(int B, int T, int H, int Dv) {
    constexpr int C = 64;
    const size_t prep = 2 * ((chunk_workspace_bytes<false, KD, C, 1>(B, T, H) + 255) & ~(size_t)255);
    const size_t at = chunk_pfrag_bytes<false, KD, C, 1>(B, T, H);
    // v' and the first output, in tile order: whole 64-token chunks
    const size_t vo = (size_t)B * H * ((T + C - 1) / C) * C * Dv * 4;
    return prep + at + 2 * vo;
}

template <int KD>
hipError_t launch_dp2(const ChunkArgs &args, hipStream_t stream) {
    constexpr int C = 64;
    ChunkArgs a = args;
    const int NT = (a.T + C - 1) / C, nbh = a.B * a.H;
    if (nbh == 0 || NT == 0) return launch_chunk_fwd<false, KD, C, 1>(a, stream);   // hT = h0 only
    char *ws = static_cast<char *>(a.tmat);
    const size_t subws = (chunk_workspace_bytes<false, KD, C, 1>(a.B, a.T, a.H) + 255) & ~(size_t)255;
    a.pfrag = ws + chunk_tmat_bytes<false, KD, C, 1>(a.B, a.T, a.H);
    a.gtab = static_cast<char *>(a.pfrag) + chunk_pfrag_bytes<false, KD, C, 1>(a.B, a.T, a.H);
    char *at = ws + 2 * subws;
    const size_t vo = (size_t)nbh * NT * C * a.Dv * 4;    // v' in tile order (whole chunks)
    float *vprime = reinterpret_cast<float *>(at + chunk_pfrag_bytes<false, KD, C, 1>(a.B, a.T, a.H));
    float *o0 = reinterpret_cast<float *>(reinterpret_cast<char *>(vprime) + vo);
    const int nchunks = 2 * nbh * NT, nwg = (nchunks + 3) / 4;     // both sub-keys
    const int pgrid = nwg < 2 * num_cus() ? nwg : 2 * num_cus();
    const int cgrid = ((nbh + 7) / 8) * 8 * (a.Dv / 16);
    const int ktot = 2 * KD;
    a.kw = KD;
    a.kst = ktot;
    a.bst = 2;
    a.hrows = ktot;
    // pass 1: sub-key 0
    ChunkArgs p1 = a;
    p1.koff = 0;
    p1.boff = 0;
    p1.hoff = 0;
    p1.atil = at;
    p1.vout = vprime;
    p1.o = o0;
    p1.out_bf16 = 0;
    // the prep of both sub-keys in one launch (sub-key 1's work space subws on)
    ChunkArgs pp = p1;
    pp.nsub = 2;
    pp.subws = subws;
    hipLaunchKernelGGL((chunk_prep2_kernel<KD, C>), dim3(pgrid), dim3(256), 0, stream, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_chain1_kernel<KD, C, 1>), dim3(cgrid), dim3(Chain1Shape<KD, C>::NTHR), 0, stream, p1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // pass 2: sub-key 1, values v', output added
    ChunkArgs p2 = a;
    p2.koff = KD;
    p2.boff = 1;
    p2.hoff = KD;
    p2.atil = nullptr;
    p2.vin = vprime;
    p2.oprev = o0;
    p2.tmat = ws + subws;
    p2.pfrag = static_cast<char *>(a.pfrag) + subws;
    p2.gtab = static_cast<char *>(a.gtab) + subws;
    hipLaunchKernelGGL((chunk_chain1_kernel<KD, C, 2>), dim3(cgrid), dim3(Chain1Shape<KD, C>::NTHR), 0, stream, p2);
    return hipGetLastError();
}

struct ChunkImpl {
    hipError_t (*launch)(const ChunkArgs &, hipStream_t);
    size_t (*workspace)(int B, int T, int H, int Dv);
};

// Each returns false when (KD, C) has no instantiation for that input type
// and step count.
bool find_chunk_bf16_r1(int KD, int C, ChunkImpl *out);
bool find_chunk_bf16_r2(int KD, int C, ChunkImpl *out);
bool find_chunk_f32(int KD, int C, int R, ChunkImpl *out);
// the two-pass DeltaProduct path for sub-keys of width dk (bf16)
bool find_dp2(int dk, ChunkImpl *out);

}  // namespace gdn

#define GDN_CASE(F32, KD_, C_, R_)                                   \
    if (KD == KD_ && C == C_) {                                      \
        out->launch = launch_chunk_fwd<F32, KD_, C_, R_>;            \
        out->workspace = chunk_fwd_workspace_bytes<F32, KD_, C_, R_>; \
        return true;                                                 \
    }
