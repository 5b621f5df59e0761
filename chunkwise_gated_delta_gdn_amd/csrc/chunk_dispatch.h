// Lookup of the chunk kernel instantiations (one source file per input type
// and step count, so they compile in parallel).
#pragma once

#include <atomic>

#include "chunk_chain1.h"
#include "chunk_kernels.h"
#include "chunk_prep2.h"

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

// Launch both kernels of one instantiation on `stream`.
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
    const int nvb = a.Dv / 16;
    const int grid = ((nbh + 7) / 8) * 8 * nvb;
    if constexpr (use_chain1<F32IN, KD, C, R>()) {
        hipLaunchKernelGGL((chunk_chain1_kernel<KD, C>), dim3(grid), dim3(Chain1Shape<KD, C>::NTHR), 0, stream, a);
    } else {
        hipLaunchKernelGGL((chunk_chain_kernel<F32IN, KD, C, R>), dim3(grid), dim3(512), 0, stream, a);
    }
    return hipGetLastError();
}

struct ChunkImpl {
    hipError_t (*launch)(const ChunkArgs &, hipStream_t);
    size_t (*workspace)(int B, int T, int H);
};

// Each returns false when (KD, C) has no instantiation for that input type
// and step count.
bool find_chunk_bf16_r1(int KD, int C, ChunkImpl *out);
bool find_chunk_bf16_r2(int KD, int C, ChunkImpl *out);
bool find_chunk_f32(int KD, int C, int R, ChunkImpl *out);

}  // namespace gdn

#define GDN_CASE(F32, KD_, C_, R_)                                   \
    if (KD == KD_ && C == C_) {                                      \
        out->launch = launch_chunk_fwd<F32, KD_, C_, R_>;            \
        out->workspace = chunk_workspace_bytes<F32, KD_, C_, R_>;    \
        return true;                                                 \
    }
