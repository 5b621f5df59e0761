// Lookup of the chunk kernel instantiations (one source file per input type
// and step count, so they compile in parallel).
#pragma once

#include "chunk_kernels.h"

namespace gdn {

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
