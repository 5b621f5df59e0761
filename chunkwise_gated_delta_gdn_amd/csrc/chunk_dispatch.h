// Dispatch of the chunk kernel instantiations (one source file per input
// type and step count, so they compile in parallel).
#pragma once

#include "chunk_fwd_kernel.h"

namespace gdn {

// Each returns hipErrorInvalidValue with *found = false when (KD, C) has no
// instantiation for that input type and step count.
hipError_t dispatch_chunk_bf16_r1(int KD, int C, const ChunkArgs &a, hipStream_t s, bool *found);
hipError_t dispatch_chunk_bf16_r2(int KD, int C, const ChunkArgs &a, hipStream_t s, bool *found);
hipError_t dispatch_chunk_f32(int KD, int C, int R, const ChunkArgs &a, hipStream_t s, bool *found);

}  // namespace gdn

#define GDN_CASE(F32, KD_, C_, R_)                                   \
    if (KD == KD_ && C == C_) {                                      \
        *found = true;                                               \
        return launch_chunk_fwd<F32, KD_, C_, R_>(a, s);             \
    }
