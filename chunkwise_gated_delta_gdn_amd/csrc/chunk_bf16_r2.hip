// bf16-input instantiations of the chunk kernel, two steps per token.
#include "chunk_dispatch.h"

namespace gdn {

hipError_t dispatch_chunk_bf16_r2(int KD, int C, const ChunkArgs &a, hipStream_t s, bool *found) {
    *found = false;
    GDN_CASE(false, 32, 16, 2) GDN_CASE(false, 32, 32, 2)
    GDN_CASE(false, 64, 16, 2) GDN_CASE(false, 64, 32, 2)
    GDN_CASE(false, 128, 16, 2) GDN_CASE(false, 128, 32, 2)
    GDN_CASE(false, 256, 16, 2) GDN_CASE(false, 256, 32, 2)
    return hipErrorInvalidValue;
}

}  // namespace gdn
