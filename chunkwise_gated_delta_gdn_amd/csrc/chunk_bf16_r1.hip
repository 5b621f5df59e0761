// bf16-input instantiations of the chunk kernels, one step per token.
#include "chunk_dispatch.h"

namespace gdn {

bool find_chunk_bf16_r1(int KD, int C, ChunkImpl *out) {
    GDN_CASE(false, 16, 16, 1) GDN_CASE(false, 16, 32, 1) GDN_CASE(false, 16, 64, 1)
    GDN_CASE(false, 32, 16, 1) GDN_CASE(false, 32, 32, 1) GDN_CASE(false, 32, 64, 1)
    GDN_CASE(false, 64, 16, 1) GDN_CASE(false, 64, 32, 1) GDN_CASE(false, 64, 64, 1)
    GDN_CASE(false, 128, 16, 1) GDN_CASE(false, 128, 32, 1) GDN_CASE(false, 128, 64, 1)
    GDN_CASE(false, 256, 16, 1) GDN_CASE(false, 256, 32, 1)
    return false;
}

}  // namespace gdn
