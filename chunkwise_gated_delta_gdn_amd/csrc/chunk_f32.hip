// fp32-input instantiations of the chunk kernels.
#include "chunk_dispatch.h"

namespace gdn {

bool find_chunk_f32(int KD, int C, int R, ChunkImpl *out) {
    if (R == 1) {
        GDN_CASE(true, 16, 16, 1) GDN_CASE(true, 16, 32, 1) GDN_CASE(true, 16, 64, 1)
        GDN_CASE(true, 32, 16, 1) GDN_CASE(true, 32, 32, 1) GDN_CASE(true, 32, 64, 1)
        GDN_CASE(true, 64, 16, 1) GDN_CASE(true, 64, 32, 1) GDN_CASE(true, 64, 64, 1)
        GDN_CASE(true, 128, 16, 1) GDN_CASE(true, 128, 32, 1)
        GDN_CASE(true, 256, 16, 1) GDN_CASE(true, 256, 32, 1)
    } else if (R == 2) {
        GDN_CASE(true, 32, 16, 2) GDN_CASE(true, 32, 32, 2)
        GDN_CASE(true, 64, 16, 2) GDN_CASE(true, 64, 32, 2)
        GDN_CASE(true, 128, 16, 2) GDN_CASE(true, 128, 32, 2)
        GDN_CASE(true, 256, 16, 2) GDN_CASE(true, 256, 32, 2)
    }
    return false;
}

}  // namespace gdn
