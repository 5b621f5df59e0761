// bf16-input instantiations of the chunk kernels, two steps per token.
#include "chunk_dispatch.h"

namespace gdn {

bool find_chunk_bf16_r2(int KD, int C, ChunkImpl *out) {
    GDN_CASE(false, 32, 16, 2) GDN_CASE(false, 32, 32, 2)
    GDN_CASE(false, 64, 16, 2) GDN_CASE(false, 64, 32, 2)
    GDN_CASE(false, 128, 16, 2) GDN_CASE(false, 128, 32, 2)
    GDN_CASE(false, 256, 16, 2) GDN_CASE(false, 256, 32, 2)
    return false;
}

bool find_dp2(int dk, ChunkImpl *out) {
    switch (dk) {
        case 32: out->launch = launch_dp2<32>; out->workspace = dp2_workspace_bytes<32>; return true;
        case 64: out->launch = launch_dp2<64>; out->workspace = dp2_workspace_bytes<64>; return true;
        case 128: out->launch = launch_dp2<128>; out->workspace = dp2_workspace_bytes<128>; return true;
        default: return false;
    }
}

}  // namespace gdn
