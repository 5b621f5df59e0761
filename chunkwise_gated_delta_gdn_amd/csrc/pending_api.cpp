// Placeholder entry points for the camera-branch operations until their
// kernels land: they validate nothing and report GDN_EUNSUPPORTED.
#include "api_common.h"

extern "C" int gdn_recurrent_fwd(const void *, const void *, const void *, const float *, const float *, float,
                                 const float *, float *, float *, int, int, int, int, int, int, void *, size_t,
                                 void *) {
    return gdn::set_error(GDN_EUNSUPPORTED, "gdn_recurrent_fwd: not available in this build");
}
extern "C" size_t gdn_recurrent_fwd_workspace_bytes(int, int, int, int, int, int) { return 0; }
extern "C" int gdn_prep(const void *, const float *, const float *, const float *, const float *, const float *,
                        const float *, float, float, void *, void *, void *, float *, float *, float *, int, int,
                        int, int, int, void *) {
    return gdn::set_error(GDN_EUNSUPPORTED, "gdn_prep: not available in this build");
}
