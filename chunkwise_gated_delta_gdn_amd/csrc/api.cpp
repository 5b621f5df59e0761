// C ABI entry points shared across operations: error reporting and version.
#include "api_common.h"

#include <string.h>

namespace gdn {

static thread_local char g_err[512] = "";

int set_error(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int check_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return GDN_OK;
    return set_error(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace gdn

extern "C" const char *gdn_last_error(void) { return gdn::g_err; }

extern "C" int gdn_abi_version(void) { return 5; }
