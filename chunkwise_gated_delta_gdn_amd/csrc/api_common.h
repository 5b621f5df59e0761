// Host-side helpers of the C ABI: thread-local error text, argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "gdn.h"

namespace gdn {

int set_error(int code, const char *fmt, ...);
int check_hip(hipError_t e, const char *what);

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace gdn

#define GDN_REQUIRE(cond, code, ...)                        \
    do {                                                    \
        if (!(cond)) return ::gdn::set_error(code, __VA_ARGS__); \
    } while (0)
