// attn_status.cpp -- status codes and the per-thread error text shared by
// every entry point of the library.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "attn_internal.h"

namespace attn {

namespace {
thread_local char g_err[512];
}

attn_status_t fail(attn_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

attn_status_t hip_check(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
    return ok();
}

}  // namespace attn

extern "C" {

const char *attn_status_string(attn_status_t status) {
    // A C caller may pass any int.  In C++ an enum value outside its
    // enumerators' range may not be read as the enum, so read its bytes as
    // an int instead.
    int code;
    static_assert(sizeof code == sizeof status, "attn_status_t is int-sized");
    memcpy(&code, &status, sizeof code);
    switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_DIM: return "invalid size";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *attn_last_error(void) {
    return attn::g_err;
}

}  // extern "C"
