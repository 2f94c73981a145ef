// Status strings, thread-local error messages and the version string.
#include "common.h"

namespace atlas {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

}  // namespace atlas

extern "C" const char* atlas_version(void) { return "atlas-w4 0.1 gfx950"; }

extern "C" const char* atlas_status_string(int s) {
    switch (s) {
        case ATLAS_OK: return "ok";
        case ATLAS_ERR_INVALID_ARG: return "invalid argument";
        case ATLAS_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case ATLAS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case ATLAS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* atlas_last_error(void) { return atlas::g_err; }
