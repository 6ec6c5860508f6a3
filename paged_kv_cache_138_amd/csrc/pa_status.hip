// Status strings and the thread-local error detail of libpa.
#include "pa_host.h"

#include <string.h>

namespace pa {

static thread_local char g_last_error[512];

pa_status fail(pa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_last_error[0] = '\0'; }

pa_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    }
    return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "null pointer";
        case PA_ERR_SHAPE: return "invalid shape";
        case PA_ERR_DTYPE: return "invalid element type";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_WORKSPACE: return "invalid workspace";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_ALIGNMENT: return "misaligned pointer";
    }
    return "unknown status";
}

extern "C" const char* pa_last_error(void) { return pa::g_last_error; }

extern "C" const char* pa_version(void) { return "0.1.0"; }
