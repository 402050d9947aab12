// Host-side error reporting shared by every entry point.
#include "common.h"

namespace shattn {

std::string& last_error() {
    static thread_local std::string msg;
    return msg;
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    last_error() = buf;
    return code;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SHATTN_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return SHATTN_OK;
}

}  // namespace shattn

extern "C" const char* shattn_last_error(void) { return shattn::last_error().c_str(); }
