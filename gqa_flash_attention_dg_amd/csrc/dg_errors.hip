// dg_errors.hip -- per-thread status message behind dg_last_error().
#include <cstring>

#include "dg_common.hpp"

namespace {
thread_local char g_msg[512] = "";
}

namespace dg {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_msg[0] = '\0';
    return DG_OK;
}

}  // namespace dg

extern "C" const char* dg_last_error(void) { return g_msg; }
