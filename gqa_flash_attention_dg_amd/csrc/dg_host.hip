// dg_host.hip -- host-side helpers of libdgattn.so: the per-thread status message behind
// dg_last_error(), and the device topology the launch plans are sized for.
#include <cstring>
#include <mutex>

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

Topology device_topology() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static Topology cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();   // leave no error for the next launch check to report
        return Topology{256, 8};
    }
    std::lock_guard<std::mutex> lock(mu);
    if (dev < kMaxDevices && cache[dev].cus > 0) return cache[dev];
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
        xcds <= 0 || xcds > cus)
        xcds = cus >= 32 ? cus / 32 : 1;   // gfx950 XCDs hold 32 active CUs each
    (void)hipGetLastError();
    const Topology t{cus, xcds};
    if (dev < kMaxDevices) cache[dev] = t;
    return t;
}

}  // namespace dg

extern "C" const char* dg_last_error(void) { return g_msg; }
