// dg_common.hpp -- helpers shared by the entry points and kernels of libdgattn.so: the
// per-thread error message, argument checks, launch-error capture, the device topology and the
// XCD placement of workgroups.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/dgattn.h"

namespace dg {

// Records the message returned by dg_last_error() on this thread and returns `status`.
int fail(int status, const char* fmt, ...);
// Clears the message (called on success).
int ok();

// Byte range [lo, hi) of a device buffer, for overlap checks.  An empty range never overlaps.
struct Span {
    uintptr_t lo = 0, hi = 0;
    Span() = default;
    Span(const void* p, size_t bytes)
        : lo(reinterpret_cast<uintptr_t>(p)), hi(reinterpret_cast<uintptr_t>(p) + bytes) {
        if (!p || bytes == 0) lo = hi = 0;
    }
    bool overlaps(const Span& o) const { return lo < hi && o.lo < o.hi && lo < o.hi && o.lo < hi; }
};

// Element count a*b*c*... in size_t, guarding against overflow of the byte count.
inline bool mul_ok(size_t& acc, long long f) {
    if (f < 0) return false;
    if (f != 0 && acc > (SIZE_MAX / 8) / static_cast<size_t>(f)) return false;
    acc *= static_cast<size_t>(f);
    return true;
}

// Compute units and XCDs (accelerator dies, each with its own L2) of the current device, read
// from the runtime once per device and cached.  Without a device to ask (a host with no GPU)
// it returns an MI355X's 256 CUs in 8 XCDs.
struct Topology {
    int cus;
    int xcds;
};
Topology device_topology();

// Workgroup id -> logical id such that consecutive logical ids share an XCD: the hardware deals
// the workgroups of a launch to the device's XCDs round robin (workgroup b runs on XCD
// b % nxcd), so logical id l runs on XCD l / (n / nxcd).  A bijection of [0, n); a grid that
// is not a multiple of nxcd keeps its order.
__host__ __device__ inline int xcd_remap(int bid, int n, int nxcd) {
    if (nxcd <= 1) return bid;
    if ((nxcd & (nxcd - 1)) == 0) {   // a power of two (8, or 4 and 1 on a partitioned MI355X)
        const int sh = __builtin_ctz(nxcd);
        if (n & (nxcd - 1)) return bid;
        return (bid & (nxcd - 1)) * (n >> sh) + (bid >> sh);
    }
    if (n % nxcd != 0) return bid;
    return (bid % nxcd) * (n / nxcd) + bid / nxcd;
}

inline int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DG_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace dg
