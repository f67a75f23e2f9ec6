// dg_common.hpp -- helpers shared by the entry points and kernels of libdgattn.so: the
// per-thread error message, argument checks, launch-error capture, and the XCD placement of
// workgroups.
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

// Workgroup id -> logical id such that consecutive logical ids share an XCD: the hardware deals
// the workgroups of a launch to the 8 XCDs round robin (workgroup b runs on XCD b % 8), so
// logical id l runs on XCD l / (n / 8).  A grid that is not a multiple of 8 keeps its order.
__device__ inline int xcd_remap(int bid, int n) {
    if ((n & 7) != 0) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

inline int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DG_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace dg
