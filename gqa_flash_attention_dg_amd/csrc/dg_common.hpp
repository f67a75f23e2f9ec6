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

// For launches whose logical workgroups alternate a full and a lighter one (l even: full, l
// odd: light; two query blocks per unit), the order within each XCD's contiguous range of
// xcd_remap ids that dispatches that range's full workgroups first: the k-th workgroup to run
// on an XCD takes the k-th even id of the range while there are any, then the odd ones.  A
// bijection of [0, n) that keeps every id on its XCD; grids that xcd_remap leaves unchanged
// (n not a multiple of nxcd) are left unchanged.
__host__ __device__ inline int full_first(int lid, int n, int nxcd) {
    if (nxcd < 1 || n % nxcd != 0) return lid;
    const int m = n / nxcd, j0 = lid % m, base = lid - j0;
    const int f = base & 1, n0 = (m - f + 1) / 2;   // ids base + f, base + f + 2, ... are even
    return base + (j0 < n0 ? f + 2 * j0 : (1 - f) + 2 * (j0 - n0));
}

// Sum of v over each aligned group of N lanes (N = 8 or 16), left in every lane of the group,
// with DPP lane moves within the lanes' own registers: two quad permutes (lane ^ 1, lane ^ 2),
// then the mirror within 8 lanes and, for 16, within 16.  Each step adds a value and its
// partner's in the same order on both sides, so every lane of a group ends with the same sum.
// (A lane shuffle goes through the LDS crossbar and waits out its latency at every step.)
template <int N>
__device__ inline float group_sum(float v) {
    static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (N == 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

inline int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DG_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace dg
