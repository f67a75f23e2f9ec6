// rope_headnorm.hip -- dg_rope_table and dg_headnorm_rope for gfx950.
//
// Follows inferencelayer 0.2.3, src/diffusion_gemma_gpu.rs: kernel DG_HEADNORM_ROPE (per
// (token, head) RMSNorm, optional weight, optional NeoX rotate-half rope, in place on
// [T, heads*hd], cos|sin table [T, 2*hd]) and the per-token rope table that `canvas_forward`
// builds for positions seq_len + t.
//
// Both are HBM-bound.  The page runs one 128-thread workgroup per (token, head) with shared
// memory trees; here one 64-lane wavefront owns one (token, head) row: lane l holds elements
// l and l+64, so every global access is one coalesced 256-byte wave load/store, the sum of
// squares is a wave butterfly (no LDS, no barrier), and the rotate-half partner is either in
// the same lane (hd = 128) or one lane shuffle away.
#include "dg_common.hpp"

namespace {

constexpr int kRowsPerBlock = 4;  // four wavefronts, one (token, head) row each

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__global__ void __launch_bounds__(256) rope_table_kernel(float* __restrict__ cs, int pos0, int T,
                                                         int hd, double theta) {
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)T * hd) return;
    const int t = (int)(idx / hd);
    const int c = (int)(idx % hd);
    const int i = c % (hd / 2);
    const double freq = pow(theta, -2.0 * (double)i / (double)hd);
    const double ang = ((double)pos0 + (double)t) * freq;
    double s, co;
    sincos(ang, &s, &co);
    cs[(size_t)t * 2 * hd + c] = (float)co;
    cs[(size_t)t * 2 * hd + hd + c] = (float)s;
}

__global__ void __launch_bounds__(256) headnorm_rope_kernel(float* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ cs,
                                                            long long units, int T, int heads,
                                                            int hd, unsigned flags, float eps) {
    const int lane = threadIdx.x & 63;
    const long long u = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (u >= units) return;  // wave-uniform
    const int t = (int)((u / heads) % T);
    float* xr = x + (size_t)u * hd;
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = e0 < hd, v1 = e1 < hd;
    float y0 = v0 ? xr[e0] : 0.0f;
    float y1 = v1 ? xr[e1] : 0.0f;
    if (!(flags & DG_NORM_SKIP)) {
        const float ss = wave_sum(y0 * y0 + y1 * y1);
        const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
        y0 *= inv;
        y1 *= inv;
        if (flags & DG_NORM_WEIGHTED) {
            if (v0) y0 *= w[e0];
            if (v1) y1 *= w[e1];
        }
    }
    if (flags & DG_NORM_ROPE) {
        const int half = hd >> 1;
        // partner of element e is e + half (e < half, enters negated) or e - half
        const int p0 = e0 < half ? e0 + half : e0 - half;
        const int p1 = e1 < half ? e1 + half : e1 - half;
        float q0, q1;
        if (hd == 128) {  // partners share the lane: e0 <-> e1
            q0 = y1;
            q1 = y0;
        } else {
            const int s0 = v0 ? (p0 & 63) : lane, s1 = v1 ? (p1 & 63) : lane;
            const float a0 = __shfl(y0, s0), b0 = __shfl(y1, s0);
            const float a1 = __shfl(y0, s1), b1 = __shfl(y1, s1);
            q0 = p0 >= 64 ? b0 : a0;
            q1 = p1 >= 64 ? b1 : a1;
        }
        const float* cr = cs + (size_t)t * 2 * hd;
        if (v0) {
            const float rot = e0 < half ? -q0 : q0;
            xr[e0] = y0 * cr[e0] + rot * cr[hd + e0];
        }
        if (v1) {
            const float rot = e1 < half ? -q1 : q1;
            xr[e1] = y1 * cr[e1] + rot * cr[hd + e1];
        }
    } else {
        if (v0) xr[e0] = y0;
        if (v1) xr[e1] = y1;
    }
}

}  // namespace

extern "C" int dg_rope_table(float* cs, int pos0, int T, int hd, double theta, void* stream) {
    if (pos0 < 0 || T < 0) return dg::fail(DG_EINVAL, "dg_rope_table: negative pos0 (%d) or T (%d)", pos0, T);
    if (hd < 2 || hd > 1024 || (hd & 1))
        return dg::fail(DG_EINVAL, "dg_rope_table: hd must be even and in [2, 1024], got %d", hd);
    if (!(theta > 0.0) || !std::isfinite(theta))
        return dg::fail(DG_EINVAL, "dg_rope_table: theta must be finite and > 0");
    if (T == 0) return dg::ok();
    if (!cs) return dg::fail(DG_EINVAL, "dg_rope_table: cs is NULL");
    const long long n = (long long)T * hd;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, cs, pos0,
                       T, hd, theta);
    return dg::launch_status("dg_rope_table");
}

extern "C" int dg_headnorm_rope(float* x, const float* w, const float* cs, int batch, int T,
                                int heads, int hd, unsigned flags, float eps, void* stream) {
    if (batch < 0 || T < 0 || heads < 0)
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: negative size (batch %d, T %d, heads %d)", batch, T, heads);
    if (hd < 1) return dg::fail(DG_EINVAL, "dg_headnorm_rope: hd must be >= 1, got %d", hd);
    if (hd > 128) return dg::fail(DG_EUNSUPPORTED, "dg_headnorm_rope: hd %d > 128 is not supported", hd);
    if (flags & ~(DG_NORM_WEIGHTED | DG_NORM_ROPE | DG_NORM_SKIP))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: unknown flag bits 0x%x", flags);
    if ((flags & DG_NORM_ROPE) && (hd & 1))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: rope needs an even hd, got %d", hd);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: eps must be finite and >= 0");
    size_t n = 1;
    if (!dg::mul_ok(n, batch) || !dg::mul_ok(n, T) || !dg::mul_ok(n, heads) || !dg::mul_ok(n, hd))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: size overflow");
    if (n == 0) return dg::ok();
    const bool need_w = (flags & DG_NORM_WEIGHTED) && !(flags & DG_NORM_SKIP);
    const bool need_cs = (flags & DG_NORM_ROPE) != 0;
    if (!x) return dg::fail(DG_EINVAL, "dg_headnorm_rope: x is NULL");
    if (need_w && !w) return dg::fail(DG_EINVAL, "dg_headnorm_rope: WEIGHTED set but w is NULL");
    if (need_cs && !cs) return dg::fail(DG_EINVAL, "dg_headnorm_rope: ROPE set but cs is NULL");
    const dg::Span xs(x, n * sizeof(float));
    if (need_w && xs.overlaps(dg::Span(w, (size_t)hd * sizeof(float))))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: w overlaps x");
    if (need_cs && xs.overlaps(dg::Span(cs, (size_t)T * 2 * hd * sizeof(float))))
        return dg::fail(DG_EINVAL, "dg_headnorm_rope: cs overlaps x");
    const long long units = (long long)batch * T * heads;
    const long long blocks = (units + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "dg_headnorm_rope: too many rows");
    hipLaunchKernelGGL(headnorm_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       x, need_w ? w : nullptr, need_cs ? cs : nullptr, units, T, heads, hd, flags, eps);
    return dg::launch_status("dg_headnorm_rope");
}
