// rope_headnorm.hip -- dg_rope_table and dg_headnorm_rope for gfx950.
//
// Follows inferencelayer 0.2.3, src/diffusion_gemma_gpu.rs: kernel DG_HEADNORM_ROPE (per
// (token, head) RMSNorm, optional weight, optional NeoX rotate-half rope, in place on
// [T, heads*hd], cos|sin table [T, 2*hd]) and the per-token rope table that `canvas_forward`
// builds for positions seq_len + t.
//
// Both are HBM-bound.  The page runs one 128-thread workgroup per (token, head) with shared
// memory trees, and dispatches q, k and v separately.  Here, for hd 64 and 128, hd/8 lanes own
// one (token, head) row, each with two 16-byte chunks hd/2 apart, so a wavefront streams 4 or 8
// rows with 16-byte accesses, the rope partner of every element is in the same lane, and the
// sum of squares is a DPP sum within the row's lanes (no LDS, no barrier).  Other head dims take
// one 64-lane wavefront per row (lane l holds elements l and l+64; the rope partner is one lane
// shuffle away).  One launch can cover the rows of q, k and v together
// (dg_qkv_headnorm_rope): at canvas sizes the three calls are launch-bound.
#include "kv16.hpp"

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

// One tensor of a headnorm launch: rows of hd floats, `heads` rows per token, normed in place
// with its own weight and flags.  A launch covers up to three of them (q, k, v of a step).
struct NormSeg {
    float* x;
    const float* w;
    long long rows;   // batch * T * heads
    int heads;
    unsigned flags;
    float* vout;      // k_eq_v: also write the weightless norm of the raw rows here, or NULL
    uint16_t* x16;    // 16-bit twin of the output rows (format NormArgs::fmt16), or NULL
    uint16_t* vout16; // 16-bit twin of vout, or NULL
};

struct NormArgs {
    NormSeg seg[3];
    int nseg;
    const float* cs;  // [T, 2*hd], shared by every segment that ropes
    int T, hd;
    float eps;
    int fmt16;        // DG_KV_F16 or DG_KV_BF16 when a segment has twins
    int kvmajor;      // exactly k and v of one shape: rows taken in (b*heads + h, k|v, t) order
    int nxcd;         // XCDs of the device (kvmajor workgroup placement)
    int kvgroup;      // 16-byte kernel, kvmajor: (b, head) pairs per XCD, rows taken in
                      // (group, k|v, t, pair) order; 0: the (b*heads + h, k|v, t) order
};

// kHD: the head dim when it is 128 or 64 (no per-lane guards), 0 for any other hd <= 128.  Lanes
// past hd read an element that exists (element 0 of the row) and discard it by selection, so
// the loads are not turned into divergent branches.  The row, its weights and its cos|sin
// entries are all loaded before any arithmetic: the wavefront waits for memory once.
template <int kHD>
__device__ inline void headnorm_row(float* __restrict__ xr, const float* __restrict__ w,
                                    const float* __restrict__ cr, int hd_rt, unsigned flags,
                                    float eps, int lane, float* __restrict__ vr,
                                    uint16_t* __restrict__ xr16, uint16_t* __restrict__ vr16,
                                    int fmt16) {
    const int hd = kHD ? kHD : hd_rt;
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = kHD ? true : e0 < hd;
    const bool v1 = kHD == 128 ? true : (kHD == 64 ? false : e1 < hd);
    const int i0 = v0 ? e0 : 0, i1 = v1 ? e1 : 0;
    const bool norm = !(flags & DG_NORM_SKIP);
    const bool weighted = norm && (flags & DG_NORM_WEIGHTED);
    const bool rope = (flags & DG_NORM_ROPE) != 0;
    const float x0 = xr[i0];
    const float x1 = kHD == 64 ? 0.0f : xr[i1];
    const float w0 = weighted ? w[i0] : 1.0f;
    const float w1 = weighted && kHD != 64 ? w[i1] : 1.0f;
    const float c0 = rope ? cr[i0] : 0.0f, s0v = rope ? cr[hd + i0] : 0.0f;
    const float c1 = rope && kHD != 64 ? cr[i1] : 0.0f;
    const float s1v = rope && kHD != 64 ? cr[hd + i1] : 0.0f;
    float y0 = v0 ? x0 : 0.0f;
    float y1 = v1 ? x1 : 0.0f;
    if (norm) {
        const float ss = wave_sum(y0 * y0 + y1 * y1);
        const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
        y0 *= inv;
        y1 *= inv;
        if (vr) {  // the v-norm of the same raw rows: weightless, un-roped
            if (v0) vr[e0] = y0;
            if (v1) vr[e1] = y1;
            if (vr16) {
                if (v0) vr16[e0] = dg::to_kv16(y0, fmt16);
                if (v1) vr16[e1] = dg::to_kv16(y1, fmt16);
            }
        }
        if (weighted) {
            y0 *= w0;
            y1 *= w1;
        }
    }
    if (rope) {
        const int half = hd >> 1;
        // partner of element e is e + half (e < half, enters negated) or e - half
        const int p0 = e0 < half ? e0 + half : e0 - half;
        const int p1 = e1 < half ? e1 + half : e1 - half;
        float q0, q1;
        if (kHD == 128) {  // partners share the lane: e0 <-> e1
            q0 = y1;
            q1 = y0;
        } else if (kHD == 64) {
            q0 = __shfl_xor(y0, 32);
            q1 = 0.0f;
        } else {
            const int s0 = v0 ? (p0 & 63) : lane, s1 = v1 ? (p1 & 63) : lane;
            const float a0 = __shfl(y0, s0), b0 = __shfl(y1, s0);
            const float a1 = __shfl(y0, s1), b1 = __shfl(y1, s1);
            q0 = p0 >= 64 ? b0 : a0;
            q1 = p1 >= 64 ? b1 : a1;
        }
        const float rot0 = e0 < half ? -q0 : q0;
        const float rot1 = e1 < half ? -q1 : q1;
        y0 = y0 * c0 + rot0 * s0v;
        y1 = y1 * c1 + rot1 * s1v;
    }
    if (v0) xr[e0] = y0;
    if (v1) xr[e1] = y1;
    if (xr16) {  // the 16-bit twin, rounded as dg_pack_kv16 rounds
        if (v0) xr16[e0] = dg::to_kv16(y0, fmt16);
        if (v1) xr16[e1] = dg::to_kv16(y1, fmt16);
    }
}

// Rows of all segments are numbered consecutively (segment 0 first); each wavefront takes one.
// With kvmajor (the k and v of a canvas step) rows go in (batch * heads + head, k|v, token)
// order instead, with workgroups placed by xcd_remap: the attention kernel reads the canvas
// rows of each (batch, kv head) on one XCD, and the norm then rewrites them on that XCD too
// (writing lines that another XCD has just read is the slow case).
template <int kHD>
__global__ void __launch_bounds__(256) headnorm_rope_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    long long u;
    // The segment is found with constant indices into the arguments, so its fields come from
    // scalar loads (a computed index would read them through per-lane memory loads).
    NormSeg g = a.seg[0];
    if (a.kvmajor) {
        const long long r =
            (long long)dg::xcd_remap(blockIdx.x, gridDim.x, a.nxcd) * kRowsPerBlock + (threadIdx.x >> 6);
        if (r >= 2 * g.rows) return;
        const long long bh = r / (2 * a.T);
        const int rem = (int)(r % (2 * a.T));
        const int t = rem % a.T;
        if (rem >= a.T) g = a.seg[1];
        u = ((bh / g.heads) * a.T + t) * g.heads + bh % g.heads;
    } else {
        u = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    }
    if (!a.kvmajor && u >= g.rows) {
        u -= g.rows;
        if (a.nseg < 2) return;
        g = a.seg[1];
        if (u >= g.rows) {
            u -= g.rows;
            if (a.nseg < 3 || u >= a.seg[2].rows) return;
            g = a.seg[2];
        }
    }
    const int t = (int)((u / g.heads) % a.T);
    const float* cr = (g.flags & DG_NORM_ROPE) ? a.cs + (size_t)t * 2 * a.hd : nullptr;
    headnorm_row<kHD>(g.x + (size_t)u * a.hd, g.w, cr, a.hd, g.flags, a.eps, lane,
                      g.vout ? g.vout + (size_t)u * a.hd : nullptr,
                      g.x16 ? g.x16 + (size_t)u * a.hd : nullptr,
                      g.vout16 ? g.vout16 + (size_t)u * a.hd : nullptr, a.fmt16);
}

// hd 64 and 128: 16-byte accesses.  A row is taken by L lanes, lane c holding chunks c, c + L,
// ... (4 floats each); chunks hd/2 apart share a lane, so the rope partner of each element is
// in the same lane, and a 64-lane wavefront takes 64/L rows at once.  The sum of squares is a DPP sum over
// the row's L lanes.  Row numbering and placement as in headnorm_rope_kernel.
template <int HD>
struct V4 {
    static constexpr int L = HD / 8;              // lanes per row
    static constexpr int kRowsPerWave = 64 / L;
    static constexpr int kRowsPerBlock = 4 * kRowsPerWave;
};

__device__ inline uint2 pack4_kv16(float4 v, int fmt) {
    return make_uint2((uint32_t)dg::to_kv16(v.x, fmt) | ((uint32_t)dg::to_kv16(v.y, fmt) << 16),
                      (uint32_t)dg::to_kv16(v.z, fmt) | ((uint32_t)dg::to_kv16(v.w, fmt) << 16));
}

__device__ inline float4 scale4(float4 v, float s) { return make_float4(v.x * s, v.y * s, v.z * s, v.w * s); }
__device__ inline float4 mul4(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }

template <int HD>
__device__ inline void headnorm_row_v4(float* __restrict__ xr, const float* __restrict__ w,
                                       const float* __restrict__ cr, unsigned flags, float eps,
                                       int c, float* __restrict__ vr, uint16_t* __restrict__ xr16,
                                       uint16_t* __restrict__ vr16, int fmt16) {
    constexpr int L = V4<HD>::L;
    constexpr int K = HD / (4 * L);   // chunks per lane: c + L*k; chunk k pairs with k + K/2
    const bool norm = !(flags & DG_NORM_SKIP);
    const bool weighted = norm && (flags & DG_NORM_WEIGHTED);
    const bool rope = (flags & DG_NORM_ROPE) != 0;
    const float4 one = make_float4(1.f, 1.f, 1.f, 1.f), zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 x[K], wv[K], co[K], si[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int ch = c + L * k;
        x[k] = reinterpret_cast<const float4*>(xr)[ch];
        wv[k] = weighted ? reinterpret_cast<const float4*>(w)[ch] : one;
        co[k] = rope ? reinterpret_cast<const float4*>(cr)[ch] : zero;
        si[k] = rope ? reinterpret_cast<const float4*>(cr + HD)[ch] : zero;
    }
    if (norm) {
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) ss += x[k].x * x[k].x + x[k].y * x[k].y + x[k].z * x[k].z + x[k].w * x[k].w;
        ss = dg::group_sum<L>(ss);
        const float inv = 1.0f / sqrtf(ss / (float)HD + eps);
#pragma unroll
        for (int k = 0; k < K; ++k) x[k] = scale4(x[k], inv);
        if (vr) {  // the v-norm of the same raw rows: weightless, un-roped
#pragma unroll
            for (int k = 0; k < K; ++k) {
                reinterpret_cast<float4*>(vr)[c + L * k] = x[k];
                if (vr16) reinterpret_cast<uint2*>(vr16)[c + L * k] = pack4_kv16(x[k], fmt16);
            }
        }
        if (weighted) {
#pragma unroll
            for (int k = 0; k < K; ++k) x[k] = mul4(x[k], wv[k]);
        }
    }
    if (rope) {   // chunk k of the first half pairs with chunk k + K/2 of the second
#pragma unroll
        for (int k = 0; k < K / 2; ++k) {
            const float4 y0 = x[k], y1 = x[k + K / 2];
            const float4 c0 = co[k], s0 = si[k], c1 = co[k + K / 2], s1 = si[k + K / 2];
            x[k] = make_float4(y0.x * c0.x - y1.x * s0.x, y0.y * c0.y - y1.y * s0.y,
                               y0.z * c0.z - y1.z * s0.z, y0.w * c0.w - y1.w * s0.w);
            x[k + K / 2] = make_float4(y1.x * c1.x + y0.x * s1.x, y1.y * c1.y + y0.y * s1.y,
                                       y1.z * c1.z + y0.z * s1.z, y1.w * c1.w + y0.w * s1.w);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        reinterpret_cast<float4*>(xr)[c + L * k] = x[k];
        if (xr16)   // the 16-bit twin, rounded as dg_pack_kv16 rounds
            reinterpret_cast<uint2*>(xr16)[c + L * k] = pack4_kv16(x[k], fmt16);
    }
}

template <int HD>
__global__ void __launch_bounds__(256) headnorm_rope_v4_kernel(NormArgs a) {
    using S = V4<HD>;
    const int lane = threadIdx.x & 63, sub = lane / S::L, c = lane % S::L;
    const long long r0 = (long long)(a.kvmajor ? dg::xcd_remap(blockIdx.x, gridDim.x, a.nxcd)
                                               : (int)blockIdx.x) * S::kRowsPerBlock +
                         (threadIdx.x >> 6) * S::kRowsPerWave + sub;
    long long u;
    NormSeg g = a.seg[0];   // constant indices: the segment's fields come from scalar loads
    if (a.kvmajor) {
        if (r0 >= 2 * g.rows) return;                  // the whole row group of L lanes
        if (a.kvgroup > 0) {
            // The (b, head) pairs of one XCD (as the attention places them) go token by token,
            // the pairs of a token next to each other: adjacent heads are adjacent rows in
            // memory, so a wavefront's rows are contiguous runs instead of rows 4 KiB apart.
            const long long per = 2LL * a.T * a.kvgroup;
            const long long grp = r0 / per, rem = r0 % per;
            const long long half = (long long)a.T * a.kvgroup;
            if (rem >= half) g = a.seg[1];
            const long long r2 = rem % half;
            const int t = (int)(r2 / a.kvgroup);
            const long long bh = grp * a.kvgroup + r2 % a.kvgroup;
            u = ((bh / g.heads) * a.T + t) * g.heads + bh % g.heads;
        } else {
            const long long bh = r0 / (2 * a.T);
            const int rem = (int)(r0 % (2 * a.T));
            const int t = rem % a.T;
            if (rem >= a.T) g = a.seg[1];
            u = ((bh / g.heads) * a.T + t) * g.heads + bh % g.heads;
        }
    } else {
        u = r0;
        if (u >= g.rows) {
            u -= g.rows;
            if (a.nseg < 2) return;
            g = a.seg[1];
            if (u >= g.rows) {
                u -= g.rows;
                if (a.nseg < 3 || u >= a.seg[2].rows) return;
                g = a.seg[2];
            }
        }
    }
    const int t = (int)((u / g.heads) % a.T);
    const float* cr = (g.flags & DG_NORM_ROPE) ? a.cs + (size_t)t * 2 * HD : nullptr;
    headnorm_row_v4<HD>(g.x + (size_t)u * HD, g.w, cr, g.flags, a.eps, c,
                        g.vout ? g.vout + (size_t)u * HD : nullptr,
                        g.x16 ? g.x16 + (size_t)u * HD : nullptr,
                        g.vout16 ? g.vout16 + (size_t)u * HD : nullptr, a.fmt16);
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

namespace {

// Checks shared by both headnorm entry points (sizes, flags, eps).
int check_norm_common(const char* fn, int batch, int T, int hd, unsigned flags, float eps) {
    if (batch < 0 || T < 0) return dg::fail(DG_EINVAL, "%s: negative size (batch %d, T %d)", fn, batch, T);
    if (hd < 1) return dg::fail(DG_EINVAL, "%s: hd must be >= 1, got %d", fn, hd);
    if (hd > 128) return dg::fail(DG_EUNSUPPORTED, "%s: hd %d > 128 is not supported", fn, hd);
    if (flags & ~(DG_NORM_WEIGHTED | DG_NORM_ROPE | DG_NORM_SKIP))
        return dg::fail(DG_EINVAL, "%s: unknown flag bits 0x%x", fn, flags);
    if ((flags & DG_NORM_ROPE) && (hd & 1))
        return dg::fail(DG_EINVAL, "%s: rope needs an even hd, got %d", fn, hd);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return dg::fail(DG_EINVAL, "%s: eps must be finite and >= 0", fn);
    return DG_OK;
}

int launch_norm(const char* fn, NormArgs& a, void* stream) {
    long long rows = 0;
    for (int i = 0; i < a.nseg; ++i) rows += a.seg[i].rows;
    if (rows == 0) return dg::ok();
    a.nxcd = dg::device_topology().xcds;
    // hd 64 and 128 take the 16-byte kernel when every tensor is 16-byte aligned
    bool v4 = a.hd == 128 || a.hd == 64;
    uintptr_t al = reinterpret_cast<uintptr_t>(a.cs);
    for (int i = 0; i < a.nseg; ++i)
        al |= reinterpret_cast<uintptr_t>(a.seg[i].x) | reinterpret_cast<uintptr_t>(a.seg[i].w) |
              reinterpret_cast<uintptr_t>(a.seg[i].vout) | reinterpret_cast<uintptr_t>(a.seg[i].x16) |
              reinterpret_cast<uintptr_t>(a.seg[i].vout16);
    if (al & 15) v4 = false;
    const int per = !v4 ? kRowsPerBlock : a.hd == 128 ? V4<128>::kRowsPerBlock : V4<64>::kRowsPerBlock;
    const long long blocks = (rows + per - 1) / per;
    a.kvgroup = 0;
    if (v4 && a.kvmajor) {   // whole XCDs of whole workgroups: the grouped order applies
        const long long pairs = a.seg[0].rows / a.T;     // (b, head) pairs
        const long long nx = a.nxcd;
        if (pairs % nx == 0 && (2LL * a.T * (pairs / nx)) % per == 0)
            a.kvgroup = (int)(pairs / nx);
    }
    if (blocks > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many rows", fn);
    auto* kern = v4 ? (a.hd == 128 ? headnorm_rope_v4_kernel<128> : headnorm_rope_v4_kernel<64>)
                    : a.hd == 128 ? headnorm_rope_kernel<128>
                                  : (a.hd == 64 ? headnorm_rope_kernel<64> : headnorm_rope_kernel<0>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
    return dg::launch_status(fn);
}

}  // namespace

extern "C" int dg_headnorm_rope(float* x, const float* w, const float* cs, int batch, int T,
                                int heads, int hd, unsigned flags, float eps, void* stream) {
    const char* fn = "dg_headnorm_rope";
    if (heads < 0) return dg::fail(DG_EINVAL, "%s: negative size (heads %d)", fn, heads);
    if (int st = check_norm_common(fn, batch, T, hd, flags, eps)) return st;
    size_t n = 1;
    if (!dg::mul_ok(n, batch) || !dg::mul_ok(n, T) || !dg::mul_ok(n, heads) || !dg::mul_ok(n, hd))
        return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    if (n == 0) return dg::ok();
    const bool need_w = (flags & DG_NORM_WEIGHTED) && !(flags & DG_NORM_SKIP);
    const bool need_cs = (flags & DG_NORM_ROPE) != 0;
    if (!x) return dg::fail(DG_EINVAL, "%s: x is NULL", fn);
    if (need_w && !w) return dg::fail(DG_EINVAL, "%s: WEIGHTED set but w is NULL", fn);
    if (need_cs && !cs) return dg::fail(DG_EINVAL, "%s: ROPE set but cs is NULL", fn);
    const dg::Span xs(x, n * sizeof(float));
    if (need_w && xs.overlaps(dg::Span(w, (size_t)hd * sizeof(float))))
        return dg::fail(DG_EINVAL, "%s: w overlaps x", fn);
    if (need_cs && xs.overlaps(dg::Span(cs, (size_t)T * 2 * hd * sizeof(float))))
        return dg::fail(DG_EINVAL, "%s: cs overlaps x", fn);
    NormArgs a{};
    a.seg[0] = NormSeg{x, need_w ? w : nullptr, (long long)batch * T * heads, heads, flags, nullptr};
    a.nseg = 1;
    a.cs = need_cs ? cs : nullptr;
    a.T = T;
    a.hd = hd;
    a.eps = eps;
    return launch_norm(fn, a, stream);
}

namespace {

// Shared body of dg_qkv_headnorm_rope and dg_qkv_headnorm_rope_kv16 (k16/v16 NULL and fmt16 0
// for the former).
int qkv_norm_call(const char* fn, float* q, const float* wq, float* k, const float* wk, float* v,
                  const float* cs, void* k16, void* v16, int fmt16, int batch, int T, int nh,
                  int nkv, int hd, unsigned flags, float eps, void* stream) {
    if (nh < 0 || nkv < 0) return dg::fail(DG_EINVAL, "%s: negative size (nh %d, nkv %d)", fn, nh, nkv);
    const bool v_from_k = (flags & DG_NORM_V_FROM_K) != 0;
    flags &= ~DG_NORM_V_FROM_K;
    if (int st = check_norm_common(fn, batch, T, hd, flags, eps)) return st;
    if (v_from_k && (flags & DG_NORM_SKIP))
        return dg::fail(DG_EINVAL, "%s: V_FROM_K needs the norm (SKIP is set)", fn);
    size_t nq = 1, nk = 1;
    if (!dg::mul_ok(nq, batch) || !dg::mul_ok(nq, T) || !dg::mul_ok(nq, nh) || !dg::mul_ok(nq, hd) ||
        !dg::mul_ok(nk, batch) || !dg::mul_ok(nk, T) || !dg::mul_ok(nk, nkv) || !dg::mul_ok(nk, hd))
        return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    if (v_from_k && nk > 0 && (!k || !v))
        return dg::fail(DG_EINVAL, "%s: V_FROM_K needs both k and v", fn);
    const bool need_w = (flags & DG_NORM_WEIGHTED) && !(flags & DG_NORM_SKIP);
    const bool need_cs = (flags & DG_NORM_ROPE) != 0;
    const bool do_q = q && nq > 0, do_k = k && nk > 0, do_v = v && nk > 0;
    if (fmt16 && ((do_k && !k16) || (do_v && !v16)))
        return dg::fail(DG_EINVAL, "%s: k16 and v16 are needed for the given k and v", fn);
    if (!do_q && !do_k && !do_v) return dg::ok();
    if (need_w && ((do_q && !wq) || (do_k && !wk)))
        return dg::fail(DG_EINVAL, "%s: WEIGHTED set but wq or wk is NULL", fn);
    if (need_cs && (do_q || do_k) && !cs)
        return dg::fail(DG_EINVAL, "%s: ROPE set but cs is NULL", fn);
    const dg::Span xs[5] = {dg::Span(do_q ? q : nullptr, nq * 4), dg::Span(do_k ? k : nullptr, nk * 4),
                            dg::Span(do_v ? v : nullptr, nk * 4),
                            dg::Span(fmt16 && do_k ? k16 : nullptr, nk * 2),
                            dg::Span(fmt16 && do_v ? v16 : nullptr, nk * 2)};
    const dg::Span ro[3] = {dg::Span(need_w && do_q ? wq : nullptr, (size_t)hd * 4),
                            dg::Span(need_w && do_k ? wk : nullptr, (size_t)hd * 4),
                            dg::Span(need_cs && (do_q || do_k) ? cs : nullptr, (size_t)T * 2 * hd * 4)};
    for (int i = 0; i < 5; ++i) {
        for (int j = i + 1; j < 5; ++j)
            if (xs[i].overlaps(xs[j])) return dg::fail(DG_EINVAL, "%s: the outputs overlap", fn);
        for (int j = 0; j < 3; ++j)
            if (xs[i].overlaps(ro[j])) return dg::fail(DG_EINVAL, "%s: wq, wk or cs overlaps an output", fn);
    }
    uint16_t* k16p = fmt16 && do_k ? static_cast<uint16_t*>(k16) : nullptr;
    uint16_t* v16p = fmt16 && do_v ? static_cast<uint16_t*>(v16) : nullptr;
    NormArgs a{};
    if (do_q)
        a.seg[a.nseg++] = NormSeg{q, need_w ? wq : nullptr, (long long)batch * T * nh, nh, flags,
                                  nullptr, nullptr, nullptr};
    if (do_k)
        a.seg[a.nseg++] = NormSeg{k, need_w ? wk : nullptr, (long long)batch * T * nkv, nkv, flags,
                                  v_from_k ? v : nullptr, k16p, v_from_k ? v16p : nullptr};
    if (do_v && !v_from_k)
        a.seg[a.nseg++] = NormSeg{v, nullptr, (long long)batch * T * nkv, nkv, 0u, nullptr, v16p,
                                  nullptr};
    a.cs = need_cs ? cs : nullptr;
    a.T = T;
    a.hd = hd;
    a.eps = eps;
    a.fmt16 = fmt16;
    a.kvmajor = !do_q && do_k && do_v && !v_from_k;   // two segments of nkv heads, T rows each
    return launch_norm(fn, a, stream);
}

}  // namespace

extern "C" int dg_qkv_headnorm_rope(float* q, const float* wq, float* k, const float* wk, float* v,
                                    const float* cs, int batch, int T, int nh, int nkv, int hd,
                                    unsigned flags, float eps, void* stream) {
    return qkv_norm_call("dg_qkv_headnorm_rope", q, wq, k, wk, v, cs, nullptr, nullptr, 0, batch,
                         T, nh, nkv, hd, flags, eps, stream);
}

extern "C" int dg_qkv_headnorm_rope_kv16(float* q, const float* wq, float* k, const float* wk,
                                         float* v, const float* cs, void* k16, void* v16,
                                         int batch, int T, int nh, int nkv, int hd,
                                         unsigned flags, float eps, int kv_format, void* stream) {
    const char* fn = "dg_qkv_headnorm_rope_kv16";
    if (kv_format != DG_KV_F16 && kv_format != DG_KV_BF16)
        return dg::fail(DG_EINVAL, "%s: kv_format must be DG_KV_F16 or DG_KV_BF16, got %d", fn,
                        kv_format);
    return qkv_norm_call(fn, q, wq, k, wk, v, cs, k16, v16, kv_format, batch, T, nh, nkv, hd,
                         flags, eps, stream);
}
