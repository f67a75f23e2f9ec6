// attn_split_gqa.hip -- dg_attn_split_gqa: GQA flash attention over the split key/value set
// [cache (ctx) | canvas (T)] on gfx950.
//
// Follows inferencelayer 0.2.3, src/diffusion_gemma_gpu.rs, kernel DG_ATTN and its dispatch in
// `canvas_forward`: q head h reads kv head h / (nh/nkv); key j < ctx is row j of the cache
// [nkv, ctx, hd], key j >= ctx is canvas row j - ctx of [T, nkv*hd]; online softmax over all
// ctx + T keys; DiffusionGemma passes scale 1.0.  `causal` and `scale` cover kernel DEP_ATTN of
// inferencelayer 0.2.4, src/moshi_gpu.rs (canvas row i sees canvas keys 0..i, scale 0.125).
//
// The page runs one workgroup per (canvas row, q head) and re-reads the whole key/value span
// for each.  Here one workgroup owns 128 query vectors of ONE kv head -- the G = nh/nkv q heads
// of a group times a block of canvas rows, flattened as (row, head-in-group) so they are
// contiguous in q and out -- and stages each 32-key K/V tile once in LDS for all of them.
// The seam between cache and canvas is resolved per key row while staging.  Scores and the
// value product run on f32 MFMA (flash_core.hpp).  Workgroups of one kv head are placed on
// the same XCD so its L2 serves the tile re-reads.
#include "dg_common.hpp"
#include "flash_core.hpp"

namespace {

using dgk::f32x16;
constexpr int kWaves = 4;
constexpr int kBlockQ = kWaves * dgk::kQuery;  // query vectors per workgroup

struct SplitArgs {
    const float* q;
    const float* kc;
    const float* vc;
    const float* k;
    const float* v;
    float* out;
    int T, ctx, nh, nkv, G;
    int qblocks;       // workgroups per (batch, kv head)
    int nblocks;       // total workgroups
    float qmul;        // scale * log2(e)
    int causal;
};

// Workgroup id -> logical id such that consecutive logical ids share an XCD (the hardware
// deals workgroups to the 8 XCDs round robin).
__device__ inline int xcd_remap(int bid, int n) {
    if ((n & 7) != 0) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

template <int HD>
__global__ void __launch_bounds__(256) attn_split_gqa_kernel(SplitArgs a) {
    using TL = dgk::Tile<HD>;
    __shared__ __attribute__((aligned(16))) float ks[dgk::kKeys * TL::kStride];
    __shared__ __attribute__((aligned(16))) float vs[dgk::kKeys * HD];

    const int lid = xcd_remap(blockIdx.x, a.nblocks);
    const int qb = lid % a.qblocks;
    const int bk = lid / a.qblocks;       // b * nkv + kv
    const int kv = bk % a.nkv;
    const int b = bk / a.nkv;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;

    const int nq = a.T * a.G;                       // query vectors of this (b, kv)
    const int qv = qb * kBlockQ + wave * dgk::kQuery + l32;
    const bool valid = qv < nq;
    const int row = valid ? qv / a.G : 0;
    const int hq = kv * a.G + (valid ? qv % a.G : 0);
    const size_t qoff = (((size_t)b * a.T + row) * a.nh + hq) * HD;
    const bool wave_active = qb * kBlockQ + wave * dgk::kQuery < nq;

    float qreg[HD / 2];
    dgk::load_q<HD>(a.q + qoff, valid, half, a.qmul, qreg);

    f32x16 o[TL::kVGroups];
#pragma unroll
    for (int t = 0; t < TL::kVGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    const int S = a.ctx + a.T;
    int kend = S;
    if (a.causal) {  // no query of this block sees canvas keys past its last row
        const int last = min(nq - 1, qb * kBlockQ + kBlockQ - 1) / a.G;
        kend = min(S, a.ctx + last + 1);
    }
    const float* kcb = a.kc + (size_t)bk * a.ctx * HD;
    const float* vcb = a.vc + (size_t)bk * a.ctx * HD;
    const size_t canvas_stride = (size_t)a.nkv * HD;
    const float* kb = a.k + ((size_t)b * a.T * a.nkv + kv) * HD;
    const float* vb = a.v + ((size_t)b * a.T * a.nkv + kv) * HD;

    constexpr int kVec = HD / 4;                        // float4 per key row
    constexpr int kPerThread = dgk::kKeys * kVec / 256; // float4 per thread per tile

    for (int t0 = 0; t0 < kend; t0 += dgk::kKeys) {
        __syncthreads();  // the previous tile has been consumed
#pragma unroll
        for (int it = 0; it < kPerThread; ++it) {
            const int f = tid + 256 * it;
            const int key = f / kVec;
            const int c = (f % kVec) * 4;
            const int j = t0 + key;
            float4 kf = make_float4(0.f, 0.f, 0.f, 0.f), vf = kf;
            if (j < a.ctx) {
                kf = *reinterpret_cast<const float4*>(kcb + (size_t)j * HD + c);
                vf = *reinterpret_cast<const float4*>(vcb + (size_t)j * HD + c);
            } else if (j < kend) {
                kf = *reinterpret_cast<const float4*>(kb + (size_t)(j - a.ctx) * canvas_stride + c);
                vf = *reinterpret_cast<const float4*>(vb + (size_t)(j - a.ctx) * canvas_stride + c);
            }
            dgk::stage_k<HD>(ks, key, c, kf);
            dgk::stage_v<HD>(vs, key, c, vf);
        }
        __syncthreads();
        if (wave_active) {
            f32x16 s = dgk::scores<HD>(ks, l32, half, qreg);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = t0 + dgk::key_of(r, half);
                const bool masked = j >= kend || (a.causal && j >= a.ctx && j - a.ctx > row);
                if (masked) s[r] = -INFINITY;
            }
            dgk::softmax_update<HD>(s, m, lsum, o);
            dgk::accumulate_pv<HD>(vs, l32, half, s, o);
        }
    }
    dgk::store_out<HD>(a.out + qoff, valid, half, lsum, o);
}

}  // namespace

extern "C" size_t dg_attn_split_gqa_workspace_size(int batch, int T, int ctx, int nh, int nkv,
                                                   int hd) {
    (void)batch; (void)T; (void)ctx; (void)nh; (void)nkv; (void)hd;
    return 0;
}

extern "C" int dg_attn_split_gqa(const float* q, const float* kc, const float* vc, const float* k,
                                 const float* v, float* out, int batch, int T, int ctx, int nh,
                                 int nkv, int hd, float scale, int causal, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    const char* fn = "dg_attn_split_gqa";
    if (batch < 0 || T < 0 || ctx < 0 || nh < 0 || nkv < 0)
        return dg::fail(DG_EINVAL, "%s: negative size (batch %d, T %d, ctx %d, nh %d, nkv %d)", fn,
                        batch, T, ctx, nh, nkv);
    if (nkv < 1 || nh < 1 || nh % nkv != 0)
        return dg::fail(DG_EINVAL, "%s: nh (%d) must be a positive multiple of nkv (%d)", fn, nh, nkv);
    if (hd < 1) return dg::fail(DG_EINVAL, "%s: hd must be >= 1, got %d", fn, hd);
    if (hd != 64 && hd != 128) return dg::fail(DG_EUNSUPPORTED, "%s: hd %d not supported (64 or 128)", fn, hd);
    if (!std::isfinite(scale)) return dg::fail(DG_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return dg::fail(DG_EINVAL, "%s: causal must be 0 or 1", fn);
    size_t nq = 1, nkvc = 1, ncache = 1;
    if (!dg::mul_ok(nq, batch) || !dg::mul_ok(nq, T) || !dg::mul_ok(nq, nh) || !dg::mul_ok(nq, hd) ||
        !dg::mul_ok(nkvc, batch) || !dg::mul_ok(nkvc, T) || !dg::mul_ok(nkvc, nkv) || !dg::mul_ok(nkvc, hd) ||
        !dg::mul_ok(ncache, batch) || !dg::mul_ok(ncache, nkv) || !dg::mul_ok(ncache, ctx) ||
        !dg::mul_ok(ncache, hd))
        return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    if (nq == 0) return dg::ok();
    if (!q || !k || !v || !out) return dg::fail(DG_EINVAL, "%s: q, k, v and out must be non-NULL", fn);
    if (ncache > 0 && (!kc || !vc)) return dg::fail(DG_EINVAL, "%s: kc/vc NULL with ctx %d > 0", fn, ctx);
    const dg::Span so(out, nq * 4);
    const dg::Span ins[5] = {dg::Span(q, nq * 4), dg::Span(k, nkvc * 4), dg::Span(v, nkvc * 4),
                             dg::Span(ncache ? kc : nullptr, ncache * 4),
                             dg::Span(ncache ? vc : nullptr, ncache * 4)};
    for (const auto& s : ins)
        if (so.overlaps(s)) return dg::fail(DG_EINVAL, "%s: out overlaps an input", fn);
    const long long qblocks = ((long long)T * (nh / nkv) + kBlockQ - 1) / kBlockQ;
    const long long nblocks = (long long)batch * nkv * qblocks;
    if (nblocks > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
    SplitArgs a;
    a.q = q; a.kc = kc; a.vc = vc; a.k = k; a.v = v; a.out = out;
    a.T = T; a.ctx = ctx; a.nh = nh; a.nkv = nkv; a.G = nh / nkv;
    a.qblocks = (int)qblocks;
    a.nblocks = (int)nblocks;
    a.qmul = scale * dgk::kLog2e;
    a.causal = causal;
    if (hd == 128)
        hipLaunchKernelGGL(attn_split_gqa_kernel<128>, dim3((unsigned)nblocks), dim3(256), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(attn_split_gqa_kernel<64>, dim3((unsigned)nblocks), dim3(256), 0,
                           (hipStream_t)stream, a);
    return dg::launch_status(fn);
}
