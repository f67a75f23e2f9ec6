// relpos_flash.hip -- relpos_flash_attn: windowless vision attention with the decomposed
// relative-position bias, flash style, on gfx950.
//
// Follows inferencelayer 0.2.8, src/deepencoder_gpu.rs: kernel SAM_SCORES fixes the score,
//   scale*<q_i,k_j> + <q_i, Rh[qy,ky]> + <q_i, Rw[qx,kx]>  (bias on the unscaled q),
// kernel DHDW hoists the two bias dot products out of the n^2 loop, `flash_reg_src` runs the
// online softmax over 64-wide chunks with hd fixed at 64, and `sam_attn_buf` fixes the fused
// qkv layout (q | k | v per token, heads contiguous) and the scale 1/sqrt(hd).
//
// The page writes dh/dw to global [heads, n, gh] / [heads, n, gw] buffers and then looks them
// up per key.  Here each workgroup computes the bias rows of its own 128 queries into LDS in
// a prologue (no global round trip, no workspace), then runs the same f32-MFMA flash loop as
// the split-GQA kernel (flash_core.hpp: 4 pairs of wavefronts on alternate 32-key tiles,
// double-buffered direct global->LDS tiles) with the two table lookups added to each score.
#include "dg_common.hpp"
#include "flash_core.hpp"

namespace {

using dgk::f32x16;
constexpr int HD = 64;
constexpr int kWaves = 8;
constexpr int kPairs = 4;
constexpr int kBlockQ = kPairs * dgk::kQuery;
constexpr int kStage = 2 * dgk::kKeys;
constexpr int kMaxGrid = 64;                 // gh, gw <= 64
constexpr int kTabStride = 2 * kMaxGrid + 1; // dh | dw per query, padded against bank conflicts

struct RelArgs {
    const float* qkv;
    const float* rh;
    const float* rw;
    float* out;
    int n, gh, gw, heads, W;
    int qblocks, nblocks;
    float qmul;  // scale * log2(e)
};

__device__ inline int xcd_remap(int bid, int n) {
    if ((n & 7) != 0) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

__global__ void __launch_bounds__(512) relpos_flash_kernel(RelArgs a) {
    using TL = dgk::Tile<HD>;
    __shared__ __attribute__((aligned(16))) float smem[2 * 2 * 2 * TL::kFloats];
    __shared__ float tab[kPairs * dgk::kQuery * kTabStride];
    auto tile_ptr = [&](int buf, int tile, int isv) {
        return smem + ((buf * 2 + tile) * 2 + isv) * TL::kFloats;
    };

    const int lid = xcd_remap(blockIdx.x, a.nblocks);
    const int qb = lid % a.qblocks;
    const int head = lid / a.qblocks;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int pair = wave & (kPairs - 1), hi = wave >> 2;
    const size_t rs = (size_t)3 * a.W;  // qkv row stride

    const int qfirst = qb * kBlockQ + pair * dgk::kQuery;
    const int qi = qfirst + l32;
    const bool valid = qi < a.n;
    const float* qrow = a.qkv + (size_t)(valid ? qi : 0) * rs + head * HD;
    const bool pair_active = qfirst < a.n;
    const bool bias = a.rh != nullptr;
    float* mytab = tab + (pair * dgk::kQuery + l32) * kTabStride;

    // Prologue: this query's bias rows in log2 units, dh[ky] = <q, Rh[qy,ky]> (even-tile wave)
    // and dw[kx] = <q, Rw[qx,kx]> (odd-tile wave); lane halves split the ky / kx range.
    if (bias && pair_active) {
        float qf[HD];
#pragma unroll
        for (int c = 0; c < HD; c += 4) {
            const float4 t = valid ? *reinterpret_cast<const float4*>(qrow + c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[c] = t.x; qf[c + 1] = t.y; qf[c + 2] = t.z; qf[c + 3] = t.w;
        }
        const int g = hi ? a.gw : a.gh;
        const int coord = valid ? (hi ? qi % a.gw : qi / a.gw) : 0;
        const float* table = hi ? a.rw : a.rh;
        for (int kk = half; kk < g; kk += 2) {
            const float* tr = table + ((size_t)coord * g + kk) * HD;
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < HD; c += 4) {
                const float4 t = *reinterpret_cast<const float4*>(tr + c);
                d += qf[c] * t.x + qf[c + 1] * t.y + qf[c + 2] * t.z + qf[c + 3] * t.w;
            }
            mytab[hi * kMaxGrid + kk] = d * dgk::kLog2e;
        }
    }

    const float* kbase = a.qkv + a.W + head * HD;
    const float* vbase = a.qkv + 2 * (size_t)a.W + head * HD;
    constexpr int kLoadsPerWave = 4 * TL::kLoadsPerTile / kWaves;
    auto issue_stage = [&](int st, int buf) {
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
            const int L = wave * kLoadsPerWave + i;
            const int part = L / TL::kLoadsPerTile;  // K0, V0, K1, V1
            const int ld = L % TL::kLoadsPerTile;
            const int tile = part >> 1, isv = part & 1;
            const int j = min(st * kStage + tile * dgk::kKeys + dgk::dma_row<HD>(ld, lane), a.n - 1);
            if (isv)
                dgk::dma_load<HD, false>(tile_ptr(buf, tile, 1), ld, vbase + (size_t)j * rs, lane);
            else
                dgk::dma_load<HD, true>(tile_ptr(buf, tile, 0), ld, kbase + (size_t)j * rs, lane);
        }
    };

    float qreg[HD / 2];
    dgk::load_q<HD>(qrow, valid, half, a.qmul, qreg);
    f32x16 o[TL::kGroups];
#pragma unroll
    for (int t = 0; t < TL::kGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    const int nstage = (a.n + kStage - 1) / kStage;
    issue_stage(0, 0);
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // stage st has landed everywhere, stage st-1 is consumed (and the
                          // bias table is complete before the first use)
        if (st + 1 < nstage) issue_stage(st + 1, buf ^ 1);
        const int t0 = st * kStage + hi * dgk::kKeys;
        if (pair_active && t0 < a.n) {
            f32x16 s = dgk::scores<HD>(tile_ptr(buf, hi, 0), l32, half, qreg, -dgk::ref_of(m));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = t0 + dgk::key_of(r, half);
                if (j >= a.n) {
                    s[r] = -INFINITY;
                } else if (bias) {
                    s[r] += mytab[j / a.gw] + mytab[kMaxGrid + j % a.gw];
                }
            }
            dgk::softmax_update<HD>(s, m, lsum, o);
            dgk::accumulate_pv<HD>(tile_ptr(buf, hi, 1), l32, half, s, o);
        }
    }

    __syncthreads();
    dgk::pair_merge<HD>(smem, pair, hi, pair_active, lane, m, lsum, o);
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (hi || !valid) return;
    dgk::store_row<HD>(a.out + (size_t)qi * a.W + head * HD, 1.0f / ltot, o, half);
}

}  // namespace

extern "C" int relpos_flash_attn(const float* qkv, const float* rh, const float* rw, float* out,
                                 int gh, int gw, int heads, int hd, float scale, void* stream) {
    const char* fn = "relpos_flash_attn";
    if (gh < 0 || gw < 0 || heads < 0)
        return dg::fail(DG_EINVAL, "%s: negative size (gh %d, gw %d, heads %d)", fn, gh, gw, heads);
    if (hd < 1) return dg::fail(DG_EINVAL, "%s: hd must be >= 1, got %d", fn, hd);
    if (hd != HD) return dg::fail(DG_EUNSUPPORTED, "%s: hd %d not supported (64 only)", fn, hd);
    if ((rh == nullptr) != (rw == nullptr))
        return dg::fail(DG_EINVAL, "%s: rh and rw must both be given or both be NULL", fn);
    if (gh > kMaxGrid || gw > kMaxGrid)
        return dg::fail(DG_EUNSUPPORTED, "%s: grid %dx%d exceeds %d per side", fn, gh, gw, kMaxGrid);
    if (!std::isfinite(scale)) return dg::fail(DG_EINVAL, "%s: scale is not finite", fn);
    const long long n = (long long)gh * gw;
    if (n == 0 || heads == 0) return dg::ok();
    if (!qkv || !out) return dg::fail(DG_EINVAL, "%s: qkv and out must be non-NULL", fn);
    const size_t W = (size_t)heads * HD;
    const dg::Span so(out, (size_t)n * W * 4);
    if (so.overlaps(dg::Span(qkv, (size_t)n * 3 * W * 4)) ||
        so.overlaps(dg::Span(rh, (size_t)gh * gh * HD * 4)) ||
        so.overlaps(dg::Span(rw, (size_t)gw * gw * HD * 4)))
        return dg::fail(DG_EINVAL, "%s: out overlaps an input", fn);
    const long long qblocks = (n + kBlockQ - 1) / kBlockQ;
    if (qblocks * heads > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
    RelArgs a;
    a.qkv = qkv; a.rh = rh; a.rw = rw; a.out = out;
    a.n = (int)n; a.gh = gh; a.gw = gw; a.heads = heads; a.W = (int)W;
    a.qblocks = (int)qblocks;
    a.nblocks = (int)(qblocks * heads);
    a.qmul = scale * dgk::kLog2e;
    hipLaunchKernelGGL(relpos_flash_kernel, dim3((unsigned)a.nblocks), dim3(512), 0,
                       (hipStream_t)stream, a);
    return dg::launch_status(fn);
}
