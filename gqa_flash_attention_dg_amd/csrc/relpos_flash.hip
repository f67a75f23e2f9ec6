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
// up per key.  Here each workgroup computes the bias rows of its own 64 queries in a prologue
// (into LDS and registers: no global round trip, no workspace), then runs the f32-MFMA flash
// loop of flash_core.hpp.  A workgroup is 2 groups of 32 queries x 4 wavefronts; the 4
// wavefronts of a group take every 4th 32-key tile (stages of 128 keys, double-buffered
// direct global->LDS tiles) and merge their softmax states at the end.  The bias enters each
// score through the MFMA accumulator's starting value.  64-query workgroups give 768
// workgroups at the 64x64-grid, 12-head shape: three full rounds on 256 CUs.
#include "dg_common.hpp"
#include "flash_core.hpp"

namespace {

using dgk::f32x16;
constexpr int HD = 64;
constexpr int kWaves = 8;
constexpr int kQGroups = 2;                   // query groups of 32 per workgroup
constexpr int kParts = 4;                     // wavefronts per group, one key tile each per stage
constexpr int kBlockQ = kQGroups * dgk::kQuery;
constexpr int kStage = kParts * dgk::kKeys;   // 128 keys per stage
constexpr int kMaxGrid = 64;                  // gh, gw <= 64

struct RelArgs {
    const float* qkv;
    const float* rh;
    const float* rw;
    const float* dhw;  // precomputed bias rows (dh [heads][n][64], then dw), or null
    float* out;
    int n, gh, gw, heads, W;
    int qblocks, nblocks;
    float qmul;  // scale * log2(e)
};

__device__ inline int xcd_remap(int bid, int n) {
    if ((n & 7) != 0) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

// Bias rows in log2 units, the page's DHDW step as small matrix products: workgroup (head,
// line) takes one grid row qy (line < gh; dh[i][ky] = <q_i, Rh[qy,ky]> for the gw queries of
// that row) or one grid column qx (dw[i][kx] = <q_i, Rw[qx,kx]> for the gh queries of that
// column).  Both operands (at most 64 x 64 each) are staged in LDS with coalesced loads; each
// thread forms 16 dot products.  Output rows are 64 wide: dh [heads][n][64], dw after it.
__global__ void __launch_bounds__(256) relpos_bias_kernel(RelArgs a, float* __restrict__ dhw) {
    __shared__ float qs[kMaxGrid * (HD + 1)];
    __shared__ float ts[kMaxGrid * (HD + 1)];
    const int head = blockIdx.x / (a.gh + a.gw);
    const int line = blockIdx.x % (a.gh + a.gw);
    const bool is_h = line < a.gh;
    const int nq = is_h ? a.gw : a.gh;      // queries on this line
    const int nr = is_h ? a.gh : a.gw;      // table rows (ky or kx)
    const size_t rs = (size_t)3 * a.W;
    auto qidx = [&](int u) { return is_h ? line * a.gw + u : u * a.gw + (line - a.gh); };
    const float* tab = is_h ? a.rh + (size_t)line * a.gh * HD : a.rw + (size_t)(line - a.gh) * a.gw * HD;
    for (int e = threadIdx.x; e < kMaxGrid * HD; e += 256) {
        const int row = e / HD, c = e % HD;
        qs[row * (HD + 1) + c] = row < nq ? a.qkv[(size_t)qidx(row) * rs + head * HD + c] : 0.0f;
        ts[row * (HD + 1) + c] = row < nr ? tab[(size_t)row * HD + c] : 0.0f;
    }
    __syncthreads();
    const int u = threadIdx.x & 63;          // query on the line
    const int r0 = (threadIdx.x >> 6) * 16;  // first of this thread's 16 table rows
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    for (int c = 0; c < HD; ++c) {
        const float qv = qs[u * (HD + 1) + c];
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[k] += qv * ts[(r0 + k) * (HD + 1) + c];
    }
    if (u >= nq) return;
    float* dst = dhw + ((is_h ? 0 : (size_t)a.heads * a.n) + (size_t)head * a.n + qidx(u)) * kMaxGrid;
#pragma unroll
    for (int k = 0; k < 16; k += 4)
        if (r0 + k < nr)
            *reinterpret_cast<float4*>(dst + r0 + k) =
                make_float4(acc[k] * dgk::kLog2e, acc[k + 1] * dgk::kLog2e, acc[k + 2] * dgk::kLog2e,
                            acc[k + 3] * dgk::kLog2e);
}

// kAligned: gw is 32 or 64, so every 32-key tile lies inside one grid row (one ky) and, as a
// stage spans 128 keys, a wavefront always sees the same 32 kx values: its 16 dw terms stay
// in registers and the dh term is one LDS read per tile.  Otherwise both terms are looked up
// per score from LDS tables.
template <bool kAligned>
__global__ void __launch_bounds__(512) relpos_flash_kernel(RelArgs a) {
    using TL = dgk::Tile<HD>;
    // staging: [buffer][tile][K, V] and bias tables [group][ky or kx][query] (dh, then dw)
    __shared__ __attribute__((aligned(16))) float smem[2 * kParts * 2 * TL::kFloats];
    __shared__ float tab[2 * kQGroups * kMaxGrid * dgk::kQuery];
    auto tile_ptr = [&](int buf, int tile, int isv) {
        return smem + ((buf * kParts + tile) * 2 + isv) * TL::kFloats;
    };

    const int lid = xcd_remap(blockIdx.x, a.nblocks);
    const int qb = lid % a.qblocks;
    const int head = lid / a.qblocks;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int grp = wave & (kQGroups - 1), part = wave >> 1;
    const size_t rs = (size_t)3 * a.W;  // qkv row stride (floats)

    const int qfirst = qb * kBlockQ + grp * dgk::kQuery;
    const int qi = qfirst + l32;
    const bool valid = qi < a.n;
    const float* qrow = a.qkv + (size_t)(valid ? qi : 0) * rs + head * HD;
    const bool active = qfirst < a.n;
    const bool bias = a.rh != nullptr;
    float* dh_tab = tab + grp * kMaxGrid * dgk::kQuery;                   // [ky][query]
    float* dw_tab = tab + (kQGroups + grp) * kMaxGrid * dgk::kQuery;      // [kx][query]
    const int kxbase = (part * dgk::kKeys) % a.gw;  // aligned case: this wave's kx offset

    // Prologue: the bias dot products of this group's queries in log2 units.  dh[ky] =
    // <q, Rh[qy,ky]> for all ky, split over the group's 4 wavefronts and 2 lane halves; dw[kx] =
    // <q, Rw[qx,kx]>, either for this lane's own 16 kx values (aligned) or for all kx (table).
    f32x16 dwreg;
#pragma unroll
    for (int r = 0; r < 16; ++r) dwreg[r] = 0.0f;
    if (bias && active && a.dhw) {
        // Gather this group's slice of the precomputed bias rows.
        const float* dhq = a.dhw + ((size_t)head * a.n + (valid ? qi : 0)) * kMaxGrid;
        const float* dwq = dhq + (size_t)a.heads * a.n * kMaxGrid;
        for (int ky = part * 2 + half; ky < a.gh; ky += 2 * kParts)
            dh_tab[ky * dgk::kQuery + l32] = valid ? dhq[ky] : 0.0f;
        if (kAligned) {
#pragma unroll
            for (int r4 = 0; r4 < 16; r4 += 4) {
                const float4 t = valid ? *reinterpret_cast<const float4*>(dwq + kxbase + dgk::key_of(r4, half))
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
                dwreg[r4] = t.x; dwreg[r4 + 1] = t.y; dwreg[r4 + 2] = t.z; dwreg[r4 + 3] = t.w;
            }
        } else {
            for (int kx = part * 2 + half; kx < a.gw; kx += 2 * kParts)
                dw_tab[kx * dgk::kQuery + l32] = valid ? dwq[kx] : 0.0f;
        }
    } else if (bias && active) {
        float qf[HD];
#pragma unroll
        for (int c = 0; c < HD; c += 4) {
            const float4 t = valid ? *reinterpret_cast<const float4*>(qrow + c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[c] = t.x; qf[c + 1] = t.y; qf[c + 2] = t.z; qf[c + 3] = t.w;
        }
        auto dot = [&](const float* tr) {
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < HD; c += 4) {
                const float4 t = *reinterpret_cast<const float4*>(tr + c);
                d += qf[c] * t.x + qf[c + 1] * t.y + qf[c + 2] * t.z + qf[c + 3] * t.w;
            }
            return d * dgk::kLog2e;
        };
        const int qy = valid ? qi / a.gw : 0, qx = valid ? qi % a.gw : 0;
        for (int ky = part * 2 + half; ky < a.gh; ky += 2 * kParts)
            dh_tab[ky * dgk::kQuery + l32] = dot(a.rh + ((size_t)qy * a.gh + ky) * HD);
        if (kAligned) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dwreg[r] = dot(a.rw + ((size_t)qx * a.gw + kxbase + dgk::key_of(r, half)) * HD);
        } else {
            for (int kx = part * 2 + half; kx < a.gw; kx += 2 * kParts)
                dw_tab[kx * dgk::kQuery + l32] = dot(a.rw + ((size_t)qx * a.gw + kx) * HD);
        }
    }

    // Loads: the four wavefronts with part < 2 (one per SIMD) issue each stage's 64 wave-wide
    // loads -- K and V of 4 tiles -- while their SIMD partners keep the matrix pipe busy.
    constexpr int kLoadsPerWave = 2 * kParts * TL::kLoadsPerTile / 4;
    constexpr int R = TL::kRowsPerLoad;
    const int pos = lane % TL::kChunks, rsub = lane / TL::kChunks;
    const char* kbase = reinterpret_cast<const char*>(a.qkv + a.W + head * HD);
    const char* vbase = reinterpret_cast<const char*>(a.qkv + 2 * (size_t)a.W + head * HD);
    const unsigned rsb = (unsigned)(rs * 4);
    const int nfull = a.n / kStage;  // stages whose 128 key rows all exist
    auto issue_stage = [&](int st, int buf) {
        if (st < nfull) {  // wave-uniform: scalar row base + loop-invariant lane offsets
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int L = wave * kLoadsPerWave + i;
                const int tpart = L / TL::kLoadsPerTile, ld = L % TL::kLoadsPerTile;
                const int tile = tpart >> 1, isv = tpart & 1;
                const int trow = ld * R + rsub;
                const unsigned coff = 16u * (isv ? pos : (pos ^ (trow % TL::kChunks)));
                const int j0 = st * kStage + tile * dgk::kKeys;
                const char* p = (isv ? vbase : kbase) + (size_t)j0 * rsb + ((unsigned)trow * rsb + coff);
                __builtin_amdgcn_global_load_lds(p, (dgk::lds_void*)(tile_ptr(buf, tile, isv) + ld * 256), 16, 0, 0);
            }
        } else {           // the partial last stage: rows past the end repeat the last key
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int L = wave * kLoadsPerWave + i;
                const int tpart = L / TL::kLoadsPerTile, ld = L % TL::kLoadsPerTile;
                const int tile = tpart >> 1, isv = tpart & 1;
                const int trow = ld * R + rsub;
                const unsigned coff = 16u * (isv ? pos : (pos ^ (trow % TL::kChunks)));
                const int j = min(st * kStage + tile * dgk::kKeys + trow, a.n - 1);
                const char* p = (isv ? vbase : kbase) + (size_t)j * rsb + coff;
                __builtin_amdgcn_global_load_lds(p, (dgk::lds_void*)(tile_ptr(buf, tile, isv) + ld * 256), 16, 0, 0);
            }
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
    if (wave < 4) issue_stage(0, 0);
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // stage st has landed everywhere, stage st-1 is consumed (and the
                          // bias tables are complete before the first use)
        if (wave < 4 && st + 1 < nstage) issue_stage(st + 1, buf ^ 1);
        const int t0 = st * kStage + part * dgk::kKeys;
        if (active && t0 < a.n) {
            const float ref = dgk::ref_of(m);
            f32x16 s;
            if (kAligned) {
                const float dhv = bias ? dh_tab[(t0 / a.gw) * dgk::kQuery + l32] : 0.0f;
                s = dgk::scores_shift<HD>(tile_ptr(buf, part, 0), l32, half, qreg, dhv - ref, dwreg);
            } else {
                s = dgk::scores<HD>(tile_ptr(buf, part, 0), l32, half, qreg, -ref);
                if (bias) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = min(t0 + dgk::key_of(r, half), a.n - 1);
                        s[r] += dh_tab[(j / a.gw) * dgk::kQuery + l32] + dw_tab[(j % a.gw) * dgk::kQuery + l32];
                    }
                }
            }
            if (t0 + dgk::kKeys > a.n) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (t0 + dgk::key_of(r, half) >= a.n) s[r] = -INFINITY;
            }
            dgk::softmax_update<HD>(s, m, lsum, o);
            dgk::accumulate_pv<HD>(tile_ptr(buf, part, 1), l32, half, s, o);
        }
    }

    __syncthreads();
    dgk::group_merge<HD>(smem, grp, part, kParts, active, lane, m, lsum, o);
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (part != 0 || !valid) return;
    dgk::store_row<HD>(a.out + (size_t)qi * a.W + head * HD, 1.0f / ltot, o, half);
}

}  // namespace

extern "C" size_t relpos_flash_attn_workspace_size(int gh, int gw, int heads, int hd) {
    if (gh < 1 || gw < 1 || heads < 1 || hd != HD || gh > kMaxGrid || gw > kMaxGrid) return 0;
    return (size_t)2 * heads * gh * gw * kMaxGrid * sizeof(float);
}

extern "C" int relpos_flash_attn(const float* qkv, const float* rh, const float* rw, float* out,
                                 int gh, int gw, int heads, int hd, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
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
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15))
        return dg::fail(DG_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    const long long n = (long long)gh * gw;
    if (n == 0 || heads == 0) return dg::ok();
    if (!qkv || !out) return dg::fail(DG_EINVAL, "%s: qkv and out must be non-NULL", fn);
    const size_t W = (size_t)heads * HD;
    const size_t need = relpos_flash_attn_workspace_size(gh, gw, heads, hd);
    if (workspace && workspace_bytes < need)
        return dg::fail(DG_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                        workspace_bytes, need);
    const bool use_ws = workspace && rh;
    const dg::Span so(out, (size_t)n * W * 4);
    const dg::Span sq(qkv, (size_t)n * 3 * W * 4), sh(rh, (size_t)gh * gh * HD * 4),
        sw(rw, (size_t)gw * gw * HD * 4), sws(use_ws ? workspace : nullptr, need);
    if (so.overlaps(sq) || so.overlaps(sh) || so.overlaps(sw) || so.overlaps(sws))
        return dg::fail(DG_EINVAL, "%s: out overlaps an input or the workspace", fn);
    if (sws.overlaps(sq) || sws.overlaps(sh) || sws.overlaps(sw))
        return dg::fail(DG_EINVAL, "%s: workspace overlaps an input", fn);
    // The kernels use 16-byte vector accesses on every tensor.
    if ((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(out) |
         reinterpret_cast<uintptr_t>(rh) | reinterpret_cast<uintptr_t>(rw)) & 15)
        return dg::fail(DG_EINVAL, "%s: tensor pointers must be 16-byte aligned", fn);
    const long long qblocks = (n + kBlockQ - 1) / kBlockQ;
    if (qblocks * heads > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
    RelArgs a;
    a.qkv = qkv; a.rh = rh; a.rw = rw; a.out = out;
    a.dhw = use_ws ? static_cast<const float*>(workspace) : nullptr;
    a.n = (int)n; a.gh = gh; a.gw = gw; a.heads = heads; a.W = (int)W;
    a.qblocks = (int)qblocks;
    a.nblocks = (int)(qblocks * heads);
    a.qmul = scale * dgk::kLog2e;
    hipStream_t s = (hipStream_t)stream;
    if (use_ws)
        hipLaunchKernelGGL(relpos_bias_kernel, dim3((unsigned)(heads * (gh + gw))), dim3(256), 0, s, a,
                           static_cast<float*>(workspace));
    if (gw == 32 || gw == 64)
        hipLaunchKernelGGL(relpos_flash_kernel<true>, dim3((unsigned)a.nblocks), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL(relpos_flash_kernel<false>, dim3((unsigned)a.nblocks), dim3(512), 0, s, a);
    return dg::launch_status(fn);
}
