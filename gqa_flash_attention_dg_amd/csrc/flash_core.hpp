// flash_core.hpp -- the f32-MFMA flash-attention pieces shared by the split-GQA and the
// rel-pos kernels (gfx950, 64-lane wavefronts).
//
// What they compute is the online softmax of inferencelayer 0.2.3 src/diffusion_gemma_gpu.rs
// kernel DG_ATTN (and of the register flash in 0.2.8 src/deepencoder_gpu.rs): per key tile a
// running max m, a correction exp(m_old - m_new) applied to the running denominator and to the
// output accumulator, and p = exp(s - m_new).  Scores are kept in log2 units (the caller folds
// log2(e) into q and into any bias), so the exponentials are exp2.
//
// Layout.  One wavefront owns 32 query vectors; a key tile holds 32 keys.  Scores are formed
// TRANSPOSED, S^T = K Q^T, with v_mfma_f32_32x32x2f32 (A = K from LDS, B = Q from registers):
// lane l then holds query column l%32 and 16 of the 32 keys, key(r, l) = 8*(r/4) + 4*(l/32) +
// r%4 for accumulator register r.  Row max and row sum need one in-lane pass and one exchange
// with lane l^32.  The output is accumulated transposed as well, O^T += V^T P^T: its B operand
// at k-step r is exactly register r of the probabilities (key(r, l) for the lane's query), so P
// never moves between lanes; the A operand is V^T, read from LDS at the matching keys.
//
// Contraction orders are free, so both are chosen for 16-byte LDS reads:
//  * scores: MFMA step s, lane half h contracts head element 8*(s/4) + 4*h + s%4, so one
//    16-byte K read feeds 4 MFMAs (Q is loaded with the same permutation);
//  * output: row m of accumulator group t holds head element m*G + t (G = hd/32 groups), so a
//    lane's G values of one V row are contiguous.
//
// Tiles live in LDS in natural row-major order (row = one key, hd floats) and are filled by
// 16-byte direct global->LDS loads (global_load_lds_dwordx4: lane i of an instruction lands at
// base + 16*i).  K rows are stored with their 16-byte chunks permuted, chunk c of key row k at
// position c ^ (k mod chunks-per-row), which makes the 32 lanes reading 32 different K rows hit
// distinct banks.  (The split-GQA kernel's f32 tiles at hd 128 use a padded layout of their own,
// with no permutation; the helpers here serve the rel-pos kernel and its other tiles.)
#pragma once

#include <hip/hip_runtime.h>

namespace dgk {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKeys = 32;    // keys per tile
constexpr int kQuery = 32;   // query vectors per wavefront
constexpr float kLog2e = 1.4426950408889634f;

template <int HD>
struct Tile {
    static constexpr int kChunks = HD / 4;            // 16-byte chunks per key row
    static constexpr int kFloats = kKeys * HD;        // one K or V tile
    static constexpr int kGroups = HD / 32;           // output accumulators per lane
    static constexpr int kRowsPerLoad = 64 / kChunks; // key rows per wave-wide 1 KiB load
    static constexpr int kLoadsPerTile = kKeys / kRowsPerLoad;
};

__device__ inline int key_of(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Loads this lane's share of a query vector: qreg[4*g + e] = q[8*g + 4*half + e] * mul.
// Elements at or past `lim` (the true head dim when a narrower head is padded to the HD-wide
// tile; a multiple of 4) read as zero.
template <int HD>
__device__ inline void load_q(const float* __restrict__ qrow, bool valid, int half, float mul,
                              float (&qreg)[HD / 2], int lim = HD) {
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        const bool in = valid && 8 * g + 4 * half < lim;
        float4 v = in ? *reinterpret_cast<const float4*>(qrow + 8 * g + 4 * half)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
        qreg[4 * g + 0] = v.x * mul;
        qreg[4 * g + 1] = v.y * mul;
        qreg[4 * g + 2] = v.z * mul;
        qreg[4 * g + 3] = v.w * mul;
    }
}

// Tile row that lane `lane` fills in wave-wide load `ld` of a tile.
template <int HD>
__device__ inline int dma_row(int ld, int lane) {
    return ld * Tile<HD>::kRowsPerLoad + lane / Tile<HD>::kChunks;
}

// Issues wave-wide 1 KiB direct load `ld` into a K tile (kSwizzle) or a V tile (plain).
// `rowptr` is the global address of this lane's key row dma_row(ld, lane).
template <int HD, bool kSwizzle>
__device__ inline void dma_load(float* tile, int ld, const float* rowptr, int lane) {
    using TL = Tile<HD>;
    const int pos = lane % TL::kChunks;
    const int chunk = kSwizzle ? (pos ^ (dma_row<HD>(ld, lane) % TL::kChunks)) : pos;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(rowptr + 4 * chunk),
                                     (lds_void*)(tile + ld * 256), 16, 0, 0);
}

// S^T tile (32 keys x 32 queries) from a swizzled K tile in LDS, accumulated onto `s`.
template <int HD>
__device__ inline f32x16 scores_from(const float* __restrict__ ks, int l32, int half,
                                     const float (&qreg)[HD / 2], f32x16 s) {
    using TL = Tile<HD>;
    const float* kr = ks + l32 * HD;
    const int sw = l32 % TL::kChunks;
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        const float4 kf = *reinterpret_cast<const float4*>(kr + 4 * ((2 * g + half) ^ sw));
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qreg[4 * g + 0], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qreg[4 * g + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qreg[4 * g + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qreg[4 * g + 3], s, 0, 0, 0);
    }
    return s;
}

// As scores_from, plus a per-query shift added to every key of the lane's query column.  The
// shift rides in one extra MFMA step (A = 1 and B = shift in the lower lane half, zeros in the
// upper half) instead of a VALU pass over the 16 accumulator registers.
template <int HD>
__device__ inline f32x16 scores_shift(const float* __restrict__ ks, int l32, int half,
                                      const float (&qreg)[HD / 2], float shift, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(half ? 0.0f : 1.0f, half ? 0.0f : shift, c, 0, 0, 0);
    return scores_from<HD>(ks, l32, half, qreg, c);
}

template <int HD>
__device__ inline f32x16 scores(const float* __restrict__ ks, int l32, int half,
                                const float (&qreg)[HD / 2], float shift) {
    const f32x16 z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    return scores_shift<HD>(ks, l32, half, qreg, shift, z);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax update on a masked S^T tile.  On entry s holds score - ref, where ref is the
// lane's softmax reference m (0 while m is still -inf); masked entries hold -inf.  The
// reference only moves when some score exceeds it by more than kHeadroom (log2 units): then
// the tile max becomes the new reference and o and lsum are rescaled.  Otherwise the
// probabilities exp2(score - m) are taken as they are (each below 2^kHeadroom, far from f32
// overflow; smaller ones lose nothing relative to the terms at or above the reference).  The
// result is the same sum as with a per-tile max; only rounding differs.  On exit s holds the
// probabilities.
constexpr float kHeadroom = 60.0f;

__device__ inline float ref_of(float m) { return m == -INFINITY ? 0.0f : m; }

template <int HD>
__device__ inline void softmax_update(f32x16& s, float& m, float& lsum,
                                      f32x16 (&o)[Tile<HD>::kGroups]) {
    float lmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) lmax = fmaxf(lmax, s[r]);
    if (__any(lmax > kHeadroom || m == -INFINITY)) {
        const float ref = ref_of(m);
        const float tmax = fmaxf(lmax, __shfl_xor(lmax, 32));
        const float m_new = fmaxf(m, ref + tmax);
        const float nref = ref_of(m_new);
        const float corr = fast_exp2(m - nref);
        const float shift = ref - nref;
        lsum *= corr;
#pragma unroll
        for (int t = 0; t < Tile<HD>::kGroups; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] *= corr;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] += shift;
        m = m_new;
    }
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(s[r]);
        psum += s[r];
    }
    lsum += psum;
}

// O^T += V^T P^T from a plain V tile in LDS; the lane reads its G contiguous head elements
// of the key row that its half supplies at k-step r.
template <int HD>
__device__ inline void accumulate_pv(const float* __restrict__ vs, int l32, int half,
                                     const f32x16& p, f32x16 (&o)[Tile<HD>::kGroups]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float* vr = vs + key_of(r, half) * HD + l32 * Tile<HD>::kGroups;
        if constexpr (HD == 128) {
            const float4 vf = *reinterpret_cast<const float4*>(vr);
            o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.x, p[r], o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.y, p[r], o[1], 0, 0, 0);
            o[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.z, p[r], o[2], 0, 0, 0);
            o[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.w, p[r], o[3], 0, 0, 0);
        } else {
            const float2 vf = *reinterpret_cast<const float2*>(vr);
            o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.x, p[r], o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf.y, p[r], o[1], 0, 0, 0);
        }
    }
}

// Head element held by accumulator register r of group t in lane half `half`.
template <int HD>
__device__ inline int out_elem(int t, int r, int half) {
    return (8 * (r >> 2) + 4 * half + (r & 3)) * Tile<HD>::kGroups + t;
}

// Writes o * scale for the lane's query (row pointer `orow`, contiguous floats); only head
// elements below `lim` (a multiple of 4) are written.
template <int HD>
__device__ inline void store_row(float* __restrict__ orow, float scale,
                                 const f32x16 (&o)[Tile<HD>::kGroups], int half, int lim = HD) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (out_elem<HD>(0, r, half) >= lim) continue;
        float* dst = orow + out_elem<HD>(0, r, half);
        if constexpr (HD == 128) {
            *reinterpret_cast<float4*>(dst) =
                make_float4(o[0][r] * scale, o[1][r] * scale, o[2][r] * scale, o[3][r] * scale);
        } else {
            *reinterpret_cast<float2*>(dst) = make_float2(o[0][r] * scale, o[1][r] * scale);
        }
    }
}

// Writes o * scale for the lane's query as row l32 of a row-major block in LDS (`rows`, row
// stride HD + 4 floats: consecutive rows start 4 banks apart, so the 16-byte writes of a
// wavefront do not collide).
template <int HD>
__device__ inline void stage_row(float* __restrict__ rows, int l32, float scale,
                                 const f32x16 (&o)[Tile<HD>::kGroups], int half) {
    float* dst = rows + l32 * (HD + 4);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float* d = dst + out_elem<HD>(0, r, half);
        if constexpr (HD == 128) {
            *reinterpret_cast<float4*>(d) =
                make_float4(o[0][r] * scale, o[1][r] * scale, o[2][r] * scale, o[3][r] * scale);
        } else {
            *reinterpret_cast<float2*>(d) = make_float2(o[0][r] * scale, o[1][r] * scale);
        }
    }
}

// Merges the softmax states of the two wavefronts of a pair (same 32 queries, disjoint keys):
// the odd-tile wavefront (hi) hands (o, m, lsum) to the even-tile one through LDS scratch
// `smem` (at least 4 * 64 * (hd/2 + 2) floats, not in use by anyone).  Every thread of the
// workgroup must call this; afterwards the even-tile wavefront holds the merged state.
template <int HD>
__device__ inline void pair_merge(float* smem, int pair, bool hi, bool active, int lane,
                                  float& m, float& lsum, f32x16 (&o)[Tile<HD>::kGroups]) {
    constexpr int kVals = Tile<HD>::kGroups * 16 + 2;
    float* mg = smem + pair * kVals * 64;
    if (hi && active) {
#pragma unroll
        for (int t = 0; t < Tile<HD>::kGroups; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mg[(t * 16 + r) * 64 + lane] = o[t][r];
        mg[(kVals - 2) * 64 + lane] = m;
        mg[(kVals - 1) * 64 + lane] = lsum;
    }
    __syncthreads();
    if (hi || !active) return;
    const float m2 = mg[(kVals - 2) * 64 + lane];
    const float l2 = mg[(kVals - 1) * 64 + lane];
    const float mn = fmaxf(m, m2);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    const float ca = fast_exp2(m - mu), cb = fast_exp2(m2 - mu);
#pragma unroll
    for (int t = 0; t < Tile<HD>::kGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = o[t][r] * ca + mg[(t * 16 + r) * 64 + lane] * cb;
    lsum = lsum * ca + l2 * cb;
    m = mn;
}

// Merges the softmax states of `nparts` wavefronts that hold the same 32 queries over disjoint
// keys: parts 1..nparts-1 hand (o, m, lsum) to part 0 through LDS scratch `smem` (at least
// ngroups * (nparts-1) * 64 * (hd/2 + 2) floats, not in use by anyone).  Every thread of the
// workgroup must call this; afterwards part 0 holds the merged state.
template <int HD>
__device__ inline void group_merge(float* smem, int grp, int part, int nparts, bool active,
                                   int lane, float& m, float& lsum,
                                   f32x16 (&o)[Tile<HD>::kGroups]) {
    constexpr int kVals = Tile<HD>::kGroups * 16 + 2;
    float* base = smem + grp * (nparts - 1) * kVals * 64;
    if (part > 0 && active) {
        float* mg = base + (part - 1) * kVals * 64;
#pragma unroll
        for (int t = 0; t < Tile<HD>::kGroups; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mg[(t * 16 + r) * 64 + lane] = o[t][r];
        mg[(kVals - 2) * 64 + lane] = m;
        mg[(kVals - 1) * 64 + lane] = lsum;
    }
    __syncthreads();
    if (part > 0 || !active) return;
    for (int p = 1; p < nparts; ++p) {
        const float* mg = base + (p - 1) * kVals * 64;
        const float m2 = mg[(kVals - 2) * 64 + lane];
        const float l2 = mg[(kVals - 1) * 64 + lane];
        const float mn = fmaxf(m, m2);
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float ca = fast_exp2(m - mu), cb = fast_exp2(m2 - mu);
#pragma unroll
        for (int t = 0; t < Tile<HD>::kGroups; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] = o[t][r] * ca + mg[(t * 16 + r) * 64 + lane] * cb;
        lsum = lsum * ca + l2 * cb;
        m = mn;
    }
}

}  // namespace dgk
