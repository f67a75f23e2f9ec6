// flash_core.hpp -- the f32-MFMA flash-attention inner step shared by the split-GQA and the
// rel-pos kernels (gfx950, 64-lane wavefronts).
//
// What it computes is the online softmax of inferencelayer 0.2.3 src/diffusion_gemma_gpu.rs
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
// Contraction order over the head dimension is permuted so that each lane fetches 4
// consecutive K (or Q) elements with one 16-byte access: MFMA step s, lane half h uses element
// pi(s, h) = 8*(s/4) + 4*h + s%4.  Q is loaded with the same permutation.
#pragma once

#include <hip/hip_runtime.h>

namespace dgk {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKeys = 32;    // keys per tile
constexpr int kQuery = 32;   // query vectors per wavefront
constexpr float kLog2e = 1.4426950408889634f;

template <int HD>
struct Tile {
    static constexpr int kStride = HD + 4;  // K row stride in LDS: conflict-free 16-byte reads
    static constexpr int kVGroups = HD / 32;  // 32-wide output tiles per query
};

__device__ inline int key_of(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Loads this lane's share of a query vector: qreg[4*g + e] = q[8*g + 4*half + e] * mul.
template <int HD>
__device__ inline void load_q(const float* __restrict__ qrow, bool valid, int half, float mul,
                              float (&qreg)[HD / 2]) {
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        float4 v = valid ? *reinterpret_cast<const float4*>(qrow + 8 * g + 4 * half)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        qreg[4 * g + 0] = v.x * mul;
        qreg[4 * g + 1] = v.y * mul;
        qreg[4 * g + 2] = v.z * mul;
        qreg[4 * g + 3] = v.w * mul;
    }
}

// S^T tile (32 keys x 32 queries) from K in LDS (row stride Tile<HD>::kStride).
template <int HD>
__device__ inline f32x16 scores(const float* __restrict__ ks, int l32, int half,
                                const float (&qreg)[HD / 2]) {
    f32x16 s = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* kr = ks + l32 * Tile<HD>::kStride + 4 * half;
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        const float4 kf = *reinterpret_cast<const float4*>(kr + 8 * g);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qreg[4 * g + 0], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qreg[4 * g + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qreg[4 * g + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qreg[4 * g + 3], s, 0, 0, 0);
    }
    return s;
}

// Online-softmax update on a masked S^T tile (masked entries hold -inf).  Turns s into
// probabilities, rescales o and the lane's partial denominator.
template <int HD>
__device__ inline void softmax_update(f32x16& s, float& m, float& lsum,
                                      f32x16 (&o)[Tile<HD>::kVGroups]) {
    float tmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = exp2f(m - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[r] = exp2f(s[r] - m_use);
        psum += s[r];
    }
    lsum = lsum * corr + psum;
    m = m_new;
#pragma unroll
    for (int t = 0; t < Tile<HD>::kVGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= corr;
}

// O^T += V^T P^T with V in LDS stored column-permuted: element c of a key row sits at
// (c % 32) * (HD/32) + c / 32, so one access returns the lane's column in every 32-wide group.
template <int HD>
__device__ inline void accumulate_pv(const float* __restrict__ vs, int l32, int half,
                                     const f32x16& p, f32x16 (&o)[Tile<HD>::kVGroups]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float* vr = vs + key_of(r, half) * HD + l32 * Tile<HD>::kVGroups;
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

// Writes o / l for the lane's query (row pointer `orow`, contiguous HD floats).
template <int HD>
__device__ inline void store_out(float* __restrict__ orow, bool valid, int half, float lsum,
                                 const f32x16 (&o)[Tile<HD>::kVGroups]) {
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!valid) return;
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int t = 0; t < Tile<HD>::kVGroups; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float4 w = make_float4(o[t][4 * b + 0] * inv, o[t][4 * b + 1] * inv,
                                   o[t][4 * b + 2] * inv, o[t][4 * b + 3] * inv);
            *reinterpret_cast<float4*>(orow + 32 * t + 8 * b + 4 * half) = w;
        }
}

// Stores one float4 of a key row into the K tile (plain) and the V tile (column-permuted).
template <int HD>
__device__ inline void stage_k(float* ks, int key, int c, float4 v) {
    *reinterpret_cast<float4*>(ks + key * Tile<HD>::kStride + c) = v;
}
template <int HD>
__device__ inline void stage_v(float* vs, int key, int c, float4 v) {
    constexpr int G = Tile<HD>::kVGroups;
    float* vr = vs + key * HD;
    vr[((c + 0) & 31) * G + ((c + 0) >> 5)] = v.x;
    vr[((c + 1) & 31) * G + ((c + 1) >> 5)] = v.y;
    vr[((c + 2) & 31) * G + ((c + 2) >> 5)] = v.z;
    vr[((c + 3) & 31) * G + ((c + 3) >> 5)] = v.w;
}

}  // namespace dgk
