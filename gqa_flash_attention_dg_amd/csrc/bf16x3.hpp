// bf16x3.hpp -- f32 arithmetic on the bf16 matrix pipe of gfx950, shared by the split-GQA and
// rel-pos kernels: f32 operands taken as three bf16 terms, products formed from exact bf16 x
// bf16 matrix products summed in f32.
#pragma once

#include <hip/hip_runtime.h>

#include "flash_core.hpp"

namespace bf3 {

using dgk::f32x16;

// A product of two bf16 values is exact in f32, and an f32 value x is exactly the sum of three
// bf16 values: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid), rounding to nearest.
// Both differences are exact (multiples of x's last significand bit, each at most half a bf16
// step, 2^-8, of the value it is taken from), x - hi keeps at most 16 significant bits and
// x - hi - mid at most 8, so lo takes it exactly (outside the subnormal range).  So with x = q
// (scores) or x = p (the value product) each MFMA step runs three v_mfma_f32_32x32x16_bf16, one
// per term, with exact products and the sums in f32: the f32 path's arithmetic up to the
// summation order, at about a fifth of the matrix-pipe time of v_mfma_f32_32x32x2f32 on the
// same tile (bf16 K/V, which are exact in bf16).  The k-slots a lane supplies are the same for
// the A and the B operand, so which 8 of the 16 a lane half holds does not matter; the 32x32
// accumulator layout is that of the f32 instruction.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// The weight pairs (-1, 0) and (0, -1) of split_bf16x3, as register values: the empty asm keeps
// the compiler from encoding them as an inline constant, which the hardware would widen as an
// f32 constant rather than place in the low half.
struct SplitWeights {
    bf16x2 n0, n1;
    __device__ SplitWeights() {
        unsigned w0 = 0x0000bf80u, w1 = 0xbf800000u;
        asm volatile("" : "+s"(w0), "+s"(w1));
        n0 = __builtin_bit_cast(bf16x2, w0);
        n1 = __builtin_bit_cast(bf16x2, w1);
    }
};

// The three terms of x0 and x1, each pair packed in one dword (x0 in the low half).  The
// differences come from v_dot2c_f32_bf16 with weights (-1, 0) and (0, -1): x - term in one
// instruction, exact since the result is representable.
__device__ inline void split_bf16x3(float x0, float x1, const SplitWeights& w, unsigned& hi,
                                    unsigned& mid, unsigned& lo) {
    const bf16x2 n0 = w.n0, n1 = w.n1;
    const bf16x2 h = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, n0, x0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, n1, x1, false);
    const bf16x2 m = __builtin_convertvector((f32x2){r0, r1}, bf16x2);
    const float t0 = __builtin_amdgcn_fdot2_f32_bf16(m, n0, r0, false);
    const float t1 = __builtin_amdgcn_fdot2_f32_bf16(m, n1, r1, false);
    const bf16x2 l = __builtin_convertvector((f32x2){t0, t1}, bf16x2);
    hi = __builtin_bit_cast(unsigned, h);
    mid = __builtin_bit_cast(unsigned, m);
    lo = __builtin_bit_cast(unsigned, l);
}

// The lane's query operand in three bf16 terms: step st, k-slot e of lane half `half` is head
// element 16*st + 8*half + e, times mul; elements at or past lim (a multiple of 4) are zero.
template <int HD>
struct QSplit {
    u32x4 h[HD / 16], m[HD / 16], l[HD / 16];
};

template <int HD>
__device__ inline void load_q_bf16x3(const float* __restrict__ qrow, bool valid, int half,
                                     float mul, QSplit<HD>& q, int lim) {
    const SplitWeights w;
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        float x[8];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int d0 = 16 * st + 8 * half + 4 * c;
            const float4 v = valid && d0 < lim ? *reinterpret_cast<const float4*>(qrow + d0)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
            x[4 * c + 0] = v.x * mul;
            x[4 * c + 1] = v.y * mul;
            x[4 * c + 2] = v.z * mul;
            x[4 * c + 3] = v.w * mul;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned th, tm, tl;
            split_bf16x3(x[2 * i], x[2 * i + 1], w, th, tm, tl);
            q.h[st][i] = th;
            q.m[st][i] = tm;
            q.l[st][i] = tl;
        }
    }
}

// f32 K/V: both operands in three terms.
// The leading products go to `c`, the five smaller ones to `d`: kept apart, the corrections
// are summed at their own magnitude (about 2^-8 of c's), so only the leading chain rounds at
// the full magnitude of the result.
__device__ inline void mfma_bf16x6(u32x4 ah, u32x4 am, u32x4 al, u32x4 bh, u32x4 bm, u32x4 bl,
                                   f32x16& c, f32x16& d) {
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(am), as_bf16x8(bm), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(bh), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bl), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(am), as_bf16x8(bh), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bm), d, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bh), c, 0, 0, 0);
}

// Splits 8 f32 values into the three bf16x8 operands of one MFMA step.
__device__ inline void split8(const float (&x)[8], const SplitWeights& w, u32x4& h, u32x4& m,
                              u32x4& l) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned th, tm, tl;
        split_bf16x3(x[2 * i], x[2 * i + 1], w, th, tm, tl);
        h[i] = th;
        m[i] = tm;
        l[i] = tl;
    }
}

// The query operand in three terms from the f32 layout of dgk::load_q: step st, k-slot e is
// qreg[8*st + e], head element 16*st + 8*(e/4) + 4*half + e%4.
template <int HD>
__device__ inline void split_q_bf16x3(const float (&qreg)[HD / 2], QSplit<HD>& q) {
    const SplitWeights w;
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qreg[8 * st + e];
        split8(x, w, q.h[st], q.m[st], q.l[st]);
    }
}

// dgk::scores_from on the bf16 pipe: S^T += K Q^T from an f32 K tile with chunk-swizzled rows
// (chunk c of key row k at position c ^ (k mod HD/4)), q from split_q_bf16x3.  Step st reads
// the lane's head elements 16*st + 4*half + 0..3 and 16*st + 8 + 4*half + 0..3 of its key row
// and splits them; the leading products and the corrections are summed apart.
template <int HD>
__device__ inline f32x16 scores_f32_bf16x6(const float* __restrict__ ks, int l32, int half,
                                           const QSplit<HD>& q, f32x16 s) {
    const SplitWeights w;
    const float* kr = ks + l32 * HD;
    const int sw = l32 % (HD / 4);
    f32x16 d = {};
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        const float4 k0 = *reinterpret_cast<const float4*>(kr + 4 * ((4 * st + half) ^ sw));
        const float4 k1 = *reinterpret_cast<const float4*>(kr + 4 * ((4 * st + 2 + half) ^ sw));
        const float x[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        u32x4 kh, km, kl;
        split8(x, w, kh, km, kl);
        mfma_bf16x6(kh, km, kl, q.h[st], q.m[st], q.l[st], s, d);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += d[r];
    return s;
}

// dgk::accumulate_pv on the bf16 pipe: O^T += V^T P^T from an f32 V tile of plain rows (output
// row m of group t is head element m*G + t); step st takes keys dgk::key_of(8*st + e, half),
// two output groups at a time.
template <int HD>
__device__ inline void accumulate_pv_f32_bf16x6(const float* __restrict__ vs, int l32, int half,
                                                const f32x16& p, f32x16 (&o)[dgk::Tile<HD>::kGroups]) {
    constexpr int G = dgk::Tile<HD>::kGroups;
    const SplitWeights w;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[8 * st + e];
        u32x4 bh, bm, bl;
        split8(x, w, bh, bm, bl);
#pragma unroll
        for (int tp = 0; tp < G; tp += 2) {
            float v0[8], v1[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 f = *reinterpret_cast<const float2*>(
                    vs + dgk::key_of(8 * st + e, half) * HD + l32 * G + tp);
                v0[e] = f.x;
                v1[e] = f.y;
            }
            u32x4 ah, am, al;
            split8(v0, w, ah, am, al);
            mfma_bf16x6(ah, am, al, bh, bm, bl, o[tp], o[tp]);
            split8(v1, w, ah, am, al);
            mfma_bf16x6(ah, am, al, bh, bm, bl, o[tp + 1], o[tp + 1]);
        }
    }
}

}  // namespace bf3
