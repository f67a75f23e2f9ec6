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

// bf16 V tiles sit in LDS row-major with each row's 16-byte chunks permuted, chunk c of key row
// k at position c ^ vswz(k): the 8 rows a wavefront's transposed reads touch at once (4 per
// lane half) then cover all 64 banks twice instead of 16 banks eight times.
template <int HD>
__device__ inline int vswz(int row) {
    return HD == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// O^T += V^T P^T from a bf16 V tile (as stored, or a plane of a split f32 tile).  Step st takes
// the 16 keys whose probabilities are the lane's registers p[8*st .. 8*st + 7] (keys
// dgk::key_of(r, half)), so the B operand is those registers split in three.  The A operand of
// output group t holds, for the lane's head element 32*t + l32, the same 16 keys; two
// ds_read_b64_tr_b16 fetch it straight from the row-major tile (vtr_offsets gives the lane's
// addresses).
// That instruction hands out, within each 16 lanes, element j%4 of the 8 bytes addressed by lane
// 4*e + j/4 as element e of lane j: so lane 4*e + c of a 16-lane group addresses key row
// (4*half + e) (plus 8 for the second read) at head elements 32*t + 16*((lane/16)%2) + 4*c.
// Output rows are therefore head elements 32*t + key_of(r, half): stage_row_blocked.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int HD>
__device__ inline void vtr_offsets(int lane, int (&off)[dgk::Tile<HD>::kGroups]) {
    const int j = lane & 15, e = j >> 2, c = j & 3, sg = (lane >> 4) & 1, half = lane >> 5;
    const int row = 4 * half + e;
#pragma unroll
    for (int t = 0; t < dgk::Tile<HD>::kGroups; ++t)
        off[t] = row * HD * 2 + 16 * ((4 * t + 2 * sg + (c >> 1)) ^ vswz<HD>(row)) + 8 * (c & 1);
}

// f32 K/V tiles split once per stage into bf16 planes.  The workgroup turns each staged f32
// tile (plain rows, so each load of the stage is a scalar offset from the last) into three bf16
// tiles hi, mid, lo: K rows with chunk c of row k at position c ^ (k mod HD/8), V rows permuted
// by vswz.  Every wavefront then reads ready MFMA operands, and the split is done once per
// element instead of once per element and query group.
template <int HD>
struct Planes {
    static constexpr int kBytes = dgk::kKeys * HD * 2;   // one bf16 plane of a tile
    static constexpr int kOct = HD / 8;                   // 8-element groups per row
    // plane p of the K (isv 0) or V (isv 1) tile `tile`
    __device__ static char* at(char* base, int tile, int isv, int p) {
        return base + ((tile * 2 + isv) * 3 + p) * kBytes;
    }
};

// The staged tile `tile` has its K at stage + 2*tile*slot_bytes and its V one slot further.
// kThreads threads (tid < kThreads) split up to kMaxTiles tiles, of which the first ntile are
// present.
template <int HD, int kThreads, int kMaxTiles>
__device__ inline void split_stage(const char* __restrict__ stage, int slot_bytes,
                                   char* __restrict__ planes, int ntile, int tid) {
    using P = Planes<HD>;
    constexpr int kPerTile = 2 * dgk::kKeys * P::kOct;    // K and V items of one tile
    static_assert(kMaxTiles * kPerTile % kThreads == 0, "whole passes");
    const SplitWeights w;
#pragma unroll
    for (int i = 0; i < kMaxTiles * kPerTile / kThreads; ++i) {
        const int it = tid + kThreads * i;
        const int tile = it / kPerTile;
        if (tile >= ntile) continue;   // uniform per iteration: whole tiles are absent
        const int o = it % P::kOct, r = (it / P::kOct) % dgk::kKeys;
        const int isv = (it / (P::kOct * dgk::kKeys)) & 1;
        const float* row = reinterpret_cast<const float*>(stage + (tile * 2 + isv) * slot_bytes) + r * HD;
        const float4 x0 = *reinterpret_cast<const float4*>(row + 8 * o);
        const float4 x1 = *reinterpret_cast<const float4*>(row + 8 * o + 4);
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        u32x4 h, m, l;
        split8(x, w, h, m, l);
        const int pos = o ^ (isv ? vswz<HD>(r) : r % P::kOct);
        char* dst = P::at(planes, tile, isv, 0) + r * HD * 2 + 16 * pos;
        *reinterpret_cast<u32x4*>(dst) = h;
        *reinterpret_cast<u32x4*>(dst + P::kBytes) = m;
        *reinterpret_cast<u32x4*>(dst + 2 * P::kBytes) = l;
    }
}

// S^T += K Q^T from the three K planes of a tile; q in the load_q_bf16x3 layout.
template <int HD>
__device__ inline f32x16 scores_planes(const char* __restrict__ kp, int l32, int half,
                                       const QSplit<HD>& q, f32x16 s) {
    using P = Planes<HD>;
    const char* kr = kp + l32 * HD * 2;
    const int sw = l32 % P::kOct;
    f32x16 d = {};
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        const int off = 16 * ((2 * st + half) ^ sw);
        const u32x4 kh = *reinterpret_cast<const u32x4*>(kr + off);
        const u32x4 km = *reinterpret_cast<const u32x4*>(kr + P::kBytes + off);
        const u32x4 kl = *reinterpret_cast<const u32x4*>(kr + 2 * P::kBytes + off);
        mfma_bf16x6(kh, km, kl, q.h[st], q.m[st], q.l[st], s, d);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += d[r];
    return s;
}

// O^T += V^T P^T from the three V planes of a tile (layout and reads as accumulate_pv_bf16x3).
template <int HD>
__device__ inline void accumulate_pv_planes(const char* __restrict__ vp,
                                            const int (&off)[dgk::Tile<HD>::kGroups],
                                            const f32x16& p, f32x16 (&o)[dgk::Tile<HD>::kGroups]) {
    constexpr int G = dgk::Tile<HD>::kGroups, PB = Planes<HD>::kBytes;
    const SplitWeights w;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[8 * st + e];
        u32x4 bh, bm, bl;
        split8(x, w, bh, bm, bl);
#pragma unroll
        for (int t = 0; t < G; ++t) {
            u32x4 a[3];
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) {
                const char* r0 = vp + pl * PB + st * 16 * HD * 2 + off[t];
                const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r0));
                const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r0 + 8 * HD * 2));
                const uint2 u0 = __builtin_bit_cast(uint2, x0), u1 = __builtin_bit_cast(uint2, x1);
                a[pl] = u32x4{u0.x, u0.y, u1.x, u1.y};
            }
            mfma_bf16x6(a[0], a[1], a[2], bh, bm, bl, o[t], o[t]);
        }
    }
}

// dgk::stage_row for the bf16 path's output layout (row m of group t is head element 32*t + m).
template <int HD>
__device__ inline void stage_row_blocked(float* __restrict__ rows, int l32, float scale,
                                         const f32x16 (&o)[dgk::Tile<HD>::kGroups], int half) {
    float* dst = rows + l32 * (HD + 4) + 4 * half;
#pragma unroll
    for (int t = 0; t < dgk::Tile<HD>::kGroups; ++t)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<float4*>(dst + 32 * t + 8 * rb) =
                make_float4(o[t][4 * rb] * scale, o[t][4 * rb + 1] * scale,
                            o[t][4 * rb + 2] * scale, o[t][4 * rb + 3] * scale);
}

}  // namespace bf3
