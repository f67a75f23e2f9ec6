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
// for each.  Here a workgroup of 8 wavefronts owns 128 query vectors of ONE kv head -- the
// G = nh/nkv q heads of a group times a block of canvas rows, flattened as (row, head-in-group)
// so they are contiguous in q and out.  Its 8 wavefronts form 4 pairs; both wavefronts of a
// pair hold the same 32 queries and take alternate 32-key tiles, so the block walks the keys in
// stages of 64.  Each stage's K and V tiles are fetched once into LDS for all 128 queries with
// direct global->LDS loads, so the next stage streams in while this one is computed; a tile
// lying wholly in the cache or wholly in the canvas is addressed from a scalar base, and only a
// tile across the seam (or the end of the keys) forms per-row addresses.  Scores and the value
// product run on the bf16 matrix pipe: f32 K/V land in one staging buffer, the workgroup splits
// each stage once into three bf16 planes (six bf16 products per f32 product; kF32OnBf16 below,
// whose false setting keeps the double-buffered f32 MFMA path of flash_core.hpp), and 16-bit
// K/V stages are double-buffered as stored.  At the end each pair merges its two partial
// softmax states through LDS, and the workgroup writes its rows out whole.
//
// dg_attn_split_gqa_qnorm takes the raw q projection instead and applies the q dispatch of
// DG_HEADNORM_ROPE (RMSNorm, weight, NeoX rope) to the workgroup's query vectors as it stages
// them in LDS before the first stage, so q never makes the extra round trip through HBM; q
// itself is left unchanged.
//
// dg_attn_split_gqa_qkvnorm also takes the raw k and v projections: the k dispatch (norm,
// weight, rope) and the weightless v dispatch run on each canvas tile after it lands in LDS and
// before any wavefront reads it, so neither makes a round trip through HBM either.  Its splits
// deal the key tiles round robin, which spreads the canvas tiles (and their norm work) over the
// workgroups of a kv head.
//
// The 16-bit K/V variants read cache and canvas rows stored as f16 or bf16.  f16 elements are
// widened to f32 as they are read from LDS and run the f32 MFMA path; bf16 tiles run both
// products on the bf16 matrix pipe, with the f32 operand taken as three bf16 terms.
//
// Shapes with too few workgroups to fill the GPU also split the key range, in whole 32-key
// tiles, across workgroups ("split-KV"): each writes an unnormalised partial (max,
// denominator, output) to the caller's workspace and a second kernel merges them.  Workgroups
// that share K/V are placed on the same XCD so its L2 serves the re-reads.
#include <mutex>

#include "bf16x3.hpp"
#include "dg_common.hpp"
#include "flash_core.hpp"

namespace {

using namespace bf3;
using dgk::f32x16;
constexpr int kWaves = 8;
constexpr int kPairs = 4;
constexpr int kBlockQ = kPairs * dgk::kQuery;  // query vectors per workgroup
constexpr int kStage = 2 * dgk::kKeys;         // keys per stage (one tile per pair member)

struct SplitArgs {
    const float* q;
    const float* kc;
    const float* vc;
    const float* k;
    const float* v;
    float* out;
    float* ws;         // split-KV partials: o [nsplit][nqtot][hd], m [nsplit][nqtot], l [...]
    size_t nqtot;      // batch * T * nh query vectors
    int hd;            // head dim (a multiple of 4; the tile width HD is 64 or 128)
    int T, ctx, nh, nkv, G;
    int qblocks;       // workgroups per (batch, kv head, split)
    int nsplit;        // key-range splits
    int nblocks;       // total workgroups
    int nxcd;          // XCDs of the device (workgroup placement)
    float qmul;        // scale * log2(e)
    int causal;
    const float* wq;   // q norm weight [hd] (qnorm entry with WEIGHTED)
    const float* wk;   // k norm weight [hd] (qkvnorm entry with WEIGHTED)
    const float* cs;   // rope table [T, 2*hd] (qnorm entry with ROPE)
    unsigned qflags;   // DG_NORM_* bits of the q norm (and of the k norm in the qkvnorm entry)
    float eps;
};

// K/V element storage: 0 = f32, DG_KV_F16, DG_KV_BF16.  16-bit tiles are loaded into LDS as
// they are stored (half the bytes of a stage).  f16 operands are widened to f32 in registers as
// they are read, so that arithmetic is the f32 path's; bf16 tiles feed bf16 MFMAs directly.
template <int HD, int kKV>
struct KVTile {
    static constexpr int kEsz = kKV ? 2 : 4;                  // bytes per element
    static constexpr int kChunks = HD * kEsz / 16;            // 16-byte chunks per key row
    static constexpr int kBytes = dgk::kKeys * HD * kEsz;     // one K or V tile
    static constexpr int kRowsPerLoad = 64 / kChunks;         // key rows per wave-wide 1 KiB load
    static constexpr int kLoadsPerTile = dgk::kKeys / kRowsPerLoad;
};

// Where the key rows of a K tile sit in LDS.  f32 tiles at HD 128 are padded: wave-wide load i
// fills key rows i and i + 16 (512 bytes each) and loads start 1040 bytes apart.  Chunk c of
// rows 0..15 (likewise of rows 16..31) then lies in 16 different 16-byte bank groups, so the 32
// lanes reading one chunk of 32 rows do not collide, and a lane's K reads are its row base
// plus a constant: no per-chunk address arithmetic.  The other tiles (HD 64, whose loads hold
// four rows each, and 16-bit rows) are plain row-major with each row's 16-byte chunks
// permuted, chunk c of row k at position c ^ (k mod chunks-per-row).
template <int HD, int kKV>
struct KLayout {
    using KT = KVTile<HD, kKV>;
    static constexpr bool kPadded = HD == 128 && kKV == 0;
    static constexpr int kLoadBytes = kPadded ? 1040 : 1024;
    static constexpr int kSlotBytes = KT::kLoadsPerTile * kLoadBytes;   // one K or V tile slot
    // Byte offset of key row `trow` (and of its chunk 0) in a K tile.
    __device__ static int row(int trow) {
        return kPadded ? (trow & 15) * kLoadBytes + (trow >> 4) * 512 : trow * HD * KT::kEsz;
    }
};

// dgk::scores_from on a padded f32 K tile: the lane's chunks 2g + half are 32 bytes apart.
template <int HD>
__device__ inline f32x16 scores_padded(const char* __restrict__ ks, int l32, int half,
                                       const float (&qreg)[HD / 2], f32x16 s) {
    const float* kr = reinterpret_cast<const float*>(ks + KLayout<HD, 0>::row(l32)) + 4 * half;
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

template <int kKV>
__device__ inline float lo16(uint32_t w) {
    if constexpr (kKV == DG_KV_BF16) return __uint_as_float(w << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

template <int kKV>
__device__ inline float hi16(uint32_t w) {
    if constexpr (kKV == DG_KV_BF16) return __uint_as_float(w & 0xffff0000u);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// dgk::scores_from on a 16-bit K tile: chunk g of a row holds elements 8g..8g+7, so the lane's
// elements 8g+4*half..+3 are the 8 bytes at offset 8*half of chunk g (swizzled like f32 rows).
template <int HD, int kKV>
__device__ inline f32x16 scores_from16(const char* __restrict__ ks, int l32, int half,
                                       const float (&qreg)[HD / 2], f32x16 s) {
    using KT = KVTile<HD, kKV>;
    const char* kr = ks + l32 * HD * 2;
    const int sw = l32 % KT::kChunks;
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        const uint2 w = *reinterpret_cast<const uint2*>(kr + 16 * (g ^ sw) + 8 * half);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(lo16<kKV>(w.x), qreg[4 * g + 0], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(hi16<kKV>(w.x), qreg[4 * g + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(lo16<kKV>(w.y), qreg[4 * g + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(hi16<kKV>(w.y), qreg[4 * g + 3], s, 0, 0, 0);
    }
    return s;
}

// dgk::accumulate_pv on a 16-bit V tile: the lane's G = HD/32 contiguous elements of a row are
// 2G bytes.
template <int HD, int kKV>
__device__ inline void accumulate_pv16(const char* __restrict__ vs, int l32, int half,
                                       const f32x16& p, f32x16 (&o)[dgk::Tile<HD>::kGroups]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const char* vr = vs + (dgk::key_of(r, half) * HD + l32 * dgk::Tile<HD>::kGroups) * 2;
        if constexpr (HD == 128) {
            const uint2 w = *reinterpret_cast<const uint2*>(vr);
            o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(lo16<kKV>(w.x), p[r], o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(hi16<kKV>(w.x), p[r], o[1], 0, 0, 0);
            o[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(lo16<kKV>(w.y), p[r], o[2], 0, 0, 0);
            o[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(hi16<kKV>(w.y), p[r], o[3], 0, 0, 0);
        } else {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(vr);
            o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(lo16<kKV>(w), p[r], o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(hi16<kKV>(w), p[r], o[1], 0, 0, 0);
        }
    }
}

// f32 K/V on the bf16 pipe.  With both operands split exactly in three terms, a = ah + am + al
// and b = bh + bm + bl, the product a*b is taken as the six terms down to order 2^-16 (ah*bh,
// ah*bm, am*bh, ah*bl, al*bh, am*bm); the dropped ones (am*bl, al*bm, al*bl) leave each product
// within 2^-23 |a||b| and typically within 2^-29, where f32 rounds a product by up to 2^-24
// (median 2^-25.5), so the result stays on the f32 bar.  Six v_mfma_f32_32x32x16_bf16 per
// step are 2.7 times less matrix-pipe time than v_mfma_f32_32x32x2f32.  The K and V tiles are
// split once per stage by the whole workgroup (split_stage), q once per wavefront, and the
// probabilities per tile (7 vector instructions per pair of values).  false: f32 MFMA.
constexpr bool kF32OnBf16 = true;

// S^T += K Q^T from a bf16 K tile (rows of HD elements, 16-byte chunks swizzled as in
// scores_from16): step st reads chunk 2*st + half of the lane's key row, 8 elements at once.
template <int HD>
__device__ inline f32x16 scores_bf16x3(const char* __restrict__ ks, int l32, int half,
                                       const QSplit<HD>& q, f32x16 s) {
    const char* kr = ks + l32 * HD * 2;
    const int sw = l32 % (HD / 8);
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        const bf16x8 k = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * ((2 * st + half) ^ sw)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, as_bf16x8(q.h[st]), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, as_bf16x8(q.m[st]), s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, as_bf16x8(q.l[st]), s, 0, 0, 0);
    }
    return s;
}

// O^T += V^T P^T from a bf16 V tile as stored (rows permuted by vswz), read transposed at the
// vtr_offsets addresses.
template <int HD>
__device__ inline void accumulate_pv_bf16x3(const char* __restrict__ vs, const int (&off)[dgk::Tile<HD>::kGroups],
                                            const f32x16& p, f32x16 (&o)[dgk::Tile<HD>::kGroups]) {
    constexpr int G = dgk::Tile<HD>::kGroups;
    const SplitWeights w;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        u32x4 bh, bm, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned th, tm, tl;
            split_bf16x3(p[8 * st + 2 * i], p[8 * st + 2 * i + 1], w, th, tm, tl);
            bh[i] = th;
            bm[i] = tm;
            bl[i] = tl;
        }
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const char* r0 = vs + st * 16 * HD * 2 + off[t];
            const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r0));
            const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r0 + 8 * HD * 2));
            const uint2 u0 = __builtin_bit_cast(uint2, x0), u1 = __builtin_bit_cast(uint2, x1);
            const bf16x8 av = as_bf16x8(u32x4{u0.x, u0.y, u1.x, u1.y});
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, as_bf16x8(bh), o[t], 0, 0, 0);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, as_bf16x8(bm), o[t], 0, 0, 0);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, as_bf16x8(bl), o[t], 0, 0, 0);
        }
    }
}

using dg::group_sum;

// Row stride (floats) of the normalised queries staged in LDS: HD + 4 keeps the 16-byte
// operand reads (32 lanes on 32 different rows) free of bank conflicts.
template <int HD>
constexpr int kQStride = HD + 4;

// The q dispatch of DG_HEADNORM_ROPE for the workgroup's QN query vectors, written to LDS
// rows qs[v][kQStride] (pre-multiplied by scale*log2(e), zero past hd and for vectors past the
// end) for the dgk::load_q layout to read back.  Row-oriented, so every global access is
// coalesced: 8 lanes share one query vector, lane c holding its float4 chunks c, c+8, c+16 and
// c+24; a wave covers 8 vectors per pass, and the sum of squares takes 3 lane exchanges.  The
// rope partner of element e (e +- hd/2, any even hd) is read back from the staged row, which
// the same wavefront wrote (LDS accesses of one wavefront complete in order).
//
// kQPlanes (hd == HD, the bf16 pipe): the vectors are written instead as three bf16 planes,
// split once here rather than by both wavefronts of a pair, for load_q_planes to read back.
// Plane p holds row v at qs + (p * QN + v) * HD bf16, its 16-byte chunk j (elements 8j..8j+7)
// at position j ^ (v mod HD/8), so the 32 rows a wavefront reads at once spread over all banks.
// The rope partner of chunk k is the lane's own chunk k ^ (HD/64): hd/2 is 8 chunks of 4
// elements away.
template <int HD>
constexpr int kQPlaneBytes = kBlockQ * HD * 2;   // one bf16 plane of the workgroup's queries

template <int HD, int QN = kBlockQ, bool kQPlanes = false>
__device__ inline void stage_q_normed(const SplitArgs& a, float* __restrict__ qs, int b, int kv,
                                      int qb, int wave, int lane, int hd) {
    constexpr int kPerLane = HD / 32;  // float4 chunks per lane
    const int sub = lane >> 3, c = lane & 7;
    const int nq = a.T * a.G;
    const bool norm = !(a.qflags & DG_NORM_SKIP);
    const bool weighted = norm && (a.qflags & DG_NORM_WEIGHTED);
    const bool rope = (a.qflags & DG_NORM_ROPE) != 0;
    const int half_hd = hd >> 1;
    float4 w[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int e0 = 4 * (c + 8 * k);
        w[k] = weighted && e0 < hd ? *reinterpret_cast<const float4*>(a.wq + e0)
                                   : make_float4(1.f, 1.f, 1.f, 1.f);
    }
    // Lane group g (8 lanes) takes vectors kPasses*g + pass, consecutive vectors in successive
    // passes: with an even G they are heads of one canvas row, and the row's cos|sin entries,
    // loaded in the first pass, serve the next as well (half the table reads of the burst
    // that opens every workgroup).
    constexpr int kPasses = QN / (8 * kWaves);
    static_assert(kPasses >= 1 && QN % (8 * kWaves) == 0, "whole passes of 8 vectors per wave");
    float4 co[kPerLane], si[kPerLane];
    int cs_row = -1;   // canvas row whose entries co/si hold
#pragma unroll 1
    for (int pass = 0; pass < kPasses; ++pass) {
        const int vloc = (wave * 8 + sub) * kPasses + pass;
        const int qv = qb * QN + vloc;
        const bool valid = qv < nq;
        const int row = valid ? qv / a.G : 0;
        const int hq = kv * a.G + (valid ? qv % a.G : 0);
        const float* qrow = a.q + (((size_t)b * a.T + row) * a.nh + hq) * hd;
        float* srow = qs + vloc * kQStride<HD>;
        float4 x[kPerLane];
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int e0 = 4 * (c + 8 * k);
            x[k] = valid && e0 < hd ? *reinterpret_cast<const float4*>(qrow + e0)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            ss += x[k].x * x[k].x + x[k].y * x[k].y + x[k].z * x[k].z + x[k].w * x[k].w;
        }
        ss = group_sum<8>(ss);
        const float inv = norm ? (valid ? 1.0f / sqrtf(ss / (float)hd + a.eps) : 0.0f) : 1.0f;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            x[k].x = x[k].x * inv * w[k].x;
            x[k].y = x[k].y * inv * w[k].y;
            x[k].z = x[k].z * inv * w[k].z;
            x[k].w = x[k].w * inv * w[k].w;
        }
        if (rope) {
            if constexpr (!kQPlanes) {
#pragma unroll
                for (int k = 0; k < kPerLane; ++k)
                    *reinterpret_cast<float4*>(srow + 4 * (c + 8 * k)) = x[k];
            }
            if (row != cs_row) {   // the same for the 8 lanes of a vector
                const float* cr = a.cs + (size_t)row * 2 * hd;
#pragma unroll
                for (int k = 0; k < kPerLane; ++k) {
                    const int e0 = 4 * (c + 8 * k);
                    co[k] = e0 < hd ? *reinterpret_cast<const float4*>(cr + e0)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                    si[k] = e0 < hd ? *reinterpret_cast<const float4*>(cr + hd + e0)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                cs_row = row;
            }
            float part[kPerLane][4];
            if constexpr (kQPlanes) {
#pragma unroll
                for (int k = 0; k < kPerLane; ++k) {
                    const float4 pk = x[k ^ (kPerLane / 2)];
                    part[k][0] = pk.x; part[k][1] = pk.y; part[k][2] = pk.z; part[k][3] = pk.w;
                }
            } else {
#pragma unroll
                for (int k = 0; k < kPerLane; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * (c + 8 * k) + i;
                        const int pe = e < half_hd ? e + half_hd : e - half_hd;
                        part[k][i] = e < hd ? srow[pe] : 0.0f;
                    }
            }
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const int e0 = 4 * (c + 8 * k);
                if (e0 < hd) {
                    const float y[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
                    const float cc[4] = {co[k].x, co[k].y, co[k].z, co[k].w};
                    const float sn[4] = {si[k].x, si[k].y, si[k].z, si[k].w};
                    float r[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float rot = e0 + i < half_hd ? -part[k][i] : part[k][i];
                        r[i] = y[i] * cc[i] + rot * sn[i];
                    }
                    x[k] = make_float4(r[0], r[1], r[2], r[3]);
                }
            }
        }
        if constexpr (kQPlanes) {
            const SplitWeights sw;
            char* prow = reinterpret_cast<char*>(qs) + vloc * HD * 2;
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const int ch = c + 8 * k;   // 4-element chunk: half ch & 1 of 16-byte chunk ch >> 1
                unsigned h0, m0, l0, h1, m1, l1;
                split_bf16x3(x[k].x * a.qmul, x[k].y * a.qmul, sw, h0, m0, l0);
                split_bf16x3(x[k].z * a.qmul, x[k].w * a.qmul, sw, h1, m1, l1);
                char* dst = prow + 16 * ((ch >> 1) ^ (vloc % (HD / 8))) + 8 * (ch & 1);
                *reinterpret_cast<uint2*>(dst) = make_uint2(h0, h1);
                *reinterpret_cast<uint2*>(dst + kQPlaneBytes<HD>) = make_uint2(m0, m1);
                *reinterpret_cast<uint2*>(dst + 2 * kQPlaneBytes<HD>) = make_uint2(l0, l1);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k)
                *reinterpret_cast<float4*>(srow + 4 * (c + 8 * k)) =
                    make_float4(x[k].x * a.qmul, x[k].y * a.qmul, x[k].z * a.qmul, x[k].w * a.qmul);
        }
    }
}

// The lane's query operand (the load_q_bf16x3 layout) from the planes stage_q_normed<kQPlanes>
// wrote: row v, step st reads 16-byte chunk 2*st + half of each plane.
template <int HD>
__device__ inline void load_q_planes(const char* __restrict__ qp, int v, int half, QSplit<HD>& q) {
    const char* row = qp + v * HD * 2;
    const int sw = v % (HD / 8);
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
        const char* src = row + 16 * ((2 * st + half) ^ sw);
        q.h[st] = *reinterpret_cast<const u32x4*>(src);
        q.m[st] = *reinterpret_cast<const u32x4*>(src + kQPlaneBytes<HD>);
        q.l[st] = *reinterpret_cast<const u32x4*>(src + 2 * kQPlaneBytes<HD>);
    }
}

// The k and v dispatches of DG_HEADNORM_ROPE on the canvas rows of one stage tile pair in LDS,
// in place (dg_attn_split_gqa_qkvnorm): a K row gets the norm, the weight and the rope of its
// canvas row (the q flags), a V row the weightless, un-roped norm.  Cache rows (key < ctx) are
// stored normalised and left alone; rows past the end of the keys hold a copy of the last key
// and are normalised like it.  L = HD/8 lanes share a row, lane c holding chunks c and c + L,
// so for the exact widths the rope partner chunk (hd/2 away) is in the same lane; padded widths
// read it back from the row, which the same wavefront wrote.  The 64 rows (32 K, then 32 V)
// go in passes of 512/L rows (one at HD 64; at HD 128 the K rows, then the V rows, which need
// no table loads), kept apart so that few registers are live beside the attention state.
// Chunks past hd keep their raw copies (they meet zero query elements, or fill output
// elements that are never stored).
template <int HD, bool kPad, bool kPadK = KLayout<HD, 0>::kPadded, bool kSwzK = true>
__device__ inline void norm_canvas_tile(const SplitArgs& a, float* __restrict__ kt,
                                        float* __restrict__ vt, int j0, int kend, int wave,
                                        int lane, int hd) {
    constexpr int kChunks = HD / 4, L = HD / 8, kRowsPerPass = 512 / L;
    const int c = lane % L;
#pragma unroll 1
    for (int r0 = 0; r0 < 2 * dgk::kKeys; r0 += kRowsPerPass) {
        const int R = r0 + wave * (64 / L) + lane / L;
        const bool isv = R >= dgk::kKeys;        // wave-uniform
        const int trow = R % dgk::kKeys;
        const int j = min(j0 + trow, kend - 1);
        if (j < a.ctx) continue;                 // a cache row; its L lanes leave together
        using KL = KLayout<HD, 0>;
        float* rowp = isv ? vt + trow * HD : kt + (kPadK ? KL::row(trow) / 4 : trow * HD);
        // K rows of unpadded tiles are stored chunk-swizzled
        const int sw = isv || kPadK || !kSwzK ? 0 : trow % kChunks;
        float4 x[2];
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int ch = c + L * k;
            x[k] = !kPad || 4 * ch < hd ? *reinterpret_cast<const float4*>(rowp + 4 * (ch ^ sw))
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
            ss += x[k].x * x[k].x + x[k].y * x[k].y + x[k].z * x[k].z + x[k].w * x[k].w;
        }
        ss = group_sum<L>(ss);
        const float inv = 1.0f / sqrtf(ss / (float)hd + a.eps);
        const bool weighted = !isv && (a.qflags & DG_NORM_WEIGHTED);
        const bool rope = !isv && (a.qflags & DG_NORM_ROPE);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int ch = c + L * k;
            const float4 w = weighted && (!kPad || 4 * ch < hd)
                                 ? *reinterpret_cast<const float4*>(a.wk + 4 * ch)
                                 : make_float4(1.f, 1.f, 1.f, 1.f);
            x[k] = make_float4(x[k].x * inv * w.x, x[k].y * inv * w.y, x[k].z * inv * w.z,
                               x[k].w * inv * w.w);
        }
        if (rope) {
            const int half_hd = hd >> 1;
            const float* cr = a.cs + (size_t)(j - a.ctx) * 2 * hd;
            float4 part[2];
            if constexpr (!kPad) {
                part[0] = x[1];
                part[1] = x[0];
            } else {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int ch = c + L * k;
                    if (4 * ch < hd) *reinterpret_cast<float4*>(rowp + 4 * (ch ^ sw)) = x[k];
                }
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    float pv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * (c + L * k) + i;
                        const int pe = e < half_hd ? e + half_hd : e - half_hd;
                        pv[i] = e < hd ? rowp[4 * ((pe >> 2) ^ sw) + (pe & 3)] : 0.0f;
                    }
                    part[k] = make_float4(pv[0], pv[1], pv[2], pv[3]);
                }
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int e0 = 4 * (c + L * k);
                if (kPad && e0 >= hd) continue;
                const float4 co = *reinterpret_cast<const float4*>(cr + e0);
                const float4 si = *reinterpret_cast<const float4*>(cr + hd + e0);
                const float y[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
                const float p[4] = {part[k].x, part[k].y, part[k].z, part[k].w};
                const float cc[4] = {co.x, co.y, co.z, co.w}, sn[4] = {si.x, si.y, si.z, si.w};
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float rot = e0 + i < half_hd ? -p[i] : p[i];
                    r[i] = y[i] * cc[i] + rot * sn[i];
                }
                x[k] = make_float4(r[0], r[1], r[2], r[3]);
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int ch = c + L * k;
            if (!kPad || 4 * ch < hd) *reinterpret_cast<float4*>(rowp + 4 * (ch ^ sw)) = x[k];
        }
    }
}

using dg::xcd_remap;

// kPad: the head dim hd is narrower than the HD-wide tile (hd < HD, a multiple of 4).  Queries
// are zero past hd; key/value rows are loaded with their chunks past hd taken from a valid
// chunk of the same row (finite values that meet zero query elements, and output elements
// past hd that are never stored).
// kNormKV (with kNormQ): k and v arrive raw; each stage that holds canvas rows normalises them
// in LDS (norm_canvas_tile) before they are read.  Split-KV then deals the tiles round robin
// (split s takes tiles s, s + nsplit, ...), so the canvas tiles, and that work, spread evenly
// over the splits instead of falling to the last ones.
template <int HD, bool kNormQ, bool kNormKV, bool kPad, int kKV>
__global__ void __launch_bounds__(512) attn_split_gqa_kernel(SplitArgs a) {
    using TL = dgk::Tile<HD>;
    using KT = KVTile<HD, kKV>;
    // [buffer][tile of the stage][K, V]; with kNormQ the normalised queries are staged over
    // buffer 1 (free until the second stage is issued) and a little past it; the pair merge
    // reuses the space at the end.
    using KL = KLayout<HD, kKV>;
    // kPlanes (f32 K/V on the bf16 pipe): one staging buffer [tile][K, V] of plain f32 tiles,
    // then the bf16 planes [tile][K, V][hi, mid, lo] the split writes; the
    // normalised queries are staged over the planes, which are free until the first split.
    constexpr bool kPlanes = kKV == 0 && kF32OnBf16;
    constexpr bool kPadK = KL::kPadded && !kPlanes;
    constexpr int kSlot = kPlanes ? KT::kBytes : KL::kSlotBytes;
    constexpr int kPlanesOff = 2 * 2 * kSlot;
    constexpr int kStageFloats = kPlanes ? (kPlanesOff + 2 * 2 * 3 * Planes<HD>::kBytes) / 4
                                         : 2 * 2 * 2 * KL::kSlotBytes / 4;
    constexpr int kQOff = kPlanes ? kPlanesOff / 4 : 2 * 2 * KL::kSlotBytes / 4;
    constexpr int kQStageEnd = kQOff + kBlockQ * kQStride<HD>;
    constexpr int kMergeFloats = kPairs * 64 * (TL::kGroups * 16 + 2) + 2 * kBlockQ;  // + row indices
    constexpr int kA = kNormQ && kQStageEnd > kStageFloats ? kQStageEnd : kStageFloats;
    constexpr int kSmemFloats = kA > kMergeFloats ? kA : kMergeFloats;
    __shared__ __attribute__((aligned(16))) float smem[kSmemFloats];
    const int hd = kPad ? a.hd : HD;
    auto tile_ptr = [&](int buf, int tile, int isv) {
        return reinterpret_cast<char*>(smem) + ((buf * 2 + tile) * 2 + isv) * kSlot;
    };
    char* const planes = reinterpret_cast<char*>(smem) + kPlanesOff;

    const int lid = xcd_remap(blockIdx.x, a.nblocks, a.nxcd);
    const int qb = lid % a.qblocks;
    const int rest = lid / a.qblocks;
    const int split = rest % a.nsplit;
    const int bk = rest / a.nsplit;           // b * nkv + kv
    const int kv = bk % a.nkv;
    const int b = bk / a.nkv;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int pair = wave & (kPairs - 1), hi = wave >> 2;

    const int nq = a.T * a.G;                 // query vectors of this (b, kv)
    const int qfirst = qb * kBlockQ + pair * dgk::kQuery;
    const int qv = qfirst + l32;
    const bool valid = qv < nq;
    const int row = valid ? qv / a.G : 0;
    const int hq = kv * a.G + (valid ? qv % a.G : 0);
    const size_t gq = ((size_t)b * a.T + row) * a.nh + hq;   // global query vector index
    const bool pair_active = qfirst < nq;
    const int row_min = pair_active ? qfirst / a.G : 0;

    const int S = a.ctx + a.T;
    int kend = S;
    if (a.causal) {  // no query of this block sees canvas keys past its last row
        const int last = min(nq - 1, qb * kBlockQ + kBlockQ - 1) / a.G;
        kend = min(S, a.ctx + last + 1);
    }
    // Splits divide the key range in whole kKeys-key tiles, so the splits of a launch differ by
    // at most one tile (stages take two tiles; a split's last stage may hold only one).
    const int ntile = (kend + dgk::kKeys - 1) / dgk::kKeys;
    const int tile_begin = (int)((long long)split * ntile / a.nsplit);
    const int tile_end = (int)((long long)(split + 1) * ntile / a.nsplit);
    const int kbeg = tile_begin * dgk::kKeys;   // this split's keys: [kbeg, kend)
    int ntl;                                    // tiles of this split
    if constexpr (kNormKV) {                    // round robin: tiles split, split + nsplit, ...
        ntl = split < ntile ? (ntile - split + a.nsplit - 1) / a.nsplit : 0;
    } else {
        kend = min(kend, tile_end * dgk::kKeys);
        ntl = tile_end - tile_begin;
    }
    const int nst = (ntl + 1) / 2;
    // First key of tile t (0 or 1) of stage st; a key at or past kend means the tile is absent.
    auto key0 = [&](int st, int t) {
        if constexpr (kNormKV) return (split + a.nsplit * (2 * st + t)) * dgk::kKeys;
        else return kbeg + st * kStage + t * dgk::kKeys;
    };

    constexpr int kEsz = KT::kEsz;
    constexpr bool kBf16 = kKV == DG_KV_BF16;    // both contractions on the bf16 pipe
    const char* kcb = reinterpret_cast<const char*>(a.kc) + (size_t)bk * a.ctx * hd * kEsz;
    const char* vcb = reinterpret_cast<const char*>(a.vc) + (size_t)bk * a.ctx * hd * kEsz;
    const size_t cstride = (size_t)a.nkv * hd;   // canvas row stride, elements
    const char* kb = reinterpret_cast<const char*>(a.k) + ((size_t)b * a.T * a.nkv + kv) * hd * kEsz;
    const char* vb = reinterpret_cast<const char*>(a.v) + ((size_t)b * a.T * a.nkv + kv) * hd * kEsz;

    // The four even-tile wavefronts issue the stage's 4 * kLoadsPerTile wave-wide loads (K and
    // V of both tiles); their odd-tile partners start on the MFMAs meanwhile (on this hardware
    // vector and scalar instructions do not overlap the f32 matrix pipe, so one member of each
    // SIMD pair keeps it fed).  A tile lying wholly in the cache or wholly in the canvas is
    // addressed from a scalar base plus a loop-invariant per-lane offset; only a tile that
    // straddles the seam or the end of the key range forms per-lane addresses.
    constexpr int kLoadsPerWave = 4 * KT::kLoadsPerTile / (kWaves / 2);
    constexpr int R = KT::kRowsPerLoad;
    const int pos = lane % KT::kChunks, rsub = lane / KT::kChunks;
    const unsigned rstride_c = (unsigned)hd * kEsz, rstride_v = (unsigned)cstride * kEsz;
    // Each issuing wavefront fills one part of the stage -- K0, V0, K1 or V1, part = pair --
    // with all kLoadsPerTile wave-wide loads of that tile, so which address form applies is
    // decided once per stage, outside the loads.
    static_assert(kLoadsPerWave == KT::kLoadsPerTile, "one tile part per issuing wavefront");
    const int ld_tile = pair >> 1, ld_isv = pair & 1;
    const char* cache_base = ld_isv ? vcb : kcb;
    const char* canvas_base = ld_isv ? vb : kb;
    const int last_chunk = hd * kEsz / 16 - 1;   // kPad: chunks past it repeat it
    auto issue_stage = [&](int st, int buf) {
        const int j0 = key0(st, ld_tile);
        if (j0 >= kend) return;              // the split's last stage holds one tile
        char* dst = tile_ptr(buf, ld_tile, ld_isv);
        // A padded K tile takes rows i and i + 16 in load i (KLayout); V tiles and unpadded K
        // tiles take rows 2i, 2i + 1 (HD 128) or 4i..4i + 3 (HD 64).
        const bool padk = kPadK && !ld_isv;
        const int load_bytes = padk ? KL::kLoadBytes : 1024;
        const bool in_cache = j0 + dgk::kKeys <= a.ctx, in_canvas = j0 >= a.ctx;
        if ((in_cache || in_canvas) && j0 + dgk::kKeys <= kend) {   // one side of the seam
            const char* b = in_cache ? cache_base + (size_t)j0 * rstride_c
                                     : canvas_base + (size_t)(j0 - a.ctx) * rstride_v;
            const unsigned rs = in_cache ? rstride_c : rstride_v;
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int trow = padk ? i + KT::kLoadsPerTile * rsub : i * R + rsub;
                int chunk = ld_isv ? (kBf16 ? pos ^ vswz<HD>(trow) : pos)
                                   : (kPadK || kPlanes ? pos : (pos ^ (trow % KT::kChunks)));
                if (kPad) chunk = min(chunk, last_chunk);
                __builtin_amdgcn_global_load_lds(b + ((unsigned)trow * rs + 16u * chunk),
                                                 (dgk::lds_void*)(dst + i * load_bytes), 16, 0, 0);
            }
        } else {                           // straddles the seam or the end: per-row addresses
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int trow = padk ? i + KT::kLoadsPerTile * rsub : i * R + rsub;
                const int j = min(j0 + trow, kend - 1);
                int chunk = ld_isv ? (kBf16 ? pos ^ vswz<HD>(trow) : pos)
                                   : (kPadK || kPlanes ? pos : (pos ^ (trow % KT::kChunks)));
                if (kPad) chunk = min(chunk, last_chunk);
                const char* p = (j < a.ctx ? cache_base + (size_t)j * rstride_c
                                           : canvas_base + (size_t)(j - a.ctx) * rstride_v) +
                                16u * chunk;
                __builtin_amdgcn_global_load_lds(p, (dgk::lds_void*)(dst + i * load_bytes), 16, 0, 0);
            }
        }
    };

    // The first stage's loads go out before the queries are fetched, so the two overlap; with
    // the q norm inside, after the queries have been staged, so that the opening burst of every
    // workgroup serves the queries first (measured: DiffusionGemma-like step 29.40 -> 29.22 us).
    if (!kNormQ && !hi && nst > 0) issue_stage(0, 0);
    constexpr bool kQ3 = kBf16 || kPlanes;   // q as three bf16 terms
    float qreg[kQ3 ? 1 : HD / 2];
    QSplit<kQ3 ? HD : 16> q3;
    if constexpr (kNormQ) {
        static_assert(!kBf16, "16-bit K/V take normalised q");
        float* qs = smem + kQOff;
        if constexpr (kPlanes && !kPad) {   // q split once, into bf16 planes over the K/V planes
            static_assert(3 * kQPlaneBytes<HD> <= 2 * 2 * 3 * Planes<HD>::kBytes, "q planes fit");
            stage_q_normed<HD, kBlockQ, true>(a, qs, b, kv, qb, wave, lane, hd);
            if (!hi && nst > 0) issue_stage(0, 0);
            __syncthreads();
            load_q_planes<HD>(reinterpret_cast<const char*>(qs), pair * dgk::kQuery + l32, half, q3);
        } else {
            stage_q_normed<HD>(a, qs, b, kv, qb, wave, lane, hd);
            if (!hi && nst > 0) issue_stage(0, 0);
            __syncthreads();
            const float* qrow = qs + (pair * dgk::kQuery + l32) * kQStride<HD>;
            if constexpr (kQ3)
                load_q_bf16x3<HD>(qrow, true, half, 1.0f, q3, HD);
            else
                dgk::load_q<HD>(qrow, true, half, 1.0f, qreg);
        }
    } else if constexpr (kQ3) {
        load_q_bf16x3<HD>(a.q + gq * hd, valid, half, a.qmul, q3, hd);
    } else {
        dgk::load_q<HD>(a.q + gq * hd, valid, half, a.qmul, qreg, hd);
    }
    f32x16 o[TL::kGroups];
#pragma unroll
    for (int t = 0; t < TL::kGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;
    int voff[TL::kGroups];   // bf16 V: the lane's transposed-read offsets
    if constexpr (kBf16 || kPlanes) vtr_offsets<HD>(lane, voff);

    for (int st = 0; st < nst; ++st) {
        const int buf = kPlanes ? 0 : st & 1;
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of stage st have landed
        __syncthreads();                 // ...everyone's; and stage st-1 is fully consumed
        if (!kPlanes && !hi && st + 1 < nst) issue_stage(st + 1, buf ^ 1);
        if constexpr (kNormKV) {
            // Canvas rows are normalised in place before anyone reads them (the next stage's
            // loads, issued just before, stream in meanwhile).
            const int ja = key0(st, 0), jb = key0(st, 1);
            const bool ca = ja < kend && ja + dgk::kKeys > a.ctx;
            const bool cb = jb < kend && jb + dgk::kKeys > a.ctx;
            if (ca || cb) {
                if (ca)
                    norm_canvas_tile<HD, kPad, kPadK, !kPlanes>(a, reinterpret_cast<float*>(tile_ptr(buf, 0, 0)),
                                               reinterpret_cast<float*>(tile_ptr(buf, 0, 1)), ja,
                                               kend, wave, lane, hd);
                if (cb)
                    norm_canvas_tile<HD, kPad, kPadK, !kPlanes>(a, reinterpret_cast<float*>(tile_ptr(buf, 1, 0)),
                                               reinterpret_cast<float*>(tile_ptr(buf, 1, 1)), jb,
                                               kend, wave, lane, hd);
                __syncthreads();
            }
        }
        if constexpr (kPlanes) {
            // the whole workgroup splits the staged tiles, then the staging buffer is free
            split_stage<HD, 64 * kWaves, 2>(tile_ptr(0, 0, 0), kSlot, planes, key0(st, 1) < kend ? 2 : 1, tid);
            __syncthreads();
            if (!hi && st + 1 < nst) issue_stage(st + 1, 0);
        }
        const int t0 = key0(st, hi);
        if (pair_active && t0 < kend) {
            f32x16 s;
            if constexpr (kPlanes) {
                const float shift = -dgk::ref_of(m);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(half ? 0.0f : 1.0f, half ? 0.0f : shift,
                                                         f32x16{}, 0, 0, 0);
                s = scores_planes<HD>(Planes<HD>::at(planes, hi, 0, 0), l32, half, q3, s);
            } else if constexpr (kKV == 0) {
                if constexpr (KL::kPadded) {
                    const float shift = -dgk::ref_of(m);
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(half ? 0.0f : 1.0f, half ? 0.0f : shift,
                                                             f32x16{}, 0, 0, 0);
                    s = scores_padded<HD>(tile_ptr(buf, hi, 0), l32, half, qreg, s);
                } else {
                    s = dgk::scores<HD>(reinterpret_cast<const float*>(tile_ptr(buf, hi, 0)), l32,
                                        half, qreg, -dgk::ref_of(m));
                }
            } else {
                const float shift = -dgk::ref_of(m);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(half ? 0.0f : 1.0f, half ? 0.0f : shift,
                                                         f32x16{}, 0, 0, 0);
                if constexpr (kBf16)
                    s = scores_bf16x3<HD>(tile_ptr(buf, hi, 0), l32, half, q3, s);
                else
                    s = scores_from16<HD, kKV>(tile_ptr(buf, hi, 0), l32, half, qreg, s);
            }
            const bool need_mask =
                t0 + dgk::kKeys > kend || (a.causal && t0 + dgk::kKeys - 1 - a.ctx > row_min);
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = t0 + dgk::key_of(r, half);
                    if (j >= kend || (a.causal && j - a.ctx > row)) s[r] = -INFINITY;
                }
            }
            dgk::softmax_update<HD>(s, m, lsum, o);
            if constexpr (kPlanes)
                accumulate_pv_planes<HD>(Planes<HD>::at(planes, hi, 1, 0), voff, s, o);
            else if constexpr (kKV == 0)
                dgk::accumulate_pv<HD>(reinterpret_cast<const float*>(tile_ptr(buf, hi, 1)), l32, half, s, o);
            else if constexpr (kBf16)
                accumulate_pv_bf16x3<HD>(tile_ptr(buf, hi, 1), voff, s, o);
            else
                accumulate_pv16<HD, kKV>(tile_ptr(buf, hi, 1), l32, half, s, o);
        }
    }

    __syncthreads();  // every wave is done with the stage buffers; reuse them for the merge
    dgk::pair_merge<HD>(smem, pair, hi, pair_active, lane, m, lsum, o);
    const float ltot = lsum + __shfl_xor(lsum, 32);
    // The even wavefront of each pair restages its 32 merged rows row-major over its own merge
    // scratch (the same LDS span: 64 * (HD/2 + 2) = 32 * (HD + 4) floats, read only by this
    // wavefront), with the rows' global query indices beside the block.  The workgroup then
    // writes the block out with 16 contiguous bytes per lane, whole rows per half-wavefront.
    constexpr int kOStride = HD + 4;
    static_assert(64 * (TL::kGroups * 16 + 2) == dgk::kQuery * kOStride, "row block overlays the merge scratch");
    long long* rowg = reinterpret_cast<long long*>(smem + kPairs * dgk::kQuery * kOStride);
    if (!hi) {
        const float oscale = a.nsplit == 1 && valid ? 1.0f / ltot : 1.0f;
        if constexpr (kBf16 || kPlanes)
            stage_row_blocked<HD>(smem + pair * dgk::kQuery * kOStride, l32, oscale, o, half);
        else
            dgk::stage_row<HD>(smem + pair * dgk::kQuery * kOStride, l32, oscale, o, half);
        if (half == 0) rowg[pair * dgk::kQuery + l32] = valid ? (long long)gq : -1;
        if (a.nsplit > 1 && valid && half == 0) {
            float* wm = a.ws + (size_t)a.nsplit * a.nqtot * hd;
            wm[(size_t)split * a.nqtot + gq] = m;
            wm[(size_t)(a.nsplit + split) * a.nqtot + gq] = ltot;
        }
    }
    __syncthreads();
    float* obase = a.nsplit == 1 ? a.out : a.ws + (size_t)split * a.nqtot * hd;
    constexpr int kChunksO = HD / 4;                       // 16-byte chunks per row
    constexpr int kRowsPerPass = kWaves * 64 / kChunksO;
#pragma unroll
    for (int r0 = 0; r0 < kBlockQ; r0 += kRowsPerPass) {
        const int rloc = r0 + tid / kChunksO, c = tid % kChunksO;
        const long long g = rowg[rloc];
        if (g < 0 || (kPad && 4 * c >= hd)) continue;
        *reinterpret_cast<float4*>(obase + (size_t)g * hd + 4 * c) =
            *reinterpret_cast<const float4*>(smem + rloc * kOStride + 4 * c);
    }
}

// Short key sets (ctx + T <= 8, e.g. the depformer's causal frames of 8 steps): there is too
// little work per query for matrix tiles, and the call is HBM-bound.  One wavefront per
// (batch entry, q head): lane (r, c) = (lane / 8, lane % 8) owns query row r and the c-th
// HD/8-wide segment of it, and loads the same segment of key/value row r into wave-private LDS.
// Each lane forms partial dots of its query segment with every key's segment; a 3-step lane
// exchange within each group of 8 completes them, the 8-entry softmax runs in registers, and
// each lane writes its segment of the output row.  All global accesses are contiguous per row.
// Elements at or past hd (kPad) are zero.  With kNormQ the q norm runs on the lane's segment
// (3 exchanges for the sum of squares) and the rope partner is read back from a staged row;
// with kNormKV the k and v norms of canvas key rows run the same way (the k rope partner is
// read back from the key's own LDS row before the row is written).
constexpr int kSmallKeys = 8;

template <int HD, bool kNormQ, bool kNormKV, bool kPad, int kKV>
__global__ void __launch_bounds__(256) attn_small_kernel(SplitArgs a, long long units) {
    constexpr int SEG = HD / 8;
    constexpr int kRows = kNormQ ? 3 : 2;   // K, V (and the staged q) per wave
    __shared__ __attribute__((aligned(16))) float kvs[4 * kRows * kSmallKeys * HD];
    const int hd = kPad ? a.hd : HD;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane >> 3, cseg = (lane & 7) * SEG;
    const long long u = (long long)blockIdx.x * 4 + wave;   // b * nh + h
    const bool active = u < units;
    const int h = active ? (int)(u % a.nh) : 0;
    const int b = active ? (int)(u / a.nh) : 0;
    const int kv = h / a.G;
    const int S = a.ctx + a.T;
    float* ks = kvs + wave * kRows * kSmallKeys * HD;
    float* vs = ks + kSmallKeys * HD;

    float qr[SEG], kr[SEG], vr[SEG];
    const bool has_key = active && r < S, has_q = active && r < a.T;
    constexpr int kEsz = kKV ? 2 : 4;
    // Every lane loads from an address that exists (key row 0 and query row 0 stand in for
    // rows past the end, a last chunk for padding) and zeroes by selection afterwards: guarded
    // loads would become divergent branches that issue the loads one at a time.
    const int rk = has_key ? r : 0, rq = has_q ? r : 0;
    const size_t off = rk < a.ctx ? (((size_t)b * a.nkv + kv) * a.ctx + rk) * hd
                                  : (((size_t)b * a.T + (rk - a.ctx)) * a.nkv + kv) * hd;
    const char* kp = reinterpret_cast<const char*>(rk < a.ctx ? a.kc : a.k) + off * kEsz;
    const char* vp = reinterpret_cast<const char*>(rk < a.ctx ? a.vc : a.v) + off * kEsz;
    const float* qrow = a.q + (((size_t)b * a.T + rq) * a.nh + h) * hd;
    constexpr int kStep = kKV ? 8 : 4;   // elements per 16-byte load
#pragma unroll
    for (int e = 0; e < SEG; e += kStep) {
        const bool in = cseg + e < hd;
        const int el = in ? cseg + e : hd - kStep;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        const uint4 kl = *reinterpret_cast<const uint4*>(kp + el * kEsz);
        const uint4 vl = *reinterpret_cast<const uint4*>(vp + el * kEsz);
        const uint4 k4 = has_key && in ? kl : z;
        const uint4 v4 = has_key && in ? vl : z;
        const uint32_t kw[4] = {k4.x, k4.y, k4.z, k4.w}, vw[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (kKV == 0) {
                kr[e + w] = __uint_as_float(kw[w]);
                vr[e + w] = __uint_as_float(vw[w]);
            } else {
                kr[e + 2 * w] = lo16<kKV>(kw[w]);
                kr[e + 2 * w + 1] = hi16<kKV>(kw[w]);
                vr[e + 2 * w] = lo16<kKV>(vw[w]);
                vr[e + 2 * w + 1] = hi16<kKV>(vw[w]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < SEG; e += 4) {
        const bool in = cseg + e < hd;
        const float4 ql = *reinterpret_cast<const float4*>(qrow + (in ? cseg + e : hd - 4));
        const float4 q4 = has_q && in ? ql : make_float4(0.f, 0.f, 0.f, 0.f);
        qr[e] = q4.x; qr[e + 1] = q4.y; qr[e + 2] = q4.z; qr[e + 3] = q4.w;
    }
    if constexpr (kNormQ) {
        if (!(a.qflags & DG_NORM_SKIP)) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < SEG; ++e) ss += qr[e] * qr[e];
            ss = group_sum<8>(ss);
            const float inv = has_q ? 1.0f / sqrtf(ss / (float)hd + a.eps) : 0.0f;
#pragma unroll
            for (int e = 0; e < SEG; ++e) {
                qr[e] *= inv;
                if ((a.qflags & DG_NORM_WEIGHTED) && cseg + e < hd) qr[e] *= a.wq[cseg + e];
            }
        }
        if (a.qflags & DG_NORM_ROPE) {
            float* qs = vs + kSmallKeys * HD + r * HD;   // this row's staging, wave-private
#pragma unroll
            for (int e = 0; e < SEG; ++e) qs[cseg + e] = qr[e];
            const int half_hd = hd >> 1;
            const float* cr = a.cs + (size_t)(has_q ? r : 0) * 2 * hd;
            float part[SEG];
#pragma unroll
            for (int e = 0; e < SEG; ++e) {
                const int el = cseg + e;
                part[e] = el < hd ? qs[el < half_hd ? el + half_hd : el - half_hd] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < SEG; ++e) {
                const int el = cseg + e;
                if (el < hd && has_q) {
                    const float rot = el < half_hd ? -part[e] : part[e];
                    qr[e] = qr[e] * cr[el] + rot * cr[hd + el];
                } else {
                    qr[e] = 0.0f;
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < SEG; ++e) qr[e] *= a.qmul;
    if constexpr (kNormKV) {
        // Canvas key rows arrive raw: the k dispatch (norm, weight, rope at canvas row r - ctx)
        // and the weightless v norm, on the lane's segment.  kr, vr are zero past hd.
        const bool canvas_key = has_key && r >= a.ctx;   // the same for the 8 lanes of a row
        float ssk = 0.0f, ssv = 0.0f;
#pragma unroll
        for (int e = 0; e < SEG; ++e) {
            ssk += kr[e] * kr[e];
            ssv += vr[e] * vr[e];
        }
        ssk = group_sum<8>(ssk);
        ssv = group_sum<8>(ssv);
        if (canvas_key) {
            const float invk = 1.0f / sqrtf(ssk / (float)hd + a.eps);
            const float invv = 1.0f / sqrtf(ssv / (float)hd + a.eps);
#pragma unroll
            for (int e = 0; e < SEG; ++e) {
                kr[e] *= invk;
                if ((a.qflags & DG_NORM_WEIGHTED) && cseg + e < hd) kr[e] *= a.wk[cseg + e];
                vr[e] *= invv;
            }
            if (a.qflags & DG_NORM_ROPE) {
                float* krow = ks + r * HD;    // the key's own row, wave-private, written below
#pragma unroll
                for (int e = 0; e < SEG; ++e) krow[cseg + e] = kr[e];
                const int half_hd = hd >> 1;
                const float* cr = a.cs + (size_t)(r - a.ctx) * 2 * hd;
                float part[SEG];
#pragma unroll
                for (int e = 0; e < SEG; ++e) {
                    const int el = cseg + e;
                    part[e] = el < hd ? krow[el < half_hd ? el + half_hd : el - half_hd] : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < SEG; ++e) {
                    const int el = cseg + e;
                    if (el < hd) {
                        const float rot = el < half_hd ? -part[e] : part[e];
                        kr[e] = kr[e] * cr[el] + rot * cr[hd + el];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < SEG; e += 4) {
        *reinterpret_cast<float4*>(ks + r * HD + cseg + e) = make_float4(kr[e], kr[e + 1], kr[e + 2], kr[e + 3]);
        *reinterpret_cast<float4*>(vs + r * HD + cseg + e) = make_float4(vr[e], vr[e + 1], vr[e + 2], vr[e + 3]);
    }
    __syncthreads();
    float sc[kSmallKeys];
#pragma unroll
    for (int j = 0; j < kSmallKeys; ++j) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
            const float4 k4 = *reinterpret_cast<const float4*>(ks + j * HD + cseg + e);
            d += qr[e] * k4.x + qr[e + 1] * k4.y + qr[e + 2] * k4.z + qr[e + 3] * k4.w;
        }
        d = group_sum<8>(d);
        const bool visible = j < S && !(a.causal && j >= a.ctx && j - a.ctx > r);
        sc[j] = visible ? d : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int j = 1; j < kSmallKeys; ++j) mx = fmaxf(mx, sc[j]);
    const float mu = (mx == -INFINITY) ? 0.0f : mx;
    float l = 0.0f;
#pragma unroll
    for (int j = 0; j < kSmallKeys; ++j) {
        sc[j] = dgk::fast_exp2(sc[j] - mu);
        l += sc[j];
    }
    float o[SEG];
#pragma unroll
    for (int e = 0; e < SEG; ++e) o[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kSmallKeys; ++j) {
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(vs + j * HD + cseg + e);
            o[e] += sc[j] * v4.x; o[e + 1] += sc[j] * v4.y; o[e + 2] += sc[j] * v4.z; o[e + 3] += sc[j] * v4.w;
        }
    }
    if (!has_q) return;
    const float inv = 1.0f / l;
    float* op = a.out + (((size_t)b * a.T + r) * a.nh + h) * hd + cseg;
#pragma unroll
    for (int e = 0; e < SEG; e += 4)
        if (cseg + e < hd)
            *reinterpret_cast<float4*>(op + e) = make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
}

// Merges split-KV partials: out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s.
// One thread per 4 output elements (hd is a multiple of 4).  Splits are taken 8 at a time with
// all their loads issued together, and the running maximum is folded in as it grows (the
// same rescaling as the online softmax), so no pass waits for a previous one.
// With `local`, threads are numbered (batch, kv head, query vector of the group, chunk) and
// workgroups are placed as the attention kernel placed its own, so each kv head's partials
// are merged on the XCD whose workgroups wrote them (the launch sets it only when both grids
// divide evenly into the device's XCDs and each kv head fills whole workgroups).
__global__ void __launch_bounds__(256) split_combine_kernel(const float* __restrict__ ws,
                                                            float* __restrict__ out,
                                                            size_t total, int nsplit, int hd,
                                                            int T, int G, int nkv, int local,
                                                            int nxcd) {
    constexpr int kBatch = 8;
    const int c4 = hd / 4;
    size_t gq;
    int c;
    if (local) {
        const size_t idx = (size_t)xcd_remap(blockIdx.x, gridDim.x, nxcd) * blockDim.x + threadIdx.x;
        if (idx >= total * c4) return;
        const size_t per_bk = (size_t)T * G * c4;
        const size_t bk = idx / per_bk, rem = idx % per_bk;
        const int qv = (int)(rem / c4);
        c = (int)(rem % c4) * 4;
        const size_t b = bk / nkv, kv = bk % nkv;
        gq = (b * T + qv / G) * ((size_t)nkv * G) + kv * G + qv % G;
    } else {
        const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (idx >= total * c4) return;
        gq = idx / c4;
        c = (int)(idx % c4) * 4;
    }
    const float* wm = ws + (size_t)nsplit * total * hd;
    const float* wl = wm + (size_t)nsplit * total;
    float M = -INFINITY, L = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
        float mv[kBatch], lv[kBatch];
        float4 ov[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int sp = min(s0 + i, nsplit - 1);   // a repeated split is masked below
            mv[i] = wm[(size_t)sp * total + gq];
            lv[i] = wl[(size_t)sp * total + gq];
            ov[i] = *reinterpret_cast<const float4*>(ws + ((size_t)sp * total + gq) * hd + c);
        }
        float bm = M;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (s0 + i < nsplit) bm = fmaxf(bm, mv[i]);
        const float ref = bm == -INFINITY ? 0.0f : bm;
        const float corr = dgk::fast_exp2(M - ref);
        L *= corr;
        acc.x *= corr; acc.y *= corr; acc.z *= corr; acc.w *= corr;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const float w = s0 + i < nsplit ? dgk::fast_exp2(mv[i] - ref) : 0.0f;
            L += lv[i] * w;
            acc.x += ov[i].x * w; acc.y += ov[i].y * w; acc.z += ov[i].z * w; acc.w += ov[i].w * w;
        }
        M = bm;
    }
    const float inv = 1.0f / L;
    *reinterpret_cast<float4*>(out + gq * hd + c) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Launch plan shared by the workspace query and the launch: which kernel, how many query
// vectors per workgroup, and how many key-range splits, for a device with `cus` compute units.
//  * ctx + T <= 8: attn_small_kernel.
//  * Otherwise attn_split_gqa_kernel (128 query vectors per workgroup).
// A shape with fewer workgroups than CUs splits its key range (not causal calls), at least two
// 64-key stages per split.  (Fewer, longer splits were measured slower on the DiffusionGemma-like
// step: 36.3 us per step at 4 to 5 splits against 29.6 us at 8.)
struct Plan {
    int kernel = DG_KERNEL_TILE32;
    int blockq = kBlockQ;
    int qblocks = 0, nsplit = 1;
    long long nblocks = 0;
    size_t ws_bytes = 0;
};

// Splits of a shape with `blocks` workgroups per key range: one workgroup per CU when the keys
// allow it (at least two 64-key stages per split; causal calls do not split).
int split_count(long long blocks, int S, int causal, int cus) {
    const int nstage = (S + kStage - 1) / kStage;   // both tiled kernels take 64-key stages
    if (blocks <= 0 || blocks >= cus || causal) return 1;
    const long long want = (cus + blocks - 1) / blocks;
    const long long cap = nstage / 2;
    return (int)std::max(1LL, std::min(want, cap));
}

Plan plan(int batch, int T, int ctx, int nh, int nkv, int hd, int causal, int kv, int cus) {
    Plan p;
    const int G = nh / nkv;
    const int S = ctx + T;
    if (S <= kSmallKeys) {
        p.kernel = DG_KERNEL_SMALL;
        p.blockq = 0;
        p.nblocks = ((long long)batch * nh + 3) / 4;
        return p;
    }
    p.qblocks = (int)(((long long)T * G + kBlockQ - 1) / kBlockQ);
    long long blocks = (long long)batch * nkv * p.qblocks;
    p.nsplit = split_count(blocks, S, causal, cus);
    p.nblocks = blocks * p.nsplit;
    if (p.nsplit > 1)
        p.ws_bytes = (size_t)p.nsplit * batch * T * nh * (size_t)(hd + 2) * sizeof(float);
    return p;
}

// The static split-KV scratch of dg_attn_split_gqa_noalloc: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory; its device address on each GPU comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = DG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that runs `stream`, which must be the current
// device (the address is looked up with that device current).
int scratch_for_stream(const char* fn, void* stream, void** out) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return dg::fail(DG_ELAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess)
            return dg::fail(DG_ELAUNCH, "%s: hipStreamGetDevice: %s", fn, hipGetErrorString(e));
        if (sdev != cur)
            return dg::fail(DG_EINVAL, "%s: the stream belongs to device %d, the current device is %d",
                            fn, (int)sdev, cur);
    }
    if (cur < 0 || cur >= kMaxDevices)
        return dg::fail(DG_EUNSUPPORTED, "%s: device %d is beyond the %d the library tracks", fn,
                        cur, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[cur]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return dg::fail(DG_ELAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn,
                            cur, hipGetErrorString(e));
        g_scratch_ptr[cur] = ptr;
    }
    *out = g_scratch_ptr[cur];
    return DG_OK;
}

}  // namespace

extern "C" size_t dg_attn_split_gqa_workspace_size(int batch, int T, int ctx, int nh, int nkv,
                                                   int hd) {
    if (batch <= 0 || T <= 0 || ctx < 0 || nkv < 1 || nh < 1 || nh % nkv != 0) return 0;
    if (hd < 4 || hd > 128 || hd % 4 != 0) return 0;
    // enough for the f32 and the 16-bit K/V entry points, whose plans may differ
    const int cus = dg::device_topology().cus;
    return std::max(plan(batch, T, ctx, nh, nkv, hd, 0, 0, cus).ws_bytes,
                    plan(batch, T, ctx, nh, nkv, hd, 0, DG_KV_BF16, cus).ws_bytes);
}

extern "C" int dg_attn_split_gqa_plan(int batch, int T, int ctx, int nh, int nkv, int hd,
                                      int causal, int kv_format, int cus, dg_attn_plan* out) {
    const char* fn = "dg_attn_split_gqa_plan";
    if (!out) return dg::fail(DG_EINVAL, "%s: plan is NULL", fn);
    if (batch < 0 || T < 0 || ctx < 0 || nh < 1 || nkv < 1 || nh % nkv != 0 || cus < 0)
        return dg::fail(DG_EINVAL, "%s: bad sizes (batch %d, T %d, ctx %d, nh %d, nkv %d, cus %d)",
                        fn, batch, T, ctx, nh, nkv, cus);
    if (hd < 4 || hd > 128 || hd % 4 != 0)
        return dg::fail(DG_EUNSUPPORTED, "%s: hd %d not supported", fn, hd);
    if (causal != 0 && causal != 1) return dg::fail(DG_EINVAL, "%s: causal must be 0 or 1", fn);
    if (kv_format != 0 && kv_format != DG_KV_F16 && kv_format != DG_KV_BF16)
        return dg::fail(DG_EINVAL, "%s: unknown kv_format %d", fn, kv_format);
    const dg::Topology topo = dg::device_topology();
    const Plan p = plan(batch, T, ctx, nh, nkv, hd, causal, kv_format, cus > 0 ? cus : topo.cus);
    out->kernel = batch == 0 || T == 0 ? DG_KERNEL_NONE : p.kernel;
    out->query_block = p.blockq;
    out->nsplit = p.nsplit;
    out->workgroups = batch == 0 || T == 0 ? 0 : p.nblocks;
    out->workspace_bytes = batch == 0 || T == 0 ? 0 : p.ws_bytes;
    return dg::ok();
}

namespace {

// Kernel variant for a head dim: the tile is 64 wide for hd <= 64 and 128 wide above; a
// narrower hd runs padded.
using SplitKernel = void (*)(SplitArgs);
using SmallKernel = void (*)(SplitArgs, long long);

// norm: 0 (k, v and q as given), 1 (q normalised in the kernel), 2 (q, k and v normalised in
// the kernel).
template <int HD, int kNorm, int kKV>
SplitKernel split_variant(int hd) {
    return hd == HD ? attn_split_gqa_kernel<HD, kNorm >= 1, kNorm == 2, false, kKV>
                    : attn_split_gqa_kernel<HD, kNorm >= 1, kNorm == 2, true, kKV>;
}

template <int HD>
SplitKernel split_norm_variant(int hd, int norm) {
    return norm == 2 ? split_variant<HD, 2, 0>(hd) : norm == 1 ? split_variant<HD, 1, 0>(hd)
                                                               : split_variant<HD, 0, 0>(hd);
}

// kv: 0 (f32), DG_KV_F16 or DG_KV_BF16; the 16-bit variants take no in-kernel norm.

SplitKernel pick_split(int hd, int norm, int kv) {
    if (kv == DG_KV_F16) return hd > 64 ? split_variant<128, 0, DG_KV_F16>(hd) : split_variant<64, 0, DG_KV_F16>(hd);
    if (kv == DG_KV_BF16) return hd > 64 ? split_variant<128, 0, DG_KV_BF16>(hd) : split_variant<64, 0, DG_KV_BF16>(hd);
    return hd > 64 ? split_norm_variant<128>(hd, norm) : split_norm_variant<64>(hd, norm);
}

template <int HD, int kNorm, int kKV>
SmallKernel small_variant(int hd) {
    return hd == HD ? attn_small_kernel<HD, kNorm >= 1, kNorm == 2, false, kKV>
                    : attn_small_kernel<HD, kNorm >= 1, kNorm == 2, true, kKV>;
}

template <int HD>
SmallKernel small_norm_variant(int hd, int norm) {
    return norm == 2 ? small_variant<HD, 2, 0>(hd) : norm == 1 ? small_variant<HD, 1, 0>(hd)
                                                               : small_variant<HD, 0, 0>(hd);
}

SmallKernel pick_small(int hd, int norm, int kv) {
    if (kv == DG_KV_F16) return hd > 64 ? small_variant<128, 0, DG_KV_F16>(hd) : small_variant<64, 0, DG_KV_F16>(hd);
    if (kv == DG_KV_BF16) return hd > 64 ? small_variant<128, 0, DG_KV_BF16>(hd) : small_variant<64, 0, DG_KV_BF16>(hd);
    return hd > 64 ? small_norm_variant<128>(hd, norm) : small_norm_variant<64>(hd, norm);
}

// Shared body of the attention entry points.  `norm` selects the in-kernel norms (0 none, 1 q,
// 2 q, k and v), whose extra arguments (wq, wk, cs, qflags, eps) were validated by the caller.
// With `use_scratch` the split-KV partials go to the library's static device scratch (the
// caller passes no workspace); a shape whose partials exceed it is refused.
int attn_call(const char* fn, const float* q, const void* kc, const void* vc, const void* k,
              const void* v, float* out, int batch, int T, int ctx, int nh, int nkv, int hd,
              float scale, int causal, void* workspace, size_t workspace_bytes, void* stream,
              int norm, const float* wq, const float* wk, const float* cs, unsigned qflags,
              float eps, int kv, bool use_scratch = false) {
    const bool normq = norm >= 1;
    if (batch < 0 || T < 0 || ctx < 0 || nh < 0 || nkv < 0)
        return dg::fail(DG_EINVAL, "%s: negative size (batch %d, T %d, ctx %d, nh %d, nkv %d)", fn,
                        batch, T, ctx, nh, nkv);
    if (nkv < 1 || nh < 1 || nh % nkv != 0)
        return dg::fail(DG_EINVAL, "%s: nh (%d) must be a positive multiple of nkv (%d)", fn, nh, nkv);
    if (hd < 1) return dg::fail(DG_EINVAL, "%s: hd must be >= 1, got %d", fn, hd);
    if (hd > 128 || hd % 4 != 0)
        return dg::fail(DG_EUNSUPPORTED, "%s: hd %d not supported (a multiple of 4, at most 128)", fn, hd);
    if (kv && hd % 8 != 0)
        return dg::fail(DG_EUNSUPPORTED, "%s: 16-bit K/V need hd a multiple of 8, got %d", fn, hd);
    // Key and query-vector indices inside the kernels are 32-bit.
    if ((long long)ctx + T > (1LL << 30) || (long long)T * (nh / nkv) > (1LL << 30))
        return dg::fail(DG_EUNSUPPORTED, "%s: ctx + T (%lld) or T * nh/nkv above 2^30", fn,
                        (long long)ctx + T);
    const size_t esz = kv ? 2 : 4;
    if (!std::isfinite(scale)) return dg::fail(DG_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return dg::fail(DG_EINVAL, "%s: causal must be 0 or 1", fn);
    size_t nq = 1, nkvc = 1, ncache = 1;
    if (!dg::mul_ok(nq, batch) || !dg::mul_ok(nq, T) || !dg::mul_ok(nq, nh) || !dg::mul_ok(nq, hd) ||
        !dg::mul_ok(nkvc, batch) || !dg::mul_ok(nkvc, T) || !dg::mul_ok(nkvc, nkv) || !dg::mul_ok(nkvc, hd) ||
        !dg::mul_ok(ncache, batch) || !dg::mul_ok(ncache, nkv) || !dg::mul_ok(ncache, ctx) ||
        !dg::mul_ok(ncache, hd))
        return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    if (workspace && workspace_bytes == 0)
        return dg::fail(DG_EINVAL, "%s: workspace given with workspace_bytes 0", fn);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15))
        return dg::fail(DG_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    if (nq == 0) return dg::ok();
    if (!q || !k || !v || !out) return dg::fail(DG_EINVAL, "%s: q, k, v and out must be non-NULL", fn);
    if (ncache > 0 && (!kc || !vc)) return dg::fail(DG_EINVAL, "%s: kc/vc NULL with ctx %d > 0", fn, ctx);
    const dg::Topology topo = dg::device_topology();
    Plan p = plan(batch, T, ctx, nh, nkv, hd, causal, kv, topo.cus);
    if (use_scratch && p.nsplit > 1) {
        if (p.ws_bytes > kScratchBytes)
            return dg::fail(DG_EUNSUPPORTED,
                            "%s: this shape needs %zu bytes of split-KV scratch, more than the "
                            "%zu bytes of the library's static scratch (use dg_attn_split_gqa "
                            "with a workspace)", fn, p.ws_bytes, kScratchBytes);
        const int st = scratch_for_stream(fn, stream, &workspace);
        if (st != DG_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (p.nsplit > 1 && (!workspace || workspace_bytes < p.ws_bytes)) {
        if (workspace)
            return dg::fail(DG_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed",
                            fn, workspace_bytes, p.ws_bytes);
        p.nsplit = 1;  // no workspace: run unsplit
        p.ws_bytes = 0;
    }
    const dg::Span so(out, nq * 4);
    const dg::Span ins[9] = {dg::Span(q, nq * 4), dg::Span(k, nkvc * esz), dg::Span(v, nkvc * esz),
                             dg::Span(ncache ? kc : nullptr, ncache * esz),
                             dg::Span(ncache ? vc : nullptr, ncache * esz),
                             dg::Span(normq ? wq : nullptr, (size_t)hd * 4),
                             dg::Span(norm == 2 ? wk : nullptr, (size_t)hd * 4),
                             dg::Span(normq ? cs : nullptr, (size_t)T * 2 * hd * 4),
                             dg::Span(p.nsplit > 1 ? workspace : nullptr, p.ws_bytes)};
    for (int i = 0; i < 9; ++i)
        if (so.overlaps(ins[i])) return dg::fail(DG_EINVAL, "%s: out overlaps an input or the workspace", fn);
    for (int i = 0; i < 8; ++i)
        if (ins[8].overlaps(ins[i])) return dg::fail(DG_EINVAL, "%s: workspace overlaps an input", fn);
    // The kernels read and write these with 16-byte vector accesses.
    const void* vec[9] = {q, k, v, out, ncache ? kc : nullptr, ncache ? vc : nullptr,
                          normq ? wq : nullptr, norm == 2 ? wk : nullptr, normq ? cs : nullptr};
    for (int i = 0; i < 9; ++i)
        if (reinterpret_cast<uintptr_t>(vec[i]) & 15)
            return dg::fail(DG_EINVAL, "%s: tensor pointers must be 16-byte aligned", fn);
    const long long nblocks = (long long)batch * nkv * p.qblocks * p.nsplit;
    if (nblocks > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
    SplitArgs a;
    a.q = q; a.out = out;   // K/V are addressed bytewise in the kernels, whatever their storage
    a.kc = static_cast<const float*>(kc); a.vc = static_cast<const float*>(vc);
    a.k = static_cast<const float*>(k); a.v = static_cast<const float*>(v);
    a.ws = static_cast<float*>(p.nsplit > 1 ? workspace : nullptr);
    a.nqtot = (size_t)batch * T * nh;
    a.hd = hd;
    a.T = T; a.ctx = ctx; a.nh = nh; a.nkv = nkv; a.G = nh / nkv;
    a.qblocks = p.qblocks;
    a.nsplit = p.nsplit;
    a.nblocks = (int)nblocks;
    a.nxcd = topo.xcds;
    a.qmul = scale * dgk::kLog2e;
    a.causal = causal;
    a.wq = normq ? wq : nullptr;
    a.wk = norm == 2 ? wk : nullptr;
    a.cs = normq ? cs : nullptr;
    a.qflags = normq ? qflags : 0u;
    a.eps = eps;
    hipStream_t s = (hipStream_t)stream;
    if (p.kernel == DG_KERNEL_SMALL) {
        const long long units = (long long)batch * nh;
        const long long blocks = (units + 3) / 4;
        if (blocks > 0x7fffffffLL) return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
        hipLaunchKernelGGL(pick_small(hd, norm, kv), dim3((unsigned)blocks), dim3(256), 0, s, a, units);
        return dg::launch_status(fn);
    }
    auto* kern = pick_split(hd, norm, kv);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(512), 0, s, a);
    if (p.nsplit > 1) {
        const size_t total = (size_t)batch * T * nh;
        const size_t threads = total * (hd / 4);
        const unsigned blocks = (unsigned)((threads + 255) / 256);
        const int nx = topo.xcds;
        const int local = nblocks % nx == 0 && blocks % nx == 0 &&
                          ((size_t)T * a.G * (hd / 4)) % 256 == 0;
        hipLaunchKernelGGL(split_combine_kernel, dim3(blocks), dim3(256), 0, s, (const float*)a.ws,
                           out, total, p.nsplit, hd, T, a.G, nkv, local, nx);
    }
    return dg::launch_status(fn);
}

}  // namespace

extern "C" int dg_attn_split_gqa(const float* q, const float* kc, const float* vc, const float* k,
                                 const float* v, float* out, int batch, int T, int ctx, int nh,
                                 int nkv, int hd, float scale, int causal, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return attn_call("dg_attn_split_gqa", q, kc, vc, k, v, out, batch, T, ctx, nh, nkv, hd, scale,
                     causal, workspace, workspace_bytes, stream, 0, nullptr, nullptr, nullptr, 0u,
                     0.0f, 0);
}

extern "C" int dg_attn_split_gqa_qnorm(const float* q, const float* wq, const float* cs,
                                       const float* kc, const float* vc, const float* k,
                                       const float* v, float* out, int batch, int T, int ctx,
                                       int nh, int nkv, int hd, unsigned qflags, float eps,
                                       float scale, int causal, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    const char* fn = "dg_attn_split_gqa_qnorm";
    if (qflags & ~(DG_NORM_WEIGHTED | DG_NORM_ROPE | DG_NORM_SKIP))
        return dg::fail(DG_EINVAL, "%s: unknown flag bits 0x%x", fn, qflags);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return dg::fail(DG_EINVAL, "%s: eps must be finite and >= 0", fn);
    const bool need_w = (qflags & DG_NORM_WEIGHTED) && !(qflags & DG_NORM_SKIP);
    const bool need_cs = (qflags & DG_NORM_ROPE) != 0;
    const bool empty = batch == 0 || T == 0;
    if (!empty && need_w && !wq) return dg::fail(DG_EINVAL, "%s: WEIGHTED set but wq is NULL", fn);
    if (!empty && need_cs && !cs) return dg::fail(DG_EINVAL, "%s: ROPE set but cs is NULL", fn);
    return attn_call(fn, q, kc, vc, k, v, out, batch, T, ctx, nh, nkv, hd, scale, causal,
                     workspace, workspace_bytes, stream, 1, need_w ? wq : nullptr, nullptr,
                     need_cs ? cs : nullptr, qflags, eps, 0);
}

extern "C" int dg_attn_split_gqa_qkvnorm(const float* q, const float* wq, const float* k,
                                         const float* wk, const float* v, const float* cs,
                                         const float* kc, const float* vc, float* out, int batch,
                                         int T, int ctx, int nh, int nkv, int hd, unsigned flags,
                                         float eps, float scale, int causal, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    const char* fn = "dg_attn_split_gqa_qkvnorm";
    if (flags & ~(DG_NORM_WEIGHTED | DG_NORM_ROPE))
        return dg::fail(DG_EINVAL, "%s: flag bits 0x%x not accepted (WEIGHTED and ROPE only)", fn,
                        flags);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return dg::fail(DG_EINVAL, "%s: eps must be finite and >= 0", fn);
    const bool need_w = (flags & DG_NORM_WEIGHTED) != 0;
    const bool need_cs = (flags & DG_NORM_ROPE) != 0;
    const bool empty = batch == 0 || T == 0;
    if (!empty && need_w && (!wq || !wk))
        return dg::fail(DG_EINVAL, "%s: WEIGHTED set but wq or wk is NULL", fn);
    if (!empty && need_cs && !cs) return dg::fail(DG_EINVAL, "%s: ROPE set but cs is NULL", fn);
    return attn_call(fn, q, kc, vc, k, v, out, batch, T, ctx, nh, nkv, hd, scale, causal,
                     workspace, workspace_bytes, stream, 2, need_w ? wq : nullptr,
                     need_w ? wk : nullptr, need_cs ? cs : nullptr, flags, eps, 0);
}

extern "C" int dg_attn_split_gqa_kv16(const float* q, const void* kc, const void* vc, const void* k,
                                      const void* v, float* out, int batch, int T, int ctx, int nh,
                                      int nkv, int hd, float scale, int causal, int kv_format,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "dg_attn_split_gqa_kv16";
    if (kv_format != DG_KV_F16 && kv_format != DG_KV_BF16)
        return dg::fail(DG_EINVAL, "%s: kv_format must be DG_KV_F16 or DG_KV_BF16, got %d", fn, kv_format);
    return attn_call(fn, q, kc, vc, k, v, out, batch, T, ctx, nh, nkv, hd, scale, causal, workspace,
                     workspace_bytes, stream, 0, nullptr, nullptr, nullptr, 0u, 0.0f, kv_format);
}

extern "C" int dg_attn_split_gqa_noalloc(const float* q, const float* kc, const float* vc,
                                         const float* k, const float* v, float* out, int batch,
                                         int T, int ctx, int nh, int nkv, int hd, float scale,
                                         int causal, void* stream) {
    return attn_call("dg_attn_split_gqa_noalloc", q, kc, vc, k, v, out, batch, T, ctx, nh, nkv,
                     hd, scale, causal, nullptr, 0, stream, 0, nullptr, nullptr, nullptr, 0u,
                     0.0f, 0, true);
}
