// relpos_flash.hip -- relpos_flash_attn(_windows): vision attention with the decomposed
// relative-position bias, flash style, on gfx950.
//
// Follows inferencelayer 0.2.8, src/deepencoder_gpu.rs: kernel SAM_SCORES fixes the score,
//   scale*<q_i,k_j> + <q_i, Rh[qy,ky]> + <q_i, Rw[qx,kx]>  (bias on the unscaled q),
// kernel DHDW hoists the two bias dot products out of the n^2 loop, `flash_reg_src` runs the
// online softmax over 64-wide chunks with hd fixed at 64, and `sam_attn_buf` fixes the fused
// qkv layout (q | k | v per token, heads contiguous) and the scale 1/sqrt(hd).  The windowed
// SAM blocks that the page's encoder cost model counts (25 windows of 14 x 14 tokens) are the
// same attention run independently per window with shared tables: a batch of grids.
//
// The hoisted bias rows (dh: gh floats, dw: gw floats per (window, head, query), in log2
// units), the page's DHDW step, are formed as small matrix products by the attention
// workgroups themselves where their queries allow it (8 x 8 patches of large grids, the
// windowed grids), else by a bias pass into the workspace; without a workspace, each
// attention workgroup forms the dot products of its own queries in a prologue.  The attention
// is the flash loop of flash_core.hpp with its tile products on the bf16 matrix pipe
// (kRelF32OnBf16).  For large grids a workgroup is 2
// groups of 32 queries x 4 wavefronts; the 4 wavefronts of a group take every 4th 32-key tile
// (stages of 128 keys, double-buffered direct global->LDS tiles) and merge their softmax
// states at the end.  Small grids use the shapes of RelShape.  The bias enters each score
// through the MFMA accumulator's starting value (see relpos_flash_kernel).  64-query
// workgroups give 768 workgroups at the 64x64-grid, 12-head shape: three full rounds on an
// MI355X's 256 CUs.
#include "bf16x3.hpp"
#include "dg_common.hpp"
#include "flash_core.hpp"

namespace {

using dgk::f32x16;
constexpr int HD = 64;
constexpr int kWaves = 8;
// A workgroup of kWavesT wavefronts is kQGroups = kWavesT / kParts query groups of 32 times
// kParts wavefronts per group, each taking every kParts-th key tile:
//  * 2 x 4 for large grids (8 wavefronts, 64 queries, 4-way key split);
//  * 4 x 2 for small ones (8 wavefronts, 128 queries, 2-way), where fewer, longer-running
//    workgroups amortise their prologue and merge;
//  * 4 x 1 for small grids of at most 16 rows of at most 32, such as 14x14 windows (4
//    wavefronts, 128 queries, no key split; row tiles only, as every wavefront takes every
//    tile): with its height-bias table cut to 16 rows and single-buffered stages (one f32
//    tile and its bf16 planes) a workgroup needs 48 KiB of LDS, so three fit on a CU beside
//    each other and the windows' workgroups run in one round, each CU's matrix pipes kept
//    busy by whichever workgroup is not waiting.  Used when the launch has more workgroups
//    than the GPU has CUs.
template <int kParts, int kWavesT = 8>
struct RelShape {
    static constexpr int kQGroups = kWavesT / kParts;
    static constexpr int kBlockQ = kQGroups * dgk::kQuery;
    static constexpr int kTabRows = kWavesT == 4 ? 16 : 64;   // height-bias table rows (>= gh)
};
constexpr int kMaxGrid = 64;                  // gh, gw <= 64
constexpr int kSmallGrid = 512;               // grids of at most this many tokens use 4 x 2 (or 4 x 1)
constexpr int kSmallRows = 16;                // ... and 4 x 1 when gh is at most this

struct RelArgs {
    const float* qkv;  // [nwin][n][3W]
    const float* rh;
    const float* rw;
    const float* dhw;  // precomputed bias rows, or null
    // the dh row of (window, head, query) row index r = (win * heads + head) * n + query sits at
    // dhw + r * dh_stride, its dw row at dhw + dw_off + r * dw_stride (floats)
    size_t dw_off;
    int dh_stride, dw_stride;
    float* out;        // [nwin][n][W]
    int n, gh, gw, heads, W, nwin;
    int qblocks, nblocks;
    int nxcd;    // XCDs of the device (workgroup placement)
    float qmul;  // scale * log2(e)
    // key tiling (see make_tiling): tile t starts at key (t >> tsh) * ta + (t & tmsk) * tb and
    // holds min(tl0 + (t & tmsk) * td, n - start) keys
    int tsh, ta, tmsk, tb, tl0, td, ntiles;
    // windowed grids (gh, gw <= 16): relpos_bias16_kernel's bias row layout, [dh (gh4 floats) |
    // dw] with stride brs floats
    int gh4, brs;
    // 4 x 1 shape on a windowed grid (gh, gw <= 16) with tables: each workgroup forms the bias
    // rows of its queries itself (no bias pass, no workspace)
    int lines;
};

using dg::xcd_remap;

// Reads the height-bias table in LDS (a separate array that the direct-to-LDS loads never
// write).
__device__ inline float tab_read(const float* __restrict__ tab, int i) { return tab[i]; }

// Bias rows in log2 units, the page's DHDW step, as small matrix products on MFMA.  A "line"
// is one grid row qy (its gw queries against the gh table rows Rh[qy, :]) or one grid column qx
// (its gh queries against Rw[qx, :]); its output is [queries x table rows] = Q_line T^T with a
// 64-long contraction.  One wavefront computes one 32x32 tile of one line: lane l supplies
// query row l%32 (A) and table row l%32 (B), both read straight from memory in the
// contraction order of the attention (half h holds chunks 8g+4h..8g+4h+3), and the 16
// accumulators hold 16 queries of table row l%32.  Output rows follow the page's buffers:
// dh [nwin][heads][n][gh], then dw [nwin][heads][n][gw].
constexpr int kBiasWaves = 4;

// Both bias kernels number their workgroups through xcd_remap over a grid padded to a multiple
// of the XCD count (the padding workgroups have no task), so the rows of one (window, head) are written on
// the XCD whose attention workgroups read them: writing lines that another XCD's L2 has just
// read was measured to be the slow case for the split-KV workspace.
//
// Lines of at most 16 queries against at most 16 table rows (windowed grids in the 8-wavefront
// shapes; the 4-wavefront shape forms its lines itself, see form_lines): one 16x16 tile per
// line with v_mfma_f32_16x16x4f32, a quarter of the 32x32 tile's matrix work.  Lane l
// supplies query row l%16 (A) and table row l%16 (B) at contraction index k = l/16; step
// 4c+e contracts element 16c+4k+e, so in each of the 4 float4 loads per operand the 4 lanes
// of a row read 64 contiguous bytes.  The 4 accumulators hold queries 4*(l/16)+r of table
// row l%16.  One wavefront per line (measured fastest: two or four lines per wavefront, with
// their loads in flight together, took 12.0 and 14.7 us against 10.3 for the SAM windows).
// The output is one row per (window, head, query), dh then dw, each part padded to a multiple
// of 4 floats (read through RelArgs' dh_stride, dw_off, dw_stride); the head is the fastest-varying task
// index, so the wavefronts running together read the q slices of all heads of the same tokens,
// which lie next to each other in each qkv row.
__global__ void __launch_bounds__(64 * kBiasWaves) relpos_bias16_kernel(RelArgs a, float* __restrict__ dhw,
                                                                       int ntasks) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, l16 = lane & 15, kq = lane >> 4;
    const int task = xcd_remap(blockIdx.x, gridDim.x, a.nxcd) * kBiasWaves +
                     __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (task >= ntasks) return;  // wave-uniform; task = (win * (gh + gw) + line) * heads + head
    const int head = task % a.heads;
    const int wl = task / a.heads;
    const int line = wl % (a.gh + a.gw), win = wl / (a.gh + a.gw);
    const int unit = win * a.heads + head;
    // line < gh: grid row `line` (gw queries) against rh[line] (gh rows); else grid column
    // p = line - gh (gh queries) against rw[p] (gw rows)
    const bool col = line >= a.gh;
    const int p = col ? line - a.gh : line;
    const int nq = col ? a.gh : a.gw, nr = col ? a.gw : a.gh;
    auto qidx = [&](int v) { return col ? v * a.gw + p : p * a.gw + v; };
    const size_t rs = (size_t)3 * a.W;
    const float* qr = a.qkv + ((size_t)win * a.n + qidx(min(l16, nq - 1))) * rs + head * HD + 4 * kq;
    const float* tr = (col ? a.rw + ((size_t)p * a.gw + min(l16, nr - 1)) * HD
                           : a.rh + ((size_t)p * a.gh + min(l16, nr - 1)) * HD) + 4 * kq;
    float qv[16], tv[16];
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qr + 4 * c);
        const float4 y = *reinterpret_cast<const float4*>(tr + 4 * c);
        qv[c] = x.x; qv[c + 1] = x.y; qv[c + 2] = x.z; qv[c + 3] = x.w;
        tv[c] = y.x; tv[c + 1] = y.y; tv[c + 2] = y.z; tv[c + 3] = y.w;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 16; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[st], tv[st], acc, 0, 0, 0);
    if (l16 >= nr) return;
    // one row of gh4 + gw4 floats per (window, head, query): dh at 0, dw at gh4
    float* base = dhw + (size_t)unit * a.n * a.brs + (col ? a.gh4 : 0) + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int v = 4 * kq + r;   // accumulator r: query on the line
        if (v < nq) base[(size_t)qidx(v) * a.brs] = acc[r] * dgk::kLog2e;
    }
}

__global__ void __launch_bounds__(64 * kBiasWaves) relpos_bias_kernel(RelArgs a, float* __restrict__ dhw,
                                                                     long long ntasks) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
    const long long task =
        (long long)xcd_remap(blockIdx.x, gridDim.x, a.nxcd) * kBiasWaves + (threadIdx.x >> 6);
    if (task >= ntasks) return;  // wave-uniform
    // task = ((unit * (gh + gw) + line) * 2 + qt) * 2 + rt, unit = win * heads + head
    const int rt = (int)(task & 1), qt = (int)((task >> 1) & 1);
    const long long lt = task >> 2;
    const int line = (int)(lt % (a.gh + a.gw));
    const int unit = (int)(lt / (a.gh + a.gw));
    const int head = unit % a.heads, win = unit / a.heads;
    const bool is_h = line < a.gh;
    const int nq = is_h ? a.gw : a.gh;      // queries on this line
    const int nr = is_h ? a.gh : a.gw;      // table rows (ky or kx)
    if (qt * 32 >= nq || rt * 32 >= nr) return;
    const int u = qt * 32 + l32, rrow = rt * 32 + l32;
    auto qidx = [&](int v) { return is_h ? line * a.gw + v : v * a.gw + (line - a.gh); };
    const size_t rs = (size_t)3 * a.W;
    const float* qr = a.qkv + ((size_t)win * a.n + qidx(min(u, nq - 1))) * rs + head * HD;
    const float* tr = (is_h ? a.rh + (size_t)line * a.gh * HD : a.rw + (size_t)(line - a.gh) * a.gw * HD) +
                      (size_t)min(rrow, nr - 1) * HD;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int g = 0; g < HD / 8; ++g) {
        const float4 qv = *reinterpret_cast<const float4*>(qr + 8 * g + 4 * half);
        const float4 tv = *reinterpret_cast<const float4*>(tr + 8 * g + 4 * half);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.x, tv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.y, tv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.z, tv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.w, tv.w, acc, 0, 0, 0);
    }
    if (rrow >= nr) return;
    float* base = dhw + (is_h ? (size_t)unit * a.n * a.gh
                              : (size_t)a.nwin * a.heads * a.n * a.gh + (size_t)unit * a.n * a.gw);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int v = qt * 32 + dgk::key_of(r, half);   // accumulator row r: query on the line
        if (v < nq) base[(size_t)qidx(v) * nr + rrow] = acc[r] * dgk::kLog2e;
    }
}

constexpr int kWinGrid = 16;   // windowed grids: gh, gw <= 16 (bias lines fit one 16 x 16 tile)
constexpr unsigned kRsrcWord3 = 0x00020000u;   // raw 32-bit buffer descriptor (gfx9 family)

// Key tiles are cut along grid rows, so that every lane sees the same kx at the same register
// slot in every tile:
//  * gw <= 32 ("row tiles"): a tile holds rpt = min(8, 32 / gw) whole grid rows (rpt * gw keys,
//    the rest of the 32 slots is padding);
//  * 32 < gw <= 64 ("half-row tiles"): a tile holds one half of a grid row, kh = ceil(gw / 2)
//    or gw - kh keys; as a wavefront takes every 4th tile it always sees the same half.
// The lane's 16 width-bias terms dw[q][kx] then stay in registers as the starting value of the
// score accumulator, with -inf at padding slots (which masks them for free), and the height
// bias dh[q][ky] - ref rides in ceil(rpt / 2) extra MFMA steps: step m contracts over the two
// rows 2m and 2m+1 of the tile, with A one-hot on the key's row within the tile.
// A compile-time double-buffer index.
template <int B>
struct BufC {
    static constexpr int value = B;
};

struct Tiling {
    int half_rows;   // 1: half-row tiles; 0: row tiles
    int rpt;         // grid rows per tile (row tiles)
    int kh;          // keys in the first half of a row (half-row tiles)
    int kpt;         // keys in a full tile
    int ntiles;
    int nshift;      // extra MFMA steps for the height bias
};

__host__ __device__ inline Tiling make_tiling(int gh, int gw) {
    Tiling t;
    if (gw > 32) {
        t.half_rows = 1; t.rpt = 1; t.kh = (gw + 1) / 2; t.kpt = t.kh;
        t.ntiles = 2 * gh; t.nshift = 1;
    } else {
        t.half_rows = 0; t.rpt = min(8, 32 / gw); t.kh = 0; t.kpt = t.rpt * gw;
        t.ntiles = (gh + t.rpt - 1) / t.rpt; t.nshift = (t.rpt + 1) / 2;
    }
    return t;
}

// Scores and the value product run on the bf16 matrix pipe: q, K, V and the probabilities taken
// as three bf16 terms, every product as six exact bf16 products summed in f32 (bf16x3.hpp);
// within 2^-23 |q||k| of each f32 product, typically 2^-29.  The 8-wavefront grid shapes split
// each K and V value in registers as it is read from LDS (two query groups share each tile, so
// each value is split twice); the 4-wavefront shape, whose four query groups all take every
// tile, splits each staged tile once into bf16 planes in LDS (bf16x3.hpp, split_stage).  The
// bias terms stay on f32 MFMA.  false: f32 MFMA throughout.
constexpr bool kRelF32OnBf16 = true;

// kFull: every tile holds 32 keys (no padding slots, no short last tile); kOneShift: the height
// bias takes one MFMA step (at most two grid rows per tile).
// kPatch: the workgroup's 64 queries are an 8 x 8 patch of the grid (both sides multiples of
// 8, half-row tiles) and the workgroup forms their bias rows itself on MFMA (see below).
template <bool kFull, bool kOneShift, int kParts, int kWavesT, bool kPatch = false>
__global__ void __launch_bounds__(64 * kWavesT)
    __attribute__((amdgpu_waves_per_eu(kWavesT == 4 ? 3 : 1))) relpos_flash_kernel(RelArgs a) {
    using TL = dgk::Tile<HD>;
    constexpr int kQGroups = RelShape<kParts, kWavesT>::kQGroups;
    constexpr int kBlockQ = RelShape<kParts, kWavesT>::kBlockQ;
    constexpr int kTabRows = RelShape<kParts, kWavesT>::kTabRows;
    // staging: [buffer][tile][K, V] and bias tables [group][ky][query] (dh)
    constexpr int kOStride = HD + 4;   // row stride of the output rows restaged at the end
    // 4-wavefront shape on the bf16 pipe: one f32 staging buffer [K, V] of one tile, then the
    // tile's six bf16 planes (single-buffered: the next tile's loads go out once the split is
    // done): 40 KiB, 48 KiB with the height-bias table, so three workgroups fit on a CU.
    constexpr bool kPl = kRelF32OnBf16 && kWavesT == 4;
    static_assert(!kPl || kParts == 1, "the planes shape takes every tile");
    constexpr int kStageFloats =
        kPl ? 2 * TL::kFloats + 2 * 3 * bf3::Planes<HD>::kBytes / 4 : 2 * kParts * 2 * TL::kFloats;
    constexpr int kSmemFloats = kStageFloats > kBlockQ * kOStride ? kStageFloats : kBlockQ * kOStride;
    __shared__ __attribute__((aligned(16))) float smem[kSmemFloats];
    __shared__ float tab[kQGroups * kTabRows * dgk::kQuery];
    auto tile_ptr = [&](int buf, int tile, int isv) {
        return smem + ((buf * kParts + tile) * 2 + isv) * TL::kFloats;
    };
    char* const planes = reinterpret_cast<char*>(smem + 2 * TL::kFloats);   // kPl only

    int lid = xcd_remap(blockIdx.x, a.nblocks, a.nxcd);
    // Two query blocks per (window, head), the second the lighter (196 queries: 128 and 68):
    // within each XCD the first blocks go out first, so the third workgroups that some CUs
    // receive are light ones.
    if (kPl && a.qblocks == 2) lid = dg::full_first(lid, a.nblocks, a.nxcd);
    const int qb = lid % a.qblocks;
    const int unit = lid / a.qblocks;          // win * heads + head
    const int head = unit % a.heads, win = unit / a.heads;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    // in the 8-wavefront shapes wavefronts w and w+4 share a SIMD: the same group, parts p and
    // p + kParts/2
    const int grp = wave & (kQGroups - 1), part = wave / kQGroups;
    const size_t rs = (size_t)3 * a.W;  // qkv row stride (floats)
    const Tiling tl = make_tiling(a.gh, a.gw);

    static_assert(!kPatch || kBlockQ == 64, "a patch is 64 queries");
    // patch mode: query p of the workgroup (p = 32 grp + l32) is patch cell (p / 8, p % 8)
    const int pxn = a.gw >> 3;
    const int py0 = kPatch ? 8 * (qb / pxn) : 0, px0 = kPatch ? 8 * (qb % pxn) : 0;
    auto patch_token = [&](int p) { return (py0 + (p >> 3)) * a.gw + px0 + (p & 7); };
    const int qfirst = qb * kBlockQ + grp * dgk::kQuery;
    const int qi = kPatch ? patch_token(grp * dgk::kQuery + l32) : qfirst + l32;
    const bool valid = qi < a.n;
    const float* qkvw = a.qkv + (size_t)win * a.n * rs;   // this window's rows
    const float* qrow = qkvw + (size_t)(valid ? qi : 0) * rs + head * HD;
    const bool active = qfirst < a.n;
    const bool bias = a.rh != nullptr;
    float* dh_tab = tab + grp * kTabRows * dgk::kQuery;   // [ky][query]

    // Where the lane's 16 score slots sit in its tiles (the same in every tile of this wave).
    const int parity = part & 1;                           // half-row tiles: which half
    const int tlen_w = tl.half_rows ? (parity ? a.gw - tl.kh : tl.kh) : tl.kpt;
    const int kx0 = tl.half_rows ? parity * tl.kh : 0;
    // A operand of the height-bias steps: this lane supplies key row l32 at contraction index
    // `half`; it is 1 in step m iff that key lies in tile row 2m + half.
    const int arow = l32 < tlen_w ? (tl.half_rows ? 0 : l32 / a.gw) : -1;
    const float aone = arow == half ? 1.0f : 0.0f;   // the single step's A (kOneShift)

    constexpr bool kBf16Pipe = kRelF32OnBf16 && kWavesT == 8;
    float qreg[kPl ? 1 : HD / 2];
    bf3::QSplit<kBf16Pipe || kPl ? HD : 16> q3;

    // Prologue: the dh rows of this group's queries (all ky) into LDS, and the lane's dw terms.
    f32x16 dwreg;
    const int qx = valid ? qi % a.gw : 0, qy = valid ? qi / a.gw : 0;
    // Windowed grids in the 4 x 1 shape on the bf16 pipe (a.lines): the bias rows of the
    // workgroup's queries as small matrix products on v_mfma_f32_16x16x4f32, as
    // relpos_bias16_kernel forms them: a row line is grid row qy's queries against rh[qy] (gh
    // table rows), a column line grid column qx's queries against rw[qx] (gw rows), each one
    // 16 x 16 tile with a 64-long contraction.  The workgroup's queries lie on grid rows
    // qy0..qy1 (at most 16), so it takes those row lines and every column line restricted to
    // those rows; wavefront w takes lines w, w + 4, ..., three at a time with all their table
    // loads in flight together.  The query operands come from the workgroup's query rows,
    // staged in LDS once (each row serves a row line and a column line).  Row products go to
    // the dh tables, column products to a [query][kx] table beside the staged rows, from which
    // each lane then takes its dw terms.  Products of queries outside the workgroup are formed
    // and dropped.  Measured on the SAM windows (per call): lines one at a time 46.4 us, three
    // at a time 46.3 us, query rows from LDS 43.8 us; forming the lines after the first
    // stage's loads had gone out, 48.0 us.
    auto form_lines = [&]() {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const int l16 = lane & 15, kq = lane >> 4;
        const int q0 = qb * kBlockQ;
        const int qy0 = q0 / a.gw, qy1 = (min(q0 + kBlockQ, a.n) - 1) / a.gw;
        const int nrl = qy1 - qy0 + 1, nl = nrl + a.gw;
        // The workgroup's query rows (this head's 64 elements) are staged in LDS first, each
        // read by one row line and one column line: row r at smem + 64 r, its 16-byte chunk j
        // at position j ^ (r mod 16), so the 16 rows of a line's operand read spread over the
        // banks.  The [query][kx] table follows them.  Both lie in the stage and plane areas,
        // free until the first stage's loads.
        constexpr int kDwStride = 16;
        static_assert(kBlockQ * (HD + kDwStride) <= kSmemFloats, "query rows and dw table fit");
        float* const qst = smem;
        float* const dwt = smem + kBlockQ * HD;   // [kBlockQ][kDwStride]
        // Line li: grid row qy0 + li (li < nrl) or grid column li - nrl.
        auto load_table = [&](int li, float4 (&y)[4]) {
            const bool col = li >= nrl;
            const int p = col ? li - nrl : qy0 + li;   // the line's grid column or row
            const int nr = col ? a.gw : a.gh;
            const float* tr = (col ? a.rw + ((size_t)p * a.gw + min(l16, nr - 1)) * HD
                                   : a.rh + ((size_t)p * a.gh + min(l16, nr - 1)) * HD) + 4 * kq;
#pragma unroll
            for (int c = 0; c < 4; ++c) y[c] = *reinterpret_cast<const float4*>(tr + 16 * c);
        };
        auto load_query = [&](int li, float4 (&x)[4]) {
            const bool col = li >= nrl;
            const int p = col ? li - nrl : qy0 + li;
            const int nq = col ? nrl : a.gw;
            const int v = min(l16, nq - 1);
            const int tok = col ? (qy0 + v) * a.gw + p : p * a.gw + v;
            // a slot outside the workgroup reads some staged row; its products are dropped
            const int r = min(max(tok - q0, 0), kBlockQ - 1);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                x[c] = *reinterpret_cast<const float4*>(qst + r * HD + 4 * ((4 * c + kq) ^ (r % 16)));
        };
        // kLB lines per round trip: all their table loads go out, then their products are
        // formed; the first batch's go out before the query rows are staged
        constexpr int kLB = 3;
        float4 y[kLB][4];
#pragma unroll
        for (int bl = 0; bl < kLB; ++bl)
            if (wave + bl * kWavesT < nl) load_table(wave + bl * kWavesT, y[bl]);
#pragma unroll
        for (int i = 0; i < kBlockQ * (HD / 4) / (64 * kWavesT); ++i) {
            const int id = tid + 64 * kWavesT * i, r = id / (HD / 4), j = id % (HD / 4);
            const float4 v = *reinterpret_cast<const float4*>(
                qkvw + (size_t)min(q0 + r, a.n - 1) * rs + head * HD + 4 * j);
            *reinterpret_cast<float4*>(qst + r * HD + 4 * (j ^ (r % 16))) = v;
        }
        if (!valid)
            for (int ky = half; ky < a.gh; ky += 2) dh_tab[ky * dgk::kQuery + l32] = 0.0f;
        __syncthreads();
        for (int l0 = wave; l0 < nl; l0 += kLB * kWavesT) {   // wave-uniform
            if (l0 != wave) {
#pragma unroll
                for (int bl = 0; bl < kLB; ++bl)
                    if (l0 + bl * kWavesT < nl) load_table(l0 + bl * kWavesT, y[bl]);
            }
            float4 x[kLB][4];
#pragma unroll
            for (int bl = 0; bl < kLB; ++bl)
                if (l0 + bl * kWavesT < nl) load_query(l0 + bl * kWavesT, x[bl]);
#pragma unroll
            for (int bl = 0; bl < kLB; ++bl) {
                const int li = l0 + bl * kWavesT;
                if (li >= nl) break;
                const bool col = li >= nrl;
                const int p = col ? li - nrl : qy0 + li;
                const int nq = col ? nrl : a.gw, nr = col ? a.gw : a.gh;
                // lane l supplies query slot l%16 (A) and table row l%16 (B) at contraction
                // index l/16; step 4c+e contracts element 16c + 4(l/16) + e; accumulator r holds
                // query slot 4(l/16) + r against table row l%16
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[bl][c].x, y[bl][c].x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[bl][c].y, y[bl][c].y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[bl][c].z, y[bl][c].z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[bl][c].w, y[bl][c].w, acc, 0, 0, 0);
                }
                if (l16 < nr) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int v = 4 * kq + r;
                        const int tok = col ? (qy0 + v) * a.gw + p : p * a.gw + v;
                        const int loc = tok - q0;   // index in the workgroup
                        if (v < nq && loc >= 0 && loc < kBlockQ && tok < a.n) {
                            const float val = acc[r] * dgk::kLog2e;
                            if (col)
                                dwt[loc * kDwStride + l16] = val;
                            else
                                tab[((loc >> 5) * kTabRows + l16) * dgk::kQuery + (loc & 31)] = val;
                        }
                    }
                }
            }
        }
        // the attention's own query operand (the load_q_bf16x3 layout), from the staged rows,
        // before the barrier after which the first stage's loads may overwrite them
        {
            const int r = grp * dgk::kQuery + l32;   // the lane's query, index in the workgroup
            const bf3::SplitWeights w;
#pragma unroll
            for (int st = 0; st < HD / 16; ++st) {
                float x[8];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int ch = 4 * st + 2 * half + c;   // elements 16 st + 8 half + 4 c ..
                    const float4 v = valid ? *reinterpret_cast<const float4*>(qst + r * HD + 4 * (ch ^ (r % 16)))
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
                    x[4 * c + 0] = v.x * a.qmul;
                    x[4 * c + 1] = v.y * a.qmul;
                    x[4 * c + 2] = v.z * a.qmul;
                    x[4 * c + 3] = v.w * a.qmul;
                }
                if constexpr (kPl) bf3::split8(x, w, q3.h[st], q3.m[st], q3.l[st]);
            }
        }
        __syncthreads();
        const float* dwq = dwt + (grp * dgk::kQuery + l32) * kDwStride;
        // kx = i mod gw without an integer division per slot: (i + 1/2) / gw lies at least
        // 1/(2 gw) from an integer, far beyond the rounding of the product, so its floor is exact
        const float inv_gw = 1.0f / (float)a.gw;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = dgk::key_of(r, half);
            const int kx = i - a.gw * (int)(((float)i + 0.5f) * inv_gw);
            dwreg[r] = i < tlen_w ? (valid ? dwq[kx] : 0.0f) : -INFINITY;
        }
    };
    if (kPatch && bias) {
        // The bias rows of the patch as small matrix products on v_mfma_f32_16x16x4f32:
        // wavefront w takes patch row w (8 queries of grid row py0 + w against rh[py0 + w]) and
        // patch column w (8 queries of grid column px0 + w against rw[px0 + w]).  A line's
        // product D^T = T Q^T has 16 table rows per tile (up to 4 tiles) and 16 columns, the 8
        // queries twice (columns n and n + 8 alike).  Lane l supplies table row l%16 (A) and
        // query l%8 (B) at contraction index k = l/16; step 4c+e contracts element 16c+4k+e.
        // Accumulator i holds table row 4*(l/16)+i of the tile for query (l%16) % 8.  Row
        // products go to the dh tables; column products to a [query][kx] table in the second
        // stage buffer (free until stage 1), from which each lane then takes its dw terms.
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const int l16 = lane & 15, kq = lane >> 4;
        float* dwt = smem + 2 * kParts * TL::kFloats;   // [64 queries][kDwStride]
        constexpr int kDwStride = 64 + 4;
        float qb_h[16], qb_w[16];
        const int qh = (py0 + wave) * a.gw + px0 + (l16 & 7);        // row segment's query
        const int qv = (py0 + (l16 & 7)) * a.gw + px0 + wave;        // column segment's query
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 x = *reinterpret_cast<const float4*>(qkvw + (size_t)qh * rs + head * HD + 16 * c + 4 * kq);
            const float4 y = *reinterpret_cast<const float4*>(qkvw + (size_t)qv * rs + head * HD + 16 * c + 4 * kq);
            qb_h[4 * c] = x.x; qb_h[4 * c + 1] = x.y; qb_h[4 * c + 2] = x.z; qb_h[4 * c + 3] = x.w;
            qb_w[4 * c] = y.x; qb_w[4 * c + 1] = y.y; qb_w[4 * c + 2] = y.z; qb_w[4 * c + 3] = y.w;
        }
        // One table tile at a time: loading all eight tiles of both lines up front made the
        // prologue slower (14.9 against 11.9 us per workgroup), every workgroup of a round
        // asking for its tables at once.
        auto line = [&](const float* table, int nrows, const float (&qv_)[16], auto put) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (16 * kt < nrows) {
                    const float* tr = table + (size_t)min(16 * kt + l16, nrows - 1) * HD + 4 * kq;
                    float tv[16];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float4 t = *reinterpret_cast<const float4*>(tr + 16 * c);
                        tv[4 * c] = t.x; tv[4 * c + 1] = t.y; tv[4 * c + 2] = t.z; tv[4 * c + 3] = t.w;
                    }
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 16; ++st)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[st], qv_[st], acc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * kt + 4 * kq + i;
                        if (l16 < 8 && row < nrows) put(row, acc[i] * dgk::kLog2e);
                    }
                }
            }
        };
        // patch row `wave`: queries p = 8 wave + c, in group p / 32 at index p % 32
        line(a.rh + (size_t)(py0 + wave) * a.gh * HD, a.gh, qb_h, [&](int ky, float v) {
            const int p = 8 * wave + l16;
            tab[((p >> 5) * kTabRows + ky) * dgk::kQuery + (p & 31)] = v;
        });
        // patch column `wave`: queries p = 8 r + wave
        line(a.rw + (size_t)(px0 + wave) * a.gw * HD, a.gw, qb_w, [&](int kx, float v) {
            dwt[(8 * l16 + wave) * kDwStride + kx] = v;
        });
        __syncthreads();
        const int p = grp * dgk::kQuery + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = dgk::key_of(r, half);
            dwreg[r] = i < tlen_w ? dwt[p * kDwStride + min(kx0 + i, a.gw - 1)] : -INFINITY;
        }
    } else if (kPl && bias && a.lines) {
        form_lines();
    } else if (bias && active && a.dhw) {
        const size_t row = (size_t)unit * a.n + (valid ? qi : 0);
        const float* dhq = a.dhw + row * a.dh_stride;
        const float* dwq = a.dhw + a.dw_off + row * a.dw_stride;
        for (int ky = part * 2 + half; ky < a.gh; ky += 2 * kParts)
            dh_tab[ky * dgk::kQuery + l32] = valid ? dhq[ky] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = dgk::key_of(r, half);
            const int kx = min(tl.half_rows ? kx0 + i : i % a.gw, a.gw - 1);   // in range even
            dwreg[r] = i < tlen_w ? (valid ? dwq[kx] : 0.0f) : -INFINITY;      // at padding slots
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
        for (int ky = part * 2 + half; ky < a.gh; ky += 2 * kParts)
            dh_tab[ky * dgk::kQuery + l32] = dot(a.rh + ((size_t)qy * a.gh + ky) * HD);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = dgk::key_of(r, half);
            const int kx = min(tl.half_rows ? kx0 + i : i % a.gw, a.gw - 1);
            dwreg[r] = i < tlen_w ? dot(a.rw + ((size_t)qx * a.gw + kx) * HD) : -INFINITY;
        }
    } else {
        for (int ky = part * 2 + half; ky < a.gh; ky += 2 * kParts) dh_tab[ky * dgk::kQuery + l32] = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) dwreg[r] = dgk::key_of(r, half) < tlen_w ? 0.0f : -INFINITY;
    }

    // Tile t's first key and length (wave-uniform, branch-free).
    auto tile_start = [&](int t) { return (t >> a.tsh) * a.ta + (t & a.tmsk) * a.tb; };
    auto tile_len = [&](int t) { return min(a.tl0 + (t & a.tmsk) * a.td, a.n - tile_start(t)); };

    // Loads: the four wavefronts with part < 2 (one per SIMD) issue each stage's wave-wide
    // loads -- K and V of kParts tiles -- while their SIMD partners keep the matrix pipe busy
    // (in the 4 x 1 shape every wavefront issues, and the partners are other workgroups').  They
    // are buffer loads straight into LDS: the window's qkv rows are one buffer, the lane's
    // offset within a full tile is loop-invariant (a row rsub of its 4-row group and a 16-byte
    // chunk, K's chunks permuted as the reads expect) and the tile, the 4-row group and the k
    // or v column are a scalar offset, so a load costs no vector instruction.  A shorter tile
    // repeats its last key in the padding rows.
    constexpr int kLoadsPerWave = 2 * kParts * TL::kLoadsPerTile / 4;
    constexpr int R = TL::kRowsPerLoad;
    static_assert(TL::kChunks == 16 && R == 4, "the offsets below assume hd 64");
    const int pos = lane % TL::kChunks, rsub = lane / TL::kChunks;
    const unsigned rsb = (unsigned)(rs * 4);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(qkvw), 0, (int)((unsigned)a.n * rsb), (int)kRsrcWord3);
    const int colk = (a.W + head * HD) * 4, colv = (2 * a.W + head * HD) * 4;
    // lane offsets of full-tile loads: row rsub of load ld's 4 rows; K's chunk pos ^ (row % 16)
    // depends on ld % 4 only (row = 4 * ld + rsub < 32)
    unsigned koffs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) koffs[j] = (unsigned)rsub * rsb + 16u * (pos ^ (4 * j + rsub));
    const unsigned voffs = (unsigned)rsub * rsb + 16u * pos;
    auto issue_stage = [&](int st, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
            const int L = wave * kLoadsPerWave + i;
            const int tpart = L / TL::kLoadsPerTile, ld = L % TL::kLoadsPerTile;
            const int tile = tpart >> 1, isv = tpart & 1;
            // a tile past the last one reloads keys that exist (its results are never used)
            const int t = min(st * kParts + tile, a.ntiles - 1);
            const int j0 = tile_start(t);
            unsigned off;
            int soff;
            if (kFull) {
                off = isv || kPl ? voffs : koffs[i % 4];   // ld % 4 == i % 4 in every shape
                soff = (isv ? colv : colk) + (j0 + R * ld) * (int)rsb;
            } else {
                const int trow = ld * R + rsub;
                const unsigned coff = 16u * (isv || kPl ? pos : (pos ^ (trow % TL::kChunks)));
                off = (unsigned)min(trow, tile_len(t) - 1) * rsb + coff;
                soff = (isv ? colv : colk) + j0 * (int)rsb;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (dgk::lds_void*)(tile_ptr(buf, tile, isv) + ld * 256), 16, (int)off, soff, 0, 0);
        }
    };

    if constexpr (kPl) {
        if (!(bias && a.lines))   // with the lines, q3 was read from the staged query rows
            bf3::load_q_bf16x3<HD>(qrow, valid, half, a.qmul, q3, HD);
    } else {
        dgk::load_q<HD>(qrow, valid, half, a.qmul, qreg);
        if constexpr (kBf16Pipe) bf3::split_q_bf16x3<HD>(qreg, q3);
    }
    f32x16 o[TL::kGroups];
#pragma unroll
    for (int t = 0; t < TL::kGroups; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    const int nstage = (a.ntiles + kParts - 1) / kParts;
    if (wave < 4) issue_stage(0, BufC<0>{});
    // One stage; the stage loop is unrolled by two so that the buffer index is a constant and
    // the LDS reads of a tile take immediate offsets.
    int voff[TL::kGroups];   // planes: the lane's transposed-read offsets into a V plane
    if constexpr (kPl) bf3::vtr_offsets<HD>(lane, voff);
    auto stage = [&](int st, auto bufc) {
        constexpr int buf = kPl ? 0 : decltype(bufc)::value;
        constexpr int nbuf = kPl ? 0 : buf ^ 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // stage st has landed everywhere, stage st-1 is consumed (and the
                          // bias tables are complete before the first use)
        if constexpr (kPl) {
            // the workgroup splits the staged tile into its planes; the staging buffer is then
            // free for the next tile's loads
            bf3::split_stage<HD, 64 * kWavesT, 1>(reinterpret_cast<const char*>(smem), TL::kFloats * 4,
                                                  planes, 1, tid);
            __syncthreads();
        }
        const int t = st * kParts + part;
        // The height-bias table values of this tile (one per step; a row tile has at most 8 rows,
        // so at most 4 steps).  An LDS read issued after the next stage's loads makes the
        // compiler wait for all of them (s_waitcnt vmcnt(0)) before the tile's first K read, so
        // the issuing wavefront stalls until its next stage has landed.  In the 4 x 1 shape,
        // where every wavefront issues, the values are read before the loads go out (measured:
        // SAM windows 65.0 -> 64.1 us); in the 8-wavefront shapes the issuing wavefront's SIMD
        // partner covers the stall, and reading early measured slower (64 x 64: 450 -> 454 us).
        constexpr int kMaxShift = 4;
        float dhv[kMaxShift] = {0.0f, 0.0f, 0.0f, 0.0f};
        auto read_dh = [&]() {
            if (!(active && t < a.ntiles)) return;
            const int row0 = tl.half_rows ? (t >> 1) : t * tl.rpt;
            if (kOneShift) {
                dhv[0] = tab_read(dh_tab, min(row0 + (tl.half_rows ? 0 : half), a.gh - 1) * dgk::kQuery + l32);
            } else {
#pragma unroll
                for (int ms = 0; ms < kMaxShift; ++ms) {
                    const int ky = row0 + 2 * ms + half;
                    if (ms < tl.nshift && ky < a.gh) dhv[ms] = tab_read(dh_tab, ky * dgk::kQuery + l32);
                }
            }
        };
        if constexpr (kParts == 1) read_dh();
        if (wave < 4 && st + 1 < nstage) issue_stage(st + 1, BufC<nbuf>{});
        if constexpr (kParts != 1) read_dh();
        if (active && t < a.ntiles) {
            const float ref = dgk::ref_of(m);
            const int row0 = tl.half_rows ? (t >> 1) : t * tl.rpt;
            f32x16 s;
            if (kOneShift) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(aone, dhv[0] - ref, dwreg, 0, 0, 0);
            } else {
                s = dwreg;
#pragma unroll
                for (int ms = 0; ms < kMaxShift; ++ms)
                    if (ms < tl.nshift)
                        s = __builtin_amdgcn_mfma_f32_32x32x2f32(arow == 2 * ms + half ? 1.0f : 0.0f,
                                                                 dhv[ms] - ref, s, 0, 0, 0);
            }
            if constexpr (kPl)
                s = bf3::scores_planes<HD>(bf3::Planes<HD>::at(planes, 0, 0, 0), l32, half, q3, s);
            else if constexpr (kBf16Pipe)
                s = bf3::scores_f32_bf16x6<HD>(tile_ptr(buf, part, 0), l32, half, q3, s);
            else
                s = dgk::scores_from<HD>(tile_ptr(buf, part, 0), l32, half, qreg, s);
            if (!kFull) {
                const int len = tile_len(t);
                if (len < tlen_w) {  // the last row tile is short
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (dgk::key_of(r, half) >= len) s[r] = -INFINITY;
                }
            }
            dgk::softmax_update<HD>(s, m, lsum, o);
            if constexpr (kPl)
                bf3::accumulate_pv_planes<HD>(bf3::Planes<HD>::at(planes, 0, 1, 0), voff, s, o);
            else if constexpr (kBf16Pipe)
                bf3::accumulate_pv_f32_bf16x6<HD>(tile_ptr(buf, part, 1), l32, half, s, o);
            else
                dgk::accumulate_pv<HD>(tile_ptr(buf, part, 1), l32, half, s, o);
        }
    };
    for (int st = 0; st < nstage; st += 2) {
        stage(st, BufC<0>{});
        if (st + 1 < nstage) stage(st + 1, BufC<1>{});
    }

    __syncthreads();
    dgk::group_merge<HD>(smem, grp, part, kParts, active, lane, m, lsum, o);
    const float ltot = lsum + __shfl_xor(lsum, 32);
    // The merged rows are restaged row-major in LDS (after every part-0 wavefront has read the
    // merge scratch) and written with 16 contiguous bytes per lane: whole 256-byte rows rather
    // than 8-byte pieces spread over 32 rows per instruction.
    __syncthreads();
    if (part == 0) {
        float* rows = smem + grp * dgk::kQuery * kOStride;
        const float inv = valid ? 1.0f / ltot : 0.0f;
        if constexpr (kPl)
            bf3::stage_row_blocked<HD>(rows, l32, inv, o, half);   // output rows of the V planes
        else
            dgk::stage_row<HD>(rows, l32, inv, o, half);
    }
    __syncthreads();
    constexpr int kChunksO = HD / 4;
    constexpr int kRowsPerPass = 64 * kWavesT / kChunksO;
#pragma unroll
    for (int r0 = 0; r0 < kBlockQ; r0 += kRowsPerPass) {
        const int rloc = r0 + tid / kChunksO, c = tid % kChunksO;
        const int q = kPatch ? patch_token(rloc) : qb * kBlockQ + rloc;
        if (q < a.n)
            *reinterpret_cast<float4*>(a.out + ((size_t)win * a.n + q) * a.W + head * HD + 4 * c) =
                *reinterpret_cast<const float4*>(smem + rloc * kOStride + 4 * c);
    }
}

}  // namespace

namespace {
// Grids whose lines fit one 16x16 tile (the windows): the 4 x 1 shape forms their bias rows
// itself; otherwise relpos_bias16_kernel writes them to the workspace.
bool win_grid(int gh, int gw) { return gh <= kWinGrid && gw <= kWinGrid; }
int round4(int x) { return (x + 3) & ~3; }
// Floats per (window, head, query) of bias rows: dh then dw, each padded to 4 floats for the
// 16x16 path; unpadded otherwise.
int bias_row_floats(int gh, int gw) { return win_grid(gh, gw) ? round4(gh) + round4(gw) : gh + gw; }

}  // namespace

extern "C" size_t relpos_flash_attn_windows_workspace_size(int nwin, int gh, int gw, int heads,
                                                          int hd) {
    if (nwin < 1 || gh < 1 || gw < 1 || heads < 1 || hd != HD || gh > kMaxGrid || gw > kMaxGrid)
        return 0;
    return (size_t)nwin * heads * gh * gw * bias_row_floats(gh, gw) * sizeof(float);
}

extern "C" size_t relpos_flash_attn_workspace_size(int gh, int gw, int heads, int hd) {
    return relpos_flash_attn_windows_workspace_size(1, gh, gw, heads, hd);
}

namespace {

template <int kParts, int kWavesT>
auto pick_flash(bool full, bool one) {
    return full ? (one ? relpos_flash_kernel<true, true, kParts, kWavesT>
                       : relpos_flash_kernel<true, false, kParts, kWavesT>)
                : (one ? relpos_flash_kernel<false, true, kParts, kWavesT>
                       : relpos_flash_kernel<false, false, kParts, kWavesT>);
}

// Grids whose attention workgroups form their own bias rows from an 8 x 8 patch of queries:
// large grids (64-query workgroups) cut into half-row tiles with both sides multiples of 8.
bool patch_grid(int gh, int gw) { return gh * gw > kSmallGrid && gw > 32 && gh % 8 == 0 && gw % 8 == 0; }

int relpos_call(const char* fn, const float* qkv, const float* rh, const float* rw, float* out,
                int nwin, int gh, int gw, int heads, int hd, float scale, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (nwin < 0 || gh < 0 || gw < 0 || heads < 0)
        return dg::fail(DG_EINVAL, "%s: negative size (nwin %d, gh %d, gw %d, heads %d)", fn, nwin,
                        gh, gw, heads);
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
    if (n == 0 || heads == 0 || nwin == 0) return dg::ok();
    if (!qkv || !out) return dg::fail(DG_EINVAL, "%s: qkv and out must be non-NULL", fn);
    size_t rows = 1;
    if (!dg::mul_ok(rows, nwin) || !dg::mul_ok(rows, n) || !dg::mul_ok(rows, 3LL * heads * HD))
        return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    const size_t W = (size_t)heads * HD;
    const size_t ntok = (size_t)nwin * n;
    const size_t need = relpos_flash_attn_windows_workspace_size(nwin, gh, gw, heads, hd);
    if (workspace && workspace_bytes < need)
        return dg::fail(DG_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                        workspace_bytes, need);
    const bool patch = rh && patch_grid(gh, gw);   // bias rows formed inside the attention
    const bool use_ws = workspace && rh && !patch;
    const dg::Span so(out, ntok * W * 4);
    const dg::Span sq(qkv, ntok * 3 * W * 4), sh(rh, (size_t)gh * gh * HD * 4),
        sw(rw, (size_t)gw * gw * HD * 4), sws(use_ws ? workspace : nullptr, need);
    if (so.overlaps(sq) || so.overlaps(sh) || so.overlaps(sw) || so.overlaps(sws))
        return dg::fail(DG_EINVAL, "%s: out overlaps an input or the workspace", fn);
    if (sws.overlaps(sq) || sws.overlaps(sh) || sws.overlaps(sw))
        return dg::fail(DG_EINVAL, "%s: workspace overlaps an input", fn);
    // The kernels use 16-byte vector accesses on every tensor.
    if ((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(out) |
         reinterpret_cast<uintptr_t>(rh) | reinterpret_cast<uintptr_t>(rw)) & 15)
        return dg::fail(DG_EINVAL, "%s: tensor pointers must be 16-byte aligned", fn);
    // every kernel addresses a window's qkv rows through one buffer descriptor
    if ((size_t)n * 12 * W > 0x7fffffffu)
        return dg::fail(DG_EUNSUPPORTED, "%s: a window of %lld tokens x %zu floats exceeds 2 GiB", fn, n,
                        3 * W);
    const bool small = n <= kSmallGrid;              // 4 x 2 workgroups for small grids
    static_assert(RelShape<1, 4>::kBlockQ == RelShape<2>::kBlockQ, "small shapes share a block");
    const long long kbq = small ? RelShape<2>::kBlockQ : RelShape<4>::kBlockQ;
    const long long qblocks = (n + kbq - 1) / kbq;
    const long long nblocks = qblocks * heads * nwin;
    // 4 x 1 for small grids of few rows cut into row tiles (gw <= 32; a wavefront of that shape
    // takes every tile, and the half-row tiling needs each wavefront to see one half only),
    // when there are more workgroups than CUs: with fewer, the 4 x 2 shape's key split halves
    // each workgroup's time.
    const dg::Topology topo = dg::device_topology();
    const bool rows16 = small && gh <= kSmallRows && gw <= 32 && nblocks > topo.cus;
    // that shape on the bf16 pipe forms the bias rows of windowed grids itself
    const bool lines = kRelF32OnBf16 && rows16 && rh && win_grid(gh, gw);
    if (nblocks > 0x7fffffffLL || (long long)nwin * heads * (gh + gw) > 0x1fffffffLL)
        return dg::fail(DG_EUNSUPPORTED, "%s: too many workgroups", fn);
    RelArgs a;
    a.qkv = qkv; a.rh = rh; a.rw = rw; a.out = out;
    a.dhw = use_ws && !lines ? static_cast<const float*>(workspace) : nullptr;
    a.lines = lines ? 1 : 0;
    a.n = (int)n; a.gh = gh; a.gw = gw; a.heads = heads; a.W = (int)W; a.nwin = nwin;
    a.qblocks = (int)qblocks;
    a.nblocks = (int)nblocks;
    a.nxcd = topo.xcds;
    a.qmul = scale * dgk::kLog2e;
    const Tiling tl = make_tiling(gh, gw);
    a.ntiles = tl.ntiles;
    if (tl.half_rows) {
        a.tsh = 1; a.ta = gw; a.tmsk = 1; a.tb = tl.kh; a.tl0 = tl.kh; a.td = gw - 2 * tl.kh;
    } else {
        a.tsh = 0; a.ta = tl.kpt; a.tmsk = 0; a.tb = 0; a.tl0 = tl.kpt; a.td = 0;
    }
    a.gh4 = round4(gh);
    a.brs = bias_row_floats(gh, gw);
    // where the bias pass puts the rows: relpos_bias16_kernel one row [dh | dw] per query
    // (windowed grids), relpos_bias_kernel a dh block and then a dw block
    if (win_grid(gh, gw)) {
        a.dh_stride = a.brs; a.dw_stride = a.brs; a.dw_off = (size_t)a.gh4;
    } else {
        a.dh_stride = gh; a.dw_stride = gw; a.dw_off = (size_t)nwin * heads * n * gh;
    }
    hipStream_t s = (hipStream_t)stream;
    const long long nx = topo.xcds;
    if (use_ws && !lines) {   // the bias rows, before the attention
        if (win_grid(gh, gw)) {
            const long long nbt = (long long)nwin * heads * (gh + gw);
            const long long nbias = (nbt + kBiasWaves - 1) / kBiasWaves;
            const dim3 bgrid((unsigned)((nbias + nx - 1) / nx * nx));
            hipLaunchKernelGGL(relpos_bias16_kernel, bgrid, dim3(64 * kBiasWaves), 0, s, a,
                               static_cast<float*>(workspace), (int)nbt);
        } else {
            const long long ntasks = (long long)nwin * heads * (gh + gw) * 4;
            const long long nbias = (ntasks + kBiasWaves - 1) / kBiasWaves;
            const dim3 grid((unsigned)((nbias + nx - 1) / nx * nx));   // whole XCD rounds for xcd_remap
            hipLaunchKernelGGL(relpos_bias_kernel, grid, dim3(64 * kBiasWaves), 0, s, a,
                               static_cast<float*>(workspace), ntasks);
        }
    }
    const bool full = tl.half_rows ? gw == 64 : (tl.kpt == dgk::kKeys && gh % tl.rpt == 0);
    const bool one = tl.nshift == 1;
    auto* kern = patch  ? (full ? relpos_flash_kernel<true, true, 4, 8, true>
                                : relpos_flash_kernel<false, true, 4, 8, true>)
               : rows16 ? pick_flash<1, 4>(full, one)
               : small  ? pick_flash<2, 8>(full, one)
                        : pick_flash<4, 8>(full, one);
    hipLaunchKernelGGL(kern, dim3((unsigned)a.nblocks), dim3(rows16 ? 256 : 512), 0, s, a);
    return dg::launch_status(fn);
}

}  // namespace

extern "C" int relpos_flash_attn_windows(const float* qkv, const float* rh, const float* rw,
                                         float* out, int nwin, int gh, int gw, int heads, int hd,
                                         float scale, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    return relpos_call("relpos_flash_attn_windows", qkv, rh, rw, out, nwin, gh, gw, heads, hd,
                       scale, workspace, workspace_bytes, stream);
}

extern "C" int relpos_flash_attn(const float* qkv, const float* rh, const float* rw, float* out,
                                 int gh, int gw, int heads, int hd, float scale, void* stream) {
    return relpos_call("relpos_flash_attn", qkv, rh, rw, out, 1, gh, gw, heads, hd, scale,
                       nullptr, 0, stream);
}

extern "C" int relpos_flash_attn_ws(const float* qkv, const float* rh, const float* rw, float* out,
                                    int gh, int gw, int heads, int hd, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return relpos_call("relpos_flash_attn_ws", qkv, rh, rw, out, 1, gh, gw, heads, hd, scale,
                       workspace, workspace_bytes, stream);
}
