/*
 * dgattn.h -- C ABI of the MI355X (gfx950) attention-block library libdgattn.so.
 *
 * The operations follow three source pages of the `inferencelayer` crate on docs.rs:
 *   - inferencelayer 0.2.3, src/diffusion_gemma_gpu.rs: kernels DG_HEADNORM_ROPE and DG_ATTN,
 *     and the rope-table, headnorm and attention dispatches of `canvas_forward`;
 *   - inferencelayer 0.2.8, src/deepencoder_gpu.rs: kernels SAM_SCORES, DHDW and the
 *     register flash generator `flash_reg_src`, driven by `sam_attn_buf`;
 *   - inferencelayer 0.2.4, src/moshi_gpu.rs: kernels COPY_KV and DEP_ATTN (causal
 *     within-frame attention with a 0.125 scale).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to contiguous, row-major float32 data that
 *     the caller allocated and owns.  The library allocates nothing, keeps no pointer after
 *     it returns, and never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  Work is
 *     enqueued on it asynchronously; nothing synchronises inside the library.  The caller
 *     keeps every buffer alive until the stream has passed the launch.
 *   - Every argument is validated on the host before any work is enqueued; the only runtime
 *     calls made before validation completes are read-only queries of the current device (its
 *     compute-unit and XCD counts, which size the launch plans).  On failure the call returns
 *     a negative status, launches nothing, writes nothing, and records a message that
 *     dg_last_error() returns (per calling thread).  The library never aborts or prints.
 *   - A call whose output is empty (T == 0, batch == 0, n == 0) returns DG_OK and launches
 *     nothing.
 *   - Calls on one stream run in order; calls that write the same buffer from different
 *     streams race.
 */
#ifndef DGATTN_H
#define DGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DG_OK = 0,
    DG_EINVAL = -1,        /* a malformed argument (negative size, NULL pointer, overlap) */
    DG_EUNSUPPORTED = -2,  /* a well-formed argument outside what the kernels implement */
    DG_ELAUNCH = -3        /* the HIP runtime rejected the launch (message holds its error) */
};

/* Flag bits of dg_headnorm_rope.  Bits 0 and 1 are the page's own flag bits of
 * DG_HEADNORM_ROPE (bit0 weighted, bit1 rope).  Bit 2 is an addition: skip the norm and
 * the weight, and only rotate -- used to rope a cache written at known positions. */
#define DG_NORM_WEIGHTED 1u
#define DG_NORM_ROPE 2u
#define DG_NORM_SKIP 4u
/* Accepted by dg_qkv_headnorm_rope only: the page's k_eq_v layers, whose v is the RAW k
 * projection.  v is then an output: each v row is the weightless, un-roped norm of the raw k
 * row (computed before k is normed and roped in place), and v's prior contents are ignored. */
#define DG_NORM_V_FROM_K 8u

/*
 * dg_rope_table -- cos|sin table for the NeoX rotate-half rope.
 * Follows `canvas_forward` in diffusion_gemma_gpu.rs (rope tables per layer type: one row per
 * canvas token at absolute position seq_len + t).  The page's table generator is not shown;
 * the frequencies are the NeoX/HF ones: pair i (0 <= i < hd/2) turns theta^(-2i/hd) radians
 * per position and both halves of a row carry the same angles.
 *   cs     out  [T, 2*hd]: cs[t, c] = cos((pos0+t) * f(c mod hd/2)), cs[t, hd+c] = sin(...).
 *               Evaluated in double precision and rounded once to float.
 *   pos0        absolute position of row 0 (>= 0);  T >= 0 rows;  hd even, 2 <= hd <= 1024.
 *   theta       rope base, > 0 (10000 for the configurations here).
 * Errors: DG_EINVAL for a negative pos0/T, odd or out-of-range hd, theta <= 0, NULL cs
 * with T > 0.
 */
int dg_rope_table(float* cs, int pos0, int T, int hd, double theta, void* stream);

/*
 * dg_headnorm_rope -- per-(token, head) RMSNorm, optional weight, optional NeoX rope, IN PLACE.
 * Follows kernel DG_HEADNORM_ROPE in diffusion_gemma_gpu.rs and its three dispatches in
 * `canvas_forward` (q: weighted + rope; k: weighted + rope; v: flags 0, the weightless,
 * un-roped v-norm).
 *   x      in/out [batch, T, heads*hd].  For every (b, t, head):
 *                 inv = 1/sqrt(sum_c x[c]^2 / hd + eps);  y[c] = x[c]*inv  (skipped with SKIP)
 *                 WEIGHTED: y[c] *= w[c]                                   (skipped with SKIP)
 *                 ROPE: x[c] = y[c]*cs[t,c] + r[c]*cs[t,hd+c],
 *                       r[c] = -y[c+hd/2] for c < hd/2, y[c-hd/2] otherwise
 *                 otherwise x[c] = y[c].
 *   w      [hd]; read iff WEIGHTED is set without SKIP (may be NULL otherwise).
 *   cs     [T, 2*hd] table from dg_rope_table (shared by all batch entries); read iff ROPE.
 *   flags  DG_NORM_* bits;  eps >= 0.
 * Errors: DG_EINVAL for negative sizes, unknown flag bits, a needed pointer that is NULL,
 * odd hd with ROPE, w or cs overlapping x, hd < 1, a negative or non-finite eps;
 * DG_EUNSUPPORTED for hd > 128 (the page's one-thread-per-element workgroup of 128).
 */
int dg_headnorm_rope(float* x, const float* w, const float* cs, int batch, int T, int heads,
                     int hd, unsigned flags, float eps, void* stream);

/*
 * dg_qkv_headnorm_rope -- the three headnorm dispatches of one canvas step in ONE launch.
 * Follows the q, k and v dispatches of DG_HEADNORM_ROPE in `canvas_forward`
 * (diffusion_gemma_gpu.rs): q and k get `flags` with their own weights, v gets the
 * weightless, un-roped norm (the page's flags 0).  Each row is computed exactly as
 * dg_headnorm_rope computes it.
 *   q   in/out [batch, T, nh*hd], or NULL to leave q alone (e.g. when the attention call
 *       normalises q itself, see dg_attn_split_gqa_qnorm)
 *   wq  [hd]; read iff q != NULL and WEIGHTED is set without SKIP
 *   k   in/out [batch, T, nkv*hd], or NULL;  wk [hd] as wq
 *   v   in/out [batch, T, nkv*hd], or NULL; with DG_NORM_V_FROM_K an output only
 *   cs  [T, 2*hd] rope table; read iff ROPE is set and q or k is given
 *   flags, eps as dg_headnorm_rope (flags apply to q and k only), plus DG_NORM_V_FROM_K.
 * Errors: as dg_headnorm_rope, plus DG_EINVAL for negative nh/nkv, overlapping q/k/v, a
 * weight or table overlapping any of them, V_FROM_K without k or v, or V_FROM_K with SKIP.
 * All of q, k, v NULL (or empty) is a no-op.
 */
int dg_qkv_headnorm_rope(float* q, const float* wq, float* k, const float* wk, float* v,
                         const float* cs, int batch, int T, int nh, int nkv, int hd,
                         unsigned flags, float eps, void* stream);

/* 16-bit storage formats of K and V (dg_pack_kv16, dg_attn_split_gqa_kv16). */
#define DG_KV_F16 1   /* IEEE binary16 */
#define DG_KV_BF16 2  /* bfloat16: the upper 16 bits of an f32 */

/*
 * dg_pack_kv16 -- f32 -> 16-bit storage of keys or values, the pack pass of deepencoder_gpu.rs
 * `flash_reg_kv16_src` (the flash reads an f16 twin of its inputs and widens each value to f32
 * before the unchanged f32 math).  Round to nearest, ties to even; values beyond the format's
 * range become infinities, NaN stays NaN.
 *   src  [n] f32;  dst [n] 16-bit values (uint16 bit patterns);  format DG_KV_F16 or DG_KV_BF16.
 *   src and dst must be 16-byte aligned and must not overlap.
 * Errors: DG_EINVAL for an unknown format, NULL pointers with n > 0, misalignment or overlap.
 */
int dg_pack_kv16(const float* src, void* dst, size_t n, int format, void* stream);

/*
 * dg_qkv_headnorm_rope_kv16 -- dg_qkv_headnorm_rope that also writes 16-bit twins of the normed
 * k and v, for dg_attn_split_gqa_kv16: the canvas step's norm launch and the pack pass of
 * deepencoder_gpu.rs `flash_reg_kv16_src` in one launch.  q, k and v are normed in place
 * exactly as dg_qkv_headnorm_rope does, and each twin element is the f32 result rounded as
 * dg_pack_kv16 rounds it (bit-identical to packing the f32 outputs).
 *   k16  out [batch, T, nkv*hd] 16-bit values; needed iff k is given
 *   v16  out [batch, T, nkv*hd] 16-bit values; needed iff v is given (with DG_NORM_V_FROM_K
 *        the twin of the v output)
 *   kv_format  DG_KV_F16 or DG_KV_BF16
 *   the other arguments as dg_qkv_headnorm_rope.
 * Errors: as dg_qkv_headnorm_rope, plus DG_EINVAL for an unknown kv_format, a missing twin,
 * or a twin that overlaps q, k, v, the other twin, a weight or the table.
 */
int dg_qkv_headnorm_rope_kv16(float* q, const float* wq, float* k, const float* wk, float* v,
                              const float* cs, void* k16, void* v16, int batch, int T, int nh,
                              int nkv, int hd, unsigned flags, float eps, int kv_format,
                              void* stream);

/*
 * dg_attn_split_gqa_workspace_size -- bytes of scratch that dg_attn_split_gqa can use to split
 * the key range of one call across more workgroups (partial results and their combine), on the
 * current device (its compute-unit count sets the split; see dg_attn_split_gqa_plan).  Enough
 * for the f32 and the 16-bit K/V entry points alike.  Returns 0 when the shape gains nothing
 * from a split.  Arguments as for dg_attn_split_gqa; returns 0 for any argument
 * dg_attn_split_gqa would reject.
 */
size_t dg_attn_split_gqa_workspace_size(int batch, int T, int ctx, int nh, int nkv, int hd);

/* Attention kernels a launch plan can name (dg_attn_plan.kernel). */
#define DG_KERNEL_NONE 0     /* empty output: nothing is launched */
#define DG_KERNEL_SMALL 1    /* ctx + T <= 8: one wavefront per (batch entry, q head) */
#define DG_KERNEL_TILE32 2   /* 32-key tiles, 128 query vectors per workgroup */

/* How a split-GQA attention call is launched (see dg_attn_split_gqa_plan). */
typedef struct dg_attn_plan {
    int kernel;              /* DG_KERNEL_* */
    int query_block;         /* query vectors per workgroup (0 for DG_KERNEL_SMALL) */
    int nsplit;              /* key-range splits (1 = unsplit) */
    long long workgroups;    /* attention workgroups launched */
    size_t workspace_bytes;  /* split-KV scratch the call uses (0 when unsplit) */
} dg_attn_plan;

/*
 * dg_attn_split_gqa_plan -- the launch plan of the dg_attn_split_gqa family for a shape on a
 * device with `cus` compute units (0 = the current device's count): which kernel runs, the
 * workgroups and the key-range splits.  The split count targets one workgroup per compute unit
 * and keeps at least two 64-key stages per split; causal calls do not split.  For sizing a
 * workspace ahead of time for another device, and for inspection.  kv_format is 0 for f32 K/V,
 * or DG_KV_F16 / DG_KV_BF16.  The plan of the actual call also depends on the workspace given
 * (none: unsplit).
 * Errors: DG_EINVAL for a NULL plan, negative sizes, nkv < 1, nh % nkv != 0, cus < 0, causal
 * not 0/1 or an unknown kv_format; DG_EUNSUPPORTED for hd not a multiple of 4 in [4, 128].
 */
int dg_attn_split_gqa_plan(int batch, int T, int ctx, int nh, int nkv, int hd, int causal,
                           int kv_format, int cus, dg_attn_plan* plan);

/*
 * dg_attn_split_gqa -- GQA flash attention over the split key/value set [cache | canvas].
 * Follows kernel DG_ATTN in diffusion_gemma_gpu.rs (online softmax over ctx cache keys then T
 * canvas keys, kv head = q head / (nh/nkv), cache layout [nkv, ctx, hd], canvas layout
 * [T, nkv*hd], scaling 1.0 because the qk norms carry the scale) and, for `causal` and
 * `scale`, kernel DEP_ATTN in moshi_gpu.rs (the step-s query sees slots 0..s, scale 0.125).
 *   q    [batch, T, nh*hd]        queries (already normed/roped by the caller)
 *   kc   [batch, nkv, ctx, hd]    cache keys;   may be NULL iff ctx == 0
 *   vc   [batch, nkv, ctx, hd]    cache values; may be NULL iff ctx == 0
 *   k    [batch, T, nkv*hd]       canvas keys
 *   v    [batch, T, nkv*hd]       canvas values
 *   out  [batch, T, nh*hd]        written; must not overlap any input
 *   For every (b, i, h), with kv = h / (nh/nkv) and keys j in [0, ctx+T):
 *     K_j = kc[b,kv,j] for j < ctx, k[b,j-ctx,kv] otherwise (V likewise),
 *     s_j = scale * <q[b,i,h], K_j>, skipping canvas keys with j-ctx > i when causal != 0,
 *     out[b,i,h] = sum_j softmax(s)_j V_j.
 *   scale      finite float (1.0f for DiffusionGemma, 0.125f for the depformer).
 *   causal     0 = bidirectional (the page); 1 = canvas row i sees canvas keys 0..i.
 *   workspace  optional device scratch of at least dg_attn_split_gqa_workspace_size() bytes,
 *              16-byte aligned, used for a split of the key range; NULL/0 runs unsplit (same
 *              results up to rounding).  Must not overlap any input or `out`.
 *   Every tensor pointer must be 16-byte aligned (the kernels use 16-byte vector accesses;
 *   torch allocations are).
 *   hd         any multiple of 4 up to 128 (the page allows hd <= 128); heads narrower than
 *              64 or 128 run in the 64- or 128-wide kernel with zero padding.
 * Arithmetic: in the 32-key tile kernel each f32 operand is taken as three bf16 terms (whose
 * sum is exactly the operand) and each product q.k and p.v as the six leading bf16 x bf16
 * products, each exact in f32, summed in f32 on the bf16 matrix pipe: every product is within
 * 2^-23 |a||b| of its value, typically 2^-29 (f32 rounds a product by up to 2^-24), and the
 * large score terms are summed apart from the small ones.  The short-key-set kernel (ctx + T <= 8) uses f32 arithmetic.
 * Errors: DG_EINVAL for negative sizes, nkv < 1, nh % nkv != 0, a NULL pointer with a
 * nonzero extent, a non-finite scale, causal not 0/1, overlapping buffers, a tensor pointer
 * that is not 16-byte aligned, or a workspace pointer that is misaligned or has
 * workspace_bytes too small; DG_EUNSUPPORTED for hd above 128 or not a multiple of 4, or
 * ctx + T or T * nh/nkv above 2^30 (the kernels index keys and query vectors in 32 bits).
 */
int dg_attn_split_gqa(const float* q, const float* kc, const float* vc, const float* k,
                      const float* v, float* out, int batch, int T, int ctx, int nh, int nkv,
                      int hd, float scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * dg_attn_split_gqa_qnorm -- dg_attn_split_gqa on the RAW q projection: each query vector gets
 * the q dispatch of DG_HEADNORM_ROPE (`canvas_forward`, diffusion_gemma_gpu.rs) in registers as
 * the attention kernel loads it, so the separate in-place pass over q is not needed.  The
 * result equals dg_headnorm_rope(q, wq, cs, ..., qflags, eps) followed by dg_attn_split_gqa,
 * up to rounding; q itself is NOT modified.  k and v must already be normalised (e.g. by
 * dg_qkv_headnorm_rope with q = NULL).
 *   q       [batch, T, nh*hd] raw queries
 *   wq      [hd]; read iff WEIGHTED is set without SKIP
 *   cs      [T, 2*hd] rope table (row t = canvas row t); read iff ROPE is set
 *   qflags  DG_NORM_* bits for q;  eps >= 0
 *   every other argument as dg_attn_split_gqa (same workspace size function).
 * Errors: as dg_attn_split_gqa, plus DG_EINVAL for unknown flag bits, a negative or
 * non-finite eps, a needed wq/cs that is NULL, or out overlapping wq or cs.
 */
int dg_attn_split_gqa_qnorm(const float* q, const float* wq, const float* cs, const float* kc,
                            const float* vc, const float* k, const float* v, float* out,
                            int batch, int T, int ctx, int nh, int nkv, int hd, unsigned qflags,
                            float eps, float scale, int causal, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * dg_attn_split_gqa_qkvnorm -- dg_attn_split_gqa on the RAW q, k and v projections of a canvas
 * step: the three headnorm dispatches of `canvas_forward` (diffusion_gemma_gpu.rs, kernel
 * DG_HEADNORM_ROPE: q weighted + roped, k weighted + roped, v the weightless, un-roped norm)
 * run inside the attention launch.  q is normalised as dg_attn_split_gqa_qnorm does it; each
 * canvas key/value row is normalised in on-chip memory after it is loaded, by every workgroup
 * that reads it.  The result equals dg_qkv_headnorm_rope(q, wq, k, wk, v, cs, ..., flags, eps)
 * followed by dg_attn_split_gqa, up to rounding; q, k and v are NOT modified.  A layer whose v
 * is the raw k projection (the page's k_eq_v layers) passes k as v.
 *   q       [batch, T, nh*hd] raw queries;   wq [hd], read iff WEIGHTED
 *   k       [batch, T, nkv*hd] raw canvas keys;   wk [hd], read iff WEIGHTED
 *   v       [batch, T, nkv*hd] raw canvas values (may be the same pointer as k)
 *   cs      [T, 2*hd] rope table (row t = canvas row t, for q and k); read iff ROPE
 *   kc, vc  the cache, stored normalised (and its keys roped), as for dg_attn_split_gqa
 *   flags   DG_NORM_WEIGHTED and/or DG_NORM_ROPE, applied to q and k;  eps >= 0
 *   every other argument as dg_attn_split_gqa (same workspace size function).
 * Errors: as dg_attn_split_gqa, plus DG_EINVAL for flag bits other than WEIGHTED and ROPE, a
 * negative or non-finite eps, a needed wq, wk or cs that is NULL, or out overlapping wq, wk
 * or cs.
 */
int dg_attn_split_gqa_qkvnorm(const float* q, const float* wq, const float* k, const float* wk,
                              const float* v, const float* cs, const float* kc, const float* vc,
                              float* out, int batch, int T, int ctx, int nh, int nkv, int hd,
                              unsigned flags, float eps, float scale, int causal,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * dg_attn_split_gqa_kv16 -- dg_attn_split_gqa with keys and values stored in 16 bits (the
 * page's kv16 twin, reduced-precision K/V storage): kc, vc, k and v hold f16 or bf16 values
 * (`kv_format`), in the same layouts as dg_attn_split_gqa's f32 tensors.  The result equals
 * dg_attn_split_gqa on the widened values up to rounding:
 *   f16   each value is widened exactly to f32 and runs the f32 MFMA arithmetic;
 *   bf16  both products run on the bf16 matrix pipe: the f32 operand (q for the scores, the
 *         probabilities for the value product) is taken as three bf16 terms whose sum is
 *         exactly it, each product of two bf16 values is exact in f32, and all sums are f32
 *         -- at about a fifth of the f32 MFMA time.
 * Stage tiles in LDS are half the bytes of f32 ones.
 *   hd must be a multiple of 8 (16-byte rows of 16-bit values); q and out are f32.
 *   Other arguments, the workspace and its size function as dg_attn_split_gqa.
 * Errors: as dg_attn_split_gqa, plus DG_EINVAL for an unknown kv_format and DG_EUNSUPPORTED
 * for hd not a multiple of 8.
 */
int dg_attn_split_gqa_kv16(const float* q, const void* kc, const void* vc, const void* k,
                           const void* v, float* out, int batch, int T, int ctx, int nh, int nkv,
                           int hd, float scale, int causal, int kv_format, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind dg_attn_split_gqa_noalloc, one copy per GPU. */
#define DG_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * dg_attn_split_gqa_noalloc -- dg_attn_split_gqa for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): it
 * takes no workspace and allocates nothing.  Where dg_attn_split_gqa would split the key range
 * across workgroups, the partial results go to a static device array of
 * DG_NOALLOC_SCRATCH_BYTES bytes inside the library instead of a caller workspace; the same
 * kernels run with the same launch plan, so the result is bit-identical to dg_attn_split_gqa
 * given a workspace of dg_attn_split_gqa_workspace_size() bytes.
 *   Every argument as dg_attn_split_gqa.  `stream` must belong to the current device (NULL is
 *   the current device's legacy default stream).
 *   The scratch is one array per GPU, shared by every call on that GPU and held until the
 *   process ends; each call writes every partial it reads, so nothing needs clearing between
 *   calls.  Calls that overlap in time on one GPU (other streams, other threads, other
 *   processes' contexts excepted) RACE on it: order them on one stream.
 * Errors: as dg_attn_split_gqa; DG_EUNSUPPORTED when the shape's split partials need more than
 * DG_NOALLOC_SCRATCH_BYTES (dg_attn_split_gqa_workspace_size() tells how many it needs);
 * DG_EINVAL when `stream` belongs to another device than the current one; DG_ELAUNCH when the
 * runtime cannot report the current device or the scratch's address.
 */
int dg_attn_split_gqa_noalloc(const float* q, const float* kc, const float* vc, const float* k,
                              const float* v, float* out, int batch, int T, int ctx, int nh,
                              int nkv, int hd, float scale, int causal, void* stream);

/*
 * relpos_flash_attn -- windowless vision attention with the decomposed relative-position bias,
 * flash style (no [heads, n, n] buffer).  Follows deepencoder_gpu.rs: kernel SAM_SCORES
 * (score definition), kernel DHDW (the bias dot products hoisted out of the n^2 loop), the
 * register flash `flash_reg_src` with bias, and `sam_attn_buf` (fused qkv layout, scale).
 *   qkv  [gh*gw, 3*heads*hd]: each row is q | k | v, each heads*hd wide, head h at h*hd.
 *   rh   [gh, gh, hd] expanded height table, or NULL
 *   rw   [gw, gw, hd] expanded width table, or NULL (both NULL = no bias; one NULL = error)
 *   out  [gh*gw, heads*hd]; must not overlap any input
 *   Token i is at grid cell (qy, qx) = (i / gw, i % gw).  For every head and query i:
 *     s_j = scale*<q_i, k_j> + <q_i, rh[qy, ky_j]> + <q_i, rw[qx, kx_j]>  (bias on unscaled q)
 *     out[i, h*hd:(h+1)*hd] = sum_j softmax(s)_j v_j
 *   scale  finite float (1/sqrt(hd) in the page's SAM block).
 *   Every tensor pointer must be 16-byte aligned.  The library allocates nothing, so without a
 *   workspace the bias dot products are formed inside each attention workgroup for its own
 *   queries; relpos_flash_attn_ws takes a workspace for them instead.
 * Arithmetic: grids above 16 x 16 form <q_i, k_j> and the value product from f32 operands taken
 * as three bf16 terms each, six exact bf16 matrix products per f32 product summed in f32
 * (within 2^-23 |q||k| of the f32 product, typically 2^-29); the bias dot products, and grids
 * up to 16 x 16, use f32 MFMA.
 * Errors: DG_EINVAL for gh, gw or heads < 0, exactly one of rh/rw NULL, a NULL qkv/out with
 * n > 0, a non-finite scale, overlapping buffers, a tensor pointer that is not 16-byte
 * aligned;
 * DG_EUNSUPPORTED for hd != 64 (the page's kernel fixes hd to its 64-wide workgroup) or gh or
 * gw above 64.
 */
int relpos_flash_attn(const float* qkv, const float* rh, const float* rw, float* out, int gh,
                      int gw, int heads, int hd, float scale, void* stream);

/*
 * relpos_flash_attn_workspace_size -- bytes of scratch relpos_flash_attn_ws uses to hold the
 * hoisted bias rows, the page's DHDW buffers dh [heads][n][gh] and dw [heads][n][gw]: per
 * (head, query) gh + gw floats, each part padded to a multiple of 4 floats when gh and gw are
 * at most 16; n = gh * gw.  Returns 0 for arguments relpos_flash_attn_ws would reject.
 */
size_t relpos_flash_attn_workspace_size(int gh, int gw, int heads, int hd);

/*
 * relpos_flash_attn_ws -- relpos_flash_attn with a caller workspace for the bias rows: a first
 * kernel computes them once per (head, query), as the page's DHDW step does, and the attention
 * reads them.  Same results as relpos_flash_attn up to rounding; faster.  Grids of more than
 * 512 tokens whose sides are multiples of 8 and whose width is above 32 (the SAM global 64 x
 * 64 map) form the bias rows inside the attention from 8 x 8 patches of queries either way, and
 * leave the workspace unused; so do grids of at most 16 x 16 (the windows) when the launch has
 * more workgroups than the GPU has CUs (128 queries of one window and head per workgroup),
 * from whole grid rows and columns of their queries.
 *   workspace  device scratch of at least relpos_flash_attn_workspace_size() bytes, 16-byte
 *              aligned, not overlapping any input or `out` (NULL/0: as relpos_flash_attn).
 * Errors: as relpos_flash_attn, plus DG_EINVAL for a misaligned or too small workspace.
 */
int relpos_flash_attn_ws(const float* qkv, const float* rh, const float* rw, float* out, int gh,
                         int gw, int heads, int hd, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * relpos_flash_attn_windows_workspace_size -- as relpos_flash_attn_workspace_size for a batch of
 * nwin windows (nwin times as many rows); 0 for arguments the call would reject.
 */
size_t relpos_flash_attn_windows_workspace_size(int nwin, int gh, int gw, int heads, int hd);

/*
 * relpos_flash_attn_windows -- relpos_flash_attn_ws over a batch of independent windows sharing
 * the tables: the windowed SAM blocks of deepencoder_gpu.rs's encoder (its cost model: 25
 * windows of 14 x 14 tokens; a 64 x 64 map padded to 70 x 70).  Window partitioning and its
 * padding belong to the caller, whose qkv already holds the padded tokens.
 *   qkv  [nwin, gh*gw, 3*heads*hd]   window w's tokens, each row q | k | v as in relpos_flash_attn
 *   out  [nwin, gh*gw, heads*hd]
 *   rh, rw, gh, gw, heads, hd, scale, workspace as relpos_flash_attn_ws (workspace size from
 *   relpos_flash_attn_windows_workspace_size; NULL/0 forms the bias inside the attention).
 *   Each window is exactly one relpos_flash_attn.
 * Errors: as relpos_flash_attn_ws, plus DG_EINVAL for nwin < 0.  nwin == 0 is a no-op.
 */
int relpos_flash_attn_windows(const float* qkv, const float* rh, const float* rw, float* out,
                              int nwin, int gh, int gw, int heads, int hd, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last nonzero status returned on the calling thread ("" if none). */
const char* dg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DGATTN_H */
