/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the attention block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Sources (the three docs.rs source pages of the `inferencelayer` crate):
 *   [DG]  inferencelayer 0.2.3, src/diffusion_gemma_gpu.rs -- kernels DG_HEADNORM_ROPE and
 *         DG_ATTN, and the rope-table / headnorm / attention dispatches in `canvas_forward`.
 *   [DE]  inferencelayer 0.2.8, src/deepencoder_gpu.rs -- kernels SAM_SCORES, DHDW,
 *         SOFTMAX, AV_MERGE and `sam_attn_buf`.
 *   [MO]  inferencelayer 0.2.4, src/moshi_gpu.rs -- kernels COPY_KV and DEP_ATTN.
 *
 * Precision: the pages fix the arithmetic at f32 ([DG] module doc: everything is f32, as is
 * the CPU reference it is gated against).  Storage and accumulation here are f32, every sum
 * runs in plain sequential index order, and no -ffast-math is used, so the result does not
 * depend on the thread count.  The one exception is the rope table (cos/sin of a position
 * times a frequency), which is evaluated in f64 and rounded once to f32.
 *
 * Parallelism: OpenMP only across independent output units ((batch, row, head) or
 * (head, query)); the work inside a unit is one sequential loop nest.
 *
 * Pins: every function here is checked by the CPU tests against closed forms, invariants,
 * hand-derived fixtures and library routines (torch's scaled_dot_product_attention, numpy
 * complex rotation).  The rope frequency schedule itself is not printed on the pages (the
 * crate's `rope_cos_sin` is absent); the reading taken is the NeoX / HF one, stated below.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NORM_WEIGHTED 1u
#define ORACLE_NORM_ROPE 2u
#define ORACLE_NORM_SKIP 4u

int oracle_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * Rope table, [DG] `canvas_forward` ("Rope tables per layer type"): one row per canvas token
 * at absolute position pos0 + t (the page uses the cache's seq_len + t).  Row layout is
 * [cos | sin], each hd wide, which is what DG_HEADNORM_ROPE reads (cos at c, sin at hd + c).
 *
 * Reading (the generator itself is not on the pages): NeoX rotate-half pairs element c with
 * c + hd/2, so both halves of a row carry the same angle; pair i (0 <= i < hd/2) turns at
 * frequency theta^(-2i/hd) radians per position.  Angles, cos and sin are taken in f64 and
 * rounded once to f32.
 */
void oracle_rope_table(float *cs, int pos0, int T, int hd, double theta) {
    const int half = hd / 2;
    for (int t = 0; t < T; ++t) {
        const double p = (double)pos0 + (double)t;
        for (int c = 0; c < hd; ++c) {
            const int i = c % half;
            const double freq = pow(theta, -2.0 * (double)i / (double)hd);
            const double ang = p * freq;
            cs[(size_t)t * 2 * hd + c] = (float)cos(ang);
            cs[(size_t)t * 2 * hd + hd + c] = (float)sin(ang);
        }
    }
}

/*
 * Per-(token, head) RMSNorm, optional weight, optional NeoX rope, in place on
 * x[batch, T, heads*hd]; [DG] DG_HEADNORM_ROPE.  Order as on the page: the norm factor is
 * 1/sqrt(sum(x^2)/hd + eps); the weight multiplies the normed value; the rope then reads the
 * normed-and-weighted values of the whole head (it pairs c with c +/- hd/2) and writes
 * y*cos + rot*sin with rot[c] = -y[c+hd/2] for c < hd/2 and y[c-hd/2] otherwise.
 * The cs table [T, 2*hd] is shared by all batch entries.
 * ORACLE_NORM_SKIP (not a page flag) leaves the values unnormalised, so the same routine can
 * rope a cache written at known positions (rope only, weight ignored).
 */
void oracle_headnorm_rope(float *x, const float *w, const float *cs, int batch, int T,
                          int heads, int hd, unsigned flags, float eps) {
    const long units = (long)batch * T * heads;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        const long bt = u / heads;
        const int t = (int)(bt % T);
        float *xh = x + (size_t)u * hd;
        float *y = (float *)malloc(sizeof(float) * (size_t)hd);
        if (flags & ORACLE_NORM_SKIP) {
            for (int c = 0; c < hd; ++c) y[c] = xh[c];
        } else {
            float ss = 0.0f;
            for (int c = 0; c < hd; ++c) ss = ss + xh[c] * xh[c];
            const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
            for (int c = 0; c < hd; ++c) {
                float v = xh[c] * inv;
                if (flags & ORACLE_NORM_WEIGHTED) v = v * w[c];
                y[c] = v;
            }
        }
        if (flags & ORACLE_NORM_ROPE) {
            const int half = hd / 2;
            const float *cosr = cs + (size_t)t * 2 * hd;
            const float *sinr = cosr + hd;
            for (int c = 0; c < hd; ++c) {
                const float rot = (c < half) ? -y[c + half] : y[c - half];
                xh[c] = y[c] * cosr[c] + rot * sinr[c];
            }
        } else {
            for (int c = 0; c < hd; ++c) xh[c] = y[c];
        }
        free(y);
    }
}

/*
 * Row softmax then weighted sum of values: the textbook definition, with the whole score row
 * materialised (no online rescale).  [DE] SOFTMAX (max, exp(s - max), sum, divide) and
 * AV_MERGE (out = sum_j p_j v_j).  `vrow(j)` is passed as a table of row pointers.
 */
static void softmax_av(const float *s, int nkeys, const float *const *vrows, int hd, float *p,
                       float *outrow) {
    float m = s[0];
    for (int j = 1; j < nkeys; ++j) m = fmaxf(m, s[j]);
    float l = 0.0f;
    for (int j = 0; j < nkeys; ++j) {
        p[j] = expf(s[j] - m);
        l = l + p[j];
    }
    for (int j = 0; j < nkeys; ++j) p[j] = p[j] / l;
    for (int c = 0; c < hd; ++c) {
        float a = 0.0f;
        for (int j = 0; j < nkeys; ++j) a = a + p[j] * vrows[j][c];
        outrow[c] = a;
    }
}

/*
 * GQA attention over the split key/value set [cache (ctx) | canvas (T)]; [DG] DG_ATTN and its
 * dispatch in `canvas_forward`.
 *   q   [batch, T, nh*hd]        kc, vc [batch, nkv, ctx, hd]      k, v [batch, T, nkv*hd]
 *   out [batch, T, nh*hd]
 * q head h reads kv head h / (nh/nkv).  Key j < ctx is cache row j of that kv head; key
 * j >= ctx is canvas row j - ctx.  Score = scale * <q, K_j>: DiffusionGemma passes 1.0 (its
 * qk norms carry the scale), the depformer 0.125 ([MO] DEP_ATTN).
 * causal = 0: every canvas row sees every key (the page's bidirectional attention).
 * causal = 1: canvas row i sees all cache keys and canvas keys 0..i ([MO] DEP_ATTN at step s
 * attends slots 0..s).
 * rows: optional list of flattened (b*T + i) canvas rows to compute (all heads of each);
 * NULL computes every row.  Other rows of `out` are left untouched.
 */
void oracle_attn_split_gqa(const float *q, const float *kc, const float *vc, const float *k,
                           const float *v, float *out, int batch, int T, int ctx, int nh,
                           int nkv, int hd, float scale, int causal, const long *rows,
                           long nrows) {
    const int G = nh / nkv;
    const long nr = rows ? nrows : (long)batch * T;
    const long units = nr * nh;
#pragma omp parallel for schedule(dynamic, 4)
    for (long u = 0; u < units; ++u) {
        const long r = u / nh;
        const int h = (int)(u % nh);
        const long bt = rows ? rows[r] : r;
        const int b = (int)(bt / T);
        const int i = (int)(bt % T);
        const int kvh = h / G;
        const int S = ctx + T;
        const float **krows = (const float **)malloc(sizeof(float *) * (size_t)S);
        const float **vrows = (const float **)malloc(sizeof(float *) * (size_t)S);
        int n = 0;
        for (int j = 0; j < S; ++j) {
            if (j < ctx) {
                const size_t off = (((size_t)b * nkv + kvh) * ctx + j) * hd;
                krows[n] = kc + off;
                vrows[n] = vc + off;
            } else {
                const int jc = j - ctx;
                if (causal && jc > i) continue;
                const size_t off = (((size_t)b * T + jc) * nkv + kvh) * hd;
                krows[n] = k + off;
                vrows[n] = v + off;
            }
            ++n;
        }
        const float *qr = q + ((size_t)bt * nh + h) * hd;
        float *s = (float *)malloc(sizeof(float) * (size_t)n);
        float *p = (float *)malloc(sizeof(float) * (size_t)n);
        for (int j = 0; j < n; ++j) {
            float dot = 0.0f;
            for (int c = 0; c < hd; ++c) dot = dot + qr[c] * krows[j][c];
            s[j] = scale * dot;
        }
        softmax_av(s, n, vrows, hd, p, out + ((size_t)bt * nh + h) * hd);
        free(s);
        free(p);
        free(krows);
        free(vrows);
    }
}

/*
 * Windowless vision attention with the decomposed relative-position bias; [DE] SAM_SCORES
 * (dense score definition), DHDW (the two bias dot products), SOFTMAX, AV_MERGE, and
 * `sam_attn_buf` (scale, fused qkv layout).
 *   qkv [n, 3*W] with W = heads*hd: q in columns [0, W), k in [W, 2W), v in [2W, 3W);
 *       head h owns columns h*hd .. h*hd + hd - 1 of each part.
 *   rh [gh, gh, hd], rw [gw, gw, hd]: the expanded tables (both NULL => no bias).
 *   out [n, W].
 * Token i sits at grid cell (qy, qx) = (i / gw, i % gw).  Score of query i against key j:
 *   scale * <q_i, k_j> + <q_i, rh[qy, ky]> + <q_i, rw[qx, kx]>
 * with the bias terms on the unscaled q.  Each row's bias dots are computed once per
 * (query, ky) and (query, kx), as DHDW does; this is the same sum, not an approximation.
 * rows: optional list of query rows (all heads of each); NULL computes every row.
 */
void oracle_relpos_attn(const float *qkv, const float *rh, const float *rw, float *out, int gh,
                        int gw, int heads, int hd, float scale, const long *rows, long nrows) {
    const int n = gh * gw;
    const int W = heads * hd;
    const long nr = rows ? nrows : (long)n;
    const long units = nr * heads;
#pragma omp parallel for schedule(dynamic, 4)
    for (long u = 0; u < units; ++u) {
        const long r = u / heads;
        const int h = (int)(u % heads);
        const int i = (int)(rows ? rows[r] : r);
        const int qy = i / gw, qx = i % gw;
        const float *qr = qkv + (size_t)i * 3 * W + (size_t)h * hd;
        float *dh = (float *)calloc((size_t)gh, sizeof(float));
        float *dw = (float *)calloc((size_t)gw, sizeof(float));
        if (rh) {
            for (int ky = 0; ky < gh; ++ky) {
                const float *t = rh + ((size_t)qy * gh + ky) * hd;
                float a = 0.0f;
                for (int c = 0; c < hd; ++c) a = a + qr[c] * t[c];
                dh[ky] = a;
            }
            for (int kx = 0; kx < gw; ++kx) {
                const float *t = rw + ((size_t)qx * gw + kx) * hd;
                float a = 0.0f;
                for (int c = 0; c < hd; ++c) a = a + qr[c] * t[c];
                dw[kx] = a;
            }
        }
        float *s = (float *)malloc(sizeof(float) * (size_t)n);
        float *p = (float *)malloc(sizeof(float) * (size_t)n);
        const float **vrows = (const float **)malloc(sizeof(float *) * (size_t)n);
        for (int j = 0; j < n; ++j) {
            const float *kr = qkv + (size_t)j * 3 * W + W + (size_t)h * hd;
            float dot = 0.0f;
            for (int c = 0; c < hd; ++c) dot = dot + qr[c] * kr[c];
            s[j] = dot * scale + dh[j / gw] + dw[j % gw];
            vrows[j] = qkv + (size_t)j * 3 * W + 2 * (size_t)W + (size_t)h * hd;
        }
        softmax_av(s, n, vrows, hd, p, out + (size_t)i * W + (size_t)h * hd);
        free(s);
        free(p);
        free(vrows);
        free(dh);
        free(dw);
    }
}

/*
 * 16-bit storage of K and V ([DE] `flash_reg_kv16_src`: the flash reads an f16-packed twin of
 * its inputs and widens each value to f32 before the unchanged f32 math).  The page does not
 * print its pack pass; the reading taken is IEEE 754 round-to-nearest, ties-to-even, for both
 * formats.  format 1 = IEEE binary16 (f16), format 2 = bfloat16 (the upper half of an f32).
 */
static uint16_t pack_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t exp = (u >> 23) & 0xffu;
    const uint32_t man = u & 0x7fffffu;
    if (exp == 0xffu) return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));  /* NaN, inf */
    if (exp == 0) return sign;              /* |f| < 2^-126: far below half the f16 minimum */
    const int e = (int)exp - 127;           /* f = sig * 2^(e-23), sig = 1.man in 24 bits */
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    const uint32_t sig = man | 0x800000u;
    /* f16 normals are (1024 + m) * 2^(E-25), E = e + 15 >= 1: keep 11 bits of sig.
     * f16 subnormals are m * 2^-24: keep sig * 2^(e+1), i.e. drop 13 + (-14 - e) bits. */
    const int shift = e >= -14 ? 13 : 13 + (-14 - e);
    if (shift > 24) return sign;            /* below 2^-25: rounds to zero */
    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t halfway = 1u << (shift - 1);
    if (rem > halfway || (rem == halfway && (q & 1u))) ++q;
    if (e >= -14) /* a carry out of the 11 bits moves into the exponent field, up to inf */
        return (uint16_t)(sign | (((uint32_t)(e + 15) << 10) + (q - 1024u)));
    return (uint16_t)(sign | q);            /* q == 1024 is the smallest normal, as wanted */
}

static float widen_f16(uint16_t h) {
    const uint32_t exp = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float v;
    if (exp == 0) v = ldexpf((float)m, -24);
    else if (exp == 0x1fu) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(1024u + m), (int)exp - 25);
    return (h & 0x8000u) ? -v : v;
}

static uint16_t pack_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);                    /* quiet NaN, sign kept */
    const uint32_t lsb = (u >> 16) & 1u;                             /* ties to even */
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

static float widen_bf16(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float v;
    memcpy(&v, &u, 4);
    return v;
}

void oracle_pack16(const float *src, uint16_t *dst, long n, int format) {
    for (long i = 0; i < n; ++i) dst[i] = format == 1 ? pack_f16(src[i]) : pack_bf16(src[i]);
}

void oracle_widen16(const uint16_t *src, float *dst, long n, int format) {
    for (long i = 0; i < n; ++i) dst[i] = format == 1 ? widen_f16(src[i]) : widen_bf16(src[i]);
}
