/*
 * kvq_oracle.c -- CPU oracle for attention over a block-quantized KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the
 * GPU library is checked against.  Only the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the library never does.
 * It shares no code, header, table or constant with the GPU path.
 *
 * Sources (web pages, cited by title and section):
 *   [RX9070]  "Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k context,
 *              via adaptive KV streaming" -- molayo1419.me insights post
 *   [ROCmKV]  "Adaptive KV streaming lands on ROCm: Qwen3.8-27B at full 262k
 *              context on a 16 GB RX 9070 XT" -- richland.au blog
 *   [OSCAR2]  "OSCAR2 KV Cache benchmark" -- molayo1419.me insights post
 *   [KVGUIDE] "Context window and KV cache" -- localaiforum.com guide
 *
 * What the pages fix: K is stored as Q8_0 and V as Q4_0 ([RX9070] first
 * paragraph; [ROCmKV] "What shipped"), Q8_0 is 136 bytes per 128 values
 * ([OSCAR2] compression-ratio table), the q8_0/q4_0 cache costs 26,624 bytes
 * per token for 16 layers ([ROCmKV] "Why it matters"), attention is exact
 * softmax attention computed without the quadratic score matrix ([KVGUIDE]
 * "levers" section, flash attention), query heads share KV heads ([KVGUIDE]
 * GQA section), and long prefill accumulates per page with an online
 * log-sum-exp ([RX9070] second paragraph).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - a block is 32 consecutive values of one (token, KV head) row;
 *   - Q8_0: d = max|x| / 127 in fp32, codes = round-half-away(x * (1/d)),
 *     int8; stored scale = fp16(d) rounded to nearest even;
 *   - Q4_0: m = the first element of largest magnitude (sign kept; +0 for an
 *     all-zero block), d = m / -8, code = min(15, trunc(fp32(fp32(x*(1/d)) + 8.5)));
 *     stored scale = fp16(d);
 *   - dequantized values use the stored fp16 scale: k = h*c, v = h*(c-8);
 *   - query i of n_q sits at position ctx_len - n_q + i and sees keys at
 *     positions <= its own (its own key included);
 *   - q head h uses KV head h / G with G = n_heads / n_kv_heads.
 *
 * Quantization is done in IEEE fp32 (so that codes are reproducible bit for
 * bit); everything in attention is fp64.  Build with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK 32

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32, written from the IEEE 754 binary16 definition.            */
/* ------------------------------------------------------------------------ */

/* Nearest binary16 value, ties to even.  Finite inputs only matter here;
 * overflow goes to infinity and NaN stays NaN. */
uint16_t orc_f32_to_f16(float f)
{
    double a = fabs((double)f);
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24 */
        double r = nearbyint(a / ldexp(1.0, -24));   /* default mode: ties to even */
        return (uint16_t)(sign | (uint16_t)r);        /* r == 1024 is the smallest normal */
    }
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;         /* a = 1.f * 2^E */
    double r = nearbyint(a / ldexp(1.0, E - 10));    /* in [1024, 2048] */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* Exact value of a binary16 bit pattern. */
float orc_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* Block quantizers ([RX9070] first paragraph; [OSCAR2] compression table). */
/* x holds n_blocks * 32 fp32 values; block b is x[32b .. 32b+31].           */
/* ------------------------------------------------------------------------ */

/* Q8_0: one fp16 scale and 32 signed 8-bit codes per block. */
void orc_quantize_q8_0(const float *x, int64_t n_blocks, int8_t *codes, uint16_t *scales)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const float *xb = x + b * ORC_BLOCK;
        float amax = 0.0f;
        for (int i = 0; i < ORC_BLOCK; ++i) {
            float ax = fabsf(xb[i]);
            if (ax > amax) amax = ax;
        }
        float d = amax / 127.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        for (int i = 0; i < ORC_BLOCK; ++i) {
            float t = xb[i] * id;
            codes[b * ORC_BLOCK + i] = (int8_t)roundf(t);   /* halves go away from zero */
        }
        scales[b] = orc_f32_to_f16(d);
    }
}

/* Q4_0: one fp16 scale and 32 unsigned 4-bit codes (stored here one per byte,
 * values 0..15) per block; the value is scale * (code - 8). */
void orc_quantize_q4_0(const float *x, int64_t n_blocks, uint8_t *codes, uint16_t *scales)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const float *xb = x + b * ORC_BLOCK;
        float amax = 0.0f, m = 0.0f;
        for (int i = 0; i < ORC_BLOCK; ++i) {
            float ax = fabsf(xb[i]);
            if (ax > amax) { amax = ax; m = xb[i]; }     /* first index wins a tie */
        }
        float d = m / -8.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        for (int i = 0; i < ORC_BLOCK; ++i) {
            float t = xb[i] * id;
            t = t + 8.5f;
            int c = (int)t;                                /* t >= 0, so this is floor */
            codes[b * ORC_BLOCK + i] = (uint8_t)(c > 15 ? 15 : c);
        }
        scales[b] = orc_f32_to_f16(d);
    }
}

/* Dequantized values (exact in fp64). */
void orc_dequant_q8_0(const int8_t *codes, const uint16_t *scales, int64_t n_blocks, double *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        double h = (double)orc_f16_to_f32(scales[b]);
        for (int i = 0; i < ORC_BLOCK; ++i) out[b * ORC_BLOCK + i] = h * (double)codes[b * ORC_BLOCK + i];
    }
}

void orc_dequant_q4_0(const uint8_t *codes, const uint16_t *scales, int64_t n_blocks, double *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        double h = (double)orc_f16_to_f32(scales[b]);
        for (int i = 0; i < ORC_BLOCK; ++i) out[b * ORC_BLOCK + i] = h * ((double)codes[b * ORC_BLOCK + i] - 8.0);
    }
}

/* ------------------------------------------------------------------------ */
/* KV bytes per token ([KVGUIDE] formula section; [ROCmKV] "Why it matters"). */
/* ------------------------------------------------------------------------ */

/* fp16 cache: K and V, each layers * kv_heads * head_dim values of 2 bytes. */
int64_t orc_kv_bytes_per_token_f16(int64_t layers, int64_t kv_heads, int64_t head_dim)
{
    return 2 * layers * kv_heads * head_dim * 2;
}

/* Q8_0 K block: fp16 scale + 32 one-byte codes.  Q4_0 V block: fp16 scale +
 * 32 four-bit codes. */
int64_t orc_q8_0_block_bytes(void) { return 2 + ORC_BLOCK; }
int64_t orc_q4_0_block_bytes(void) { return 2 + ORC_BLOCK / 2; }

/* ------------------------------------------------------------------------ */
/* INT2 codec (a 2-bit cache for K and V alike).  [OSCAR2] compression-ratio */
/* table: 36 bytes per 128 values (2.25 bit), with fp16 zero-point metadata; */
/* the same codec for K and V.  Readings where the page is silent: a block  */
/* is 128 consecutive values of one (token, KV head) row; per block         */
/* mn = min x, mx = max x, d = (mx - mn) / 3 in fp32; id = 1/d (0 when d =  */
/* 0); code = min(3, trunc(fp32(fp32(fp32(x - mn) * id) + 0.5))), i.e. the  */
/* nearest of the 4 levels with ties upward; stored: scale fp16(d) and zero  */
/* fp16(mn), nearest even; value = zero + scale * code.                     */
/* codes: one value 0..3 per byte here (the packing is a storage matter).   */
/* ------------------------------------------------------------------------ */
#define ORC_BLOCK2 128

void orc_quantize_int2(const float *x, int64_t n_blocks, uint8_t *codes, uint16_t *scales, uint16_t *zeros)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const float *xb = x + b * ORC_BLOCK2;
        float mn = xb[0], mx = xb[0];
        for (int i = 1; i < ORC_BLOCK2; ++i) {
            if (xb[i] < mn) mn = xb[i];
            if (xb[i] > mx) mx = xb[i];
        }
        float d = (mx - mn) / 3.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        for (int i = 0; i < ORC_BLOCK2; ++i) {
            float t = xb[i] - mn;
            t = t * id;
            t = t + 0.5f;
            int c = (int)t;                                /* t >= 0.5: this is floor */
            codes[b * ORC_BLOCK2 + i] = (uint8_t)(c > 3 ? 3 : c);
        }
        scales[b] = orc_f32_to_f16(d);
        zeros[b] = orc_f32_to_f16(mn);
    }
}

void orc_dequant_int2(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t n_blocks,
                      double *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        double h = (double)orc_f16_to_f32(scales[b]), z = (double)orc_f16_to_f32(zeros[b]);
        for (int i = 0; i < ORC_BLOCK2; ++i) out[b * ORC_BLOCK2 + i] = z + h * (double)codes[b * ORC_BLOCK2 + i];
    }
}

/* Bytes per 128 values: 32 bytes of 2-bit codes, an fp16 scale, an fp16 zero. */
int64_t orc_int2_block_bytes(void) { return ORC_BLOCK2 / 4 + 2 + 2; }

int64_t orc_kv_bytes_per_token_q8k_q4v(int64_t layers, int64_t kv_heads, int64_t head_dim)
{
    int64_t blocks = head_dim / ORC_BLOCK;
    return layers * kv_heads * blocks * (orc_q8_0_block_bytes() + orc_q4_0_block_bytes());
}

/* ------------------------------------------------------------------------ */
/* Attention over the dequantized cache, fp64 ([KVGUIDE] flash-attention     */
/* lever: exact attention; [KVGUIDE] GQA section: shared KV heads).          */
/*                                                                          */
/* Logical layouts (token-major):                                           */
/*   q        [n_q][n_heads][D]            fp32                             */
/*   k_codes  [ctx][n_kv][D]               int8                             */
/*   k_scales [ctx][n_kv][D/32]            fp16 bits                        */
/*   v_codes  [ctx][n_kv][D]               uint8 (0..15)                    */
/*   v_scales [ctx][n_kv][D/32]            fp16 bits                        */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t n_q, n_heads, n_kv, D, ctx;
    const float *q;
    const int8_t *kc; const uint16_t *ks;
    const uint8_t *vc; const uint16_t *vs;
    double scale;
    /* given dequantized values [ctx][n_kv][D] (any codec), or NULL */
    const double *kd, *vd;
} orc_problem;

static double khat(const orc_problem *p, int64_t j, int kv, int d)
{
    if (p->kd) return p->kd[(j * p->n_kv + kv) * p->D + d];
    int nb = p->D / ORC_BLOCK;
    double h = (double)orc_f16_to_f32(p->ks[(j * p->n_kv + kv) * nb + d / ORC_BLOCK]);
    return h * (double)p->kc[(j * p->n_kv + kv) * p->D + d];
}

static double vhat(const orc_problem *p, int64_t j, int kv, int d)
{
    if (p->vd) return p->vd[(j * p->n_kv + kv) * p->D + d];
    int nb = p->D / ORC_BLOCK;
    double h = (double)orc_f16_to_f32(p->vs[(j * p->n_kv + kv) * nb + d / ORC_BLOCK]);
    return h * ((double)p->vc[(j * p->n_kv + kv) * p->D + d] - 8.0);
}

/* Score of query row (i, h) against key j: scale * sum_d q[d] * k[j][d]. */
static double score(const orc_problem *p, int i, int h, int64_t j)
{
    int G = p->n_heads / p->n_kv;
    int kv = h / G;
    const float *qr = p->q + ((int64_t)i * p->n_heads + h) * p->D;
    double s = 0.0;
    for (int d = 0; d < p->D; ++d) s += (double)qr[d] * khat(p, j, kv, d);
    return p->scale * s;
}

/* Unnormalized softmax state of one query row over keys [j0, j1) that the
 * row may see: m = max score, l = sum exp(s - m), acc = sum exp(s - m) v.
 * An empty range gives m = -inf, l = 0, acc = 0. */
static void partial_row(const orc_problem *p, int i, int h, int64_t j0, int64_t j1,
                        double *m_out, double *l_out, double *acc)
{
    int64_t pos = (int64_t)p->ctx - p->n_q + i;
    if (j1 > pos + 1) j1 = pos + 1;
    for (int d = 0; d < p->D; ++d) acc[d] = 0.0;
    if (j0 >= j1) { *m_out = -INFINITY; *l_out = 0.0; return; }
    int G = p->n_heads / p->n_kv;
    int kv = h / G;
    double *s = (double *)malloc(sizeof(double) * (size_t)(j1 - j0));
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        s[j - j0] = score(p, i, h, j);
        if (s[j - j0] > m) m = s[j - j0];        /* max over complete scores */
    }
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double w = exp(s[j - j0] - m);
        l += w;
        for (int d = 0; d < p->D; ++d) acc[d] += w * vhat(p, j, kv, d);
    }
    free(s);
    *m_out = m;
    *l_out = l;
}

/* Full attention for a list of query rows.  rows = n_rows (i, h) pairs, or
 * NULL for every row in (i, h) order.  out: [n_rows][D]; lse: [n_rows]
 * (natural log of the sum of exp(score)).  Returns the thread count used. */
static int attention_rows(const orc_problem *pp, int32_t n_rows, const int32_t *rows, double *out, double *lse);

int orc_attention(int32_t n_q, int32_t n_heads, int32_t n_kv, int32_t D, int32_t ctx,
                  const float *q, const int8_t *kc, const uint16_t *ks,
                  const uint8_t *vc, const uint16_t *vs, double scale,
                  int32_t n_rows, const int32_t *rows, double *out, double *lse)
{
    orc_problem p = {n_q, n_heads, n_kv, D, ctx, q, kc, ks, vc, vs, scale, NULL, NULL};
    return attention_rows(&p, n_rows, rows, out, lse);
}

/* The same attention over given dequantized K and V ([ctx][n_kv][D], fp64):
 * the plain definition for any codec (the INT2 cache uses it). */
int orc_attention_dense(int32_t n_q, int32_t n_heads, int32_t n_kv, int32_t D, int32_t ctx,
                        const float *q, const double *khat_in, const double *vhat_in, double scale,
                        int32_t n_rows, const int32_t *rows, double *out, double *lse)
{
    orc_problem p = {n_q, n_heads, n_kv, D, ctx, q, NULL, NULL, NULL, NULL, scale, khat_in, vhat_in};
    return attention_rows(&p, n_rows, rows, out, lse);
}

static int attention_rows(const orc_problem *pp, int32_t n_rows, const int32_t *rows, double *out, double *lse)
{
    const orc_problem p = *pp;
    const int32_t n_heads = p.n_heads, D = p.D, ctx = p.ctx, n_q = p.n_q;
    int64_t total = rows ? n_rows : (int64_t)n_q * n_heads;
    int threads = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < total; ++r) {
            int i = rows ? rows[2 * r] : (int)(r / n_heads);
            int h = rows ? rows[2 * r + 1] : (int)(r % n_heads);
            double m, l;
            double *o = out + r * D;
            partial_row(&p, i, h, 0, ctx, &m, &l, o);
            for (int d = 0; d < D; ++d) o[d] /= l;
            if (lse) lse[r] = m + log(l);
        }
    }
    return threads;
}

/* Softmax state of every row over key range [j0, j1): m, l [n_q*n_heads],
 * acc [n_q*n_heads][D].  Used to check split-and-merge ([RX9070] second
 * paragraph: per-page online log-sum-exp accumulation). */
void orc_attention_partial(int32_t n_q, int32_t n_heads, int32_t n_kv, int32_t D, int32_t ctx,
                           const float *q, const int8_t *kc, const uint16_t *ks,
                           const uint8_t *vc, const uint16_t *vs, double scale,
                           int64_t j0, int64_t j1, double *m, double *l, double *acc)
{
    orc_problem p = {n_q, n_heads, n_kv, D, ctx, q, kc, ks, vc, vs, scale, NULL, NULL};
    int64_t total = (int64_t)n_q * n_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r)
        partial_row(&p, (int)(r / n_heads), (int)(r % n_heads), j0, j1, &m[r], &l[r], acc + r * D);
}

/* Combine n_splits softmax states of one row: M = max m_s,
 * L = sum l_s e^(m_s - M), o = sum acc_s e^(m_s - M) / L, lse = M + ln L. */
void orc_merge(int32_t n_splits, int32_t D, const double *m, const double *l, const double *acc,
               double *out, double *lse)
{
    double M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) if (m[s] > M) M = m[s];
    double L = 0.0;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int s = 0; s < n_splits; ++s) {
        if (l[s] == 0.0) continue;                     /* empty split */
        double w = exp(m[s] - M);
        L += l[s] * w;
        for (int d = 0; d < D; ++d) out[d] += acc[(int64_t)s * D + d] * w;
    }
    for (int d = 0; d < D; ++d) out[d] /= L;
    *lse = M + log(L);
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
