/*
 * oracle_sanitize_driver.c -- runs every exported function of the C oracle
 * (oracle/kvq_oracle.c, included below so that it is compiled with this
 * file's flags) on small seeded inputs.  tests/test_oracle_sanitize.py builds
 * it with -fsanitize=address,undefined and checks that it exits cleanly: any
 * out-of-bounds access, leak, or undefined operation (signed overflow, a bad
 * shift, misaligned access) in the oracle aborts the run.
 *
 * A few cheap consistency checks ride along (the real pins live in the
 * Python tests): one key returns its dequantized value, and splitting the keys
 * then merging by log-sum-exp gives the unsplit result.
 *
 * Test infrastructure only; nothing in the GPU library includes it.
 */
#include "../oracle/kvq_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64, then a Box-Muller normal; only the input values depend on it */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float normal(void)
{
    double u1 = ((next_u64() >> 11) + 1.0) / 9007199254740993.0;
    double u2 = (next_u64() >> 11) / 9007199254740992.0;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "check failed: " __VA_ARGS__); \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

int main(void)
{
    enum { NQ = 3, NH = 4, NKV = 2, D = 128, CTX = 37 };
    const int nb = D / ORC_BLOCK, nb2 = D / ORC_BLOCK2;
    const size_t n_kv_vals = (size_t)CTX * NKV * D;

    /* scalars over every fp16 pattern and a spread of floats */
    for (uint32_t h = 0; h < 65536; ++h) (void)orc_f16_to_f32((uint16_t)h);
    for (int i = 0; i < 4096; ++i) (void)orc_f32_to_f16(normal() * ldexpf(1.0f, i % 40 - 10));
    CHECK(orc_f32_to_f16(1.0f) == 0x3C00, "fp16(1)");

    float *k = malloc(sizeof(float) * n_kv_vals), *v = malloc(sizeof(float) * n_kv_vals);
    float *q = malloc(sizeof(float) * NQ * NH * D);
    for (size_t i = 0; i < n_kv_vals; ++i) { k[i] = normal(); v[i] = normal(); }
    for (int i = 0; i < NQ * NH * D; ++i) q[i] = normal();
    /* a zero block and a block of equal magnitudes of both signs */
    for (int d = 0; d < ORC_BLOCK; ++d) { k[d] = 0.0f; v[d] = 0.0f; k[D + d] = (d & 1) ? -3.0f : 3.0f; }

    int8_t *kc = malloc(n_kv_vals);
    uint8_t *vc = malloc(n_kv_vals);
    uint16_t *ks = malloc(sizeof(uint16_t) * CTX * NKV * nb), *vs = malloc(sizeof(uint16_t) * CTX * NKV * nb);
    orc_quantize_q8_0(k, (int64_t)CTX * NKV * nb, kc, ks);
    orc_quantize_q4_0(v, (int64_t)CTX * NKV * nb, vc, vs);
    double *kd = malloc(sizeof(double) * n_kv_vals), *vd = malloc(sizeof(double) * n_kv_vals);
    orc_dequant_q8_0(kc, ks, (int64_t)CTX * NKV * nb, kd);
    orc_dequant_q4_0(vc, vs, (int64_t)CTX * NKV * nb, vd);
    for (size_t i = 0; i < n_kv_vals; ++i) CHECK(vc[i] <= 15, "Q4_0 code %zu out of range", i);

    uint8_t *c2 = malloc(n_kv_vals);
    uint16_t *s2 = malloc(sizeof(uint16_t) * CTX * NKV * nb2), *z2 = malloc(sizeof(uint16_t) * CTX * NKV * nb2);
    double *d2 = malloc(sizeof(double) * n_kv_vals);
    orc_quantize_int2(k, (int64_t)CTX * NKV * nb2, c2, s2, z2);
    orc_dequant_int2(c2, s2, z2, (int64_t)CTX * NKV * nb2, d2);
    for (size_t i = 0; i < n_kv_vals; ++i) CHECK(c2[i] <= 3, "INT2 code %zu out of range", i);

    CHECK(orc_kv_bytes_per_token_f16(32, 8, 128) == 131072, "fp16 bytes per token");
    CHECK(orc_kv_bytes_per_token_q8k_q4v(16, 4, 256) == 26624, "quantized bytes per token");
    CHECK(orc_q8_0_block_bytes() == 34 && orc_q4_0_block_bytes() == 18 && orc_int2_block_bytes() == 36,
          "block bytes");

    /* attention: every row, a row list, the dense form, the split form */
    const double scale = 1.0 / sqrt((double)D);
    double *out = malloc(sizeof(double) * NQ * NH * D), *lse = malloc(sizeof(double) * NQ * NH);
    (void)orc_attention(NQ, NH, NKV, D, CTX, q, kc, ks, vc, vs, scale, 0, NULL, out, lse);
    int32_t rows[4] = {2, 3, 0, 1};
    double out2[2 * D], lse2[2];
    (void)orc_attention(NQ, NH, NKV, D, CTX, q, kc, ks, vc, vs, scale, 2, rows, out2, lse2);
    for (int d = 0; d < D; ++d) CHECK(out2[d] == out[(2 * NH + 3) * D + d], "row list, dim %d", d);
    double *outd = malloc(sizeof(double) * NQ * NH * D), *lsed = malloc(sizeof(double) * NQ * NH);
    (void)orc_attention_dense(NQ, NH, NKV, D, CTX, q, kd, vd, scale, 0, NULL, outd, lsed);
    for (int i = 0; i < NQ * NH * D; ++i) CHECK(fabs(outd[i] - out[i]) <= 1e-12 * (1 + fabs(out[i])), "dense %d", i);
    (void)orc_attention_dense(NQ, NH, NKV, D, CTX, q, d2, d2, scale, 0, NULL, outd, lsed);

    /* split at 0 | 11 | 30 | CTX, merge, compare with the unsplit rows */
    enum { S = 3 };
    const int64_t cut[S + 1] = {0, 11, 30, CTX};
    double *m = malloc(sizeof(double) * S * NQ * NH), *l = malloc(sizeof(double) * S * NQ * NH);
    double *acc = malloc(sizeof(double) * S * NQ * NH * D);
    for (int s = 0; s < S; ++s)
        orc_attention_partial(NQ, NH, NKV, D, CTX, q, kc, ks, vc, vs, scale, cut[s], cut[s + 1],
                              m + s * NQ * NH, l + s * NQ * NH, acc + (size_t)s * NQ * NH * D);
    for (int r = 0; r < NQ * NH; ++r) {
        double ms[S], ls[S], as[S * D], o[D], lr;
        for (int s = 0; s < S; ++s) {
            ms[s] = m[s * NQ * NH + r];
            ls[s] = l[s * NQ * NH + r];
            memcpy(as + s * D, acc + ((size_t)s * NQ * NH + r) * D, sizeof(double) * D);
        }
        orc_merge(S, D, ms, ls, as, o, &lr);
        for (int d = 0; d < D; ++d) CHECK(fabs(o[d] - out[r * D + d]) <= 1e-12 * (1 + fabs(out[r * D + d])), "merge");
        CHECK(fabs(lr - lse[r]) <= 1e-12 * (1 + fabs(lse[r])), "merge lse");
    }

    /* one key: the output is that key's dequantized value */
    double o1[NH * D], l1[NH];
    (void)orc_attention(1, NH, NKV, D, 1, q, kc, ks, vc, vs, scale, 0, NULL, o1, l1);
    for (int h = 0; h < NH; ++h)
        for (int d = 0; d < D; ++d) CHECK(o1[h * D + d] == vd[(h / (NH / NKV)) * D + d], "one key h=%d d=%d", h, d);

    (void)orc_max_threads();
    free(k); free(v); free(q); free(kc); free(vc); free(ks); free(vs); free(kd); free(vd);
    free(c2); free(s2); free(z2); free(d2); free(out); free(lse); free(outd); free(lsed);
    free(m); free(l); free(acc);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitize driver: ok\n");
    return 0;
}
