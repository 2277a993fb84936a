/*
 * Runs every entry point of the CPU oracle (oracle/moe_oracle.c, compiled into this file)
 * on small seeded shapes, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_layout.py: an out-of-bounds access, a use after free, a leak or undefined
 * arithmetic in the oracle aborts the run.  It also checks the invariants every routing must
 * satisfy and the documented error returns.  Prints "<n> failures".
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/moe_oracle.c"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            printf("FAIL line %d: %s\n", __LINE__, #c);                 \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
/* uniform in [-1, 1) as a bf16 bit pattern (upper half of the binary32) */
static uint16_t rand_bf16(void)
{
    float v = (float)(next_u32() % 65536u) / 32768.0f - 1.0f;
    uint32_t u;
    memcpy(&u, &v, 4);
    return (uint16_t)(u >> 16);
}

static void run_shape(int64_t B, int64_t d, int64_t f, int64_t E, int64_t k, int with_bias)
{
    printf("shape B=%lld d=%lld f=%lld E=%lld k=%lld bias=%d\n", (long long)B, (long long)d, (long long)f,
           (long long)E, (long long)k, with_bias);
    const int64_t Bm = B > 0 ? B : 1;
    uint16_t *x = malloc((size_t)(Bm * d) * 2);
    float *Wr = malloc((size_t)(d * E) * 4);
    float *bias = malloc((size_t)E * 4);
    uint16_t *W1 = malloc((size_t)(E * d * f) * 2), *W3 = malloc((size_t)(E * d * f) * 2);
    uint16_t *W2 = malloc((size_t)(E * f * d) * 2);
    for (int64_t i = 0; i < Bm * d; ++i) x[i] = rand_bf16();
    for (int64_t i = 0; i < d * E; ++i) Wr[i] = (float)(next_u32() % 2001u) / 1000.0f - 1.0f;
    for (int64_t i = 0; i < E; ++i) bias[i] = -0.5f * (float)i;
    for (int64_t i = 0; i < E * d * f; ++i) {
        W1[i] = rand_bf16();
        W3[i] = rand_bf16();
        W2[i] = rand_bf16();
    }
    float *logits = malloc((size_t)(Bm * E) * 4);
    int32_t *idx = malloc((size_t)(Bm * k) * 4);
    double *w = malloc((size_t)(Bm * k) * 8);
    int32_t *hist = malloc((size_t)E * 4), *indptr = malloc((size_t)(E + 1) * 4);
    int32_t *perm = malloc((size_t)(Bm * k) * 4), *inv = malloc((size_t)(Bm * k) * 4);
    const float *bp = with_bias ? bias : NULL;

    CHECK(oracle_router_logits(x, Wr, bp, B, d, E, logits) == 0);
    CHECK(oracle_topk(logits, B, E, k, idx) == 0);
    CHECK(oracle_softmax_topk(logits, idx, B, E, k, w) == 0);
    CHECK(oracle_histogram(idx, B, k, E, hist, indptr) == 0);
    CHECK(oracle_permutation(idx, indptr, B, k, E, perm, inv) == 0);

    int64_t total = 0;
    for (int64_t e = 0; e < E; ++e) total += hist[e];
    CHECK(total == B * k);
    CHECK(indptr[0] == 0 && indptr[E] == B * k);
    for (int64_t b = 0; b < B; ++b) {
        double s = 0.0;
        for (int64_t i = 0; i < k; ++i) {
            s += w[b * k + i];
            for (int64_t j = 0; j < i; ++j) CHECK(idx[b * k + i] != idx[b * k + j]);
            if (i > 0) CHECK(logits[b * E + idx[b * k + i - 1]] >= logits[b * E + idx[b * k + i]]);
        }
        CHECK(fabs(s - 1.0) < 1e-12);
    }
    for (int64_t a = 0; a < B * k; ++a) CHECK(perm[inv[a]] == a);
    for (int64_t e = 0; e < E; ++e)
        for (int64_t p = indptr[e] + 1; p < indptr[e + 1]; ++p) CHECK(perm[p - 1] < perm[p]);

    if (B > 0) {
        const uint16_t **t1 = malloc((size_t)E * sizeof(void *)), **t3 = malloc((size_t)E * sizeof(void *));
        const uint16_t **t2 = malloc((size_t)E * sizeof(void *));
        for (int64_t e = 0; e < E; ++e) {
            t1[e] = W1 + e * d * f;
            t3[e] = W3 + e * d * f;
            t2[e] = W2 + e * f * d;
        }
        int64_t *tokens = malloc((size_t)B * 8);
        for (int64_t b = 0; b < B; ++b) tokens[b] = B - 1 - b;
        double *out = malloc((size_t)(B * d) * 8), *one = malloc((size_t)d * 8), *row = malloc((size_t)d * 8);
        CHECK(oracle_moe_tokens(x, d, tokens, B, k, idx, w, t1, t3, t2, f, out) == 0);
        /* the last listed token through the single-token entry, and slot 0 through one expert */
        const int64_t b0 = tokens[B - 1];
        CHECK(oracle_moe_token(x + b0 * d, k, idx + b0 * k, w + b0 * k, t1, t3, t2, d, f, one) == 0);
        for (int64_t j = 0; j < d; ++j) CHECK(one[j] == out[(B - 1) * d + j]);
        const int32_t e0 = idx[b0 * k];
        CHECK(oracle_expert_row(x + b0 * d, t1[e0], t3[e0], t2[e0], d, f, row) == 0);
        for (int64_t j = 0; j < d; ++j) CHECK(isfinite(row[j]));
        /* documented failures: a negative token index, an expert table entry that is NULL */
        tokens[0] = -1;
        CHECK(oracle_moe_tokens(x, d, tokens, 1, k, idx, w, t1, t3, t2, f, out) == -2);
        t1[e0] = NULL;
        CHECK(oracle_moe_token(x + b0 * d, k, idx + b0 * k, w + b0 * k, t1, t3, t2, d, f, one) == -2);
        free(t1); free(t3); free(t2); free(tokens); free(out); free(one); free(row);
    }
    free(x); free(Wr); free(bias); free(W1); free(W3); free(W2);
    free(logits); free(idx); free(w); free(hist); free(indptr); free(perm); free(inv);
}

int main(void)
{
    run_shape(0, 64, 32, 4, 2, 0);    /* empty batch */
    run_shape(1, 64, 32, 4, 4, 1);    /* k = E */
    run_shape(37, 128, 96, 8, 3, 1);  /* ragged: d not a multiple of the column block */
    run_shape(65, 64, 300, 16, 1, 0); /* k = 1, f past one 256-column block */

    /* argument errors and NaN logits */
    float lg[4] = {1.0f, NAN, 0.0f, 2.0f};
    int32_t id[2];
    CHECK(oracle_topk(lg, 1, 4, 5, id) == -1);
    CHECK(oracle_topk(lg, 1, 4, 2, id) == -2);
    int32_t h[4], ip[5], bad[2] = {0, 7};
    CHECK(oracle_histogram(bad, 1, 2, 4, h, ip) == -2);
    CHECK(oracle_router_logits(NULL, NULL, NULL, -1, 8, 4, NULL) == -1);

    printf("%d failures\n", failures);
    return failures != 0;
}
