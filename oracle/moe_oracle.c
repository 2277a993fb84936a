/*
 * moe_oracle.c -- plain, slow CPU reference of one top-k Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never links,
 * loads or calls it, and the two share no code: no headers, helpers or tables.
 *
 * What the layer computes.  "Event Tensor: A Unified Abstraction for Compiling
 * Dynamic Megakernel" (MLSys 2026), section "Problem", names the data-dependent
 * steps of an MoE layer: routing by the runtime top-k, token grouping, and a
 * GroupGEMM over the experts.  Its section "Core method" says that grouping updates
 * the event of the expert each token was routed to, and that the exp_indptr prefix
 * sum (the per-expert row offsets) decides how many GroupGEMM tiles each expert
 * triggers.  The pages do not print the arithmetic, so this file writes out the
 * standard layer, with these readings:
 *
 *   router   logit[b,e] = sum_j x[b,j] * Wr[j,e]  (+ bias[e]), fp32, in the fixed
 *            order described at oracle_router_logits (the order decides top-k near
 *            ties, so it is part of the contract);
 *   top-k    the k largest logits of each token, ties to the lowest expert index;
 *   weights  softmax over the k selected logits;
 *   grouping histogram of rows per expert, exclusive prefix sum exp_indptr[E+1],
 *            stable counting sort of the assignments a = b*k + i by expert;
 *   experts  SwiGLU: h = silu(x W1[e]) * (x W3[e]),  y = h W2[e],
 *            W1/W3 are [E, d, f] (gate / up), W2 is [E, f, d];
 *   combine  out[b,:] = sum_i w[b,i] * y(b,i)[:].
 *
 * Precision.  The router and top-k run in fp32 because the top-k decision has to be
 * taken in the same precision as the GPU path.  Everything after the decision
 * (softmax weights, expert FFN, combine) is computed in fp64 from the bf16 inputs
 * taken as exact values.  Compile with -O2 -ffp-contract=off and without fast-math.
 *
 * Every function returns 0 on success and a negative value on bad arguments.
 * OpenMP parallelism is only over independent outputs, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_LANES 64

/* bfloat16 is the upper half of an IEEE binary32; the conversion to float is exact. */
static float bf16_value(uint16_t v)
{
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Router logits, fp32.  For every (token b, expert e):
 *   64 partial sums s[0..63] start at +0.0f;
 *   for j = 0, 1, ..., d-1 in ascending order: s[j mod 64] = fmaf(x[b,j], Wr[j,e], s[j mod 64]);
 *   the partial sums are folded in halves: for t = 32, 16, 8, 4, 2, 1 and every l < t,
 *   s[l] = s[l] + s[l+t];
 *   logit = s[0] + bias[e]   (bias taken as +0.0f when absent, still added).
 * x is bf16 [B, d], Wr fp32 [d, E] row-major, bias fp32 [E] or NULL, logits fp32 [B, E].
 */
int oracle_router_logits(const uint16_t *x, const float *Wr, const float *bias,
                         int64_t B, int64_t d, int64_t E, float *logits)
{
    if (B < 0 || d <= 0 || E <= 0) return -1;
    if (B == 0) return 0;
    if (!x || !Wr || !logits) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t e = 0; e < E; ++e) {
            float s[ORACLE_LANES];
            for (int l = 0; l < ORACLE_LANES; ++l) s[l] = 0.0f;
            for (int64_t j = 0; j < d; ++j) {
                int l = (int)(j % ORACLE_LANES);
                s[l] = fmaf(bf16_value(x[b * d + j]), Wr[j * E + e], s[l]);
            }
            for (int t = ORACLE_LANES / 2; t >= 1; t /= 2)
                for (int l = 0; l < t; ++l) s[l] = s[l] + s[l + t];
            float bias_e = bias ? bias[e] : 0.0f;
            logits[b * E + e] = s[0] + bias_e;
        }
    }
    return 0;
}

/*
 * Top-k selection: for each token, slot 0 holds the largest logit, slot 1 the next,
 * and so on.  Ordering is IEEE comparison (so -0.0 == +0.0); equal logits go to the
 * lower expert index.  NaN logits are rejected (-2).
 */
int oracle_topk(const float *logits, int64_t B, int64_t E, int64_t k, int32_t *idx)
{
    if (B < 0 || E <= 0 || k <= 0 || k > E) return -1;
    if (B == 0) return 0;
    if (!logits || !idx) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        const float *l = logits + b * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        if (!taken) { bad |= 1; continue; }
        for (int64_t e = 0; e < E; ++e)
            if (isnan(l[e])) bad |= 1;
        for (int64_t s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;  /* strict: ties keep the lower index */
            }
            taken[best] = 1;
            idx[b * k + s] = (int32_t)best;
        }
        free(taken);
    }
    return bad ? -2 : 0;
}

/*
 * Softmax over the k selected logits, fp64:  w_i = exp(l_i - l_0) / sum_j exp(l_j - l_0),
 * summed in slot order.  l_0 is the largest selected logit.
 */
int oracle_softmax_topk(const float *logits, const int32_t *idx, int64_t B, int64_t E,
                        int64_t k, double *w)
{
    if (B < 0 || E <= 0 || k <= 0 || k > E) return -1;
    if (B == 0) return 0;
    if (!logits || !idx || !w) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double m = (double)logits[b * E + idx[b * k]];
        double sum = 0.0;
        for (int64_t i = 0; i < k; ++i) {
            double ex = exp((double)logits[b * E + idx[b * k + i]] - m);
            w[b * k + i] = ex;
            sum += ex;
        }
        for (int64_t i = 0; i < k; ++i) w[b * k + i] = w[b * k + i] / sum;
    }
    return 0;
}

/*
 * Rows per expert and the exclusive prefix sum exp_indptr (length E+1):
 * hist[e] = #{(b,i) : idx[b,i] = e},  exp_indptr[0] = 0,  exp_indptr[e+1] = exp_indptr[e] + hist[e].
 */
int oracle_histogram(const int32_t *idx, int64_t B, int64_t k, int64_t E,
                     int32_t *hist, int32_t *exp_indptr)
{
    if (B < 0 || E <= 0 || k <= 0) return -1;
    if (!hist || !exp_indptr || (B > 0 && !idx)) return -1;
    for (int64_t e = 0; e < E; ++e) hist[e] = 0;
    for (int64_t a = 0; a < B * k; ++a) {
        int32_t e = idx[a];
        if (e < 0 || e >= E) return -2;
        hist[e] += 1;
    }
    exp_indptr[0] = 0;
    for (int64_t e = 0; e < E; ++e) exp_indptr[e + 1] = exp_indptr[e] + hist[e];
    return 0;
}

/*
 * Token grouping: a stable counting sort of the assignments a = b*k + i (taken in
 * ascending a) by expert.  perm[p] = a puts assignment a at row p of its expert's
 * segment [exp_indptr[e], exp_indptr[e+1]); inv[a] = p is the inverse.  Within a
 * segment the token index ascends.
 */
int oracle_permutation(const int32_t *idx, const int32_t *exp_indptr, int64_t B, int64_t k,
                       int64_t E, int32_t *perm, int32_t *inv)
{
    if (B < 0 || E <= 0 || k <= 0) return -1;
    if (B == 0) return 0;
    if (!idx || !exp_indptr || !perm || !inv) return -1;
    int64_t *next = (int64_t *)malloc((size_t)E * sizeof(int64_t));
    if (!next) return -3;
    for (int64_t e = 0; e < E; ++e) next[e] = exp_indptr[e];
    for (int64_t a = 0; a < B * k; ++a) {
        int32_t e = idx[a];
        if (e < 0 || e >= E) { free(next); return -2; }
        int64_t p = next[e]++;
        perm[p] = (int32_t)a;
        inv[a] = (int32_t)p;
    }
    free(next);
    return 0;
}

/*
 * One expert applied to one row, fp64:
 *   g[n] = sum_c x[c] W1[c,n],  u[n] = sum_c x[c] W3[c,n]        (W1, W3: [d, f])
 *   h[n] = g[n] / (1 + exp(-g[n])) * u[n]                           (SwiGLU, W1 = gate)
 *   y[j] = sum_n h[n] W2[n,j]                                       (W2: [f, d])
 * x is one bf16 row of length d; y has length d.
 *
 * The work is split into blocks of output columns.  Every column is computed by the
 * same loop (c ascending for g and u, n ascending for y) whichever thread runs its
 * block, so the result does not depend on how the blocks are shared out.
 */
#define ORACLE_COL_BLOCK 256

/* Gate/up columns [n0, n1): g and u (zero on entry) summed over c, then h. */
static void expert_gateup_block(const uint16_t *xrow, const uint16_t *W1e, const uint16_t *W3e,
                                int64_t d, int64_t f, int64_t n0, int64_t n1,
                                double *g, double *u, double *h)
{
    for (int64_t c = 0; c < d; ++c) {
        double xc = (double)bf16_value(xrow[c]);
        const uint16_t *w1 = W1e + c * f;
        const uint16_t *w3 = W3e + c * f;
        for (int64_t n = n0; n < n1; ++n) {
            g[n] += xc * (double)bf16_value(w1[n]);
            u[n] += xc * (double)bf16_value(w3[n]);
        }
    }
    for (int64_t n = n0; n < n1; ++n) h[n] = g[n] / (1.0 + exp(-g[n])) * u[n];
}

/* Down-projection columns [j0, j1): y[j] summed over n. */
static void expert_down_block(const double *h, const uint16_t *W2e, int64_t d, int64_t f,
                              int64_t j0, int64_t j1, double *y)
{
    for (int64_t j = j0; j < j1; ++j) y[j] = 0.0;
    for (int64_t n = 0; n < f; ++n) {
        const uint16_t *w2 = W2e + n * d;
        for (int64_t j = j0; j < j1; ++j) y[j] += h[n] * (double)bf16_value(w2[j]);
    }
}

/* parallel_blocks: share the column blocks over OpenMP threads (one row at a time), or
 * run them in order on the calling thread (when rows are shared out instead). */
static int expert_row_impl(const uint16_t *xrow, const uint16_t *W1e, const uint16_t *W3e,
                           const uint16_t *W2e, int64_t d, int64_t f, double *y, int parallel_blocks)
{
    double *g = (double *)calloc((size_t)f, sizeof(double));
    double *u = (double *)calloc((size_t)f, sizeof(double));
    double *h = (double *)malloc((size_t)f * sizeof(double));
    if (!g || !u || !h) { free(g); free(u); free(h); return -3; }
    const int64_t NB = ORACLE_COL_BLOCK;
#pragma omp parallel for schedule(static) if (parallel_blocks)
    for (int64_t n0 = 0; n0 < f; n0 += NB)
        expert_gateup_block(xrow, W1e, W3e, d, f, n0, n0 + NB < f ? n0 + NB : f, g, u, h);
#pragma omp parallel for schedule(static) if (parallel_blocks)
    for (int64_t j0 = 0; j0 < d; j0 += NB)
        expert_down_block(h, W2e, d, f, j0, j0 + NB < d ? j0 + NB : d, y);
    free(g);
    free(u);
    free(h);
    return 0;
}

int oracle_expert_row(const uint16_t *xrow, const uint16_t *W1e, const uint16_t *W3e,
                      const uint16_t *W2e, int64_t d, int64_t f, double *y)
{
    if (d <= 0 || f <= 0) return -1;
    if (!xrow || !W1e || !W3e || !W2e || !y) return -1;
    return expert_row_impl(xrow, W1e, W3e, W2e, d, f, y, 1);
}

/*
 * One token's layer output, fp64: out[j] = sum_{i<k} w[i] * y_i[j], slot order,
 * where y_i is expert idx[i] applied to the token's row.
 */
static int moe_token_impl(const uint16_t *xrow, int64_t k, const int32_t *idx, const double *w,
                          const uint16_t *const *W1, const uint16_t *const *W3,
                          const uint16_t *const *W2, int64_t d, int64_t f, double *out,
                          int parallel_blocks)
{
    double *y = (double *)malloc((size_t)d * sizeof(double));
    if (!y) return -3;
    for (int64_t j = 0; j < d; ++j) out[j] = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        int32_t e = idx[i];
        if (e < 0 || !W1[e] || !W3[e] || !W2[e]) { free(y); return -2; }
        int rc = expert_row_impl(xrow, W1[e], W3[e], W2[e], d, f, y, parallel_blocks);
        if (rc) { free(y); return rc; }
        for (int64_t j = 0; j < d; ++j) out[j] += w[i] * y[j];
    }
    free(y);
    return 0;
}

/*
 * Expert weights are passed as per-expert pointer tables W1[e], W3[e], W2[e] (entries of
 * experts the token does not use may be NULL), so callers can hold only the experts they
 * need.  The column blocks of each expert row are shared over OpenMP threads.
 */
int oracle_moe_token(const uint16_t *xrow, int64_t k, const int32_t *idx, const double *w,
                     const uint16_t *const *W1, const uint16_t *const *W3,
                     const uint16_t *const *W2, int64_t d, int64_t f, double *out)
{
    if (k <= 0 || d <= 0 || f <= 0) return -1;
    if (!xrow || !idx || !w || !W1 || !W3 || !W2 || !out) return -1;
    return moe_token_impl(xrow, k, idx, w, W1, W3, W2, d, f, out, 1);
}

/*
 * The layer output of n listed tokens, fp64: out[r, :] is oracle_moe_token of token
 * tokens[r] (row tokens[r] of x [*, d], its slots idx[tokens[r], :] and weights
 * w[tokens[r], :], both [*, k]).  The tokens are shared over OpenMP threads, one token per
 * thread at a time; each token's arithmetic is exactly that of oracle_moe_token.
 */
int oracle_moe_tokens(const uint16_t *x, int64_t d, const int64_t *tokens, int64_t n, int64_t k,
                      const int32_t *idx, const double *w, const uint16_t *const *W1,
                      const uint16_t *const *W3, const uint16_t *const *W2, int64_t f,
                      double *out)
{
    if (n < 0 || k <= 0 || d <= 0 || f <= 0) return -1;
    if (n == 0) return 0;
    if (!x || !tokens || !idx || !w || !W1 || !W3 || !W2 || !out) return -1;
    int rc_all = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc_all)
    for (int64_t r = 0; r < n; ++r) {
        const int64_t t = tokens[r];
        int rc = t < 0 ? -1
                       : moe_token_impl(x + t * d, k, idx + t * k, w + t * k, W1, W3, W2, d, f,
                                        out + r * d, 0);
        if (rc) rc_all |= 1;
    }
    return rc_all ? -2 : 0;
}
