/*
 * fp64 CPU oracle for the fused no-KV-cache multi-head attention forward
 * (the mo.mha.no_cache operator).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library. The HIP library never calls it,
 * and it shares no code, header or table with the HIP library.
 *
 * What it computes is the plain definition of the operator:
 *   - "FlashAttentionGPU" API page (max.modular.com), section "execute",
 *     Steps 0-4: transpose BSHD to BHSD, attention matrix = Q @ K^T, scale,
 *     mask functor, softmax per row, @ V, transpose back to BSHD;
 *   - same page, grouped attention ("Step -1"): K and V may carry fewer
 *     heads (BShD); the result equals running plain attention on K and V
 *     with their heads repeated up to H;
 *   - "Custom Operations: Applications in AI Models" (builds.modular.com),
 *     section "Limitations of classic attention": bmm, softmax, bmm with
 *     the full [B, H, S, S] intermediate materialised.
 *
 * Readings taken where the pages leave a step open:
 *   - query head h reads key/value head h / (H / Hkv) (contiguous groups);
 *   - causal: key j is visible to query i iff j <= i;
 *     sliding window of width W: iff i - W < j <= i (exactly W keys);
 *   - a hidden score is -infinity, so it gets probability exactly 0;
 *   - softmax is the textbook max-subtracted form, evaluated in fp64.
 *
 * Inputs are fp64 arrays holding the exact values the GPU sees (bf16, fp16
 * or fp32 values widened to fp64); the output is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_SLIDING_WINDOW = 2 };
enum { ORACLE_OK = 0, ORACLE_INVALID_ARG = 1, ORACLE_NO_MEMORY = 3 };

/* Flat offsets of the BSHD (queries, output) and BShD (keys, values) layouts. */
static int64_t q_offset(int64_t b, int64_t i, int64_t h, int S, int H, int D)
{
    return ((b * S + i) * H + h) * D;
}

static int64_t kv_offset(int64_t b, int64_t j, int64_t g, int S, int Hkv, int D)
{
    return ((b * S + j) * Hkv + g) * D;
}

/* Grouped attention: H / Hkv consecutive query heads share one K/V head. */
static int kv_head_of(int h, int H, int Hkv)
{
    return h / (H / Hkv);
}

/* The mask functor: is key j visible to query i? */
static int visible(int mask_kind, int64_t window, int64_t i, int64_t j)
{
    switch (mask_kind) {
    case MASK_NONE:
        return 1;
    case MASK_CAUSAL:
        return j <= i;
    case MASK_SLIDING_WINDOW:
        return j <= i && j > i - window;
    default:
        return 0;
    }
}

static int check_args(int B, int S, int H, int Hkv, int D, int mask_kind, int window)
{
    if (B < 1 || S < 1 || H < 1 || Hkv < 1 || D < 1)
        return ORACLE_INVALID_ARG;
    if (H % Hkv != 0)
        return ORACLE_INVALID_ARG;
    if (mask_kind != MASK_NONE && mask_kind != MASK_CAUSAL && mask_kind != MASK_SLIDING_WINDOW)
        return ORACLE_INVALID_ARG;
    if (mask_kind == MASK_SLIDING_WINDOW && window < 1)
        return ORACLE_INVALID_ARG;
    return ORACLE_OK;
}

/*
 * Steps 1 and 3 for one row of the attention matrix:
 *   row[j] = scale * sum_d Q[b,i,h,d] * K[b,j,g,d]   if key j is visible,
 *   row[j] = -infinity                                otherwise.
 */
static void score_row(const double *q, const double *k, int b, int i, int h, int S, int H,
                      int Hkv, int D, double scale, int mask_kind, int window, double *row)
{
    const int g = kv_head_of(h, H, Hkv);
    const double *qi = q + q_offset(b, i, h, S, H, D);
    for (int j = 0; j < S; ++j) {
        if (!visible(mask_kind, window, i, j)) {
            row[j] = -INFINITY;
            continue;
        }
        const double *kj = k + kv_offset(b, j, g, S, Hkv, D);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qi[d] * kj[d];
        row[j] = dot * scale;
    }
}

/* Step 4, softmax of one row in place: p_j = exp(s_j - max) / sum_t exp(s_t - max). */
static void softmax_row(double *row, int S)
{
    double m = -INFINITY;
    for (int j = 0; j < S; ++j)
        if (row[j] > m)
            m = row[j];
    double sum = 0.0;
    for (int j = 0; j < S; ++j) {
        row[j] = exp(row[j] - m);
        sum += row[j];
    }
    for (int j = 0; j < S; ++j)
        row[j] /= sum;
}

/* Step 4, reprojection of one row: out[d] = sum_j p_j * V[b,j,g,d]. */
static void reproject_row(const double *p, const double *v, int b, int h, int S, int H, int Hkv,
                          int D, double *out)
{
    const int g = kv_head_of(h, H, Hkv);
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int j = 0; j < S; ++j) {
        if (p[j] == 0.0)
            continue; /* adds exactly +0 * finite */
        const double *vj = v + kv_offset(b, j, g, S, Hkv, D);
        for (int d = 0; d < D; ++d)
            out[d] += p[j] * vj[d];
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Whole operator. For every (b, h) the full S x S attention matrix is
 * materialised, scaled, masked and softmaxed row by row, then multiplied by
 * V; the answer is written in BSHD, like q. Rows are split across threads.
 */
int fa355_oracle_attention(const double *q, const double *k, const double *v, double *out,
                           int B, int S, int H, int Hkv, int D, double scale, int mask_kind,
                           int window, int nthreads)
{
    int rc = check_args(B, S, H, Hkv, D, mask_kind, window);
    if (rc != ORACLE_OK)
        return rc;
    if (!q || !k || !v || !out)
        return ORACLE_INVALID_ARG;
    double *att = (double *)malloc(sizeof(double) * (size_t)S * (size_t)S);
    if (!att)
        return ORACLE_NO_MEMORY;
    set_threads(nthreads);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
#pragma omp parallel for schedule(dynamic, 4)
            for (int i = 0; i < S; ++i) {
                double *row = att + (size_t)i * S;
                score_row(q, k, b, i, h, S, H, Hkv, D, scale, mask_kind, window, row);
                softmax_row(row, S);
            }
#pragma omp parallel for schedule(dynamic, 4)
            for (int i = 0; i < S; ++i)
                reproject_row(att + (size_t)i * S, v, b, h, S, H, Hkv, D,
                              out + q_offset(b, i, h, S, H, D));
        }
    }
    free(att);
    return ORACLE_OK;
}

/*
 * Selected output rows only, for checks at sizes where the whole operator
 * is too slow. rows holds nrows triples (b, h, i); out receives nrows x D.
 * Each row of the attention matrix is materialised on its own.
 */
int fa355_oracle_rows(const double *q, const double *k, const double *v, int B, int S, int H,
                      int Hkv, int D, double scale, int mask_kind, int window,
                      const int64_t *rows, int64_t nrows, double *out, int nthreads)
{
    int rc = check_args(B, S, H, Hkv, D, mask_kind, window);
    if (rc != ORACLE_OK)
        return rc;
    if (!q || !k || !v || !out || (nrows > 0 && !rows) || nrows < 0)
        return ORACLE_INVALID_ARG;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S)
            return ORACLE_INVALID_ARG;
    }
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)S);
        if (!row) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!row)
                continue;
            const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
            score_row(q, k, b, i, h, S, H, Hkv, D, scale, mask_kind, window, row);
            softmax_row(row, S);
            reproject_row(row, v, b, h, S, H, Hkv, D, out + r * D);
        }
        free(row);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* One row of the softmaxed attention matrix (probabilities p[b,h,i,:]). */
int fa355_oracle_probs(const double *q, const double *k, int B, int S, int H, int Hkv, int D,
                       double scale, int mask_kind, int window, int b, int h, int i, double *p)
{
    int rc = check_args(B, S, H, Hkv, D, mask_kind, window);
    if (rc != ORACLE_OK)
        return rc;
    if (!q || !k || !p || b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S)
        return ORACLE_INVALID_ARG;
    score_row(q, k, b, i, h, S, H, Hkv, D, scale, mask_kind, window, p);
    softmax_row(p, S);
    return ORACLE_OK;
}

/* Number of visible (query, key) pairs of one head under the mask. */
int64_t fa355_oracle_visible_pairs(int S, int mask_kind, int window)
{
    int64_t n = 0;
    for (int64_t i = 0; i < S; ++i)
        for (int64_t j = 0; j < S; ++j)
            n += visible(mask_kind, window, i, j);
    return n;
}

/* Threads an OpenMP region of this library would use (1 without OpenMP). */
int fa355_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
