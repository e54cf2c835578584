/*
 * attn_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, double-precision CPU definition of causal grouped-query
 * attention for a chunk of C query rows at positions P..P+C-1 against a cache
 * of P+C key/value positions.  Only tests, the smoke check and the CPU leg of
 * the benchmark may call it.  It shares no code, header or constant with the
 * GPU library.
 *
 * What it computes, and where the pages define it:
 *   - "Inference Attention 1: The Full Score Matrix", Lesson: for each query,
 *     score every key, softmax the scores, take the weighted sum of the
 *     values; subtract the row maximum before exponentiating.
 *   - "Inference Attention 2: Flash Prefill Against a Cached Prefix", Lesson:
 *     query row i sees keys j <= P + i; 32 query heads, 8 KV heads, head
 *     size 64; query head h reads KV head h / 4; the scale is exactly 1/8;
 *     the reference sums in double.
 *
 * For every row i in [0, C), head h in [0, 32), g = h / 4, and n = P + i + 1
 * visible keys:
 *   s_j  = (1/8) * sum_{k<64} q[i][h][k] * K[j][g][k]          j = 0 .. P+i
 *   M    = max_j s_j
 *   w_j  = exp(s_j - M)
 *   L    = sum_j w_j
 *   out[i][h][d] = (float)( (sum_j w_j * V[j][g][d]) / L )
 * All sums run in ascending index order in double; the result is rounded to
 * float once.  Inputs are float32 arrays; bfloat16 inputs are passed widened
 * to float32 (an exact widening).
 *
 * Paged caches ("FlashAttention and inference kernels", section PagedAttention):
 * the cache is cut into pages of pageSize positions; position t lives at slot
 * t % pageSize of physical page blockTable[t / pageSize].  The paged entry
 * gathers the logical cache position by position and then computes exactly the
 * definition above.
 *
 * Parity pins: see the oracle tests (golden worked example, single visible
 * key, planted 4.0 rows, zero keys giving exact prefix means, convex-hull and
 * permutation invariants, numpy float64 formulation on tiny shapes; paged
 * gather against the contiguous layout).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_HQ 32
#define OR_HKV 8
#define OR_D 64
#define OR_GROUP (OR_HQ / OR_HKV)

/* One (row, head) output vector of 64 floats, written to orow.
 * s is scratch for n = P+i+1 doubles. */
static void oracle_one_row(const float* q, const float* kc, const float* vc, float* orow,
                           int i, int h, int P, double* s) {
    const int g = h / OR_GROUP;
    const int n = P + i + 1;
    const float* qrow = q + ((size_t)i * OR_HQ + h) * OR_D;

    /* step 1: score every visible key */
    for (int j = 0; j < n; ++j) {
        const float* krow = kc + ((size_t)j * OR_HKV + g) * OR_D;
        double dot = 0.0;
        for (int k = 0; k < OR_D; ++k) dot += (double)qrow[k] * (double)krow[k];
        s[j] = dot * 0.125;
    }

    /* step 2: stable softmax weights (max subtracted before exp) */
    double M = s[0];
    for (int j = 1; j < n; ++j)
        if (s[j] > M) M = s[j];
    double L = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - M);
        L += s[j];
    }

    /* step 3: weighted sum of V (each acc[d] summed in ascending j), one
     * division, one rounding */
    double acc[OR_D];
    for (int d = 0; d < OR_D; ++d) acc[d] = 0.0;
    for (int j = 0; j < n; ++j) {
        const float* vrow = vc + ((size_t)j * OR_HKV + g) * OR_D;
        for (int d = 0; d < OR_D; ++d) acc[d] += s[j] * (double)vrow[d];
    }
    for (int d = 0; d < OR_D; ++d) orow[d] = (float)(acc[d] / L);
}

/* Full output.  Returns 0 on success, nonzero on bad arguments or memory. */
int oracle_attn_prefill(const float* q, const float* kc, const float* vc, float* out,
                        int C, int P, int nthreads) {
    if (C < 0 || P < 0) return 1;
    if (C == 0) return 0;
    if (!q || !kc || !vc || !out) return 2;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(P + C));
        if (!s) {
#pragma omp atomic write
            bad = 3;
        }
#pragma omp for schedule(dynamic, 4)
        for (long t = 0; t < (long)C * OR_HQ; ++t)
            if (s)
                oracle_one_row(q, kc, vc, out + (size_t)t * OR_D, (int)(t / OR_HQ),
                               (int)(t % OR_HQ), P, s);
        free(s);
    }
    return bad;
}

/* Selected (row, head) outputs only: rows[t], heads[t] for t < count, each
 * written to out_rows + t*64.  Used to check sampled outputs at sizes where
 * the full oracle is too slow.  Returns 0 on success. */
int oracle_attn_rows(const float* q, const float* kc, const float* vc, float* out_rows,
                     int C, int P, const int* rows, const int* heads, int count, int nthreads) {
    if (C <= 0 || P < 0 || count < 0) return 1;
    if (!q || !kc || !vc || !out_rows || (count > 0 && (!rows || !heads))) return 2;
    for (int t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= C || heads[t] < 0 || heads[t] >= OR_HQ) return 1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(P + C));
        if (!s) {
#pragma omp atomic write
            bad = 3;
        }
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < count; ++t)
            if (s) oracle_one_row(q, kc, vc, out_rows + (size_t)t * OR_D, rows[t], heads[t], P, s);
        free(s);
    }
    return bad;
}

/* Paged cache: kPages/vPages are [numBlocks][pageSize][8][64]; blockTable has
 * ceil((P+C)/pageSize) entries, each in [0, numBlocks).  Returns 0 on success,
 * 1 on bad sizes or a table entry out of range, 3 if memory runs out. */
int oracle_attn_prefill_paged(const float* q, const float* kPages, const float* vPages,
                              const int* blockTable, int numBlocks, int pageSize, float* out,
                              int C, int P, int nthreads) {
    if (C < 0 || P < 0 || pageSize <= 0 || numBlocks < 0) return 1;
    if (C == 0) return 0;
    const long T = (long)P + C;
    const long nblk = (T + pageSize - 1) / pageSize;
    for (long b = 0; b < nblk; ++b)
        if (blockTable[b] < 0 || blockTable[b] >= numBlocks) return 1;
    const size_t row = (size_t)OR_HKV * OR_D;
    float* kc = (float*)malloc(sizeof(float) * (size_t)T * row);
    float* vc = (float*)malloc(sizeof(float) * (size_t)T * row);
    int rc = 3;
    if (kc && vc) {
        for (long t = 0; t < T; ++t) {
            const size_t src = ((size_t)blockTable[t / pageSize] * pageSize + (size_t)(t % pageSize)) * row;
            for (size_t e = 0; e < row; ++e) {
                kc[(size_t)t * row + e] = kPages[src + e];
                vc[(size_t)t * row + e] = vPages[src + e];
            }
        }
        rc = oracle_attn_prefill(q, kc, vc, out, C, P, nthreads);
    }
    free(kc);
    free(vc);
    return rc;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
