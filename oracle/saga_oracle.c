/*
 * saga_oracle.c -- plain fp64 CPU oracle for SAGA + Atop-N decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded input generator.
 *
 * What it computes (source: "More Value per Key: Asymmetric Sparse Attention
 * for Faster LLM Decoding", picx.dev structured summary):
 *   - scores  A = q K^T / sqrt(d)                 (Attention Mechanism
 *     Formalization, eqs. 2-4)
 *   - threshold tau = N-th largest entry of a score row, found by a full
 *     descending sort                             (Top-N Attention, eq. 6;
 *     Methodology > Atop-N Attention, item 1)
 *   - selection S = { t : A_t >= tau }            (Atop-N, item 1)
 *   - tau recomputed exactly once every R decode steps and reused between
 *     refreshes                                   (Atop-N, item 2)
 *   - O = softmax(A[S]) V[S]                      (Atop-N, eq. 7)
 *   - SAGA head decoupling: h_k key heads, h_v value heads (SAGA
 *     Architecture).  The pages give no head-to-head map; the reading used
 *     here is contiguous groups: query head j reads key head
 *     floor(j*h_k/h_q) and value head floor(j*h_v/h_q).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - ">=" against tau, ties at tau all kept (so |S| may exceed N);
 *   - a refresh happens at steps t with t mod R == 0, from that same step's
 *     scores, and is used in that step;
 *   - an empty S (tau above every score) gives O = 0 and count 0;
 *   - -0.0 and +0.0 are the same score (the fp32 order used for the tau check
 *     compares values, not bit patterns).
 *
 * Arithmetic: bf16 inputs are widened exactly to double; every sum, the
 * division by sqrt(d), exp and the normalisation are done in double with
 * libm, in plain loop order.  OpenMP only splits independent rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32: widen exactly. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int key_head_of(int j, int h_q, int h_k) { return (int)(((int64_t)j * h_k) / h_q); }
static int value_head_of(int j, int h_q, int h_v) { return (int)(((int64_t)j * h_v) / h_q); }

int sao_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void sao_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Eq. 2 for one query row against one key head: a[t] = <q, k_t> / sqrt(d). */
void sao_scores_row(const uint16_t *q, const uint16_t *Khead, int d, int64_t l_kv, double *a)
{
    double inv = 1.0 / sqrt((double)d);
    for (int64_t t = 0; t < l_kv; ++t) {
        const uint16_t *k = Khead + t * (int64_t)d;
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += bf16_to_double(q[c]) * bf16_to_double(k[c]);
        a[t] = s * inv;
    }
}

/* Scores for a whole decode step: A[b][j][t], Q [B][h_q][d], K [B][h_k][l_kv][d]. */
void sao_scores(const uint16_t *Q, const uint16_t *K, int B, int h_q, int h_k, int d, int64_t l_kv,
                double *A)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < B * h_q; ++r) {
        int b = r / h_q, j = r % h_q, g = key_head_of(j, h_q, h_k);
        sao_scores_row(Q + (int64_t)r * d, K + ((int64_t)b * h_k + g) * l_kv * d, d, l_kv,
                       A + (int64_t)r * l_kv);
    }
}

static int cmp_desc_double(const void *x, const void *y)
{
    double a = *(const double *)x, b = *(const double *)y;
    return (a < b) - (a > b);
}

static int cmp_desc_float(const void *x, const void *y)
{
    float a = *(const float *)x, b = *(const float *)y;
    return (a < b) - (a > b);
}

/* Eq. 6 / Atop-N item 1: the N-th largest entry (1-based N) of a row, by a
 * full sort of a copy in descending order. Returns NAN on bad arguments. */
double sao_nth_largest(const double *a, int64_t n, int64_t N)
{
    if (N < 1 || N > n) return NAN;
    double *c = (double *)malloc((size_t)n * sizeof *c);
    if (!c) return NAN;
    memcpy(c, a, (size_t)n * sizeof *c);
    qsort(c, (size_t)n, sizeof *c, cmp_desc_double);
    double v = c[N - 1];
    free(c);
    return v;
}

/* The same selection over fp32 values, used to check a GPU threshold
 * bit-for-bit against the GPU's own fp32 scores. */
float sao_nth_largest_f32(const float *a, int64_t n, int64_t N)
{
    if (N < 1 || N > n) return NAN;
    float *c = (float *)malloc((size_t)n * sizeof *c);
    if (!c) return NAN;
    memcpy(c, a, (size_t)n * sizeof *c);
    qsort(c, (size_t)n, sizeof *c, cmp_desc_float);
    float v = c[N - 1];
    free(c);
    return v;
}

/* Eq. 7 for one row: softmax over the selected scores, times the selected
 * value rows.  mask[t] != 0 marks t in S.  Returns |S|; O row is all zero
 * when S is empty. */
int64_t sao_attend_row(const double *a, const uint8_t *mask, const uint16_t *Vhead, int d,
                       int64_t l_kv, double *o)
{
    int64_t cnt = 0;
    double m = -INFINITY;
    for (int64_t t = 0; t < l_kv; ++t)
        if (mask[t]) {
            ++cnt;
            if (a[t] > m) m = a[t];
        }
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (cnt == 0) return 0;
    double den = 0.0;
    for (int64_t t = 0; t < l_kv; ++t)
        if (mask[t]) den += exp(a[t] - m);
    for (int64_t t = 0; t < l_kv; ++t) {
        if (!mask[t]) continue;
        double p = exp(a[t] - m) / den;
        const uint16_t *v = Vhead + t * (int64_t)d;
        for (int c = 0; c < d; ++c) o[c] += p * bf16_to_double(v[c]);
    }
    return cnt;
}

/* Atop-N comparison (item 1): mask[t] = (a[t] >= tau). Returns |S|. */
int64_t sao_select_row(const double *a, int64_t l_kv, double tau, uint8_t *mask)
{
    int64_t cnt = 0;
    for (int64_t t = 0; t < l_kv; ++t) {
        mask[t] = (uint8_t)(a[t] >= tau);
        cnt += mask[t];
    }
    return cnt;
}

/*
 * A whole Atop-N decode trajectory over T steps with a static cache.
 *   Q     [T][B][h_q][d]   bf16 query of every step
 *   K     [B][h_k][l_kv][d] bf16,  V [B][h_v][l_kv][d] bf16
 *   O     [T][B][h_q][d]   out, double
 *   tau   [T][B][h_q]      out, the threshold in force at each step
 *   count [T][B][h_q]      out, |S|
 *   mask  [T][B][h_q][l_kv] out, nullable: the selection of every step
 * A refresh (exact tau from this step's scores) happens when t % R == 0.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int sao_trajectory(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int T, int B, int h_q,
                   int h_k, int h_v, int d, int64_t l_kv, int64_t N, int R, double *O, double *tau,
                   int64_t *count, uint8_t *mask_out)
{
    if (T < 1 || B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || h_k > h_q || h_v > h_q || d < 1 ||
        l_kv < 1 || N < 1 || N > l_kv || R < 1)
        return -1;
    int rows = B * h_q;
    double *tau_cur = (double *)malloc((size_t)rows * sizeof *tau_cur);
    if (!tau_cur) return -1;
    int fail = 0;
    for (int t = 0; t < T; ++t) {
        int refresh = (t % R) == 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
        for (int r = 0; r < rows; ++r) {
            int b = r / h_q, j = r % h_q;
            int g = key_head_of(j, h_q, h_k), v = value_head_of(j, h_q, h_v);
            double *a = (double *)malloc((size_t)l_kv * sizeof *a);
            uint8_t *mk = (uint8_t *)malloc((size_t)l_kv);
            if (!a || !mk) {
                free(a);
                free(mk);
                fail |= 1;
                continue;
            }
            const uint16_t *q = Q + (((int64_t)t * B + b) * h_q + j) * d;
            sao_scores_row(q, K + ((int64_t)b * h_k + g) * l_kv * d, d, l_kv, a);
            if (refresh) tau_cur[r] = sao_nth_largest(a, l_kv, N);
            int64_t idx = (int64_t)t * rows + r;
            tau[idx] = tau_cur[r];
            sao_select_row(a, l_kv, tau_cur[r], mk);
            count[idx] = sao_attend_row(a, mk, V + ((int64_t)b * h_v + v) * l_kv * d, d, l_kv,
                                        O + idx * d);
            if (mask_out) memcpy(mask_out + idx * l_kv, mk, (size_t)l_kv);
            free(a);
            free(mk);
        }
    }
    free(tau_cur);
    return fail ? -1 : 0;
}

/*
 * A whole Atop-N decode trajectory over a GROWING cache: the decode loop's
 * key/value cache (Introduction > Background: keys and values of earlier
 * tokens are cached and reused) receives the current token's key and value
 * rows before the step attends, so step t attends over the first
 *     len_t = l0 + t + 1
 * cache rows, the newest being the current token's.  The threshold follows
 * Atop-N items 1-2 exactly as in sao_trajectory: at t mod R == 0 it is the
 * exact N-th largest of this step's len_t scores; at every other step the
 * threshold of the last refresh is reused, and the rows appended since then
 * (the new keys) are compared with it like every other position.
 *   Q    [T][B][h_q][d]          bf16 query of every step
 *   K    [B][h_k][cap][d], V [B][h_v][cap][d]  bf16; rows 0 .. l0+T-1 used
 *   O    [T][B][h_q][d]          out, double
 *   tau  [T][B][h_q]             out, the threshold in force at each step
 *   count[T][B][h_q]             out, |S|
 *   mask [T][B][h_q][cap]        out, nullable; positions >= len_t are 0
 * Requires 0 <= l0, l0 + T <= cap and N <= l0 + 1 (the first step's length).
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int sao_trajectory_growing(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int T, int B,
                           int h_q, int h_k, int h_v, int d, int64_t cap, int64_t l0, int64_t N,
                           int R, double *O, double *tau, int64_t *count, uint8_t *mask_out)
{
    if (T < 1 || B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || h_k > h_q || h_v > h_q || d < 1 ||
        cap < 1 || l0 < 0 || l0 + T > cap || N < 1 || N > l0 + 1 || R < 1)
        return -1;
    int rows = B * h_q;
    double *tau_cur = (double *)malloc((size_t)rows * sizeof *tau_cur);
    if (!tau_cur) return -1;
    int fail = 0;
    for (int t = 0; t < T; ++t) {
        const int64_t len = l0 + t + 1; /* the token of step t sits at row l0 + t */
        const int refresh_step = t % R == 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
        for (int r = 0; r < rows; ++r) {
            int b = r / h_q, j = r % h_q;
            int g = key_head_of(j, h_q, h_k), v = value_head_of(j, h_q, h_v);
            double *a = (double *)malloc((size_t)len * sizeof *a);
            uint8_t *mk = (uint8_t *)malloc((size_t)len);
            if (!a || !mk) {
                free(a);
                free(mk);
                fail |= 1;
                continue;
            }
            const uint16_t *q = Q + (((int64_t)t * B + b) * h_q + j) * d;
            sao_scores_row(q, K + ((int64_t)b * h_k + g) * cap * d, d, len, a);
            if (refresh_step) tau_cur[r] = sao_nth_largest(a, len, N);
            int64_t idx = (int64_t)t * rows + r;
            tau[idx] = tau_cur[r];
            sao_select_row(a, len, tau_cur[r], mk);
            count[idx] = sao_attend_row(a, mk, V + ((int64_t)b * h_v + v) * cap * d, d, len,
                                        O + idx * d);
            if (mask_out) {
                memset(mask_out + idx * cap, 0, (size_t)cap);
                memcpy(mask_out + idx * cap, mk, (size_t)len);
            }
            free(a);
            free(mk);
        }
    }
    free(tau_cur);
    return fail ? -1 : 0;
}

/*
 * One decode step with a selection supplied from outside ("given-mask"
 * mode): O = softmax(A[S]) V[S] with S = mask, eq. 7.  Lets an output be
 * checked independently of which entries sit right at the threshold.
 *   Q [B][h_q][d], mask [B][h_q][l_kv], O [B][h_q][d], count [B][h_q].
 */
int sao_given_mask(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int B, int h_q,
                   int h_k, int h_v, int d, int64_t l_kv, const uint8_t *mask, double *O,
                   int64_t *count)
{
    if (B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || h_k > h_q || h_v > h_q || d < 1 || l_kv < 1)
        return -1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (int r = 0; r < B * h_q; ++r) {
        int b = r / h_q, j = r % h_q;
        int g = key_head_of(j, h_q, h_k), v = value_head_of(j, h_q, h_v);
        double *a = (double *)malloc((size_t)l_kv * sizeof *a);
        if (!a) {
            fail |= 1;
            continue;
        }
        sao_scores_row(Q + (int64_t)r * d, K + ((int64_t)b * h_k + g) * l_kv * d, d, l_kv, a);
        count[r] = sao_attend_row(a, mask + (int64_t)r * l_kv,
                                  V + ((int64_t)b * h_v + v) * l_kv * d, d, l_kv,
                                  O + (int64_t)r * d);
        free(a);
    }
    return fail ? -1 : 0;
}

/*
 * Dense GQA decode, eqs. 2-4: every position selected, h_kv heads shared by
 * key and value (query head j reads head floor(j*h_kv/h_q)).
 */
int sao_dense(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int B, int h_q, int h_kv,
              int d, int64_t l_kv, double *O)
{
    if (B < 1 || h_q < 1 || h_kv < 1 || h_kv > h_q || d < 1 || l_kv < 1) return -1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (int r = 0; r < B * h_q; ++r) {
        int b = r / h_q, j = r % h_q, g = key_head_of(j, h_q, h_kv);
        double *a = (double *)malloc((size_t)l_kv * sizeof *a);
        uint8_t *mk = (uint8_t *)malloc((size_t)l_kv);
        if (!a || !mk) {
            free(a);
            free(mk);
            fail |= 1;
            continue;
        }
        const uint16_t *kh = K + ((int64_t)b * h_kv + g) * l_kv * d;
        sao_scores_row(Q + (int64_t)r * d, kh, d, l_kv, a);
        memset(mk, 1, (size_t)l_kv);
        sao_attend_row(a, mk, V + ((int64_t)b * h_kv + g) * l_kv * d, d, l_kv, O + (int64_t)r * d);
        free(a);
        free(mk);
    }
    return fail ? -1 : 0;
}
