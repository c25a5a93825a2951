/*
 * Drives every entry point of the fp64 oracle (oracle/saga_oracle.c) on small
 * seeded inputs and edge cases, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and runs
 * it on the CPU).  Exits non-zero if a call rejects valid arguments or a basic
 * invariant fails; the sanitizers abort on any out-of-bounds access, leak or
 * undefined operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int sao_trajectory(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int T, int B, int h_q,
                   int h_k, int h_v, int d, int64_t l_kv, int64_t N, int R, double *O, double *tau,
                   int64_t *count, uint8_t *mask_out);
int sao_trajectory_growing(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int T, int B,
                           int h_q, int h_k, int h_v, int d, int64_t cap, int64_t l0, int64_t N,
                           int R, double *O, double *tau, int64_t *count, uint8_t *mask_out);
int sao_given_mask(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int B, int h_q,
                   int h_k, int h_v, int d, int64_t l_kv, const uint8_t *mask, double *O,
                   int64_t *count);
int sao_dense(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int B, int h_q, int h_kv,
              int d, int64_t l_kv, double *O);
void sao_scores(const uint16_t *Q, const uint16_t *K, int B, int h_q, int h_k, int d, int64_t l_kv,
                double *A);
double sao_nth_largest(const double *a, int64_t n, int64_t N);
float sao_nth_largest_f32(const float *a, int64_t n, int64_t N);

static uint64_t rng = 88172645463325252ull;
static double uniform(void)
{
    rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
/* a float rounded toward zero to bf16 bits (any bf16 pattern is a valid input) */
static uint16_t bf16(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}
static uint16_t *rand_bf16(size_t n, double scale)
{
    uint16_t *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = bf16((uniform() * 2.0 - 1.0) * scale);
    return p;
}

static int fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
            ++fails;                                                          \
        }                                                                     \
    } while (0)

static void run(int T, int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N, int R)
{
    size_t nq = (size_t)T * B * h_q * d, nk = (size_t)B * h_k * l_kv * d, nv = (size_t)B * h_v * l_kv * d;
    uint16_t *Q = rand_bf16(nq, 3.0), *K = rand_bf16(nk, 1.0), *V = rand_bf16(nv, 1.0);
    size_t rows = (size_t)T * B * h_q;
    double *O = malloc(rows * d * sizeof *O), *tau = malloc(rows * sizeof *tau);
    int64_t *cnt = malloc(rows * sizeof *cnt);
    uint8_t *mask = malloc(rows * (size_t)l_kv);
    CHECK(sao_trajectory(Q, K, V, T, B, h_q, h_k, h_v, d, l_kv, N, R, O, tau, cnt, mask) == 0);
    for (size_t r = 0; r < rows; ++r) {
        int64_t m = 0;
        for (int64_t t = 0; t < l_kv; ++t) m += mask[r * l_kv + t];
        CHECK(m == cnt[r]);
        if ((r / (B * h_q)) % R == 0) CHECK(cnt[r] >= N);
    }
    /* given-mask mode on the first step's selection reproduces it */
    double *O2 = malloc((size_t)B * h_q * d * sizeof *O2);
    int64_t *c2 = malloc((size_t)B * h_q * sizeof *c2);
    CHECK(sao_given_mask(Q, K, V, B, h_q, h_k, h_v, d, l_kv, mask, O2, c2) == 0);
    for (int r = 0; r < B * h_q; ++r) CHECK(c2[r] == cnt[r]);
    /* growing cache: the first l0 + 1 rows, then one more per step */
    if (l_kv >= T && N <= l_kv - T + 1) {
        int64_t l0 = l_kv - T;
        uint8_t *gm = malloc(rows * (size_t)l_kv);
        CHECK(sao_trajectory_growing(Q, K, V, T, B, h_q, h_k, h_v, d, l_kv, l0, N, R, O, tau, cnt,
                                     gm) == 0);
        free(gm);
    }
    if (h_k == h_v) {
        double *O3 = malloc((size_t)B * h_q * d * sizeof *O3);
        CHECK(sao_dense(Q, K, V, B, h_q, h_k, d, l_kv, O3) == 0);
        free(O3);
    }
    double *A = malloc((size_t)B * h_q * l_kv * sizeof *A);
    sao_scores(Q, K, B, h_q, h_k, d, l_kv, A);
    float *Af = malloc((size_t)l_kv * sizeof *Af);
    for (int64_t t = 0; t < l_kv; ++t) Af[t] = (float)A[t];
    CHECK(sao_nth_largest(A, l_kv, N) == sao_nth_largest(A, l_kv, N));
    CHECK(!isnan(sao_nth_largest_f32(Af, l_kv, N)));
    CHECK(isnan(sao_nth_largest(A, l_kv, l_kv + 1)));  /* out-of-range rank is rejected */
    free(Q), free(K), free(V), free(O), free(tau), free(cnt), free(mask), free(O2), free(c2);
    free(A), free(Af);
}

int main(void)
{
    run(5, 2, 6, 4, 5, 16, 301, 37, 3);    /* non-integer head ratios */
    run(3, 1, 8, 2, 2, 32, 64, 64, 1);     /* N = l_kv, h_k = h_v */
    run(4, 1, 4, 1, 2, 8, 50, 1, 2);       /* N = 1 */
    run(2, 3, 4, 4, 4, 8, 1, 1, 1);        /* a single cache position */
    run(6, 1, 12, 1, 4, 64, 500, 40, 4);   /* a group of 12 */
    /* rejected arguments return -1 without touching the outputs */
    CHECK(sao_trajectory(NULL, NULL, NULL, 0, 1, 1, 1, 1, 8, 8, 1, 1, NULL, NULL, NULL, NULL) == -1);
    CHECK(sao_trajectory_growing(NULL, NULL, NULL, 1, 1, 1, 1, 1, 8, 8, 8, 1, 1, NULL, NULL, NULL,
                                 NULL) == -1);
    if (fails) return 1;
    puts("oracle sanitizer run ok");
    return 0;
}
