/* Drives every entry point of the fp64 oracle (oracle/race_oracle.c) on small
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * the sanitizers catch out-of-bounds or use-after-free accesses and undefined
 * arithmetic; the checks below catch wrong sizes passed between the steps.
 * Shapes span one and several of the oracle's row blocks (2048 rows), P = 1
 * to 4, causal and not, soft and hard, a zero row and un-normalised rows.
 * Exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int race_oracle_threads(int n);
int race_oracle_hash(const double *x, int64_t n, int d, const double *W, int L, int P, double tau,
                     int hard, double *phi, double *z);
int race_oracle_forward(const double *q, const double *k, const double *v, const double *W, int L,
                        int P, double tau, int causal, int hard, int64_t BH, int64_t N, int d,
                        double *o, double *den);
int race_oracle_forward_backward_w(const double *q, const double *k, const double *v,
                                   const double *g, const double *W, int L, int P, double tau,
                                   int causal, int64_t BH, int64_t N, int d, double *o, double *den,
                                   double *dq, double *dk, double *dv, double *dW);
int race_oracle_stream_forward(const double *q, const double *k, const double *v, const double *W,
                               int L, int P, double tau, int64_t n, int d, double *M, double *o,
                               double *den);
int race_oracle_stream_backward(const double *q, const double *k, const double *v, const double *g,
                                const double *o, const double *den, const double *W, int L, int P,
                                double tau, int64_t n, int d, double *S, double *G, double *dq,
                                double *dk, double *dv);
int race_oracle_block_sums(const double *x, const double *y, int ycols, int64_t n, int d,
                           const double *W, int L, int P, double tau, double *M);

static int failures = 0;
#define CHECK(c, ...)                                             \
    do {                                                          \
        if (!(c)) {                                               \
            ++failures;                                           \
            fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                         \
            fputc('\n', stderr);                                  \
        }                                                         \
    } while (0)

/* 64-bit LCG (Knuth's MMIX constants) and a Box-Muller normal draw */
static uint64_t rng = 88172645463325252ull;
static double unif(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return ((rng >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static double normal(void) { return sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()); }

static double *alloc(size_t n)
{
    double *p = malloc(sizeof(double) * (n ? n : 1));
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static double *randn(size_t n, double scale)
{
    double *p = alloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = scale * normal();
    return p;
}
static int finite_all(const double *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}
static double max_rel(const double *a, const double *b, size_t n)
{
    double num = 0, den = 0;
    for (size_t i = 0; i < n; ++i) {
        num = fmax(num, fabs(a[i] - b[i]));
        den = fmax(den, fabs(b[i]));
    }
    return den > 0 ? num / den : num;
}

static void run_case(int BH, int N, int d, int L, int P, double tau, int causal)
{
    const int R = 1 << P, F = L * R, d1 = d + 1;
    const size_t nx = (size_t)BH * N * d, nr = (size_t)BH * N;
    double *W = randn((size_t)L * P * d, 1.0);
    double *q = randn(nx, 1.0), *k = randn(nx, 3.0), *v = randn(nx, 1.0), *g = randn(nx, 1.0);
    memset(q, 0, sizeof(double) * d);            /* a zero query row */
    double *o = alloc(nx), *den = alloc(nr), *dq = alloc(nx), *dk = alloc(nx), *dv = alloc(nx);
    double *dW = alloc((size_t)L * P * d);

    /* soft and hard assignments: each table's weights sum to 1 */
    for (int hard = 0; hard < 2; ++hard) {
        double *phi = alloc((size_t)N * F), *z = alloc((size_t)N * L * P);
        CHECK(race_oracle_hash(k, N, d, W, L, P, tau, hard, phi, z) == 0, "hash");
        for (int i = 0; i < N; ++i)
            for (int l = 0; l < L; ++l) {
                double s = 0;
                for (int r = 0; r < R; ++r) s += phi[(size_t)i * F + l * R + r];
                CHECK(fabs(s - 1.0) < 1e-12, "phi sum %g (hard %d)", s, hard);
            }
        CHECK(finite_all(z, (size_t)N * L * P), "z finite");
        free(phi);
        free(z);
    }

    /* forward, soft and hard; constant values come back unchanged (soft) */
    CHECK(race_oracle_forward(q, k, v, W, L, P, tau, causal, 1, BH, N, d, o, den) == 0, "hard fwd");
    CHECK(finite_all(o, nx) && finite_all(den, nr), "hard fwd finite");
    double *vc = alloc(nx);
    for (size_t i = 0; i < nx; ++i) vc[i] = 0.25 * (double)(i % d) - 1.0;
    CHECK(race_oracle_forward(q, k, vc, W, L, P, tau, causal, 0, BH, N, d, o, den) == 0, "fwd");
    CHECK(max_rel(o, vc, nx) < 1e-12, "constant values: %g", max_rel(o, vc, nx));
    free(vc);

    /* forward + backward with dW */
    CHECK(race_oracle_forward_backward_w(q, k, v, g, W, L, P, tau, causal, BH, N, d, o, den, dq, dk,
                                         dv, dW) == 0, "fwd+bwd");
    CHECK(finite_all(dq, nx) && finite_all(dk, nx) && finite_all(dv, nx) &&
              finite_all(dW, (size_t)L * P * d), "gradients finite");

    /* head 0 streamed in two blocks equals the one-shot causal result */
    if (causal && N >= 2) {
        const int n0 = N / 2 + 1, n1 = N - n0;
        double *M = alloc((size_t)d1 * F), *so = alloc((size_t)N * d), *sd = alloc(N);
        memset(M, 0, sizeof(double) * d1 * F);
        CHECK(race_oracle_stream_forward(q, k, v, W, L, P, tau, n0, d, M, so, sd) == 0, "sf0");
        double *S1 = alloc((size_t)d1 * F);
        memcpy(S1, M, sizeof(double) * d1 * F);
        if (n1 > 0)
            CHECK(race_oracle_stream_forward(q + (size_t)n0 * d, k + (size_t)n0 * d,
                                             v + (size_t)n0 * d, W, L, P, tau, n1, d, M,
                                             so + (size_t)n0 * d, sd + n0) == 0, "sf1");
        CHECK(max_rel(so, o, (size_t)N * d) < 1e-12 && max_rel(sd, den, N) < 1e-12,
              "stream forward %g", max_rel(so, o, (size_t)N * d));
        /* backward: the later block first, then the earlier one */
        double *G = alloc((size_t)d1 * F), *S = alloc((size_t)d1 * F);
        double *sq = alloc((size_t)N * d), *sk = alloc((size_t)N * d), *sv = alloc((size_t)N * d);
        memset(G, 0, sizeof(double) * d1 * F);
        if (n1 > 0) {
            memcpy(S, S1, sizeof(double) * d1 * F);
            const size_t off = (size_t)n0 * d;
            CHECK(race_oracle_stream_backward(q + off, k + off, v + off, g + off, so + off, sd + n0,
                                              W, L, P, tau, n1, d, S, G, sq + off, sk + off,
                                              sv + off) == 0, "sb1");
        }
        memset(S, 0, sizeof(double) * d1 * F);
        CHECK(race_oracle_stream_backward(q, k, v, g, so, sd, W, L, P, tau, n0, d, S, G, sq, sk,
                                          sv) == 0, "sb0");
        CHECK(max_rel(sq, dq, (size_t)N * d) < 1e-10 && max_rel(sk, dk, (size_t)N * d) < 1e-10 &&
                  max_rel(sv, dv, (size_t)N * d) < 1e-10,
              "stream backward %g %g %g", max_rel(sq, dq, (size_t)N * d),
              max_rel(sk, dk, (size_t)N * d), max_rel(sv, dv, (size_t)N * d));
        /* the key sums of all of head 0 equal its bucket sums */
        double *y = alloc((size_t)N * d1), *Mb = alloc((size_t)d1 * F);
        for (int i = 0; i < N; ++i) {
            memcpy(y + (size_t)i * d1, v + (size_t)i * d, sizeof(double) * d);
            y[(size_t)i * d1 + d] = 1.0;
        }
        memset(Mb, 0, sizeof(double) * d1 * F);
        CHECK(race_oracle_block_sums(k, y, d1, N, d, W, L, P, tau, Mb) == 0, "block sums");
        CHECK(max_rel(Mb, M, (size_t)d1 * F) < 1e-12, "block sums %g", max_rel(Mb, M, (size_t)d1 * F));
        free(M); free(so); free(sd); free(S1); free(G); free(S); free(sq); free(sk); free(sv);
        free(y); free(Mb);
    }
    free(W); free(q); free(k); free(v); free(g); free(o); free(den); free(dq); free(dk); free(dv);
    free(dW);
}

int main(void)
{
    race_oracle_threads(2);
    run_case(1, 1, 8, 1, 1, 1.0, 1);
    run_case(2, 37, 8, 3, 2, 0.5, 1);
    run_case(2, 37, 8, 3, 3, 1.0, 0);
    run_case(1, 2100, 8, 2, 4, 1.0, 1);
    run_case(1, 300, 16, 5, 4, 0.25, 0);
    /* invalid arguments are refused before any access */
    double x = 0;
    CHECK(race_oracle_forward(&x, &x, &x, &x, 1, 0, 1.0, 1, 0, 1, 1, 1, &x, &x) == 1, "P = 0");
    CHECK(race_oracle_forward(&x, &x, &x, &x, 1, 1, -1.0, 1, 0, 1, 1, 1, &x, &x) == 1, "tau < 0");
    CHECK(race_oracle_forward(&x, &x, &x, &x, 1, 1, NAN, 1, 0, 1, 1, 1, &x, &x) == 1, "tau NaN");
    CHECK(race_oracle_forward(&x, &x, &x, &x, 0, 1, 1.0, 1, 0, 1, 1, 1, &x, &x) == 1, "L = 0");
    CHECK(race_oracle_stream_forward(&x, &x, &x, &x, 1, 1, 1.0, 1, 1, NULL, &x, &x) == 1, "no M");
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
