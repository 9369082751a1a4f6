/* Host driver that runs every export of oracle/kda_oracle.c on small seeded
 * inputs, for builds with AddressSanitizer and UndefinedBehaviorSanitizer:
 * odd sizes, T = 0 and T below one chunk, column subsets, several thread
 * counts.  It checks only that outputs are finite; the values themselves are
 * pinned by the Python tests.  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void kda_oracle_gate(long n, const double* theta, double* g);
void kda_oracle_gate_softplus(long n, const double* theta, double* g);
void kda_oracle_output_gate(long n, const double* o, const double* z, double* out);
void kda_oracle_gate_cumsum(int B, int T, int H, int dk, const double* g, double* gcum);
int kda_oracle_recurrence(int B, int T, int H, int dk, int dv, const double* q, const double* k,
                          const double* v, const double* g, const double* beta, const double* S0,
                          const int* cols, int ncols, double* o, double* S_T, int nthreads);
int kda_oracle_chunk_fwd(int B, int T, int H, int dk, int dv, const double* q, const double* k,
                         const double* v, const double* theta, const double* beta, const double* S0,
                         const int* cols, int ncols, double* o, double* S_T, int nthreads);
int kda_oracle_decode_step(int B, int H, int dk, int dv, const double* q, const double* k,
                           const double* v, const double* theta, const double* beta, double* S,
                           double* o, int nthreads);
int kda_oracle_backward(int B, int T, int H, int dk, int dv, const double* q, const double* k,
                        const double* v, const double* g, const double* beta, const double* S0,
                        const double* dout, const double* dS_T, double* dq, double* dkk, double* dvv,
                        double* dg, double* dbeta, double* dS0);
void kda_oracle_gate_backward(long n, const double* theta, const double* dg, double* dtheta);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* xorshift64*, uniform in [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n, double scale) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = scale * urand();
    return p;
}
static int finite_all(const double* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}
#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                               \
        }                                                           \
    } while (0)

static int run_case(int B, int T, int H, int dk, int dv, int nthreads, int ncols) {
    const size_t nq = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv, nb = (size_t)B * T * H;
    const size_t ns = (size_t)B * H * dk * dv;
    double *q = fill(nq, 1.0), *k = fill(nq, 0.3), *v = fill(nv, 1.0), *th = fill(nq, 4.0);
    double *beta = fill(nb, 0.5), *S0 = fill(ns, 0.1), *g = fill(nq, 0.0), *gc = fill(nq, 0.0);
    for (size_t i = 0; i < nb; ++i) beta[i] = 0.5 + beta[i];   /* in [0, 1) */
    kda_oracle_gate((long)nq, th, g);
    CHECK(finite_all(g, nq));
    kda_oracle_gate_cumsum(B, T, H, dk, g, gc);
    CHECK(finite_all(gc, nq));
    int* cols = (int*)malloc(sizeof(int) * (size_t)(ncols > 0 ? ncols : 1));
    for (int j = 0; j < ncols; ++j) cols[j] = (j * 7 + 3) % dv;
    const int nc = ncols > 0 ? ncols : dv;
    double *o = fill((size_t)B * T * H * nc, 0.0), *ST = fill((size_t)B * H * dk * nc, 0.0);
    CHECK(kda_oracle_chunk_fwd(B, T, H, dk, dv, q, k, v, th, beta, S0, ncols > 0 ? cols : NULL, ncols, o,
                               ST, nthreads) == 0);
    CHECK(finite_all(o, (size_t)B * T * H * nc) && finite_all(ST, (size_t)B * H * dk * nc));
    CHECK(kda_oracle_recurrence(B, T, H, dk, dv, q, k, v, g, beta, NULL, ncols > 0 ? cols : NULL, ncols, o,
                                ST, nthreads) == 0);
    CHECK(finite_all(o, (size_t)B * T * H * nc));
    double *dout = fill(nv, 1.0), *dST = fill(ns, 1.0);
    double *dq = fill(nq, 0.0), *dk_ = fill(nq, 0.0), *dv_ = fill(nv, 0.0), *dg = fill(nq, 0.0);
    double *db = fill(nb, 0.0), *dS0 = fill(ns, 0.0), *dth = fill(nq, 0.0);
    CHECK(kda_oracle_backward(B, T, H, dk, dv, q, k, v, g, beta, S0, dout, dST, dq, dk_, dv_, dg, db, dS0) == 0);
    CHECK(finite_all(dq, nq) && finite_all(dk_, nq) && finite_all(dv_, nv) && finite_all(dg, nq));
    CHECK(finite_all(db, nb) && finite_all(dS0, ns));
    CHECK(kda_oracle_backward(B, T, H, dk, dv, q, k, v, g, beta, NULL, dout, NULL, dq, dk_, dv_, dg, db, NULL) == 0);
    kda_oracle_gate_backward((long)nq, th, dg, dth);
    CHECK(finite_all(dth, nq));
    kda_oracle_gate_softplus((long)nq, th, g);
    CHECK(finite_all(g, nq));
    kda_oracle_output_gate((long)nv, v, dout, dv_);
    CHECK(finite_all(dv_, nv));
    if (T > 0) {   /* one decode step on the first token of every sequence */
        double* S = fill(ns, 0.1);
        double* od = fill((size_t)B * H * dv, 0.0);
        CHECK(kda_oracle_decode_step(B, H, dk, dv, q, k, v, th, beta, S, od, nthreads) == 0);
        CHECK(finite_all(S, ns) && finite_all(od, (size_t)B * H * dv));
        free(S);
        free(od);
    }
    free(q); free(k); free(v); free(th); free(beta); free(S0); free(g); free(gc); free(cols);
    free(o); free(ST); free(dout); free(dST); free(dq); free(dk_); free(dv_); free(dg); free(db);
    free(dS0); free(dth);
    return 0;
}

int main(void) {
    static const int cases[][7] = {
        /* B, T, H, dk, dv, threads, ncols */
        {1, 0, 1, 16, 16, 1, 0},  {1, 5, 1, 16, 16, 1, 0},   {2, 17, 3, 16, 16, 4, 0},
        {1, 33, 2, 32, 32, 3, 5}, {2, 48, 1, 16, 16, 16, 0}, {1, 21, 2, 8, 12, 2, 0},
    };
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
        const int* c = cases[i];
        if (run_case(c[0], c[1], c[2], c[3], c[4], c[5], c[6])) {
            fprintf(stderr, "case %zu failed\n", i);
            return 1;
        }
    }
    puts("oracle driver: ok");
    return 0;
}
