/*
 * oracle_sanitize.c -- the fp64 oracle (oracle/kda_oracle.c, linked in) under the C
 * sanitizers: AddressSanitizer + UndefinedBehaviorSanitizer in one build, ThreadSanitizer
 * in another (the oracle splits (sequence, head) pairs over threads).  Built and run by
 * tests/test_sanitizers.py.  Inputs are small and seeded (a 64-bit LCG here, nothing of
 * the method's arithmetic); the program checks return codes and properties any correct
 * run has: the threaded run equals the one-thread run bit for bit, a zero-length sequence
 * passes its state and conv cache through unchanged, invalid arguments are refused.
 * Exit status 0 when every check holds; a sanitizer report aborts with a nonzero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_run(int n_seqs, int n_heads, int dk, int dv, const int64_t *cu,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *log_alpha, const double *beta,
                   const double *wq, const double *wk, const double *wv,
                   const double *cq_in, const double *ck_in, const double *cv_in,
                   const double *rms_w, const double *s_in, double scale,
                   double l2_eps, double rms_eps, int prologue, int epilogue,
                   double *o, double *s_out, double *cq_out, double *ck_out,
                   double *cv_out, int n_threads);
int kda_oracle_lowrank_log_alpha(int64_t T, int H, int d, int r, const double *z, const double *w,
                                 const double *b, const double *a, double *out);
int kda_oracle_softplus_log_alpha(int64_t T, int H, int d, int r, const double *z, const double *w,
                                  const double *b, const double *a, double *out);
int kda_oracle_beta_from_logit(int64_t n, const double *w, double *beta);

static uint64_t lcg = 0x9e3779b97f4a7c15ull;
static double uni(void) { /* [0, 1) */
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}
static double *fill(size_t n, double lo, double hi) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}
static double *zeros(size_t n) { return (double *)calloc(n ? n : 1, sizeof(double)); }

static int failures = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

int main(void) {
    enum { N = 5, H = 2, DK = 8, DV = 8 };
    const int64_t cu[N + 1] = {0, 0, 1, 4, 21, 26};  /* lengths 0, 1, 3, 17, 5 */
    const int64_t T = cu[N];
    const size_t tk = (size_t)T * H * DK, tv = (size_t)T * H * DV, sd = (size_t)N * H * DK * DV;
    const size_t ck = (size_t)N * 3 * H * DK, cvn = (size_t)N * 3 * H * DV;
    double *q = fill(tk, -1, 1), *k = fill(tk, -1, 1), *v = fill(tv, -1, 1), *g = fill(tv, -2, 2);
    double *la = fill(tk, -5, 0), *beta = fill((size_t)T * H, 0, 1);
    double *wq = fill((size_t)H * DK * 4, -0.5, 0.5), *wk = fill((size_t)H * DK * 4, -0.5, 0.5);
    double *wv = fill((size_t)H * DV * 4, -0.5, 0.5), *rw = fill(DV, 0.5, 1.5);
    double *cq = fill(ck, -1, 1), *ckk = fill(ck, -1, 1), *cv = fill(cvn, -1, 1), *s0 = fill(sd, -0.1, 0.1);

    double *o1 = zeros(tv), *s1 = zeros(sd), *cq1 = zeros(ck), *ck1 = zeros(ck), *cv1 = zeros(cvn);
    double *o3 = zeros(tv), *s3 = zeros(sd), *cq3 = zeros(ck), *ck3 = zeros(ck), *cv3 = zeros(cvn);
    CHECK(kda_oracle_run(N, H, DK, DV, cu, q, k, v, g, la, beta, wq, wk, wv, cq, ckk, cv, rw, s0,
                         0.35, 1e-6, 1e-6, 1, 1, o1, s1, cq1, ck1, cv1, 1) == 0);
    CHECK(kda_oracle_run(N, H, DK, DV, cu, q, k, v, g, la, beta, wq, wk, wv, cq, ckk, cv, rw, s0,
                         0.35, 1e-6, 1e-6, 1, 1, o3, s3, cq3, ck3, cv3, 3) == 0);
    CHECK(memcmp(o1, o3, tv * sizeof(double)) == 0);
    CHECK(memcmp(s1, s3, sd * sizeof(double)) == 0);
    CHECK(memcmp(cq1, cq3, ck * sizeof(double)) == 0 && memcmp(cv1, cv3, cvn * sizeof(double)) == 0);
    /* sequence 0 has no tokens: its state and conv cache pass through */
    CHECK(memcmp(s1, s0, (size_t)H * DK * DV * sizeof(double)) == 0);
    for (int j = 0; j < 3; ++j)
        CHECK(memcmp(ck1 + (size_t)j * H * DK, ckk + (size_t)j * H * DK, (size_t)H * DK * sizeof(double)) == 0);

    /* the bare recurrence: no prologue, epilogue, initial state or caches */
    CHECK(kda_oracle_run(N, H, DK, DV, cu, q, k, v, NULL, la, beta, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 0.35, 1e-6, 1e-6, 0, 0, o1, s1, NULL, NULL, NULL, 4) == 0);
    CHECK(kda_oracle_run(0, H, DK, DV, cu, q, k, v, NULL, la, beta, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 0.35, 1e-6, 1e-6, 0, 0, o1, NULL, NULL, NULL, NULL, 2) == 0);
    /* refusals */
    const int64_t bad_cu[3] = {0, 5, 3};
    CHECK(kda_oracle_run(2, H, DK, DV, bad_cu, q, k, v, NULL, la, beta, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 0.35, 1e-6, 1e-6, 0, 0, o1, NULL, NULL, NULL, NULL, 1) != 0);
    CHECK(kda_oracle_run(N, H, DK, DV, cu, q, k, v, NULL, la, beta, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 0.35, 1e-6, 1e-6, 1, 0, o1, NULL, NULL, NULL, NULL, 1) != 0);
    CHECK(kda_oracle_run(N, H, DK, DV, cu, q, k, v, NULL, la, beta, wq, wk, wv, NULL, NULL, NULL,
                         NULL, NULL, 0.35, 1e-6, 1e-6, 1, 1, o1, NULL, NULL, NULL, NULL, 1) != 0);

    /* the gate pre-activations */
    enum { R = 4 };
    double *z = fill((size_t)T * R, -1, 1), *w = fill((size_t)H * DK * R, -1, 1);
    double *bias = fill((size_t)H * DK, -1, 1), *a = fill(H, -1, 1), *out = zeros(tk);
    CHECK(kda_oracle_lowrank_log_alpha(T, H, DK, R, z, w, bias, a, out) == 0);
    for (size_t i = 0; i < tk; ++i) CHECK(out[i] < 0.0 && out[i] > -5.0);
    CHECK(kda_oracle_softplus_log_alpha(T, H, DK, R, z, w, bias, a, out) == 0);
    for (size_t i = 0; i < tk; ++i) CHECK(out[i] < 0.0);
    CHECK(kda_oracle_lowrank_log_alpha(T, H, DK, 0, z, w, bias, a, out) != 0);
    const double logits[4] = {-800.0, -1.0, 0.0, 800.0};
    double bl[4];
    CHECK(kda_oracle_beta_from_logit(4, logits, bl) == 0);
    CHECK(bl[0] == 0.0 && bl[2] == 0.5 && bl[3] == 1.0 && bl[1] > 0.26 && bl[1] < 0.27);
    CHECK(kda_oracle_beta_from_logit(0, NULL, NULL) == 0);
    CHECK(kda_oracle_beta_from_logit(-1, logits, bl) != 0);

    double *bufs[] = {q, k, v, g, la, beta, wq, wk, wv, rw, cq, ckk, cv, s0, o1, s1, cq1, ck1, cv1,
                      o3, s3, cq3, ck3, cv3, z, w, bias, a, out};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) free(bufs[i]);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
