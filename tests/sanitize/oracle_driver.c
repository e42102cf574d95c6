/* Drives the fp64 oracle (oracle/gdn_oracle.c) through its entry points on small inputs for a
 * build under AddressSanitizer + UndefinedBehaviorSanitizer, or ThreadSanitizer
 * (tests/test_sanitize_cpu.py): both directions, start state or none, l2 norm on and off,
 * eps = 0, one thread and several, T = 0 and 1, row blocks that do not divide d_v, and the
 * gradient.  Checks that every output is finite and that the argument checks refuse bad sizes.
 * Exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_scan(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, const double* q, const double* k,
                    const double* v, const double* a, const double* beta, const double* S0, int reverse, int l2norm,
                    double eps, double scale, double* o, double* S_final, int nthreads, int64_t row_block);
int gdn_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, const double* q, const double* k,
                        const double* v, const double* a, const double* beta, const double* S0, const double* dO,
                        const double* dS_final, int reverse, int l2norm, double eps, double scale, double* dq,
                        double* dk, double* dv, double* da, double* dbeta, double* dS0, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double uniform(void) { /* xorshift64, values in [-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ull << 52) - 1.0;
}
static double* fill(int64_t n, double lo, double hi) {
    double* x = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return x;
}
static int finite_all(const double* x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) if (!isfinite(x[i])) return 0;
    return 1;
}

static int failures = 0;
static void check(int ok, const char* what) {
    if (!ok) { printf("FAIL %s\n", what); ++failures; }
}

static void one(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int reverse, int state, int l2norm,
                double eps, int threads, int64_t row_block) {
    const int64_t nq = B * T * H * Dk, nv = B * T * H * Dv, ng = B * T * H, ns = B * H * Dv * Dk;
    double *q = fill(nq, -1, 1), *k = fill(nq, -1, 1), *v = fill(nv, -1, 1);
    double *a = fill(ng, 0.85, 1.0), *beta = fill(ng, 0.0, 1.0);
    double* S0 = state ? fill(ns, -0.1, 0.1) : NULL;
    if (!l2norm) for (int64_t i = 0; i < nq; ++i) { q[i] /= sqrt((double)Dk); k[i] /= sqrt((double)Dk); }
    double *o = fill(nv, 0, 0), *Sf = fill(ns, 0, 0);
    int rc = gdn_oracle_scan(B, T, H, Dk, Dv, q, k, v, a, beta, S0, reverse, l2norm, eps, 0.7, o, Sf, threads, row_block);
    check(rc == 0, "scan rc");
    check(finite_all(o, nv) && finite_all(Sf, ns), "scan finite");
    double *dO = fill(nv, -1, 1), *dSf = fill(ns, -1, 1);
    double *dq = fill(nq, 0, 0), *dk = fill(nq, 0, 0), *dv = fill(nv, 0, 0), *da = fill(ng, 0, 0),
           *db = fill(ng, 0, 0), *dS0 = fill(ns, 0, 0);
    rc = gdn_oracle_backward(B, T, H, Dk, Dv, q, k, v, a, beta, reverse ? NULL : S0, dO, dSf, reverse, l2norm, eps,
                             0.7, dq, dk, dv, da, db, dS0, threads);
    check(rc == 0, "backward rc");
    check(finite_all(dq, nq) && finite_all(dk, nq) && finite_all(dv, nv) && finite_all(da, ng) &&
          finite_all(db, ng) && finite_all(dS0, ns), "backward finite");
    free(q); free(k); free(v); free(a); free(beta); free(S0); free(o); free(Sf);
    free(dO); free(dSf); free(dq); free(dk); free(dv); free(da); free(db); free(dS0);
}

int main(void) {
    one(2, 37, 3, 16, 32, 0, 1, 1, 1e-6, 1, 16);
    one(2, 37, 3, 16, 32, 1, 0, 1, 1e-6, 4, 16);
    one(1, 64, 2, 32, 32, 0, 1, 0, 0.0, 3, 5);     /* no norm, a row block that does not divide d_v */
    one(1, 50, 2, 48, 16, 0, 1, 1, 0.0, 8, 16);    /* eps = 0, more threads than work items */
    one(1, 1, 1, 16, 16, 1, 0, 1, 1e-6, 2, 16);
    one(1, 0, 2, 16, 16, 0, 1, 1, 1e-6, 2, 16);    /* T = 0: the start state comes back */
    double x = 0.0;
    check(gdn_oracle_scan(1, 4, 1, 0, 16, &x, &x, &x, &x, &x, NULL, 0, 1, 1e-6, 1.0, &x, NULL, 1, 16) == -1,
          "scan refuses d_k = 0");
    check(gdn_oracle_scan(1, 4, 1, 16, 16, NULL, &x, &x, &x, &x, NULL, 0, 1, 1e-6, 1.0, &x, NULL, 1, 16) == -1,
          "scan refuses NULL q");
    check(gdn_oracle_backward(-1, 4, 1, 16, 16, &x, &x, &x, &x, &x, NULL, &x, NULL, 0, 1, 1e-6, 1.0, &x, &x, &x, &x,
                              &x, NULL, 1) == -1, "backward refuses B < 0");
    printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
