/* Host-only driver for the oracle under AddressSanitizer and UBSan: every
 * oracle entry point on small inputs with ties, signed zeros, phases,
 * temperatures 1, 1/2 and 0, empty and one-element sides, rows and columns
 * subsets.  Besides running clean under the sanitizers it checks that the
 * sweeps agree with the dense definition, so a read of a wrong element shows
 * up even where it stays inside an allocation.  Exit status 0 = all good.
 * Built and run by tests/test_oracle_sanitize.py; not part of the library. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int lo_argsort(const float* a, int64_t n, uint32_t* perm);
int lo_apply_dense(const float* out_anchor, const float* out_phase, int64_t n_out, const float* in_anchor,
                   const float* in_phase, int64_t n_in, const float* x, int64_t batch, const int64_t* rows,
                   int64_t n_rows, double t, double* y);
int lo_dense_matrix(const float* out_anchor, const float* out_phase, int64_t n_out, const float* in_anchor,
                    const float* in_phase, int64_t n_in, double t, double* K);
int lo_apply_sym_sweep(const float* a, const float* po, const float* pi, int64_t n, const float* x,
                       int64_t batch, double t, double* y);
int lo_apply_general_sweep(const float* out_anchor, const float* out_phase, int64_t n_out,
                           const float* in_anchor, const float* in_phase, int64_t n_in, const float* x,
                           int64_t batch, double t, double* y);
int lo_grad_dense(const float* a, const float* phi, int64_t n, const float* b, const float* psi, int64_t k,
                  double t, const float* u, const float* w, int64_t batch, const int64_t* rows, int64_t n_rows,
                  const int64_t* cols, int64_t n_cols, double* da, double* db, double* dphi, double* dpsi);
int lo_gram_direct(const float* a, const float* phi, int64_t n, const float* b, const float* psi, int64_t k,
                   const float* D, const int64_t* rows, int64_t n_rows, const int64_t* cols, int64_t n_cols,
                   double t, double* M);

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) /* xorshift64, uniform in [0, 1) */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static int failures = 0;
static void expect(int cond, const char* what, int64_t n, int64_t k, double t)
{
    if (!cond) {
        fprintf(stderr, "FAIL %s (n=%lld k=%lld t=%g)\n", what, (long long)n, (long long)k, t);
        ++failures;
    }
}

static double rel_err(const double* y, const double* ref, int64_t m)
{
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < m; ++i) {
        num += (y[i] - ref[i]) * (y[i] - ref[i]);
        den += ref[i] * ref[i];
    }
    return den > 0.0 ? sqrt(num / den) : sqrt(num);
}

/* anchors with ties and a -0.0 / +0.0 pair; exactly `n` entries (malloc'ed
 * to size so the sanitizer sees any read past the end) */
static float* anchors(int64_t n, double scale)
{
    float* a = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) a[i] = (float)((urand() - 0.5) * scale);
    for (int64_t i = 0; i + 3 < n; i += 4) a[i + 3] = a[i];
    if (n >= 2) {
        a[0] = -0.0f;
        a[n - 1] = 0.0f;
    }
    return a;
}

static float* values(int64_t n)
{
    float* v = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) v[i] = (float)(2.0 * urand() - 1.0);
    return v;
}

static double* dalloc(int64_t n) { return (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)); }

static void run_case(int64_t n, int64_t k, int phased, double t)
{
    const int64_t B = 2;
    float* a = anchors(n, 6.0);
    float* b = anchors(k, 6.0);
    float* phi = phased ? values(n) : NULL;
    float* psi = phased ? values(k) : NULL;
    float* psi_n = phased ? values(n) : NULL;
    float* x = values(B * k);
    float* xs = values(B * n);
    float* D = values(k);
    uint32_t* perm = (uint32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint32_t));

    expect(lo_argsort(a, n, perm) == 0, "argsort", n, k, t);
    for (int64_t r = 1; r < n; ++r) expect(a[perm[r - 1]] <= a[perm[r]], "argsort order", n, k, t);

    /* general: sweep vs dense, both directions */
    double* y = dalloc(B * n);
    double* yd = dalloc(B * n);
    expect(lo_apply_general_sweep(a, phi, n, b, psi, k, x, B, t, y) == 0, "general sweep", n, k, t);
    expect(lo_apply_dense(a, phi, n, b, psi, k, x, B, NULL, 0, t, yd) == 0, "dense", n, k, t);
    expect(rel_err(y, yd, B * n) < 1e-12, "general sweep = dense", n, k, t);
    float* w = values(B * n);
    double* z = dalloc(B * k);
    double* zd = dalloc(B * k);
    expect(lo_apply_general_sweep(b, psi, k, a, phi, n, w, B, t, z) == 0, "general sweep T", n, k, t);
    expect(lo_apply_dense(b, psi, k, a, phi, n, w, B, NULL, 0, t, zd) == 0, "dense T", n, k, t);
    expect(rel_err(z, zd, B * k) < 1e-12, "general sweep T = dense", n, k, t);

    /* symmetric */
    double* ys = dalloc(B * n);
    double* ysd = dalloc(B * n);
    expect(lo_apply_sym_sweep(a, phi, psi_n, n, xs, B, t, ys) == 0, "sym sweep", n, k, t);
    expect(lo_apply_dense(a, phi, n, a, psi_n, n, xs, B, NULL, 0, t, ysd) == 0, "sym dense", n, k, t);
    expect(rel_err(ys, ysd, B * n) < 1e-12, "sym sweep = dense", n, k, t);

    /* dense matrix, sampled rows */
    double* K = dalloc(n * k);
    expect(lo_dense_matrix(a, phi, n, b, psi, k, t, K) == 0, "dense matrix", n, k, t);
    int64_t rows[3] = {0, n > 1 ? n - 1 : 0, n / 2};
    const int64_t nr = n > 0 ? 3 : 0;
    double* yr = dalloc(B * nr);
    expect(lo_apply_dense(a, phi, n, b, psi, k, x, B, rows, nr, t, yr) == 0, "dense rows", n, k, t);
    for (int64_t v = 0; v < B; ++v)
        for (int64_t r = 0; r < nr; ++r) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j) acc += K[rows[r] * k + j] * x[v * k + j];
            expect(fabs(acc - yr[v * nr + r]) <= 1e-12 * (1.0 + fabs(acc)), "matrix row = dense row", n, k, t);
        }

    /* Gram, all entries and a subset */
    double* M = dalloc(n * n);
    expect(lo_gram_direct(a, phi, n, b, psi, k, D, NULL, 0, NULL, 0, t, M) == 0, "gram", n, k, t);
    int64_t cols[2] = {0, n > 2 ? 2 : 0};
    const int64_t nc = n > 0 ? 2 : 0;
    double* Ms = dalloc(nr * nc);
    expect(lo_gram_direct(a, phi, n, b, psi, k, D, rows, nr, cols, nc, t, Ms) == 0, "gram subset", n, k, t);
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t c = 0; c < nc; ++c)
            expect(fabs(Ms[r * nc + c] - M[rows[r] * n + cols[c]]) <= 1e-12 * (1.0 + fabs(M[rows[r] * n + cols[c]])),
                   "gram subset = gram", n, k, t);

    /* gradients */
    double* da = dalloc(n);
    double* db = dalloc(k);
    double* dphi = dalloc(n);
    double* dpsi = dalloc(k);
    expect(lo_grad_dense(a, phi, n, b, psi, k, t, w, x, B, NULL, 0, NULL, 0, da, db, phased ? dphi : NULL,
                         phased ? dpsi : NULL) == 0,
           "grad", n, k, t);
    for (int64_t i = 0; i < n; ++i) expect(isfinite(da[i]), "grad finite", n, k, t);

    free(a); free(b); free(phi); free(psi); free(psi_n); free(x); free(xs); free(D); free(perm);
    free(y); free(yd); free(w); free(z); free(zd); free(ys); free(ysd); free(K); free(yr);
    free(M); free(Ms); free(da); free(db); free(dphi); free(dpsi);
}

int main(void)
{
    const int64_t sizes[][2] = {{1, 1}, {2, 3}, {3, 2}, {17, 40}, {64, 5}, {300, 257}};
    const double temps[] = {1.0, 0.5, 0.0};
    for (size_t s = 0; s < sizeof(sizes) / sizeof(sizes[0]); ++s)
        for (int ph = 0; ph < 2; ++ph)
            for (size_t q = 0; q < 3; ++q) run_case(sizes[s][0], sizes[s][1], ph, temps[q]);
    /* argument checks: bad sizes and non-finite anchors are refused, not read past */
    float bad[3] = {0.0f, NAN, 1.0f};
    uint32_t p[3];
    expect(lo_argsort(bad, 3, p) != 0, "argsort refuses NaN", 3, 0, 1.0);
    expect(lo_argsort(bad, -1, p) != 0, "argsort refuses n < 0", -1, 0, 1.0);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}
