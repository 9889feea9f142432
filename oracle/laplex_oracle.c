/*
 * LAPLEX fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check of the package entry module and the
 * CPU-baseline leg of the benchmark may load or call this library.  The GPU
 * library never links, includes or calls it, and shares no code with it:
 * everything here is written from the mathematics of the operator, in plain
 * serial C with double precision (OpenMP is used only to spread independent
 * output entries of the dense definition over host cores).
 *
 * Source: the gist.science technical summaries of "LAPLEX: The FFT of
 * Learnable Laplace Kernels" (Struski, Blazhko, Kubaty, Tabor; Hindi,
 * Spanish and Portuguese pages, identical section numbering).  Sections are
 * cited as "summary §2.1" etc.
 *
 *   summary §2.1  operator K(a,b)_ij = exp(-|a_i - b_j|), and the phased
 *                 operator exp(-|a_j - b_k|) * cos(phi_j - psi_k).
 *   summary §2.2  symmetric case: sort the anchors; the lower-triangular
 *                 part obeys y_{i+1} = x_{i+1} + exp(a_i - a_{i+1}) y_i, the
 *                 upper part the mirrored suffix recurrence.
 *                 general case: contributions of b are collected into the
 *                 intervals of the sorted a (vectors u and v) and then
 *                 propagated by the same two recurrences.
 *                 Gram: M = A diag(D) A^T.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - temperature: the formula of §2.1 carries no t; every function takes
 *     t and evaluates exp(-|a - b| / t), with t = 1 the printed operator and
 *     t = 0 the zero-temperature limit of §2.1/§2.3 taken literally: the
 *     equality-routing matrix [a_i == b_j] (times the phase factor);
 *   - derivatives of |a - b| at a == b use the symmetric subgradient 0 (the
 *     mean of the two one-sided derivatives);
 *   - sort order: ascending IEEE order of the float bit patterns with -0.0
 *     before +0.0, ties broken by ascending original index;
 *   - NaN or infinite anchors are rejected (return code 1);
 *   - both triangular parts include the diagonal, so the symmetric result is
 *     L + U - x;
 *   - an input anchor equal to an output anchor, or outside the output range,
 *     is bucketed into the interval (s_{t-1}, s_t] with t = #{s < b}.
 *
 * Parity status per function (what pins it independently of itself is in
 * the CPU test suite):
 *   lo_argsort             pinned (numpy stable argsort of the ordered keys)
 *   lo_apply_dense         pinned (Kac-Murdock-Szego closed form and inverse,
 *                          Toeplitz FFT, zero-temperature permutations and
 *                          CountSketch sums, adjoint identity)
 *   lo_apply_sym_sweep     pinned (dense definition, KMS, Toeplitz FFT)
 *   lo_apply_general_sweep pinned (dense definition, zero temperature)
 *   lo_grad_dense          pinned (central finite differences of the dense
 *                          definition, including ties; adjoint identity)
 *   lo_gram_direct         pinned (KMS inverse on both sides, zero-temperature
 *                          diagonal, Gram-apply consistency; phased: reduces
 *                          to the unphased Gram at zero phases, zero-temperature
 *                          signed diagonal, Gram-apply consistency)
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define LO_OK 0
#define LO_NONFINITE 1
#define LO_BADARG 2
#define LO_NOMEM 3

/* ---------------------------------------------------------------- sorting */

/* Order-preserving map of a float's bits to an unsigned key: negative floats
 * have all bits inverted, non-negative floats get the sign bit set.  Unsigned
 * comparison of keys is then the IEEE order, with -0.0 just below +0.0. */
static uint32_t order_key(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static int cmp_u64(const void* p, const void* q)
{
    uint64_t x = *(const uint64_t*)p, y = *(const uint64_t*)q;
    return (x > y) - (x < y);
}

/* perm[r] = original index of the element of rank r (summary §2.2, "after
 * sorting the anchors").  Sorting the pairs (key, index) as one 64-bit
 * number makes the order total, so ties keep ascending index order. */
int lo_argsort(const float* a, int64_t n, uint32_t* perm)
{
    if (n < 0 || (n > 0 && (!a || !perm)) || n > 0xFFFFFFFFll) return LO_BADARG;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return LO_NONFINITE;
    uint64_t* pairs = (uint64_t*)malloc((size_t)(n ? n : 1) * sizeof(uint64_t));
    if (!pairs) return LO_NOMEM;
    for (int64_t i = 0; i < n; ++i)
        pairs[i] = ((uint64_t)order_key(a[i]) << 32) | (uint64_t)i;
    qsort(pairs, (size_t)n, sizeof(uint64_t), cmp_u64);
    for (int64_t r = 0; r < n; ++r)
        perm[r] = (uint32_t)(pairs[r] & 0xFFFFFFFFu);
    free(pairs);
    return LO_OK;
}

/* ------------------------------------------------------------ definition */

/* Decay over a distance d >= 0 at temperature t: exp(-d / t); at t = 0 the
 * limit, 1 for d == 0 and 0 otherwise. */
static double decay_t(double d, double t)
{
    if (t == 0.0) return d == 0.0 ? 1.0 : 0.0;
    return exp(-d / t);
}

/* One entry of the (phased) operator, summary §2.1:
 *   K_ij = exp(-|o_i - q_j| / t) * cos(po_i - pq_j); phases absent -> factor 1. */
static double entry(double o, double po, double q, double pq, int phased, double t)
{
    double k = decay_t(fabs(o - q), t);
    if (phased) k *= cos(po - pq);
    return k;
}

static int bad_temperature(double t) { return !(t >= 0.0) || isinf(t); }

/* Dense definition: y[v][r] = sum_j K(out[rows[r]], in[j]) * x[v][j].
 * rows == NULL means every output.  phases: both NULL or both given. */
int lo_apply_dense(const float* out_anchor, const float* out_phase, int64_t n_out,
                   const float* in_anchor, const float* in_phase, int64_t n_in,
                   const float* x, int64_t batch,
                   const int64_t* rows, int64_t n_rows, double t, double* y)
{
    if (n_out < 0 || n_in < 0 || batch < 0 || !out_anchor || !in_anchor || !x || !y)
        return LO_BADARG;
    if (bad_temperature(t)) return LO_BADARG;
    if ((out_phase == NULL) != (in_phase == NULL)) return LO_BADARG;
    const int phased = out_phase != NULL;
    const int64_t m = rows ? n_rows : n_out;
    for (int64_t r = 0; r < m; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n_out)) return LO_BADARG;

    const int many_rows = m * batch >= 64;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) if (many_rows)
    for (int64_t v = 0; v < batch; ++v) {
        for (int64_t r = 0; r < m; ++r) {
            const int64_t i = rows ? rows[r] : r;
            const double o = out_anchor[i];
            const double po = phased ? out_phase[i] : 0.0;
            const float* xv = x + v * n_in;
            double acc = 0.0;
            if (many_rows) {
                for (int64_t j = 0; j < n_in; ++j)
                    acc += entry(o, po, in_anchor[j], phased ? in_phase[j] : 0.0, phased, t) * xv[j];
            } else {
                /* few outputs over a long input: split the sum over threads */
#pragma omp parallel for schedule(static) reduction(+ : acc)
                for (int64_t j = 0; j < n_in; ++j)
                    acc += entry(o, po, in_anchor[j], phased ? in_phase[j] : 0.0, phased, t) * xv[j];
            }
            y[v * m + r] = acc;
        }
    }
    return LO_OK;
}

/* Dense matrix K[i][j] (row-major n_out x n_in), for small tests only. */
int lo_dense_matrix(const float* out_anchor, const float* out_phase, int64_t n_out,
                    const float* in_anchor, const float* in_phase, int64_t n_in, double t, double* K)
{
    if (n_out < 0 || n_in < 0 || !out_anchor || !in_anchor || !K) return LO_BADARG;
    if (bad_temperature(t)) return LO_BADARG;
    if ((out_phase == NULL) != (in_phase == NULL)) return LO_BADARG;
    const int phased = out_phase != NULL;
    for (int64_t i = 0; i < n_out; ++i)
        for (int64_t j = 0; j < n_in; ++j)
            K[i * n_in + j] = entry(out_anchor[i], phased ? out_phase[i] : 0.0, in_anchor[j],
                                    phased ? in_phase[j] : 0.0, phased, t);
    return LO_OK;
}

/* ------------------------------------------------------- symmetric sweep */

/* Summary §2.2, symmetric case, for K(a,a) with output phases po and input
 * phases pi (both NULL: unphased).  Steps in the pages' order:
 *   1. sort the anchors: s_r = a[p_r];
 *   2. lower part  L_r = xs_r + exp(s_{r-1} - s_r) L_{r-1}  (prefix);
 *   3. upper part  U_r = xs_r + exp(s_r - s_{r+1}) U_{r+1}  (suffix, mirror);
 *   4. y at rank r is L_r + U_r - xs_r (the diagonal is in both parts).
 * A phase factor cos(po_i - pi_j) = cos po_i cos pi_j + sin po_i sin pi_j
 * turns one phased product into two unphased ones with inputs scaled by
 * cos pi_j and sin pi_j and outputs by cos po_i and sin po_i. */
int lo_apply_sym_sweep(const float* a, const float* po, const float* pi, int64_t n,
                       const float* x, int64_t batch, double t, double* y)
{
    if (n < 0 || batch < 0 || (n > 0 && (!a || !x || !y))) return LO_BADARG;
    if (bad_temperature(t)) return LO_BADARG;
    if ((po == NULL) != (pi == NULL)) return LO_BADARG;
    if (n == 0 || batch == 0) return LO_OK;
    const int phased = po != NULL;
    uint32_t* p = (uint32_t*)malloc((size_t)n * sizeof(uint32_t));
    double* s = (double*)malloc((size_t)n * sizeof(double));
    double* xs = (double*)malloc((size_t)n * sizeof(double));
    double* L = (double*)malloc((size_t)n * sizeof(double));
    double* U = (double*)malloc((size_t)n * sizeof(double));
    double* acc = (double*)malloc((size_t)n * sizeof(double));
    int rc = LO_NOMEM;
    if (!p || !s || !xs || !L || !U || !acc) goto out;
    rc = lo_argsort(a, n, p);
    if (rc != LO_OK) goto out;
    for (int64_t r = 0; r < n; ++r) s[r] = a[p[r]];

    for (int64_t v = 0; v < batch; ++v) {
        const float* xv = x + v * n;
        for (int64_t r = 0; r < n; ++r) acc[r] = 0.0;
        for (int ch = 0; ch < (phased ? 2 : 1); ++ch) {
            for (int64_t r = 0; r < n; ++r) {
                double f = 1.0;
                if (phased) f = ch == 0 ? cos((double)pi[p[r]]) : sin((double)pi[p[r]]);
                xs[r] = f * xv[p[r]];
            }
            L[0] = xs[0];
            for (int64_t r = 1; r < n; ++r) L[r] = xs[r] + decay_t(s[r] - s[r - 1], t) * L[r - 1];
            U[n - 1] = xs[n - 1];
            for (int64_t r = n - 2; r >= 0; --r) U[r] = xs[r] + decay_t(s[r + 1] - s[r], t) * U[r + 1];
            for (int64_t r = 0; r < n; ++r) {
                double g = 1.0;
                if (phased) g = ch == 0 ? cos((double)po[p[r]]) : sin((double)po[p[r]]);
                acc[r] += g * (L[r] + U[r] - xs[r]);
            }
        }
        for (int64_t r = 0; r < n; ++r) y[v * n + p[r]] = acc[r];
    }
    rc = LO_OK;
out:
    free(p); free(s); free(xs); free(L); free(U); free(acc);
    return rc;
}

/* --------------------------------------------------------- general sweep */

/* Summary §2.2, general case a != b: y = K(out, in) x with outputs on the
 * sorted output anchors s and inputs at anchors q_j (weights x_j).
 *   1. sort the output anchors: s_r = out[p_r];
 *   2. bucket every input into the interval of the sorted outputs that holds
 *      it: c_j = #{r : s_r < q_j}, so q_j lies in (s_{c-1}, s_c];
 *      u_c     += exp(-(s_c - q_j)) x_j   (if c < n: it reaches ranks >= c)
 *      v_{c-1} += exp(-(q_j - s_{c-1})) x_j (if c > 0: ranks <= c-1);
 *   3. propagate with the two recurrences of the symmetric case
 *      L_r = u_r + exp(s_{r-1} - s_r) L_{r-1},
 *      R_r = v_r + exp(s_r - s_{r+1}) R_{r+1},  y at rank r = L_r + R_r.
 * Phases split into cos and sin channels as in the symmetric sweep. */
int lo_apply_general_sweep(const float* out_anchor, const float* out_phase, int64_t n_out,
                           const float* in_anchor, const float* in_phase, int64_t n_in,
                           const float* x, int64_t batch, double t, double* y)
{
    if (n_out < 0 || n_in < 0 || batch < 0) return LO_BADARG;
    if (bad_temperature(t)) return LO_BADARG;
    if ((out_phase == NULL) != (in_phase == NULL)) return LO_BADARG;
    if (n_out == 0 || batch == 0) return LO_OK;
    if (!out_anchor || !y || (n_in > 0 && (!in_anchor || !x))) return LO_BADARG;
    for (int64_t j = 0; j < n_in; ++j)
        if (!isfinite(in_anchor[j])) return LO_NONFINITE;
    const int phased = out_phase != NULL;
    const int64_t n = n_out;
    uint32_t* p = (uint32_t*)malloc((size_t)n * sizeof(uint32_t));
    double* s = (double*)malloc((size_t)n * sizeof(double));
    int64_t* bk = (int64_t*)malloc((size_t)(n_in ? n_in : 1) * sizeof(int64_t));
    double* u = (double*)malloc((size_t)n * sizeof(double));
    double* w = (double*)malloc((size_t)n * sizeof(double));
    double* L = (double*)malloc((size_t)n * sizeof(double));
    double* R = (double*)malloc((size_t)n * sizeof(double));
    double* acc = (double*)malloc((size_t)n * sizeof(double));
    int rc = LO_NOMEM;
    if (!p || !s || !bk || !u || !w || !L || !R || !acc) goto out;
    rc = lo_argsort(out_anchor, n, p);
    if (rc != LO_OK) goto out;
    for (int64_t r = 0; r < n; ++r) s[r] = out_anchor[p[r]];
    for (int64_t j = 0; j < n_in; ++j) {
        /* lower bound by bisection: first rank whose anchor is >= q_j */
        const double q = in_anchor[j];
        int64_t lo = 0, hi = n;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (s[mid] < q) lo = mid + 1; else hi = mid;
        }
        bk[j] = lo;
    }
    for (int64_t v = 0; v < batch; ++v) {
        const float* xv = x + v * n_in;
        for (int64_t r = 0; r < n; ++r) acc[r] = 0.0;
        for (int ch = 0; ch < (phased ? 2 : 1); ++ch) {
            for (int64_t r = 0; r < n; ++r) { u[r] = 0.0; w[r] = 0.0; }
            for (int64_t j = 0; j < n_in; ++j) {
                double f = 1.0;
                if (phased) f = ch == 0 ? cos((double)in_phase[j]) : sin((double)in_phase[j]);
                const double xj = f * xv[j];
                const double q = in_anchor[j];
                if (bk[j] < n) u[bk[j]] += decay_t(s[bk[j]] - q, t) * xj;
                if (bk[j] > 0) w[bk[j] - 1] += decay_t(q - s[bk[j] - 1], t) * xj;
            }
            L[0] = u[0];
            for (int64_t r = 1; r < n; ++r) L[r] = u[r] + decay_t(s[r] - s[r - 1], t) * L[r - 1];
            R[n - 1] = w[n - 1];
            for (int64_t r = n - 2; r >= 0; --r) R[r] = w[r] + decay_t(s[r + 1] - s[r], t) * R[r + 1];
            for (int64_t r = 0; r < n; ++r) {
                double g = 1.0;
                if (phased) g = ch == 0 ? cos((double)out_phase[p[r]]) : sin((double)out_phase[p[r]]);
                acc[r] += g * (L[r] + R[r]);
            }
        }
        for (int64_t r = 0; r < n; ++r) y[v * n + p[r]] = acc[r];
    }
    rc = LO_OK;
out:
    free(p); free(s); free(bk); free(u); free(w); free(L); free(R); free(acc);
    return rc;
}

/* ------------------------------------------------------------- gradients */

/* Gradients of the bilinear form F = sum_v sum_ij u[v][i] K_ij w[v][j], with
 * K = K(a, phi; b, psi) at temperature t (summary §2.1; the layer is trained
 * through its anchors and phases, so these are the derivatives a training
 * step needs: for y = K x and an upstream gradient g, u = g and w = x; for
 * y = K^T x, u = x and w = g).  From the definition, entry by entry:
 *   dK_ij/da_i   = -sgn(a_i - b_j) / t * K_ij,   dK_ij/db_j = -dK_ij/da_i,
 *   dK_ij/dphi_i = -exp(-|a_i - b_j| / t) sin(phi_i - psi_j),
 *   dK_ij/dpsi_j = -dK_ij/dphi_i,
 * with sgn(0) = 0 (the mean of the one-sided derivatives at a tie) and all
 * anchor derivatives 0 at t = 0 (the routing matrix is piecewise constant).
 * da/dphi are evaluated at the anchors rows[] of a (all n if rows == NULL),
 * db/dpsi at cols[] of b (all k if NULL); any output may be NULL.  O((|rows|
 * k + |cols| n) batch). */
int lo_grad_dense(const float* a, const float* phi, int64_t n, const float* b, const float* psi,
                  int64_t k, double t, const float* u, const float* w, int64_t batch,
                  const int64_t* rows, int64_t n_rows, const int64_t* cols, int64_t n_cols,
                  double* da, double* db, double* dphi, double* dpsi)
{
    if (n < 0 || k < 0 || batch < 0 || bad_temperature(t)) return LO_BADARG;
    if ((phi == NULL) != (psi == NULL)) return LO_BADARG;
    if ((n > 0 && (!a || !u)) || (k > 0 && (!b || !w))) return LO_BADARG;
    const int phased = phi != NULL;
    if (!phased && (dphi || dpsi)) return LO_BADARG;
    const int64_t mr = rows ? n_rows : n, mc = cols ? n_cols : k;
    for (int64_t r = 0; r < mr; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n)) return LO_BADARG;
    for (int64_t c = 0; c < mc; ++c)
        if (cols && (cols[c] < 0 || cols[c] >= k)) return LO_BADARG;
    const double inv_t = t > 0.0 ? 1.0 / t : 0.0;

    /* row side: a_i and phi_i collect sum over v, j of u_vi w_vj dK_ij */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < mr; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double ga = 0.0, gp = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double d = (double)a[i] - (double)b[j];
            const double e = decay_t(fabs(d), t);
            const double c = phased ? cos((double)phi[i] - (double)psi[j]) : 1.0;
            const double sn = phased ? sin((double)phi[i] - (double)psi[j]) : 0.0;
            const double sg = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
            double uw = 0.0;
            for (int64_t v = 0; v < batch; ++v) uw += (double)u[v * n + i] * (double)w[v * k + j];
            ga += uw * (-sg * inv_t * e * c);
            gp += uw * (-e * sn);
        }
        if (da) da[r] = ga;
        if (dphi) dphi[r] = gp;
    }
    /* column side: b_j and psi_j */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t q = 0; q < mc; ++q) {
        const int64_t j = cols ? cols[q] : q;
        double gb = 0.0, gq = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double d = (double)a[i] - (double)b[j];
            const double e = decay_t(fabs(d), t);
            const double c = phased ? cos((double)phi[i] - (double)psi[j]) : 1.0;
            const double sn = phased ? sin((double)phi[i] - (double)psi[j]) : 0.0;
            const double sg = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
            double uw = 0.0;
            for (int64_t v = 0; v < batch; ++v) uw += (double)u[v * n + i] * (double)w[v * k + j];
            gb += uw * (sg * inv_t * e * c);
            gq += uw * (e * sn);
        }
        if (db) db[q] = gb;
        if (dpsi) dpsi[q] = gq;
    }
    return LO_OK;
}

/* ------------------------------------------------------------------- Gram */

/* Weighted Gram matrix of summary §2.2, by its definition M = A diag(D) A^T
 * with A = K(a, phi; b, psi) (n x k, phases optional: both NULL or both given),
 * evaluated directly in O(k) per entry:
 *   M[r][c] = sum_l A[rows_r][l] * D_l * A[cols_c][l].
 * rows/cols == NULL mean all n.  Output is n_rows x n_cols row-major. */
int lo_gram_direct(const float* a, const float* phi, int64_t n, const float* b, const float* psi,
                   int64_t k, const float* D, const int64_t* rows, int64_t n_rows, const int64_t* cols,
                   int64_t n_cols, double t, double* M)
{
    if (n < 0 || k < 0 || !a || !M || (k > 0 && (!b || !D))) return LO_BADARG;
    if (bad_temperature(t)) return LO_BADARG;
    if ((phi == NULL) != (psi == NULL)) return LO_BADARG;
    const int phased = phi != NULL;
    const int64_t mr = rows ? n_rows : n, mc = cols ? n_cols : n;
    for (int64_t r = 0; r < mr; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n)) return LO_BADARG;
    for (int64_t c = 0; c < mc; ++c)
        if (cols && (cols[c] < 0 || cols[c] >= n)) return LO_BADARG;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < mr; ++r) {
        for (int64_t c = 0; c < mc; ++c) {
            const int64_t i = rows ? rows[r] : r, j = cols ? cols[c] : c;
            const double pi = phased ? phi[i] : 0.0, pj = phased ? phi[j] : 0.0;
            double acc = 0.0;
            for (int64_t l = 0; l < k; ++l) {
                const double ql = phased ? psi[l] : 0.0;
                acc += entry(a[i], pi, b[l], ql, phased, t) * (double)D[l] * entry(a[j], pj, b[l], ql, phased, t);
            }
            M[r * mc + c] = acc;
        }
    }
    return LO_OK;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int lo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
