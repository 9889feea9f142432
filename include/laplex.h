/*
 * laplex.h -- C ABI of the MI355X (gfx950) LAPLEX operator library.
 *
 * LAPLEX is the exact Laplace-kernel operator of "LAPLEX: The FFT of
 * Learnable Laplace Kernels" (Struski, Blazhko, Kubaty, Tabor).  Citations
 * below name the section of the technical summary published with the
 * gist.science pages of that title ("summary §2.1" ...).
 *
 *   operator (summary §2.1):  K = LAPLEX(a, phi; b, psi),
 *       K_ij = exp(-|a_i - b_j|) * cos(phi_i - psi_j),   a in R^n, b in R^k.
 *   Without phases the cosine factor is 1.  A symmetric plan has b = a.
 *   A plan's temperature t (laplex_plan_set_temperature, default 1) divides
 *   the exponent: exp(-|a_i - b_j| / t); t = 0 is the zero-temperature limit
 *   of summary §2.1 and §2.3, the equality-routing matrix [a_i == b_j].
 *
 *   algorithm (summary §2.2): sort the anchors; apply the lower and upper
 *   triangular parts by a prefix and a suffix scan of the recurrence
 *   y_{i+1} = x_{i+1} + exp(a_i - a_{i+1}) y_i; for a != b collect the
 *   contributions of one side into the intervals of the other (vectors u, v)
 *   and run the same scans; weighted Gram M = A diag(D) A^T in O(n^2 + k log n).
 *   The dense matrix is never formed.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers to float32 (fp32) data on the
 *     current HIP device, except where stated.  Vectors are contiguous; a
 *     batch of vectors is row-major [batch][length].  Offsets are 64-bit.
 *   - `stream` is a hipStream_t passed as void* (NULL = legacy default stream).
 *   - Functions return a laplex_status and never abort or throw.  Argument
 *     checks run on the host before any HIP call, so an invalid call returns
 *     LAPLEX_ERR_INVALID_ARGUMENT without touching the device.
 *   - Outputs are overwritten, never accumulated into.
 *   - Inputs are borrowed only for the duration of the call.
 *
 * Environment (read once per process):
 *   LAPLEX_REPLAY_MIN  sides of at least this many anchors (default 2^20)
 *                      move x into sorted order and y back by replaying the
 *                      sort's per-pass records (streaming passes); shorter
 *                      sides gather and scatter through the permutation.
 *                      Results agree to rounding (the summation order can
 *                      differ); the permutation is the same.
 */
#ifndef LAPLEX_H
#define LAPLEX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct laplex_plan_s* laplex_plan;

typedef enum {
    LAPLEX_OK = 0,
    LAPLEX_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, flag or overlap */
    LAPLEX_ERR_NONFINITE_ANCHOR = 2, /* NaN or +-Inf in a, b, phi or psi       */
    LAPLEX_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed               */
    LAPLEX_ERR_UNSUPPORTED = 4,      /* valid request this build does not do   */
    LAPLEX_ERR_DEVICE = 5,           /* a HIP call failed: see laplex_last_error */
    LAPLEX_ERR_NO_DEVICE = 6         /* no HIP device visible                  */
} laplex_status;

/* Plan flags reported by laplex_plan_info. */
#define LAPLEX_PLAN_SYMMETRIC 1
#define LAPLEX_PLAN_PHASED 2

/*
 * laplex_plan_create -- sort the anchors and keep what apply/gram need.
 *   (summary §2.2: "after sorting the anchors")
 *
 *   out    host pointer; receives the plan, or NULL on any error.
 *   a      device, float32[n], the row anchors.  1 <= n <= 2^30.
 *   b      device, float32[k], the column anchors, or NULL for a symmetric
 *          plan (b := a; then k must be 0 or n).  1 <= k <= 2^30.
 *          (Longer sides give INVALID_ARGUMENT: element offsets are formed
 *          as 32-bit byte offsets.)
 *   phi    device, float32[n] row phases, and
 *   psi    device, float32[k] (float32[n] if symmetric) column phases;
 *          both NULL (unphased) or both non-NULL (phased operator).
 *   stream stream on which all device work is ordered.
 *
 *   The sort order of each anchor set is ascending IEEE order with -0.0
 *   before +0.0 and ties kept in ascending original index (a stable sort),
 *   so the permutation is deterministic.  NaN/Inf anchors or phases give
 *   LAPLEX_ERR_NONFINITE_ANCHOR.  The plan copies everything it needs into
 *   device memory it owns; the call synchronizes `stream` once before it
 *   returns, after which a, b, phi, psi may be freed.
 */
laplex_status laplex_plan_create(laplex_plan* out, const float* a, int64_t n,
                                 const float* b, int64_t k,
                                 const float* phi, const float* psi, void* stream);

/*
 * laplex_plan_create_apply -- a symmetric plan (b = a) and y = K x at once.
 *   (summary §2.2: sort the anchors, then the two scans; for a layer whose
 *   anchors change every training step the sort and the first product
 *   always come together)
 *
 *   Arguments as laplex_plan_create with b = NULL, plus x, y: device float32
 *   [batch][n], row-major, not overlapping; batch >= 1.  y = K x as
 *   laplex_apply(plan, x, y, batch, 0) would give, bit for bit.  For long
 *   anchor sets the rows of x (up to 18 with phases, 20 without) travel
 *   through the radix passes with the anchors, which saves one pass over
 *   x per radix digit; otherwise it is plan_create followed by apply.
 *   Synchronizes `stream` once, like laplex_plan_create; *out receives the
 *   plan (NULL on error), which stays usable for apply, gram and backward.
 *   The plan keeps its own copy of x (batch * n floats, sorted or as given)
 *   for laplex_backward with x = NULL; it is released with the plan.
 */
laplex_status laplex_plan_create_apply(laplex_plan* out, const float* a, int64_t n,
                                       const float* phi, const float* psi, const float* x,
                                       float* y, int64_t batch, void* stream);

/*
 * laplex_apply -- y = K x (transpose = 0) or y = K^T x (transpose = 1).
 *   (summary §2.2: prefix/suffix scans; general case via vectors u, v)
 *
 *   x, y   device float32 arrays, [batch][in] and [batch][out] row-major with
 *          (in, out) = (k, n) for transpose = 0 and (n, k) for transpose = 1
 *          (a symmetric plan has k = n).  x and y must not overlap.
 *   batch  number of vectors, >= 1.
 *   Asynchronous on `stream`; the caller keeps x and y alive until the stream
 *   reaches this work.  One apply or gram per plan may be in flight at a
 *   time (they share the plan's workspace).  The workspace grows on demand
 *   (the only allocation on this path).  NaN/Inf in x propagate per IEEE.
 */
laplex_status laplex_apply(laplex_plan plan, const float* x, float* y, int64_t batch,
                           int transpose, void* stream);

/*
 * laplex_apply_noalloc -- laplex_apply without any device allocation.
 *   For callers that cannot allocate: code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc.
 *
 *   Arguments, results and errors as laplex_apply (bit for bit the same
 *   y), but the workspace is a fixed scratch array inside the library, one
 *   copy per GPU of LAPLEX_NOALLOC_SCRATCH_BYTES, held until the process
 *   ends, instead of the plan's growing workspace; no hipMalloc, hipFree or
 *   allocating library call is made.  A call whose workspace would exceed
 *   the array returns LAPLEX_ERR_INVALID_ARGUMENT (laplex_last_error says
 *   how much it needs); roughly, a symmetric plan takes batch * n up to
 *   about 7.5 million (2^20 <= n) or 15 million (shorter n).  Every call on
 *   one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   (other streams or threads) race and must be ordered by the caller.
 */
#define LAPLEX_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
laplex_status laplex_apply_noalloc(laplex_plan plan, const float* x, float* y, int64_t batch,
                                   int transpose, void* stream);

/*
 * laplex_gram -- weighted Gram matrix M = A diag(D) A^T with A = K (n x k).
 *   (summary §2.2, Gram operators: O(n^2 + k log n), not O(n^2 k))
 *
 *   D      device float32[k] weights (k = n for a symmetric plan); any finite
 *          real values.
 *   M      device float32[n][n], row-major, rows and columns in the original
 *          order of a.  Needs n * n <= 2^40 (else INVALID_ARGUMENT).
 *   For a phased plan A carries the phases too (A_il = exp(-|a_i - b_l|)
 *   cos(phi_i - psi_l)); the product of two cosines splits into three
 *   unphased Grams with weights D cos^2 psi, D cos psi sin psi, D sin^2 psi.
 *   Precision: interval sums, scans and the per-entry combination in
 *   float64 (each input's decay to about 1e-7 relative, the decays between
 *   anchors exact to float64), M rounded once to float32.
 *   Asynchronous on `stream`.  The first call on a plan also makes tables
 *   the plan keeps for later calls (interval bounds and ranks, 4 (n + 2) +
 *   4 n + 32 (n + 1) bytes; b's inputs grouped by interval and by eighth
 *   of the original order, 8 k bytes, 16 k when phased); the workspace
 *   grows on demand as for laplex_apply.
 */
laplex_status laplex_gram(laplex_plan plan, const float* D, float* M, void* stream);

/*
 * laplex_backward -- gradients of a training step through y = K x
 *   (transpose = 0) or y = K^T x (transpose = 1), K at the plan's temperature.
 *   (summary §2.1: a LAPLEX layer is trained through its anchors and phases;
 *   the derivatives are those of the definition, entry by entry)
 *
 *   x      device float32 [batch][in]: the forward input ((in, out) as in
 *          laplex_apply).  NULL for a plan made by laplex_plan_create_apply
 *          (then transpose = 0 and batch as in that call): the plan kept that
 *          call's x, by rank when its rows travelled with the sort, so the
 *          backward does not move x into sorted order again.
 *   g      device float32 [batch][out]: the upstream gradient dL/dy.
 *   dx     [batch][in]: dL/dx = K^T g (transpose = 0) or K g (transpose = 1).
 *   da     [n]: dL/da summed over the batch.  For y = K x,
 *            dL/da_i = -(1/t) sum_v g_vi sum_j sgn(a_i - b_j) K_ij x_vj;
 *          a symmetric plan (b = a) adds the column-side term, so da is the
 *          full gradient of its one anchor vector.
 *   db     [k]: dL/db (general plans only; must be NULL for a symmetric plan).
 *   dphi   [n], dpsi [k] (symmetric: [n]): phase gradients, phased plans only
 *          (must be NULL otherwise).  dL/dphi_i = -sum_v g_vi sum_j
 *          exp(-|a_i - b_j| / t) sin(phi_i - psi_j) x_vj for transpose = 0.
 *   Each output may be NULL to skip it; outputs are overwritten and must not
 *   overlap each other, x or g.  sgn(0) = 0: equal anchors exert no force on
 *   each other (the mean of the two one-sided derivatives).  At t = 0 the
 *   anchor gradients are 0 (the routing matrix is piecewise constant).
 *   Asynchronous on `stream`; shares the plan's workspace with apply/gram.
 */
laplex_status laplex_backward(laplex_plan plan, const float* x, const float* g, int64_t batch,
                              int transpose, float* dx, float* da, float* db, float* dphi,
                              float* dpsi, void* stream);

/* Releases all device memory of the plan (synchronizes the device first).
 * NULL is accepted. */
laplex_status laplex_plan_destroy(laplex_plan plan);

/*
 * Introspection.  laplex_plan_perm: *perm_dev receives a DEVICE pointer to the
 * plan's permutation uint32[len] (rank r -> original index) of side 0 (a) or
 * side 1 (b; the same as side 0 for a symmetric plan).  It stays valid until
 * the plan is destroyed.  laplex_plan_sorted likewise gives the sorted
 * anchors float32[len].  laplex_plan_info reports n, k and LAPLEX_PLAN_* flags.
 */
laplex_status laplex_plan_perm(laplex_plan plan, int side, const uint32_t** perm_dev);
laplex_status laplex_plan_sorted(laplex_plan plan, int side, const float** sorted_dev);
laplex_status laplex_plan_info(laplex_plan plan, int64_t* n, int64_t* k, int* flags);

/*
 * Algorithm choice for a != b (both give the same operator, exactly up to
 * rounding):
 *   LAPLEX_ALGO_AUTO      scan over the smaller side (default);
 *   LAPLEX_ALGO_BUCKET    the pages' general case: bucket the input side into
 *                         the intervals of the sorted output side (u, v), scan
 *                         over the output side, write back in original order;
 *   LAPLEX_ALGO_EVALUATE  scan over the sorted input side, then evaluate each
 *                         output by bisection into the sorted input side.
 * Symmetric plans ignore the setting.
 */
#define LAPLEX_OPT_GENERAL_ALGO 1
#define LAPLEX_ALGO_AUTO 0
#define LAPLEX_ALGO_BUCKET 1
#define LAPLEX_ALGO_EVALUATE 2
laplex_status laplex_plan_set_option(laplex_plan plan, int option, int64_t value);

/*
 * laplex_plan_set_temperature -- entries exp(-|a_i - b_j| / t) cos(phi_i - psi_j)
 *   for every later apply / gram / backward of the plan.
 *   (summary §2.1: the temperature t -> 0 regime; §2.3: zero-temperature
 *   limit, equality routing that recovers permutations and CountSketch)
 *
 *   t      1 is the operator as printed (the default).  t = 0 selects the
 *          limit: 1 where a_i == b_j (-0.0 == +0.0), else 0, so y routes x by
 *          exact equality of anchors.  Otherwise FLT_MIN <= t <= FLT_MAX;
 *          anything else (negative, NaN, Inf, subnormal) is INVALID_ARGUMENT.
 *   The sort order does not depend on t, so the plan is reused as is.  Not
 *   ordered with in-flight work: call it between applies on the same thread.
 */
laplex_status laplex_plan_set_temperature(laplex_plan plan, double t);

/* Kernel timing: while enabled, every kernel the library launches is
 * bracketed by HIP events on its stream (timing-only events, recorded
 * without a system-scope fence, so they order no memory for the host).
 * laplex_profile_collect waits for the recorded events and folds their
 * durations into per-kernel totals;
 * laplex_profile_entry reads entry `i` (returns INVALID_ARGUMENT past the
 * end).  Names are static strings.  Not thread-safe; for benchmarks. */
laplex_status laplex_profile_enable(int on);
/* While enabled, bracket only the launches whose label equals `label`
 * (copied; NULL or "" brackets every launch, the default): fewer event
 * records between launches when only one kernel's time is wanted. */
laplex_status laplex_profile_only(const char* label);
laplex_status laplex_profile_reset(void);
laplex_status laplex_profile_collect(void);
laplex_status laplex_profile_entry(int i, const char** name, int64_t* launches, double* total_ms);

const char* laplex_status_str(laplex_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* laplex_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LAPLEX_H */
