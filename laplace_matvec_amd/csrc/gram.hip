// Weighted Gram matrix M = A diag(D) A^T, A = K(a, b) (n x k), gfx950.
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2
// (Gram operators): the sorted order gives M exactly in O(n^2 + k log n)
// instead of O(n^2 k).  With sorted row anchors s_0 <= ... <= s_{n-1} and
// ranks r <= c, split the sum over b by position:
//   b <= s_r       : D e^{-(s_r-b)} e^{-(s_c-b)} = e^{-(s_c-s_r)} D e^{-2(s_r-b)}
//   s_r < b <= s_c : D e^{-(b-s_r)} e^{-(s_c-b)} = e^{-(s_c-s_r)} D
//   b > s_c        : D e^{-(b-s_r)} e^{-(b-s_c)} = e^{-(s_c-s_r)} D e^{-2(b-s_c)}
// so M_rc = e^{-(s_c - s_r)} (P_r + (S_c - S_r) + Q_c) with (at temperature t
// every exponent divided by t)
//   S_r = sum of D over b <= s_r,
//   P_r = sum over b <= s_r of D e^{-2(s_r - b)},
//   Q_c = sum over b >  s_c of D e^{-2(b - s_c)}.
// These are prefix sums of exp(+-2b) D rescaled to the interval end points,
// so nothing overflows for large |b|; S is kept in float64 because S_c - S_r
// cancels.  Per interval r (b in (s_{r-1}, s_r], r = 0..n) the kernels sum
//   sigma_r = sum D,  p_r = sum D e^{-2(s_r - b)},  q_{r-1} = sum D e^{-2(b - s_{r-1})}
// and then run P_r = e^{-2(s_r - s_{r-1})} P_{r-1} + p_r (forward),
// Q_r = e^{-2(s_{r+1} - s_r)} Q_{r+1} + q_r (backward), S by a prefix sum.
// Equal anchors get equal (S, P, Q), so the order among ties is irrelevant.
//
// A phased operator, cos(phi_i - psi_l) in every entry, expands into three
// such Grams with weights D cos^2 psi, D cos psi sin psi, D sin^2 psi,
// combined per entry with cos/sin of phi_i and phi_j.
//
//   lx_gram_bins : one workgroup per interval; its b-range in the sorted b
//                  by bisection (k log n in total), fixed-order reduction.
//   lx_gram_scan : one workgroup, the three scans, stats in original order.
//   lx_gram_tile : 64 x 64 tiles of M in the original order, O(1) per entry.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

constexpr int kBinThreads = 256;
constexpr int kGramScanThreads = 1024;
constexpr int kGT = 64;  // tile edge

__device__ __forceinline__ double block_sum_d(double x, double* sh)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) x += __shfl_down(x, d);
    if (lane == 0) sh[w] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kBinThreads / kWave; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// Weight sets: one (D) for the plain operator; three for a phased one,
// D cos^2 psi, D cos psi sin psi and D sin^2 psi, since
// cos(p_i - q) cos(p_j - q) = cp_i cp_j c^2 + (cp_i sp_j + sp_i cp_j) c s + sp_i sp_j s^2.
// Stats per original index i: s_i, then (P, S, Q) per weight set, then
// cos/sin of phi_i when phased.
template <int NW>
constexpr int gram_stride() { return 1 + 3 * NW + (NW == 3 ? 2 : 0); }

template <int NW>
__global__ __launch_bounds__(kBinThreads) void lx_gram_bins(GramArgs A, double* __restrict__ sigma,
                                                           double* __restrict__ p, double* __restrict__ q)
{
    __shared__ double sh[kBinThreads / kWave];
    const int64_t n = A.n, k = A.k;
    const int64_t r = blockIdx.x;  // interval (s_{r-1}, s_r], r = 0..n
    const int64_t lo = r == 0 ? 0 : upper_bound_f(A.sb, k, A.sa[r - 1]);
    const int64_t hi = r == n ? k : upper_bound_f(A.sb, k, A.sa[r]);
    const double right = r < n ? (double)A.sa[r] : 0.0;
    const double left = r > 0 ? (double)A.sa[r - 1] : 0.0;
    double sg[NW], pp[NW], qq[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) sg[w] = pp[w] = qq[w] = 0.0;
    for (int64_t j = lo + threadIdx.x; j < hi; j += kBinThreads) {
        const double d = (double)A.D[A.pb[j]];
        double wt[NW];
        if (NW == 3) {
            const double c = A.cpsi_r[j], sn = A.spsi_r[j];
            wt[0] = d * c * c;
            wt[NW > 1 ? 1 : 0] = d * c * sn;
            wt[NW - 1] = d * sn * sn;
        } else {
            wt[0] = d;
        }
        const double b = (double)A.sb[j];
        const double er = r < n ? decay_dist(2.0 * (right - b), A.inv_t) : 0.0;
        const double el = r > 0 ? decay_dist(2.0 * (b - left), A.inv_t) : 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            sg[w] += wt[w];
            pp[w] += wt[w] * er;
            qq[w] += wt[w] * el;
        }
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const double a1 = block_sum_d(sg[w], sh);
        const double a2 = block_sum_d(pp[w], sh);
        const double a3 = block_sum_d(qq[w], sh);
        if (threadIdx.x == 0) {
            sigma[w * (n + 1) + r] = a1;
            if (r < n) p[w * n + r] = a2;
            if (r > 0) q[w * n + r - 1] = a3;
        }
    }
}

template <int NW>
__global__ __launch_bounds__(kGramScanThreads) void lx_gram_scan(GramArgs A, const double* __restrict__ sigma,
                                                                const double* __restrict__ p,
                                                                const double* __restrict__ q,
                                                                double* __restrict__ st)
{
    __shared__ Aff<double> sh[kGramScanThreads / kWave];
    constexpr int SW = gram_stride<NW>();
    const int64_t n = A.n;
    const float* s = A.sa;
    const int64_t per = (n + kGramScanThreads - 1) / kGramScanThreads;
    int64_t r0 = (int64_t)threadIdx.x * per;
    if (r0 > n) r0 = n;
    int64_t r1 = r0 + per;
    if (r1 > n) r1 = n;
    for (int64_t r = r0; r < r1; ++r) {
        double* o = st + (int64_t)A.pa[r] * SW;
        o[0] = (double)s[r];
        if (NW == 3) {
            o[SW - 2] = A.cphi_r[r];
            o[SW - 1] = A.sphi_r[r];
        }
    }
#pragma unroll 1
    for (int w = 0; w < NW; ++w) {
        const double* sg = sigma + w * (n + 1);
        const double* pw = p + w * n;
        const double* qw = q + w * n;
        // forward: S (multiplier 1) and P (multiplier e^{-2 gap}); rank 0 starts both
        Aff<double> S = aff_identity<double>(), P = aff_identity<double>();
        for (int64_t r = r0; r < r1; ++r) {
            const double m = r > 0 ? decay_dist(2.0 * ((double)s[r] - (double)s[r - 1]), A.inv_t) : 0.0;
            S = compose(S, Aff<double>{1.0, sg[r]});
            P = compose(P, Aff<double>{m, pw[r]});
        }
        Aff<double> tot;
        double runS = block_exscan_up<double, kGramScanThreads / kWave>(S, sh, tot).v;
        double runP = block_exscan_up<double, kGramScanThreads / kWave>(P, sh, tot).v;
        for (int64_t r = r0; r < r1; ++r) {
            const double m = r > 0 ? decay_dist(2.0 * ((double)s[r] - (double)s[r - 1]), A.inv_t) : 0.0;
            runS += sg[r];
            runP = m * runP + pw[r];
            double* o = st + (int64_t)A.pa[r] * SW + 1 + 3 * w;
            o[0] = runP;
            o[1] = runS;
        }
        Aff<double> Q = aff_identity<double>();
        for (int64_t r = r1 - 1; r >= r0; --r) {
            const double m = r + 1 < n ? decay_dist(2.0 * ((double)s[r + 1] - (double)s[r]), A.inv_t) : 0.0;
            Q = compose(Q, Aff<double>{m, qw[r]});
        }
        double runQ = block_exscan_down<double, kGramScanThreads / kWave>(Q, sh, tot).v;
        for (int64_t r = r1 - 1; r >= r0; --r) {
            const double m = r + 1 < n ? decay_dist(2.0 * ((double)s[r + 1] - (double)s[r]), A.inv_t) : 0.0;
            runQ = m * runQ + qw[r];
            st[(int64_t)A.pa[r] * SW + 3 + 3 * w] = runQ;
        }
    }
}

template <int NW>
__global__ __launch_bounds__(256) void lx_gram_tile(const double* __restrict__ st, int64_t n, double inv_t,
                                                   float* __restrict__ M)
{
    constexpr int SW = gram_stride<NW>();
    __shared__ double rs[kGT][SW];
    __shared__ double cs[kGT][SW];
    const int64_t i0 = (int64_t)blockIdx.y * kGT, j0 = (int64_t)blockIdx.x * kGT;
    for (int t = threadIdx.x; t < kGT * SW; t += 256) {
        const int e = t / SW, f = t % SW;
        rs[e][f] = (i0 + e < n) ? st[(i0 + e) * SW + f] : 0.0;
        cs[e][f] = (j0 + e < n) ? st[(j0 + e) * SW + f] : 0.0;
    }
    __syncthreads();
    const int jj = threadIdx.x % kGT;
    const int64_t j = j0 + jj;
#pragma unroll 4
    for (int ii = threadIdx.x / kGT; ii < kGT; ii += 256 / kGT) {
        const int64_t i = i0 + ii;
        if (i < n && j < n) {
            // lo: the smaller anchor (equal anchors carry equal stats)
            const bool row_first = rs[ii][0] <= cs[jj][0];
            const double* lo = row_first ? rs[ii] : cs[jj];
            const double* hi = row_first ? cs[jj] : rs[ii];
            double g[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) g[w] = lo[1 + 3 * w] + (hi[2 + 3 * w] - lo[2 + 3 * w]) + hi[3 + 3 * w];
            double val;
            if (NW == 3) {
                const double ci = rs[ii][SW - 2], si = rs[ii][SW - 1], cj = cs[jj][SW - 2], sj = cs[jj][SW - 1];
                val = ci * cj * g[0] + (ci * sj + si * cj) * g[NW > 1 ? 1 : 0] + si * sj * g[NW - 1];
            } else {
                val = g[0];
            }
            M[i * n + j] = (float)(decay_dist(hi[0] - lo[0], inv_t) * val);
        }
    }
}

size_t gram_scratch_bytes(int64_t n, int nw)
{
    const int sw = 1 + 3 * nw + (nw == 3 ? 2 : 0);
    return (size_t)(nw * ((n + 1) + 2 * n) + sw * n + 64) * 8;
}

template <int NW>
static hipError_t gram_launch_t(const GramArgs& a, hipStream_t s)
{
    const int64_t n = a.n;
    double* sigma = a.stats;
    double* p = sigma + NW * (n + 1);
    double* q = p + NW * n;
    double* st = q + NW * n;
    LX_LAUNCH("gram_bins", s, (lx_gram_bins<NW><<<(unsigned)(n + 1), kBinThreads, 0, s>>>(a, sigma, p, q)));
    LX_LAUNCH("gram_scan", s, (lx_gram_scan<NW><<<1, kGramScanThreads, 0, s>>>(a, sigma, p, q, st)));
    const unsigned nb = (unsigned)((n + kGT - 1) / kGT);
    LX_LAUNCH("gram_tile", s, (lx_gram_tile<NW><<<dim3(nb, nb), 256, 0, s>>>(st, n, a.inv_t, a.M)));
    return hipSuccess;
}

hipError_t gram_launch(const GramArgs& a, hipStream_t s)
{
    if (a.n <= 0) return hipSuccess;
    return a.cpsi_r ? gram_launch_t<3>(a, s) : gram_launch_t<1>(a, s);
}

}  // namespace lx
