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
//   lx_gram_bounds : once per plan, the first sorted-b position of every
//                    interval (bisection of each a over the sorted b);
//   lx_gram_ranks  : once per plan, the rank of each original index of a;
//   lx_gram_bins   : per slice of the inputs (see "slices" below), one wave
//                    per interval: its run of sorted b summed (sigma, p, q
//                    per weight set) in float64 and a fixed order, and the
//                    decay between the interval's two a;
//   lx_gram_fold   : the slices' sums added in a fixed order, and each
//                    anchor's decay factors about the centre of all of them
//                    when that centre serves every tile;
//   lx_gram_scan   : two workgroups, S and P forward and Q backward over
//                    the intervals, written by rank;
//   lx_gram_tile   : 64 x 64 tiles of M in the original order, O(1) per entry,
//                    each row's and column's stats fetched through its rank.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

constexpr int kGramScanThreads = 512;
constexpr int kGT = 64;  // tile edge

// Weight sets: one (D) for the plain operator; three for a phased one,
// D cos^2 psi, D cos psi sin psi and D sin^2 psi, since
// cos(p_i - q) cos(p_j - q) = cp_i cp_j c^2 + (cp_i sp_j + sp_i cp_j) c s + sp_i sp_j s^2.
// Stats row per rank: (P, S, Q) per weight set, then E+ and E- of the
// anchor about the global centre (made when every tile can use it, see
// gram_global_factors).
template <int NW>
constexpr int gram_srow() { return 3 * NW + 2; }

// The decay between two anchors splits into per-anchor factors about one
// centre c, e^{-(hi - lo)/t} = E+_lo E-_hi with E+ = e^{(a - c)/t} and
// E- = e^{-(a - c)/t}, as long as no |a - c|/t comes near overflow: with
// the centre of all the anchors (sa sorted), when their whole span is at
// most 600 t (and t > 0).
__device__ __forceinline__ bool gram_global_factors(const float* sa, int64_t n, double inv_t, double* centre)
{
    const double lo = sa[0], hi = sa[n - 1];
    *centre = 0.5 * (lo + hi);
    return inv_t <= 1.0e300 && (hi - lo) * inv_t <= 600.0;
}

// Scratch (doubles, 256-byte aligned regions):
//   sigma [NW][n+1], p [NW][n], q [NW][n], mdec [n] (e^{-2(s_r - s_{r-1})/t}),
//   st [n][3 NW + 2] (P, S, Q of each weight set, E+, E-, by rank),
//   part [slice][3 NW][n+1] (each slice's sums per interval)
struct GramScratch {
    double *sigma, *p, *q, *mdec, *st, *part;
};

static inline size_t al256g(size_t b) { return (b + 255) & ~(size_t)255; }

static GramScratch gram_scratch_at(void* base, int64_t n, int nw)
{
    GramScratch g;
    char* c = (char*)base;
    g.sigma = (double*)c; c += al256g((size_t)nw * (n + 1) * 8);
    g.p = (double*)c; c += al256g((size_t)nw * n * 8);
    g.q = (double*)c; c += al256g((size_t)nw * n * 8);
    g.mdec = (double*)c; c += al256g((size_t)n * 8);
    g.st = (double*)c; c += al256g((size_t)n * (3 * nw + 2) * 8);
    g.part = (double*)c;
    return g;
}

size_t gram_scratch_bytes(int64_t n, int64_t k, int nw)
{
    (void)k;
    const int sw = 3 * nw + 2;
    return al256g((size_t)nw * (n + 1) * 8) + 2 * al256g((size_t)nw * n * 8) + al256g((size_t)n * 8) +
           al256g((size_t)n * sw * 8) + al256g((size_t)kGramSlices * 3 * nw * (n + 1) * 8);
}

// bound[r] = #{l : b_l <= s_{r-1}} for r = 1 .. n, bound[0] = 0,
// bound[n+1] = k: interval r (b in (s_{r-1}, s_r]) is sorted b [bound[r], bound[r+1]).
__global__ __launch_bounds__(256) void lx_gram_bounds(const float* __restrict__ sa, int64_t n,
                                                     const float* __restrict__ sb, int64_t k,
                                                     uint32_t* __restrict__ bound)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r > n + 1) return;
    bound[r] = (uint32_t)(r == 0 ? 0 : (r == n + 1 ? k : upper_bound_f(sb, k, sa[r - 1])));
}

hipError_t gram_bounds_launch(const float* sa, int64_t n, const float* sb, int64_t k, uint32_t* bound, hipStream_t s)
{
    if (n <= 0 || k <= 0) return hipSuccess;
    LX_LAUNCH("gram_bounds", s, (lx_gram_bounds<<<(unsigned)((n + 2 + 255) / 256), 256, 0, s>>>(sa, n, sb, k, bound)));
    return hipSuccess;
}

// ---------------------------------------------------------------- slices
//
// The weights D arrive in the original order of b, and an interval's inputs
// sit at random original indices: gathering D for sorted b pulls a whole
// cache line per 4-byte weight from all of D.  So the inputs are split by
// original index into kGramSlices ranges, one per compute die, and each
// interval's inputs of one slice are stored together (made once per plan):
// the workgroups summing slice s run on die s, whose L2 then holds the
// 1/8 of D they gather from.  Each slice gives partial sums per interval;
// a fold adds the slices in a fixed order, so results stay deterministic.

__device__ __forceinline__ uint32_t gram_slice_of(uint32_t l, int64_t k)
{
    return (uint32_t)(((uint64_t)l * kGramSlices) / (uint64_t)k);
}

// cnt[s (n+1) + r] = inputs of interval r in slice s; one workgroup per interval.
__global__ __launch_bounds__(256) void lx_gram_slice_count(const uint32_t* __restrict__ pb,
                                                          const uint32_t* __restrict__ bound, int64_t n,
                                                          int64_t k, uint32_t* __restrict__ cnt)
{
    __shared__ uint32_t sc[kGramSlices];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    if (tid < kGramSlices) sc[tid] = 0;
    __syncthreads();
    uint32_t c[kGramSlices] = {};
    for (int64_t j = bound[r] + tid; j < bound[r + 1]; j += 256) {
        const uint32_t sl = gram_slice_of(pb[j], k);
#pragma unroll
        for (int q = 0; q < kGramSlices; ++q) c[q] += sl == (uint32_t)q ? 1u : 0u;
    }
#pragma unroll
    for (int q = 0; q < kGramSlices; ++q) {
        uint32_t x = c[q];
#pragma unroll
        for (int d = kWave / 2; d > 0; d >>= 1) x += __shfl_down(x, d);
        if (lane_id() == 0 && x) atomicAdd(&sc[q], x);  // integer sums: any order gives the same
    }
    __syncthreads();
    if (tid < kGramSlices) cnt[(int64_t)tid * (n + 1) + r] = sc[tid];
}

// In place: off[i] = sum of cnt[0 .. i), off[len] = the total (one workgroup).
__global__ __launch_bounds__(1024) void lx_gram_slice_scan(uint32_t* __restrict__ off, int64_t len)
{
    __shared__ uint32_t sh[1024 / kWave];
    uint32_t carry = 0;
    for (int64_t base = 0; base < len; base += 1024) {
        const int64_t i = base + threadIdx.x;
        const uint32_t v = i < len ? off[i] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exsum_u32<1024 / kWave>(v, sh, tot);
        if (i < len) off[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) off[len] = carry;
}

// Places every input of interval r at its slice's next free position, in
// ascending sorted position within each (slice, interval): the original
// index, b, and (phased) the cos / sin of psi.  One workgroup per interval.
__global__ __launch_bounds__(256) void lx_gram_slice_place(GramArgs A, const uint32_t* __restrict__ off,
                                                          uint32_t* __restrict__ s_src, float* __restrict__ s_b,
                                                          float* __restrict__ s_c, float* __restrict__ s_s)
{
    constexpr int kW = 256 / kWave;
    __shared__ uint32_t base[kGramSlices];
    __shared__ uint32_t wcnt[kW][kGramSlices + 1];
    const int tid = threadIdx.x, w = tid / kWave;
    const int64_t n = A.n, r = blockIdx.x;
    const int64_t lo = A.bound[r], hi = A.bound[r + 1];
    if (tid < kGramSlices) base[tid] = off[(int64_t)tid * (n + 1) + r];
    for (int64_t c0 = lo; c0 < hi; c0 += 256) {
        if (tid < kW * (kGramSlices + 1)) (&wcnt[0][0])[tid] = 0;
        __syncthreads();  // also: the previous chunk's bases are final
        const int64_t j = c0 + tid;
        const bool valid = j < hi;
        const uint32_t l = valid ? A.pb[j] : 0u;
        const uint32_t sl = valid ? gram_slice_of(l, A.k) : (uint32_t)kGramSlices;
        const uint64_t peers = match_bits<4>(sl);
        const uint32_t below = count_below(peers);
        if (below == 0) wcnt[w][sl] = (uint32_t)__popcll(peers);
        __syncthreads();
        uint32_t chunk = 0;  // this chunk's inputs of slice tid
        if (tid < kGramSlices)
            for (int i = 0; i < kW; ++i) chunk += wcnt[i][tid];
        if (valid) {
            uint32_t dst = base[sl] + below;
            for (int i = 0; i < w; ++i) dst += wcnt[i][sl];
            s_src[dst] = l;
            s_b[dst] = A.sb[j];
            if (s_c) {
                s_c[dst] = A.cpsi_r[j];
                s_s[dst] = A.spsi_r[j];
            }
        }
        __syncthreads();  // every read of the bases and counts of this chunk is done
        if (tid < kGramSlices) base[tid] += chunk;
    }
}

hipError_t gram_slices_launch(const GramArgs& a, uint32_t* off, uint32_t* s_src, float* s_b, float* s_c, float* s_s,
                              hipStream_t s)
{
    if (a.n <= 0 || a.k <= 0) return hipSuccess;
    const unsigned iv = (unsigned)(a.n + 1);
    LX_LAUNCH("gram_slices", s, (lx_gram_slice_count<<<iv, 256, 0, s>>>(a.pb, a.bound, a.n, a.k, off)));
    LX_LAUNCH("gram_slices", s, (lx_gram_slice_scan<<<1, 1024, 0, s>>>(off, (int64_t)kGramSlices * (a.n + 1))));
    LX_LAUNCH("gram_slices", s, (lx_gram_slice_place<<<iv, 256, 0, s>>>(a, off, s_src, s_b, s_c, s_s)));
    return hipSuccess;
}

// Interval sums of one slice: workgroup b takes slice b % kGramSlices (so
// on die b % 8) and four intervals, one per wave; each lane takes the
// slice's inputs of its wave's interval at stride 64, kBinLoads at a time
// with every load in flight before any is used, and the wave folds its
// lanes in a fixed order.  The per-input decays use exp_nonpos_fast: the
// float64 library exp, whose branch on the argument also splits the wave,
// made this kernel bound by its vector instructions.
constexpr int kBinThreads = 256;
constexpr int kBinWaves = kBinThreads / kWave;
constexpr int kBinLoads = 2;  // 3 * 2^20 inputs over 4097 intervals and 8 slices: about 96 per wave

template <int NW>
__global__ __launch_bounds__(kBinThreads) void lx_gram_bins(GramArgs A, GramScratch G)
{
    constexpr int K = 3 * NW;  // per weight set: sigma, p, q
    const int64_t n = A.n;
    const int sl = (int)(blockIdx.x % kGramSlices);
    const int64_t r = (int64_t)(blockIdx.x / kGramSlices) * kBinWaves + threadIdx.x / kWave;
    if (r > n) return;  // a whole wave; no barriers below
    const int lane = lane_id();
    const double it2 = 2.0 * A.inv_t;  // e^{-2 d / t}
    const int64_t io = (int64_t)sl * (n + 1) + r;
    const uint32_t lo = A.slice_off[io], hi = A.slice_off[io + 1];
    // the interval's end anchors; +inf / -inf where it has none (no decay term)
    const float right = r < n ? A.sa[r] : INFINITY;
    const float left = r > 0 ? A.sa[r - 1] : -INFINITY;
    double acc[K];
#pragma unroll
    for (int q = 0; q < K; ++q) acc[q] = 0.0;
    for (uint32_t m0 = lo + (uint32_t)lane; m0 < hi; m0 += (uint32_t)(kWave * kBinLoads)) {
        uint32_t src[kBinLoads];
        float bv[kBinLoads], cc[kBinLoads], ss[kBinLoads];
#pragma unroll
        for (int u = 0; u < kBinLoads; ++u) {
            const uint32_t m = m0 + (uint32_t)(u * kWave);
            const uint32_t mc = m < hi ? m : lo;  // a valid position; its terms are not used
            src[u] = A.slice_src[mc];
            bv[u] = A.slice_b[mc];
            cc[u] = NW == 3 ? A.slice_c[mc] : 1.f;
            ss[u] = NW == 3 ? A.slice_s[mc] : 0.f;
        }
        float dv[kBinLoads];
#pragma unroll
        for (int u = 0; u < kBinLoads; ++u) dv[u] = A.D[src[u]];
#pragma unroll
        for (int u = 0; u < kBinLoads; ++u) {
            const bool in = m0 + (uint32_t)(u * kWave) < hi;
            const double d = in ? (double)dv[u] : 0.0;
            double wt[NW];
            if (NW == 3) {
                const double c = cc[u], sn = ss[u];
                wt[0] = d * c * c;
                wt[NW > 1 ? 1 : 0] = d * c * sn;
                wt[NW - 1] = d * sn * sn;
            } else {
                wt[0] = d;
            }
            // each term to about 1e-7 (all are positive, so the sums too);
            // the decays between anchors, which the scans multiply along
            // the whole order, stay exact to float64
            const double er = decay_fast(bv[u], right, it2);  // 0 past the last anchor
            const double el = decay_fast(left, bv[u], it2);   // 0 before the first
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                acc[3 * w] += wt[w];
                acc[3 * w + 1] = fma(wt[w], er, acc[3 * w + 1]);
                acc[3 * w + 2] = fma(wt[w], el, acc[3 * w + 2]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < K; ++q) acc[q] = wave_sum_dpp(acc[q]);
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < K; ++q) G.part[((int64_t)sl * K + q) * (n + 1) + r] = acc[q];
        if (sl == 0 && r < n) G.mdec[r] = r > 0 ? decay(left, right, it2) : 0.0;
    }
}

// sigma, p, q of every interval: the slices' sums added in slice order;
// and, where the centre of all the anchors serves every tile, each
// anchor's decay factors about it (E+, E- in the stats row of its rank).
template <int NW>
__global__ __launch_bounds__(256) void lx_gram_fold(const float* __restrict__ sa, double inv_t, int64_t n,
                                                    GramScratch G)
{
    constexpr int K = 3 * NW;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= K * (n + 1)) return;
    const int q = (int)(i / (n + 1));
    const int64_t r = i - (int64_t)q * (n + 1);
    double v[kGramSlices];
#pragma unroll
    for (int sl = 0; sl < kGramSlices; ++sl) v[sl] = G.part[((int64_t)sl * K + q) * (n + 1) + r];
    double t = 0.0;
#pragma unroll
    for (int sl = 0; sl < kGramSlices; ++sl) t += v[sl];
    const int w = q / 3, kind = q % 3;
    if (kind == 0) G.sigma[w * (n + 1) + r] = t;
    else if (kind == 1) { if (r < n) G.p[w * n + r] = t; }
    else if (r > 0) G.q[w * n + r - 1] = t;
    double c;
    if (q == 0 && r < n && gram_global_factors(sa, n, inv_t, &c)) {
        const double xe = ((double)sa[r] - c) * inv_t;
        double* o = G.st + r * gram_srow<NW>() + 3 * NW;
        o[0] = exp(xe);
        o[1] = exp(-xe);
    }
}

// Two workgroups: the first runs S and P forward over the intervals, the
// second Q backward (the recurrences are independent), each writing its
// stats by rank (P, S, Q of each weight set).  A
// round covers kRound ranks, gram_run() consecutive ones per thread; every
// global load of a round is issued first, coalesced (consecutive threads,
// consecutive ranks), and each array is then turned into the per-thread
// runs through LDS; the results go back the same way, so the stores are
// coalesced too.  (Loads and stores of per-thread runs straight from
// memory touch a cache line per lane, and one workgroup's memory pipeline
// then spends several microseconds on each array.)
template <int NW>
constexpr int gram_run() { return NW == 3 ? 2 : 8; }  // three weight sets hold three times the values

// LDS position of element e of a round: one pad double per eight, so the
// per-thread runs (stride gram_run()) fall on different banks.
__device__ __forceinline__ int gram_pad(int e) { return e + (e >> 3); }

template <int NW>
__global__ __launch_bounds__(kGramScanThreads) void lx_gram_scan(GramArgs A, GramScratch G)
{
    constexpr int R = gram_run<NW>();
    constexpr int kWaves = kGramScanThreads / kWave;
    constexpr int SR = gram_srow<NW>();  // doubles per rank
    constexpr int kRound = kGramScanThreads * R;
    __shared__ Aff<double> sh[kWaves];
    __shared__ double buf[kRound + kRound / 8];
    const int tid = threadIdx.x;
    const int64_t n = A.n;
    double* st = G.st;

    // element i * threads + tid of a round (coalesced layout) -> this
    // thread's run, element tid * R + i
    auto to_runs = [&](const double (&c)[R], double (&out)[R]) {
#pragma unroll
        for (int i = 0; i < R; ++i) buf[gram_pad(i * kGramScanThreads + tid)] = c[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < R; ++i) out[i] = buf[gram_pad(tid * R + i)];
        __syncthreads();
    };
    // and back: this thread's run -> coalesced layout
    auto from_runs = [&](const double (&run)[R], double (&c)[R]) {
#pragma unroll
        for (int i = 0; i < R; ++i) buf[gram_pad(tid * R + i)] = run[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < R; ++i) c[i] = buf[gram_pad(i * kGramScanThreads + tid)];
        __syncthreads();
    };

    if (blockIdx.x == 0) {
        // ---- forward: S_r = S_{r-1} + sigma_r, P_r = e^{-2 d_{r-1}} P_{r-1} + p_r
        double carS[NW], carP[NW];  // carried in from earlier rounds (the same in every thread)
#pragma unroll
        for (int w = 0; w < NW; ++w) carS[w] = carP[w] = 0.0;
#pragma unroll 1
        for (int64_t base = 0; base < n; base += kRound) {
            double cs[NW][R], cp[NW][R], cm[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t r = base + i * kGramScanThreads + tid;
                const bool ok = r < n;
                const int64_t rc = ok ? r : 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    cs[w][i] = ok ? G.sigma[w * (n + 1) + rc] : 0.0;
                    cp[w][i] = ok ? G.p[w * n + rc] : 0.0;
                }
                cm[i] = ok ? G.mdec[rc] : 1.0;
            }
            double m[R];
            to_runs(cm, m);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                double vs[R], vp[R];
                to_runs(cs[w], vs);
                to_runs(cp[w], vp);
                Aff<double> S = aff_identity<double>(), P = aff_identity<double>();
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    S = compose(S, Aff<double>{1.0, vs[i]});
                    P = compose(P, Aff<double>{m[i], vp[i]});
                }
                Aff<double> totS, totP;
                const Aff<double> xS = block_exscan_up<double, kWaves>(S, sh, totS);
                const Aff<double> xP = block_exscan_up<double, kWaves>(P, sh, totP);
                double runS = xS.m * carS[w] + xS.v, runP = xP.m * carP[w] + xP.v;
                carS[w] = totS.m * carS[w] + totS.v;
                carP[w] = totP.m * carP[w] + totP.v;
                double oS[R], oP[R];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    runS += vs[i];
                    runP = m[i] * runP + vp[i];
                    oS[i] = runS;
                    oP[i] = runP;
                }
                double c[R];
                from_runs(oP, c);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const int64_t r = base + i * kGramScanThreads + tid;
                    if (r < n) st[r * SR + 3 * w] = c[i];
                }
                from_runs(oS, c);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const int64_t r = base + i * kGramScanThreads + tid;
                    if (r < n) st[r * SR + 3 * w + 1] = c[i];
                }
            }
        }
        return;
    }

    // ---- backward: Q_r = e^{-2 (s_{r+1} - s_r)} Q_{r+1} + q_r, rounds from the top
    double carQ[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) carQ[w] = 0.0;
    const int64_t rounds = (n + kRound - 1) / kRound;
#pragma unroll 1
    for (int64_t rd = rounds - 1; rd >= 0; --rd) {
        const int64_t base = rd * kRound;
        double cq[NW][R], cm[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t r = base + i * kGramScanThreads + tid;
            const int64_t rc = r < n ? r : 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) cq[w][i] = r < n ? G.q[w * n + rc] : 0.0;
            cm[i] = r + 1 < n ? G.mdec[r + 1] : (r + 1 == n ? 0.0 : 1.0);
        }
        double m1[R];
        to_runs(cm, m1);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            double vq[R];
            to_runs(cq[w], vq);
            Aff<double> Q = aff_identity<double>();
#pragma unroll
            for (int i = R - 1; i >= 0; --i) Q = compose(Q, Aff<double>{m1[i], vq[i]});
            Aff<double> totQ;
            const Aff<double> xQ = block_exscan_down<double, kWaves>(Q, sh, totQ);
            double runQ = xQ.m * carQ[w] + xQ.v;
            carQ[w] = totQ.m * carQ[w] + totQ.v;
            double oQ[R];
#pragma unroll
            for (int i = R - 1; i >= 0; --i) {
                runQ = m1[i] * runQ + vq[i];
                oQ[i] = runQ;
            }
            double c[R];
            from_runs(oQ, c);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t r = base + i * kGramScanThreads + tid;
                if (r < n) st[r * SR + 3 * w + 2] = c[i];
            }
        }
    }
}

// rank[perm[r]] = r: the rank of each original index.
__global__ __launch_bounds__(256) void lx_gram_ranks(const uint32_t* __restrict__ perm, int64_t n,
                                                    uint32_t* __restrict__ rank)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r < n) rank[perm[r]] = (uint32_t)r;
}

hipError_t gram_ranks_launch(const uint32_t* perm, int64_t n, uint32_t* rank, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    LX_LAUNCH("gram_ranks", s, (lx_gram_ranks<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(perm, n, rank)));
    return hipSuccess;
}

// Tiles of M, 64 x 64 entries in the original order.  Thread (column jj,
// row group) computes column jj of 16 rows and stores a wave's 64 columns
// of one row at once.  The stats of a row or column come by its rank (the
// rank of each original index is kept with the plan).  With lo / hi the
// entry's smaller / larger anchor,
//   M = e^{-(hi - lo)/t} (P_lo + (S_hi - S_lo) + Q_hi)
// (weight sets combined with the cos/sin of phi when phased).  The decay
// is split into per-anchor factors, e^{-(hi - lo)/t} = E+_lo E-_hi: about
// the centre of all the anchors when their span allows (the factors then
// come with the stats), else about the tile's own centre when its anchors
// span at most 600 t (one exp per anchor per tile); otherwise, and at
// t = 0, each entry takes its own decay.  (The sum keeps S_hi - S_lo as one
// difference, exact for equal anchors, so small entries next to a large S
// keep their precision.)
template <int NW>
__global__ __launch_bounds__(256) void lx_gram_tile(GramArgs A, const double* __restrict__ st)
{
    const int64_t n = A.n;
    const double inv_t = A.inv_t;
    float* __restrict__ M = A.M;
    constexpr int SR = gram_srow<NW>();
    constexpr int FW = 3 + 3 * NW + (NW == 3 ? 2 : 0);  // a, E+, E-, (P, S, Q) per set, (cos, sin)
    __shared__ __align__(16) double fr[2][kGT][FW + (FW & 1)];  // [rows, columns][anchor][term]
    __shared__ float sred[4][2];
    const int tid = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.y * kGT, j0 = (int64_t)blockIdx.x * kGT;
    double centre;
    const bool global_f = gram_global_factors(A.sa, n, inv_t, &centre);
    // the stats of the tile's 64 rows and 64 columns, by rank
    for (int t = tid; t < 2 * kGT; t += 256) {
        const int e = t % kGT, side = t / kGT;
        const int64_t i = (side ? j0 : i0) + e;
        double* f = fr[side][e];
        if (i < n) {
            const uint32_t r = A.rank_a[i];
            const double* x = st + (int64_t)r * SR;
            f[0] = (double)A.sa[r];
            f[1] = x[3 * NW];  // the global factors (made when global_f)
            f[2] = x[3 * NW + 1];
#pragma unroll
            for (int q = 0; q < 3 * NW; ++q) f[3 + q] = x[q];
            if (NW == 3) {
                f[FW - 2] = A.cphi_r[r];
                f[FW - 1] = A.sphi_r[r];
            }
        } else {
#pragma unroll
            for (int q = 0; q < FW; ++q) f[q] = 0.0;
        }
    }
    __syncthreads();
    bool factored = global_f;
    if (!global_f) {
        // the tile's anchor range (valid rows and columns only), for its centre
        float mn = INFINITY, mx = -INFINITY;
        if (tid < 2 * kGT) {
            const int e = tid % kGT, side = tid / kGT;
            if ((side ? j0 : i0) + e < n) mn = mx = (float)fr[side][e][0];
        }
        for (int d = 32; d > 0; d >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, d));
            mx = fmaxf(mx, __shfl_xor(mx, d));
        }
        if (lane_id() == 0) {
            sred[tid / kWave][0] = mn;
            sred[tid / kWave][1] = mx;
        }
        __syncthreads();
        const double lo_a = fmin(sred[0][0], sred[1][0]), hi_a = fmax(sred[0][1], sred[1][1]);
        const double tc = 0.5 * (lo_a + hi_a);
        // factors only when every |a - c|/t stays far from overflow (and t > 0)
        factored = inv_t <= 1.0e300 && (hi_a - lo_a) * inv_t <= 600.0;
        if (factored) {
            if (tid < 2 * kGT) {
                double* f = fr[tid / kGT][tid % kGT];
                const double xe = (f[0] - tc) * inv_t;
                f[1] = exp(xe);
                f[2] = exp(-xe);
            }
            __syncthreads();
        }
    }
    const int jj = tid % kGT;
    const int64_t j = j0 + jj;
    if (factored) {
        double cf[FW];
#pragma unroll
        for (int q = 0; q < FW; ++q) cf[q] = fr[1][jj][q];
#pragma unroll 4
        for (int ii = tid / kGT; ii < kGT; ii += 256 / kGT) {
            const int64_t i = i0 + ii;
            // the row's terms, the same for the whole wave (broadcast reads),
            // read as 16-byte pairs: a single 8-byte read feeding one arm of
            // the per-lane choice below is moved into that arm by the
            // compiler, a divergent branch with its own LDS wait
            double rf[FW + (FW & 1)];
#pragma unroll
            for (int q = 0; q < (FW + 1) / 2; ++q) {
                const double2 v = reinterpret_cast<const double2*>(fr[0][ii])[q];
                rf[2 * q] = v.x;
                rf[2 * q + 1] = v.y;
            }
            const bool row_first = rf[0] <= cf[0];
            // stats of lo and hi: P, S, Q of weight set w at 3 + 3 w .. 5 + 3 w
            double g[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const double p_lo = row_first ? rf[3 + 3 * w] : cf[3 + 3 * w];
                const double s_lo = row_first ? rf[4 + 3 * w] : cf[4 + 3 * w];
                const double s_hi = row_first ? cf[4 + 3 * w] : rf[4 + 3 * w];
                const double q_hi = row_first ? cf[5 + 3 * w] : rf[5 + 3 * w];
                g[w] = p_lo + (s_hi - s_lo) + q_hi;
            }
            const double dec = row_first ? rf[1] * cf[2] : cf[1] * rf[2];
            double val;
            if (NW == 3) {
                const double ci = rf[FW - 2], si = rf[FW - 1], cj = cf[FW - 2], sj = cf[FW - 1];
                val = ci * cj * g[0] + (ci * sj + si * cj) * g[NW > 1 ? 1 : 0] + si * sj * g[NW - 1];
            } else {
                val = g[0];
            }
            if (i < n && j < n) M[i * n + j] = (float)(dec * val);
        }
        return;
    }
#pragma unroll 4
    for (int ii = tid / kGT; ii < kGT; ii += 256 / kGT) {
        const int64_t i = i0 + ii;
        if (i < n && j < n) {
            // lo: the smaller anchor (equal anchors carry equal stats)
            const bool row_first = fr[0][ii][0] <= fr[1][jj][0];
            const double* lo = row_first ? fr[0][ii] : fr[1][jj];
            const double* hi = row_first ? fr[1][jj] : fr[0][ii];
            double g[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) g[w] = lo[3 + 3 * w] + (hi[4 + 3 * w] - lo[4 + 3 * w]) + hi[5 + 3 * w];
            double val;
            if (NW == 3) {
                const double ci = fr[0][ii][FW - 2], si = fr[0][ii][FW - 1];
                const double cj = fr[1][jj][FW - 2], sj = fr[1][jj][FW - 1];
                val = ci * cj * g[0] + (ci * sj + si * cj) * g[NW > 1 ? 1 : 0] + si * sj * g[NW - 1];
            } else {
                val = g[0];
            }
            M[i * n + j] = (float)(decay_dist(hi[0] - lo[0], inv_t) * val);
        }
    }
}

template <int NW>
static hipError_t gram_launch_t(const GramArgs& a, hipStream_t s)
{
    const GramScratch G = gram_scratch_at(a.stats, a.n, NW);
    const int64_t groups = (a.n + 1 + kBinWaves - 1) / kBinWaves;
    LX_LAUNCH("gram_bins", s, (lx_gram_bins<NW><<<(unsigned)(groups * kGramSlices), kBinThreads, 0, s>>>(a, G)));
    const int64_t fold = 3 * NW * (a.n + 1);
    LX_LAUNCH("gram_fold", s, (lx_gram_fold<NW><<<(unsigned)((fold + 255) / 256), 256, 0, s>>>(a.sa, a.inv_t, a.n, G)));
    LX_LAUNCH("gram_scan", s, (lx_gram_scan<NW><<<2, kGramScanThreads, 0, s>>>(a, G)));
    const unsigned nb = (unsigned)((a.n + kGT - 1) / kGT);
    LX_LAUNCH("gram_tile", s, (lx_gram_tile<NW><<<dim3(nb, nb), 256, 0, s>>>(a, G.st)));
    return hipSuccess;
}

hipError_t gram_launch(const GramArgs& a, hipStream_t s)
{
    if (a.n <= 0 || a.k <= 0) return hipSuccess;
    return a.cpsi_r ? gram_launch_t<3>(a, s) : gram_launch_t<1>(a, s);
}

}  // namespace lx
