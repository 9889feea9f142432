// Small symmetric plans in one workgroup (gfx950).
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2:
// sort the anchors, then the prefix and suffix recurrences give the product
// as L + U - x.  For n <= 8192 anchors the whole plan -- the stable sort,
// the permutation, the phase factors by rank and, with x, y = K x -- fits
// in one workgroup's LDS and registers, so one launch replaces the sixteen
// or so of the large path, whose cost at such sizes is launch latency.
//
//   sort : four stable LSD passes of 8-bit digits inside LDS (keys and
//          original indices), ranked with wave64 ballots like the large
//          radix passes, without any look-back (one tile);
//   plan : sorted anchors, the permutation, cos/sin of the phases by rank
//          (float64 sincos rounded once), a flag for NaN/Inf;
//   scan : 1024 threads x 8 consecutive ranks, float64 decays and
//          recurrences, block scans across the 16 waves, y scattered
//          through the permutation.
// Every combine order is fixed, so results are deterministic.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;  // 16
constexpr int kSmallItems = kSmallMax / kSmallThreads;  // 8
constexpr int kSmallRadix = 256;
static_assert(kSmallThreads * kSmallItems == kSmallMax, "small plan size");

// ITEMS keys per thread: 8 covers kSmallMax anchors, 4 covers up to 4096
// with half the ranking and scan work.
template <int ITEMS>
__global__ __launch_bounds__(kSmallThreads) void lx_small_sym(SmallSymArgs A)
{
    __shared__ uint32_t s_key[kSmallMax];
    __shared__ uint16_t s_idx[kSmallMax];
    __shared__ uint16_t s_hist[kSmallWaves][kSmallRadix];  // per-wave counts, then slot of each wave's first key
    __shared__ uint32_t s_red[kSmallWaves];
    __shared__ Aff<double> s_aff[kSmallWaves];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / kWave;
    const int n = (int)A.n;
    const int wpos = w * (ITEMS * kWave);

    // Keys in wave-striped order (item j of lane l is position wpos + 64 j +
    // l), so a wave's items in (j, lane) order are its keys in index order;
    // positions past n take the largest key and rank last.
    uint32_t key[ITEMS], idx[ITEMS];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int p = wpos + j * kWave + lane;
        idx[j] = (uint32_t)p;
        const float f = p < n ? A.a[p] : 0.f;
        bad |= p < n && !finite_bits(f);
        key[j] = p < n ? key_of(f) : 0xFFFFFFFFu;
    }
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 8 * pass;
        if (pass > 0) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const int p = wpos + j * kWave + lane;
                key[j] = s_key[p];
                idx[j] = s_idx[p];
            }
        }
        for (int i = tid; i < kSmallWaves * kSmallRadix; i += kSmallThreads) (&s_hist[0][0])[i] = 0;
        __syncthreads();  // also: every item of the previous order has been read
        uint32_t pos[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t d = (key[j] >> shift) & 0xFFu;
            const uint64_t peers = match_digit8(d);
            const uint32_t below = count_below(peers);
            const uint32_t prev = s_hist[w][d];
            pos[j] = prev + below;
            if (below == 0) s_hist[w][d] = (uint16_t)(prev + (uint32_t)__popcll(peers));
        }
        __syncthreads();
        uint32_t count = 0;
        if (tid < kSmallRadix) {
            uint32_t run = 0;
#pragma unroll
            for (int i = 0; i < kSmallWaves; ++i) {
                const uint32_t c = s_hist[i][tid];
                s_hist[i][tid] = (uint16_t)run;
                run += c;
            }
            count = run;
        }
        uint32_t total;
        const uint32_t start = block_exsum_u32<kSmallWaves>(tid < kSmallRadix ? count : 0u, s_red, total);
        if (tid < kSmallRadix) {
#pragma unroll
            for (int i = 0; i < kSmallWaves; ++i) s_hist[i][tid] = (uint16_t)(s_hist[i][tid] + start);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t dst = s_hist[w][(key[j] >> shift) & 0xFFu] + pos[j];
            s_key[dst] = key[j];
            s_idx[dst] = (uint16_t)idx[j];
        }
        __syncthreads();
    }

    // This thread's ranks r0 .. r0+7: the plan's arrays, the phase factors.
    const int r0 = tid * ITEMS;
    float ci[ITEMS], si[ITEMS], co[ITEMS], so[ITEMS];  // input (psi), output (phi)
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int r = r0 + i;
        ci[i] = co[i] = 1.f;
        si[i] = so[i] = 0.f;
        if (r < n) {
            const uint32_t p = s_idx[r];
            A.sa[r] = float_of_key(s_key[r]);
            A.perm[r] = p;
            if (A.phi) {
                const float fp = A.phi[p], fq = A.psi[p];
                bad |= !finite_bits(fp) || !finite_bits(fq);
                double sd, cd;
                sincos((double)fp, &sd, &cd);
                co[i] = (float)cd;
                so[i] = (float)sd;
                sincos((double)fq, &sd, &cd);
                ci[i] = (float)cd;
                si[i] = (float)sd;
                A.cphi[r] = co[i];
                A.sphi[r] = so[i];
                A.cpsi[r] = ci[i];
                A.spsi[r] = si[i];
            }
        }
    }
    // the flag word is written here, whole: no clear is needed before
    const int any_bad = __syncthreads_or(bad ? 1 : 0);
    if (tid == 0) *A.flag = any_bad ? 1u : 0u;
    if (A.x == nullptr) return;  // uniform: a plan without a product
    // the plan's own copy of x (original order) for a later backward
    if (A.x_keep)
        for (int64_t i = tid; i < (int64_t)A.batch * n; i += kSmallThreads) A.x_keep[i] = A.x[i];

    // decays between neighbouring ranks; 0 before rank 0 and from rank n on
    double e[ITEMS + 1];
    {
        float s[ITEMS + 2];
#pragma unroll
        for (int i = 0; i < ITEMS + 2; ++i) {
            const int r = r0 - 1 + i;
            s[i] = (r >= 0 && r < n) ? float_of_key(s_key[r]) : 0.f;
        }
#pragma unroll
        for (int i = 0; i <= ITEMS; ++i) {
            const int r = r0 + i;  // e[i] joins ranks r - 1 and r
            e[i] = (r > 0 && r < n) ? decay(s[i], s[i + 1], A.inv_t) : 0.0;
        }
    }
    const int C = A.phi ? 2 : 1;
    for (int v = 0; v < A.batch; ++v) {  // uniform loops: every thread takes part in the scans
        const float* xv = A.x + (int64_t)v * n;
        float out[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) out[i] = 0.f;
        for (int c = 0; c < C; ++c) {
            float val[ITEMS];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const int r = r0 + i;
                const float xr = r < n ? xv[s_idx[r]] : 0.f;
                val[i] = C == 2 ? (c == 0 ? ci[i] : si[i]) * xr : xr;
            }
            Aff<double> f = aff_identity<double>(), b = aff_identity<double>();
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) f = compose(f, Aff<double>{e[i], (double)val[i]});
#pragma unroll
            for (int i = ITEMS - 1; i >= 0; --i) b = compose(b, Aff<double>{e[i + 1], (double)val[i]});
            const Aff<double> fx = block_exscan_up_lean<double, kSmallWaves>(f, s_aff);
            const Aff<double> bx = block_exscan_down_lean<double, kSmallWaves>(b, s_aff);
            double Lr[ITEMS];
            double L = fx.v;
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                L = e[i] * L + (double)val[i];
                Lr[i] = L;
            }
            double U = bx.v;
#pragma unroll
            for (int i = ITEMS - 1; i >= 0; --i) {
                U = e[i + 1] * U + (double)val[i];
                const float yc = (float)(Lr[i] + U - (double)val[i]);
                out[i] = C == 2 ? fmaf(c == 0 ? co[i] : so[i], yc, out[i]) : yc;
            }
        }
        float* yv = A.y + (int64_t)v * n;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
            if (r0 + i < n) yv[s_idx[r0 + i]] = out[i];
    }
}

}  // namespace

hipError_t small_sym_launch(const SmallSymArgs& a, hipStream_t s)
{
    if (a.n < 1 || a.n > kSmallMax || a.flag == nullptr) return hipErrorInvalidValue;
    if (a.n <= kSmallThreads * 4) LX_LAUNCH("small_sym", s, (lx_small_sym<4><<<1, kSmallThreads, 0, s>>>(a)));
    else LX_LAUNCH("small_sym", s, (lx_small_sym<8><<<1, kSmallThreads, 0, s>>>(a)));
    return hipSuccess;
}

}  // namespace lx
