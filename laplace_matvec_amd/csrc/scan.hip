// Prefix and suffix scans along a sorted anchor set (gfx950).
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2:
// after sorting, the lower-triangular product obeys
//     L_r = x_r + exp(s_{r-1} - s_r) L_{r-1}
// and the upper part the mirrored recurrence
//     U_r = x_r + exp(s_r - s_{r+1}) U_{r+1},
// each O(n) work and O(log n) depth as a scan of affine maps.  Both parts
// contain the diagonal, so the symmetric product is L + U - x.  For a != b
// the values are the interval sums u (forward) and v (backward) and the
// product is L + R.  The "evaluate" path keeps L and U apart (PL, PR).
//
// Three launches (reduce-then-scan; every workgroup runs to completion
// without waiting on another, and the combine tree is fixed, so results are
// deterministic):
//   lx_scan_reduce : per tile of 4096 ranks and per vector, the composite
//                    affine map of the tile in both directions.  In the
//                    gathering modes it also reads x through the permutation
//                    (x[perm[r]]) and stores the sorted copy xs.
//   lx_scan_carry  : per vector, an exclusive scan of the tile composites in
//                    both directions -> the value entering each tile.
//   lx_scan_apply  : per tile and vector, the final recurrences from the
//                    carries; writes y[perm[r]] (scatter back to the original
//                    order) or the sorted PL/PR tables.
// Arithmetic is float64 (storage stays float32): the decay factors and the
// recurrence would otherwise accumulate the rounding of exp(-gap), which is
// the same for every equal gap.  Layout: vectors [batch][n]; channels (the
// cos/sin split of a phased operator) outermost.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kScanItems = 16;
static_assert(kScanThreads * kScanItems == kScanTile, "scan tile size");

// Loads p[r0 .. r0+N) (zero past n) with 16-byte loads when the run is whole.
template <int N, class T>
__device__ __forceinline__ void load_run(const T* __restrict__ p, int64_t r0, int64_t n, T (&out)[N])
{
    static_assert(sizeof(T) == 4 && N % 4 == 0, "run of 32-bit values");
    if (r0 + N <= n) {
        const uint4* q = reinterpret_cast<const uint4*>(p + r0);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const uint4 t = q[i];
            out[4 * i + 0] = __builtin_bit_cast(T, t.x);
            out[4 * i + 1] = __builtin_bit_cast(T, t.y);
            out[4 * i + 2] = __builtin_bit_cast(T, t.z);
            out[4 * i + 3] = __builtin_bit_cast(T, t.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = (r0 + i < n) ? p[r0 + i] : T(0);
    }
}

template <int N>
__device__ __forceinline__ void store_run(float* __restrict__ p, int64_t r0, int64_t n, const float (&v)[N])
{
    if (r0 + N <= n) {
        float4* q = reinterpret_cast<float4*>(p + r0);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (r0 + i < n) p[r0 + i] = v[i];
    }
}

// e[i] = exp(s[r0-1+i] - s[r0+i]), i = 0..N: the decay between consecutive
// ranks around this thread's run.  e[i] multiplies the forward carry into
// rank r0+i, e[i+1] the backward carry into rank r0+i.  Missing neighbours
// (before rank 0, after rank n-1) give 0, which cuts the chain there.
template <int N>
__device__ __forceinline__ void load_decays(const float* __restrict__ s, int64_t r0, int64_t n, double (&e)[N + 1])
{
    float mid[N];
    load_run<N>(s, r0, n, mid);
    const float left = (r0 > 0 && r0 - 1 < n) ? s[r0 - 1] : 0.f;
    const float right = (r0 + N < n) ? s[r0 + N] : 0.f;
    e[0] = (r0 > 0 && r0 < n) ? decay(left, mid[0]) : 0.0;
#pragma unroll
    for (int i = 1; i < N; ++i) e[i] = (r0 + i < n) ? decay(mid[i - 1], mid[i]) : 0.0;
    e[N] = (r0 + N < n) ? decay(mid[N - 1], right) : 0.0;
}

__device__ __forceinline__ int64_t row_off(const ScanArgs& A, int c, int64_t vec)
{
    return ((int64_t)c * A.batch + vec) * A.ld;
}

template <int C, int MODE>
__global__ __launch_bounds__(kScanThreads) void lx_scan_reduce(ScanArgs A)
{
    __shared__ Aff<double> sh[kScanWaves];
    const int64_t vec = blockIdx.x / A.tiles;
    const int64_t tile = blockIdx.x - vec * A.tiles;
    const int64_t n = A.n;
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kScanItems;

    double e[kScanItems + 1];
    load_decays<kScanItems>(A.s, r0, n, e);

    float fv[C][kScanItems];  // forward values
    float bv[C][kScanItems];  // backward values (same as forward unless UV)
    if (MODE == kScanUV) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            load_run<kScanItems>(A.u + row_off(A, c, vec), r0, n, fv[c]);
            load_run<kScanItems>(A.v + row_off(A, c, vec), r0, n, bv[c]);
        }
    } else {
        uint32_t idx[kScanItems];
        load_run<kScanItems>(A.perm, r0, n, idx);
        const float* xv = A.x + vec * n;
        float g[kScanItems];
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) g[i] = (r0 + i < n) ? xv[idx[i]] : 0.f;
        if (C == 2) {
            float fc[kScanItems], fs[kScanItems];
            load_run<kScanItems>(A.in_c, r0, n, fc);
            load_run<kScanItems>(A.in_s, r0, n, fs);
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) {
                fv[0][i] = fc[i] * g[i];
                fv[C - 1][i] = fs[i] * g[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) fv[0][i] = g[i];
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            store_run<kScanItems>(A.xs + row_off(A, c, vec), r0, n, fv[c]);
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) bv[c][i] = fv[c][i];
        }
    }

#pragma unroll
    for (int c = 0; c < C; ++c) {
        Aff<double> f = aff_identity<double>();
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) f = compose(f, Aff<double>{e[i], (double)fv[c][i]});
        Aff<double> b = aff_identity<double>();
#pragma unroll
        for (int i = kScanItems - 1; i >= 0; --i) b = compose(b, Aff<double>{e[i + 1], (double)bv[c][i]});
        Aff<double> ft, bt;
        (void)block_exscan_up<double, kScanWaves>(f, sh, ft);
        (void)block_exscan_down<double, kScanWaves>(b, sh, bt);
        if (threadIdx.x == 0) {
            double* ag = A.agg + ((((int64_t)c * A.batch + vec) * A.tiles) + tile) * 4;
            ag[0] = ft.m;
            ag[1] = ft.v;
            ag[2] = bt.m;
            ag[3] = bt.v;
        }
    }
}

constexpr int kCarryThreads = 1024;

__global__ __launch_bounds__(kCarryThreads) void lx_scan_carry(const double* __restrict__ agg,
                                                              double* __restrict__ carry, int64_t T)
{
    __shared__ Aff<double> sh[kCarryThreads / kWave];
    const int64_t row = blockIdx.x;
    const double* ag = agg + row * T * 4;
    double* ca = carry + row * T * 2;
    const int64_t per = (T + kCarryThreads - 1) / kCarryThreads;
    int64_t t0 = (int64_t)threadIdx.x * per;
    if (t0 > T) t0 = T;
    int64_t t1 = t0 + per;
    if (t1 > T) t1 = T;

    Aff<double> f = aff_identity<double>();
    for (int64_t t = t0; t < t1; ++t) f = compose(f, Aff<double>{ag[4 * t], ag[4 * t + 1]});
    Aff<double> tot;
    Aff<double> run = block_exscan_up<double, kCarryThreads / kWave>(f, sh, tot);
    for (int64_t t = t0; t < t1; ++t) {
        ca[2 * t] = run.v;  // value entering tile t from the left (start value 0)
        run = compose(run, Aff<double>{ag[4 * t], ag[4 * t + 1]});
    }

    Aff<double> b = aff_identity<double>();
    for (int64_t t = t1 - 1; t >= t0; --t) b = compose(b, Aff<double>{ag[4 * t + 2], ag[4 * t + 3]});
    run = block_exscan_down<double, kCarryThreads / kWave>(b, sh, tot);
    for (int64_t t = t1 - 1; t >= t0; --t) {
        ca[2 * t + 1] = run.v;  // value entering tile t from the right
        run = compose(run, Aff<double>{ag[4 * t + 2], ag[4 * t + 3]});
    }
}

template <int C, int MODE>
__global__ __launch_bounds__(kScanThreads) void lx_scan_apply(ScanArgs A)
{
    __shared__ Aff<double> sh[kScanWaves];
    const int64_t vec = blockIdx.x / A.tiles;
    const int64_t tile = blockIdx.x - vec * A.tiles;
    const int64_t n = A.n;
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kScanItems;

    double e[kScanItems + 1];
    load_decays<kScanItems>(A.s, r0, n, e);

    float out[kScanItems];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) out[i] = 0.f;

#pragma unroll
    for (int c = 0; c < C; ++c) {
        float fv[kScanItems], bv[kScanItems];
        if (MODE == kScanUV) {
            load_run<kScanItems>(A.u + row_off(A, c, vec), r0, n, fv);
            load_run<kScanItems>(A.v + row_off(A, c, vec), r0, n, bv);
        } else {
            load_run<kScanItems>(A.xs + row_off(A, c, vec), r0, n, fv);
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) bv[i] = fv[i];
        }
        Aff<double> f = aff_identity<double>();
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) f = compose(f, Aff<double>{e[i], (double)fv[i]});
        Aff<double> b = aff_identity<double>();
#pragma unroll
        for (int i = kScanItems - 1; i >= 0; --i) b = compose(b, Aff<double>{e[i + 1], (double)bv[i]});
        Aff<double> tot;
        const Aff<double> fx = block_exscan_up<double, kScanWaves>(f, sh, tot);
        const Aff<double> bx = block_exscan_down<double, kScanWaves>(b, sh, tot);
        const double* cr = A.carry + ((((int64_t)c * A.batch + vec) * A.tiles) + tile) * 2;
        double L = fx.m * cr[0] + fx.v;
        double U = bx.m * cr[1] + bx.v;
        double Lr[kScanItems];
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            L = e[i] * L + (double)fv[i];
            Lr[i] = L;
        }
        if (MODE == kScanPLPR) {
            float pl[kScanItems], pr[kScanItems];
#pragma unroll
            for (int i = kScanItems - 1; i >= 0; --i) {
                U = e[i + 1] * U + (double)bv[i];
                pl[i] = (float)Lr[i];
                pr[i] = (float)U;
            }
            store_run<kScanItems>(A.pl + row_off(A, c, vec), r0, n, pl);
            store_run<kScanItems>(A.pr + row_off(A, c, vec), r0, n, pr);
        } else {
            float g[kScanItems];
            if (C == 2) load_run<kScanItems>(c == 0 ? A.out_c : A.out_s, r0, n, g);
#pragma unroll
            for (int i = kScanItems - 1; i >= 0; --i) {
                U = e[i + 1] * U + (double)bv[i];
                const double y = (MODE == kScanSym) ? Lr[i] + U - (double)fv[i] : Lr[i] + U;
                out[i] = (C == 2) ? fmaf(g[i], (float)y, out[i]) : (float)y;
            }
        }
    }
    if (MODE != kScanPLPR) {
        uint32_t idx[kScanItems];
        load_run<kScanItems>(A.perm, r0, n, idx);
        float* yv = A.y + vec * n;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i)
            if (r0 + i < n) yv[idx[i]] = out[i];
    }
}

template <int C, int MODE>
static hipError_t scan_launch_t(const ScanArgs& a, hipStream_t s)
{
    const int64_t blocks = a.tiles * a.batch;
    LX_LAUNCH(MODE == kScanUV ? "scan_reduce_uv" : "scan_reduce_gather", s,
              (lx_scan_reduce<C, MODE><<<(unsigned)blocks, kScanThreads, 0, s>>>(a)));
    LX_LAUNCH("scan_carry", s,
              (lx_scan_carry<<<(unsigned)(a.channels * a.batch), kCarryThreads, 0, s>>>(a.agg, a.carry, a.tiles)));
    LX_LAUNCH(MODE == kScanPLPR ? "scan_apply_tables" : "scan_apply_scatter", s,
              (lx_scan_apply<C, MODE><<<(unsigned)blocks, kScanThreads, 0, s>>>(a)));
    return hipSuccess;
}

hipError_t scan_launch(const ScanArgs& a, hipStream_t s)
{
    if (a.n <= 0 || a.batch <= 0) return hipSuccess;
    if (a.tiles * a.batch > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const bool two = a.channels == 2;
    switch (a.mode) {
        case kScanSym: return two ? scan_launch_t<2, kScanSym>(a, s) : scan_launch_t<1, kScanSym>(a, s);
        case kScanUV: return two ? scan_launch_t<2, kScanUV>(a, s) : scan_launch_t<1, kScanUV>(a, s);
        case kScanPLPR: return two ? scan_launch_t<2, kScanPLPR>(a, s) : scan_launch_t<1, kScanPLPR>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lx
