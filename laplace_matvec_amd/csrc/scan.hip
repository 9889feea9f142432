// Prefix and suffix scans along a sorted anchor set (gfx950).
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2:
// after sorting, the lower-triangular product obeys
//     L_r = x_r + exp(s_{r-1} - s_r) L_{r-1}
// (at temperature t the exponent is divided by t)
// and the upper part the mirrored recurrence
//     U_r = x_r + exp(s_r - s_{r+1}) U_{r+1},
// each O(n) work and O(log n) depth as a scan of affine maps.  Both parts
// contain the diagonal, so the symmetric product is L + U - x.  For a != b
// the values are the interval sums u (forward) and v (backward) and the
// product is L + R.  The "evaluate" path keeps L and U apart (PL, PR), and
// the gradient of a small output side keeps L and R apart (UV in, PL/PR out).
//
// Reduce-then-scan (every workgroup runs to completion without waiting on
// another, and the combine tree is fixed, so results are deterministic):
//   lx_scan_reduce : per tile of 4096 ranks and per vector, the composite
//                    affine map of the tile in both directions.  In random
//                    mode it reads x through the permutation (x[perm[r]]) and
//                    stores the copy by rank, xs; otherwise xs was filled by
//                    replaying the sort.
//   lx_scan_carry_*: per vector, exclusive scans of the tile composites in
//                    both directions (two levels) -> the value entering each
//                    tile.
//   lx_scan_apply  : per tile and vector, the final recurrences from the
//                    carries; writes y by rank (ys, replayed back to the
//                    original order afterwards), y[perm[r]] in random mode,
//                    or the PL/PR tables.
// Arithmetic is float64 (storage stays float32): the decay factors and the
// recurrence would otherwise accumulate the rounding of exp(-gap), which is
// the same for every equal gap.  Layout: vectors [batch][n]; channels (the
// cos/sin split of a phased operator) outermost.
#include "lx_device.h"
#include "lx_internal.h"
#include "lx_tile.h"

namespace lx {

__device__ __forceinline__ int64_t row_off(const ScanArgs& A, int c, int64_t vec)
{
    return ((int64_t)c * A.batch + vec) * A.ld;
}

// Values of this thread's ranks for every channel.  Sym/PLPR: one value per
// rank (x[perm[r]] when random, else xs by rank), times cos/sin of the input
// phase for a phased operator.  UV: the u (forward) and v (backward) rows.
template <int C, int MODE, bool RANDOM, bool WRITE_XS>
__device__ __forceinline__ void load_values(const ScanArgs& A, int64_t vec, int64_t r0,
                                            float (&fv)[C][kScanItems], float (&bv)[C][kScanItems])
{
    const int64_t n = A.n;
    if (MODE == kScanUV || MODE == kScanUVLR) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            load_run<kScanItems>(A.u + row_off(A, c, vec), r0, n, fv[c]);
            load_run<kScanItems>(A.v + row_off(A, c, vec), r0, n, bv[c]);
        }
        return;
    }
    float g[kScanItems];
    if (RANDOM) {
        uint32_t idx[kScanItems];
        load_run<kScanItems>(A.perm, r0, n, idx);
        const float* xv = A.x + vec * n;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) g[i] = (r0 + i < n) ? xv[idx[i]] : 0.f;
        if (WRITE_XS) store_run<kScanItems>(A.xs + vec * A.ld, r0, n, g);
    } else {
        load_run<kScanItems>(A.xs + vec * A.ld, r0, n, g);
    }
    if (C == 2) {
        float fc[kScanItems], fs[kScanItems];
        load_run<kScanItems>(A.in_c, r0, n, fc);
        load_run<kScanItems>(A.in_s, r0, n, fs);
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            fv[0][i] = bv[0][i] = fc[i] * g[i];
            fv[C - 1][i] = bv[C - 1][i] = fs[i] * g[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) fv[0][i] = bv[0][i] = g[i];
    }
}

// Vectors per scan workgroup: the decays of a tile are computed once and
// serve every vector of the group.
constexpr int kScanVB = 8;

template <int C, int MODE, bool RANDOM, int VB>
__global__ __launch_bounds__(kScanThreads) void lx_scan_reduce(ScanArgs A)
{
    // wave totals of every (vector, channel) row, both directions; one
    // barrier for the whole group, then one thread per row and direction
    // folds the waves
    __shared__ Aff<double> sh[VB * C][kScanWaves][2];
    const int64_t vg = blockIdx.x / A.tiles;
    const int64_t tile = blockIdx.x - vg * A.tiles;
    const int64_t v0 = vg * VB;
    const int nv = VB == 1 ? 1 : (int)(A.batch - v0 < VB ? A.batch - v0 : VB);
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kScanItems;
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;

    double e[kScanItems + 1];
    load_decays<kScanItems>(A.s, r0, A.n, A.inv_t, e);
#pragma unroll 1
    for (int vi = 0; vi < nv; ++vi) {
        const int64_t vec = v0 + vi;
        float fv[C][kScanItems], bv[C][kScanItems];
        load_values<C, MODE, RANDOM, true>(A, vec, r0, fv, bv);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            Aff<double> f = aff_identity<double>();
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) f = compose(f, Aff<double>{e[i], (double)fv[c][i]});
            Aff<double> b = aff_identity<double>();
#pragma unroll
            for (int i = kScanItems - 1; i >= 0; --i) b = compose(b, Aff<double>{e[i + 1], (double)bv[c][i]});
            const Aff<double> fi = wave_scan_up(f);
            const Aff<double> bi = wave_scan_down(b);
            if (lane == kWave - 1) sh[vi * C + c][w][0] = fi;
            if (lane == 0) sh[vi * C + c][w][1] = bi;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < nv * C * 2) {
        const int row = (int)threadIdx.x / 2, dir = (int)threadIdx.x & 1;
        const int vi = row / C, c = row - vi * C;
        Aff<double> acc = aff_identity<double>();
        if (dir == 0) {
#pragma unroll
            for (int i = 0; i < kScanWaves; ++i) acc = compose(acc, sh[row][i][0]);
        } else {
#pragma unroll
            for (int i = kScanWaves - 1; i >= 0; --i) acc = compose(acc, sh[row][i][1]);
        }
        double* ag = A.agg + ((((int64_t)c * A.batch + v0 + vi) * A.tiles) + tile) * 4;
        ag[2 * dir] = acc.m;
        ag[2 * dir + 1] = acc.v;
    }
}

// Carries in two levels: composites of groups of kCarryGroup tiles, then
// each group rescans its tiles from the fold of the groups before (after) it.
constexpr int kCarryThreads = 256;
constexpr int kCarryPer = kCarryGroup / kCarryThreads;  // 16 tiles per thread

__global__ __launch_bounds__(kCarryThreads) void lx_scan_carry_groups(const double* __restrict__ agg,
                                                                     double* __restrict__ gagg, int64_t T,
                                                                     int64_t G)
{
    __shared__ Aff<double> sh[kCarryThreads / kWave];
    const int64_t row = blockIdx.x / G;
    const int64_t g = blockIdx.x - row * G;
    const double* ag = agg + row * T * 4;
    int64_t t0 = g * kCarryGroup + (int64_t)threadIdx.x * kCarryPer;
    int64_t t1 = t0 + kCarryPer;
    if (t0 > T) t0 = T;
    if (t1 > T) t1 = T;
    Aff<double> f = aff_identity<double>(), b = aff_identity<double>();
    for (int64_t t = t0; t < t1; ++t) f = compose(f, Aff<double>{ag[4 * t], ag[4 * t + 1]});
    for (int64_t t = t1 - 1; t >= t0; --t) b = compose(b, Aff<double>{ag[4 * t + 2], ag[4 * t + 3]});
    Aff<double> ft, bt;
    (void)block_exscan_up<double, kCarryThreads / kWave>(f, sh, ft);
    (void)block_exscan_down<double, kCarryThreads / kWave>(b, sh, bt);
    if (threadIdx.x == 0) {
        double* o = gagg + (row * G + g) * 4;
        o[0] = ft.m;
        o[1] = ft.v;
        o[2] = bt.m;
        o[3] = bt.v;
    }
}

__global__ __launch_bounds__(kCarryThreads) void lx_scan_carry_tiles(const double* __restrict__ agg,
                                                                    const double* __restrict__ gagg,
                                                                    double* __restrict__ carry, int64_t T,
                                                                    int64_t G)
{
    __shared__ Aff<double> sh[kCarryThreads / kWave];
    __shared__ double cin[2];
    const int64_t row = blockIdx.x / G;
    const int64_t g = blockIdx.x - row * G;
    const double* ag = agg + row * T * 4;
    double* ca = carry + row * T * 2;
    if (threadIdx.x == 0) {
        const double* gg = gagg + row * G * 4;
        double lf = 0.0, lb = 0.0;  // values entering the group from the left / right
        for (int64_t q = 0; q < g; ++q) lf = gg[4 * q] * lf + gg[4 * q + 1];
        for (int64_t q = G - 1; q > g; --q) lb = gg[4 * q + 2] * lb + gg[4 * q + 3];
        cin[0] = lf;
        cin[1] = lb;
    }
    int64_t t0 = g * kCarryGroup + (int64_t)threadIdx.x * kCarryPer;
    int64_t t1 = t0 + kCarryPer;
    if (t0 > T) t0 = T;
    if (t1 > T) t1 = T;
    Aff<double> f = aff_identity<double>(), b = aff_identity<double>();
    for (int64_t t = t0; t < t1; ++t) f = compose(f, Aff<double>{ag[4 * t], ag[4 * t + 1]});
    for (int64_t t = t1 - 1; t >= t0; --t) b = compose(b, Aff<double>{ag[4 * t + 2], ag[4 * t + 3]});
    Aff<double> tot;
    const Aff<double> fx = block_exscan_up<double, kCarryThreads / kWave>(f, sh, tot);
    const Aff<double> bx = block_exscan_down<double, kCarryThreads / kWave>(b, sh, tot);
    double lv = fx.m * cin[0] + fx.v;
    for (int64_t t = t0; t < t1; ++t) {
        ca[2 * t] = lv;  // value entering tile t from the left
        lv = ag[4 * t] * lv + ag[4 * t + 1];
    }
    double rv = bx.m * cin[1] + bx.v;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        ca[2 * t + 1] = rv;  // value entering tile t from the right
        rv = ag[4 * t + 2] * rv + ag[4 * t + 3];
    }
}

// Exclusive block scans of one forward and one backward row with one
// barrier: wave scans, wave totals in LDS, then each wave folds the waves
// before (after) it.  `sh` holds two buffers used in turns (`parity`), so
// the next call can write without a second barrier.
__device__ __forceinline__ void block_exscan2(Aff<double> f, Aff<double> b, Aff<double>* sh, int parity,
                                              Aff<double>& xf, Aff<double>& xb)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    Aff<double>* buf = sh + parity * (kScanWaves * 2);
    const Aff<double> fi = wave_scan_up(f);
    const Aff<double> bi = wave_scan_down(b);
    const Aff<double> ef = wave_shift_up(fi);
    const Aff<double> eb = wave_shift_down(bi);
    if (lane == kWave - 1) buf[w * 2] = fi;
    if (lane == 0) buf[w * 2 + 1] = bi;
    __syncthreads();
    Aff<double> pf = aff_identity<double>(), pb = aff_identity<double>();
#pragma unroll
    for (int i = 0; i < kScanWaves; ++i)
        if (i < w) pf = compose(pf, buf[i * 2]);
#pragma unroll
    for (int i = kScanWaves - 1; i >= 0; --i)
        if (i > w) pb = compose(pb, buf[i * 2 + 1]);
    xf = compose(pf, ef);
    xb = compose(pb, eb);
}

template <int C, int MODE, bool RANDOM, int VB>
__global__ __launch_bounds__(kScanThreads) void lx_scan_apply(ScanArgs A)
{
    __shared__ Aff<double> sh[2 * kScanWaves * 2];
    int parity = 0;
    const int64_t vg = blockIdx.x / A.tiles;
    const int64_t tile = blockIdx.x - vg * A.tiles;
    const int64_t v0 = vg * VB;
    const int nv = VB == 1 ? 1 : (int)(A.batch - v0 < VB ? A.batch - v0 : VB);
    const int64_t n = A.n;
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kScanItems;

    double e[kScanItems + 1];
    load_decays<kScanItems>(A.s, r0, n, A.inv_t, e);
#pragma unroll 1
    for (int vi = 0; vi < nv; ++vi) {
        const int64_t vec = v0 + vi;
        float fv[C][kScanItems], bv[C][kScanItems];
        // the reduce step already stored x by rank: read it back
        load_values<C, MODE, false, false>(A, vec, r0, fv, bv);

        float out[kScanItems];
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) out[i] = 0.f;

#pragma unroll
        for (int c = 0; c < C; ++c) {
            Aff<double> f = aff_identity<double>();
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) f = compose(f, Aff<double>{e[i], (double)fv[c][i]});
            Aff<double> b = aff_identity<double>();
#pragma unroll
            for (int i = kScanItems - 1; i >= 0; --i) b = compose(b, Aff<double>{e[i + 1], (double)bv[c][i]});
            Aff<double> fx, bx;
            block_exscan2(f, b, sh, parity, fx, bx);
            parity ^= 1;
            const double* cr = A.carry + ((((int64_t)c * A.batch + vec) * A.tiles) + tile) * 2;
            double L = fx.m * cr[0] + fx.v;
            double U = bx.m * cr[1] + bx.v;
            double Lr[kScanItems];
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) {
                L = e[i] * L + (double)fv[c][i];
                Lr[i] = L;
            }
            if (MODE == kScanPLPR || MODE == kScanUVLR) {
                float pl[kScanItems], pr[kScanItems];
#pragma unroll
                for (int i = kScanItems - 1; i >= 0; --i) {
                    U = e[i + 1] * U + (double)bv[c][i];
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
                    U = e[i + 1] * U + (double)bv[c][i];
                    const double y = (MODE == kScanSym) ? Lr[i] + U - (double)fv[c][i] : Lr[i] + U;
                    out[i] = (C == 2) ? fmaf(g[i], (float)y, out[i]) : (float)y;
                }
            }
        }
        if (MODE != kScanPLPR && MODE != kScanUVLR) {
            if (RANDOM) {
                uint32_t idx[kScanItems];
                load_run<kScanItems>(A.perm, r0, n, idx);
                float* yv = A.y + vec * n;
#pragma unroll
                for (int i = 0; i < kScanItems; ++i)
                    if (r0 + i < n) yv[idx[i]] = out[i];
            } else {
                store_run<kScanItems>(A.ys + vec * A.ld, r0, n, out);
            }
        }
    }
}

hipError_t scan_carry_launch(const double* agg, double* gagg, double* carry, int64_t tiles, int64_t rows,
                             hipStream_t s)
{
    const int64_t G = (tiles + kCarryGroup - 1) / kCarryGroup;
    const unsigned cb = (unsigned)(rows * G);
    LX_LAUNCH("scan_carry", s, (lx_scan_carry_groups<<<cb, kCarryThreads, 0, s>>>(agg, gagg, tiles, G)));
    LX_LAUNCH("scan_carry", s, (lx_scan_carry_tiles<<<cb, kCarryThreads, 0, s>>>(agg, gagg, carry, tiles, G)));
    return hipSuccess;
}

template <int C, int MODE, bool RANDOM, int VB>
static hipError_t scan_launch_t(const ScanArgs& a, hipStream_t s)
{
    const int64_t blocks = a.tiles * ((a.batch + VB - 1) / VB);
    LX_LAUNCH(MODE == kScanUV || MODE == kScanUVLR ? "scan_reduce_uv" : (RANDOM ? "scan_reduce_gather" : "scan_reduce"), s,
              (lx_scan_reduce<C, MODE, RANDOM, VB><<<(unsigned)blocks, kScanThreads, 0, s>>>(a)));
    const hipError_t e = scan_carry_launch(a.agg, a.gagg, a.carry, a.tiles, (int64_t)a.channels * a.batch, s);
    if (e != hipSuccess) return e;
    LX_LAUNCH(MODE == kScanPLPR || MODE == kScanUVLR ? "scan_apply_tables" : (RANDOM ? "scan_apply_scatter" : "scan_apply"), s,
              (lx_scan_apply<C, MODE, RANDOM, VB><<<(unsigned)blocks, kScanThreads, 0, s>>>(a)));
    return hipSuccess;
}

hipError_t scan_launch(const ScanArgs& a, hipStream_t s)
{
    if (a.n <= 0 || a.batch <= 0) return hipSuccess;
    if (a.tiles * a.batch > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const bool two = a.channels == 2;
    // one vector: no vector loop, the leaner kernel keeps more waves resident
    const bool one = a.batch == 1;
#define LX_SCAN(M, R)                                                                            \
    (one ? (two ? scan_launch_t<2, M, R, 1>(a, s) : scan_launch_t<1, M, R, 1>(a, s))              \
         : (two ? scan_launch_t<2, M, R, kScanVB>(a, s) : scan_launch_t<1, M, R, kScanVB>(a, s)))
    switch (a.mode) {
        case kScanSym: return a.random ? LX_SCAN(kScanSym, true) : LX_SCAN(kScanSym, false);
        case kScanUV: return a.random ? LX_SCAN(kScanUV, true) : LX_SCAN(kScanUV, false);
        case kScanPLPR: return a.random ? LX_SCAN(kScanPLPR, true) : LX_SCAN(kScanPLPR, false);
        case kScanUVLR: return LX_SCAN(kScanUVLR, false);
        default: return hipErrorInvalidValue;
    }
#undef LX_SCAN
}

}  // namespace lx
