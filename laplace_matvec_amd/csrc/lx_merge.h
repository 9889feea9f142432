// Merge-path helpers (gfx950): two sorted float sequences merged with the
// first sequence's element placed before an equal element of the second,
// cut into tiles of equal length, and segmented sums along the merged order
// whose segments end at elements of the second sequence.  Used where one
// anchor set is collected into the intervals (s_{t-1}, s_t] of another
// ("LAPLEX: The FFT of Learnable Laplace Kernels", technical summary §2.2,
// general case and Gram operators).
#pragma once
#include "lx_device.h"

namespace lx {

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMergeItems = 8;
constexpr int kMergeTile = kMergeThreads * kMergeItems;  // merged items per tile

// Inputs among the first d merged items: the least i with input i not
// before output d - i - 1 (input i goes first iff s_in[i] <= s_out[d-i-1]).
__device__ __forceinline__ int64_t merge_search(const float* __restrict__ si, int64_t ni, const float* __restrict__ so,
                                                int64_t no, int64_t d)
{
    int64_t lo = d > no ? d - no : 0;
    int64_t hi = d < ni ? d : ni;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (si[mid] <= so[d - mid - 1]) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Exclusive segmented scan of K values per thread across the workgroup, in
// thread order: a thread holding an output (m = 0) restarts the sum.  The
// elements are the affine maps t -> m t + v (m 0 or 1, exact), so the wave
// scans of the float64 composites serve.  Returns through vex the sum
// entering this thread, through mex 1 if no earlier thread holds an output,
// through vtot the sum after the workgroup's last output (or of everything).
// sh: [2][K][kMergeWaves], used in turns by `parity`.
template <int K>
__device__ __forceinline__ void block_segscan(double m, const double (&v)[K], Aff<double>* sh, int parity, double& mex,
                                              double (&vex)[K], double (&vtot)[K])
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    Aff<double>* buf = sh + parity * (K * kMergeWaves);
    Aff<double> ex[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const Aff<double> inc = wave_scan_up(Aff<double>{m, v[k]});
        ex[k] = wave_shift_up(inc);
        if (lane == kWave - 1) buf[k * kMergeWaves + w] = inc;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        Aff<double> pre = aff_identity<double>(), tot = aff_identity<double>();
#pragma unroll
        for (int i = 0; i < kMergeWaves; ++i) {
            const Aff<double> a = buf[k * kMergeWaves + i];
            if (i < w) pre = compose(pre, a);
            tot = compose(tot, a);
        }
        const Aff<double> r = compose(pre, ex[k]);
        vex[k] = r.v;
        if (k == 0) mex = r.m;
        vtot[k] = tot.v;
    }
}

}  // namespace lx
