// Per-thread runs of a scan tile (gfx950): 256 threads x 16 consecutive ranks
// = 4096 ranks per tile; loads and stores of whole runs use 16-byte accesses.
#pragma once
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
__device__ __forceinline__ void load_decays(const float* __restrict__ s, int64_t r0, int64_t n, double inv_t,
                                            double (&e)[N + 1])
{
    float mid[N];
    load_run<N>(s, r0, n, mid);
    const float left = (r0 > 0 && r0 - 1 < n) ? s[r0 - 1] : 0.f;
    const float right = (r0 + N < n) ? s[r0 + N] : 0.f;
    e[0] = (r0 > 0 && r0 < n) ? decay(left, mid[0], inv_t) : 0.0;
#pragma unroll
    for (int i = 1; i < N; ++i) e[i] = (r0 + i < n) ? decay(mid[i - 1], mid[i], inv_t) : 0.0;
    e[N] = (r0 + N < n) ? decay(mid[N - 1], right, inv_t) : 0.0;
}

// The same decays plus a tie mask: bit i set where the two anchors meeting
// at e[i] are equal.  It gives the multipliers (1 across equal neighbours,
// 0 elsewhere and past the ends) of a scan that sums only within runs of
// equal anchors.
template <int N>
__device__ __forceinline__ void load_decays_ties(const float* __restrict__ s, int64_t r0, int64_t n, double inv_t,
                                                 double (&e)[N + 1], uint32_t& ties)
{
    static_assert(N < 32, "tie mask width");
    float mid[N];
    load_run<N>(s, r0, n, mid);
    const float left = (r0 > 0 && r0 - 1 < n) ? s[r0 - 1] : 0.f;
    const float right = (r0 + N < n) ? s[r0 + N] : 0.f;
    const bool h0 = r0 > 0 && r0 < n;
    e[0] = h0 ? decay(left, mid[0], inv_t) : 0.0;
    uint32_t m = (h0 && left == mid[0]) ? 1u : 0u;
#pragma unroll
    for (int i = 1; i < N; ++i) {
        const bool h = r0 + i < n;
        e[i] = h ? decay(mid[i - 1], mid[i], inv_t) : 0.0;
        m |= (h && mid[i - 1] == mid[i]) ? (1u << i) : 0u;
    }
    const bool hn = r0 + N < n;
    e[N] = hn ? decay(mid[N - 1], right, inv_t) : 0.0;
    m |= (hn && mid[N - 1] == right) ? (1u << N) : 0u;
    ties = m;
}

__device__ __forceinline__ double tie_mult(uint32_t ties, int i) { return ((ties >> i) & 1u) ? 1.0 : 0.0; }

}  // namespace lx
