// Device primitives for the LAPLEX kernels (gfx950, wave64).
//
// The scans of the operator (technical summary of "LAPLEX: The FFT of
// Learnable Laplace Kernels", §2.2) are scans of affine maps: the recurrence
// y_r = x_r + w * y_{r-1} is the map t -> w*t + x, and running two such
// steps one after the other is again affine.  `Aff` holds (m, v) for
// t -> m*t + v and `compose(p, q)` is "p, then q".
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lx {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Order-preserving map of float bits to uint32 (IEEE order, -0.0 < +0.0).
__device__ __forceinline__ uint32_t key_of(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_key(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool finite_bits(float f)
{
    return (__float_as_uint(f) & 0x7F800000u) != 0x7F800000u;
}

// Agent-scope relaxed atomics: look-back state words are read by workgroups
// on other XCDs, so they must bypass the per-XCD caches.
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t count_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Active lanes of this wave whose BITS-bit value equals ours: for each bit,
// keep the lanes whose ballot bit agrees with ours, i.e. AND with
// ~(ballot ^ m) where m is our bit spread over the word (0 or all ones).
template <int BITS>
__device__ __forceinline__ uint64_t match_bits(uint32_t d)
{
    const uint64_t act = __ballot(1);
    uint32_t lo = (uint32_t)act, hi = (uint32_t)(act >> 32);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const uint32_t m = (uint32_t)((int32_t)(d << (31 - b)) >> 31);  // bit b spread: 0 or ~0
        const uint64_t bal = __ballot(m != 0u);
        // v_bitop3 truth table indexed (S0 << 2 | S1 << 1 | S2): S0 & ~(S1 ^ S2) -> 0x90
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bal, m, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bal >> 32), m, 0x90);
    }
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t match_digit8(uint32_t d) { return match_bits<8>(d); }

// Workgroups of a launch are dealt to the compute dies (8 XCDs, each with
// its own L2) in turn: workgroup b runs on die b % 8.  For launches whose
// workgroups are independent, this bijection of [0, tiles) gives the
// workgroups of one die a contiguous range of tiles, taken in order, so
// neighbouring tiles share an L2 (their partly covered cache lines at the
// seams are fetched or merged once).  Any other dispatch only changes the
// order in which tiles are done.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t tiles)
{
    constexpr int64_t kDies = 8;
    const int64_t q = tiles / kDies, r = tiles % kDies;
    const int64_t x = b % kDies, j = b / kDies;
    return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// For a grid of chunks x groups in which the groups of one chunk read the
// same inputs (vector groups over one range of anchors), workgroup b is
// given chunk (b / 8 / groups) * 8 + b % 8 and group (b / 8) % groups: the
// groups of a chunk run on one die in consecutive dispatch slots, so that
// die's L2 serves the shared inputs to all of them after one read from
// HBM.  The grid is rounded up to whole dies; returns false for a
// workgroup past the last chunk.
__device__ __forceinline__ bool die_chunk_group(int64_t b, int64_t chunks, int groups, int64_t* chunk, int* g)
{
    constexpr int64_t kDies = 8;
    const int64_t k = b / kDies;
    *g = (int)(k % groups);
    *chunk = (k / groups) * kDies + b % kDies;
    return *chunk < chunks;
}
__host__ __device__ inline int64_t die_chunk_group_blocks(int64_t chunks, int groups)
{
    return (chunks + 7) / 8 * 8 * groups;
}

template <class T>
struct Aff {
    T m, v;
};

template <class T>
__device__ __forceinline__ Aff<T> aff_identity()
{
    return Aff<T>{T(1), T(0)};
}

// p first, then q:  t -> q.m*(p.m*t + p.v) + q.v
template <class T>
__device__ __forceinline__ Aff<T> compose(Aff<T> p, Aff<T> q)
{
    return Aff<T>{p.m * q.m, q.m * p.v + q.v};
}

// A 64-bit value moved between lanes by DPP (vector ALU moves, without the
// LDS round trip of a shuffle).  CTRL 0x110+d (row_shr:d) reads lane - d and
// 0x100+d (row_shl:d) lane + d inside each row of 16 lanes; 0x142
// (row_bcast:15) gives the rows in ROW_MASK lane 15 of the row below them,
// 0x143 (row_bcast:31) lane 31; 0x138 (wave_shr:1) reads lane - 1 and 0x130
// (wave_shl:1) lane + 1 across the whole wave.  Lanes without a source, or
// outside ROW_MASK, get `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_move(double x, double old)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint64_t o = (uint64_t)__double_as_longlong(old);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)b, CTRL, ROW_MASK,
                                                              0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32), (int)(uint32_t)(b >> 32),
                                                              CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// A composite moved by DPP; lanes without a source get the identity map, so
// composing with the result leaves them unchanged (1*m = m, 0*m + v = v
// exactly) and no lane needs a select.  With every row enabled, the three
// zero words of the identity (both words of v, the low word of m = 1.0)
// come from the hardware's zero for a lane without a source (bound_ctrl),
// so only the high word of m needs an initialised old value.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ Aff<double> dpp_move(Aff<double> x)
{
    if constexpr (ROW_MASK == 0xF) {
        const uint64_t bm = (uint64_t)__double_as_longlong(x.m);
        const uint64_t bv = (uint64_t)__double_as_longlong(x.v);
        const uint32_t mlo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bm, CTRL, 0xF, 0xF, true);
        const uint32_t mhi =
            (uint32_t)__builtin_amdgcn_update_dpp(0x3FF00000, (int)(uint32_t)(bm >> 32), CTRL, 0xF, 0xF, false);
        const uint32_t vlo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bv, CTRL, 0xF, 0xF, true);
        const uint32_t vhi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(bv >> 32), CTRL, 0xF, 0xF, true);
        return Aff<double>{__longlong_as_double((long long)(((uint64_t)mhi << 32) | mlo)),
                           __longlong_as_double((long long)(((uint64_t)vhi << 32) | vlo))};
    } else {
        return Aff<double>{dpp_move<CTRL, ROW_MASK>(x.m, 1.0), dpp_move<CTRL, ROW_MASK>(x.v, 0.0)};
    }
}

// The value of lane L (a constant), in scalar registers.
__device__ __forceinline__ double read_lane(double x, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ Aff<double> read_lane(Aff<double> x, int l)
{
    return Aff<double>{read_lane(x.m, l), read_lane(x.v, l)};
}

// Sum of x over the 64 lanes of a wave, returned in every lane, in a fixed
// order: distances 1, 2, 4, 8 inside each row of 16 lanes by DPP (lane 15
// of each row then holds its row's sum), rows 0 + 1 and 2 + 3 by a row
// broadcast of lane 15, the two halves by a broadcast of lane 31; lane 63
// holds the total.  All lanes of the wave must be active.  No LDS round
// trip, unlike a shuffle per step.
__device__ __forceinline__ double wave_sum_dpp(double x)
{
    x += dpp_move<0x111>(x, 0.0);
    x += dpp_move<0x112>(x, 0.0);
    x += dpp_move<0x114>(x, 0.0);
    x += dpp_move<0x118>(x, 0.0);
    x += dpp_move<0x142, 0xA>(x, 0.0);  // rows 1, 3 += lane 15 of rows 0, 2
    x += dpp_move<0x143, 0xC>(x, 0.0);  // rows 2, 3 += lane 31
    return read_lane(x, kWave - 1);
}

// Inclusive scan over the lanes of a wave in ascending lane order.  All
// lanes of the wave must be active.  Float64 composites: distances 1, 2, 4,
// 8 inside each row of 16 lanes by DPP, then each row takes the composite
// of all rows below it (row broadcasts of lanes 15 and 31); lanes with
// nothing to take compose with the identity.  Other types: shuffles at
// distances 1 .. 32.
template <class T>
__device__ __forceinline__ Aff<T> wave_scan_up(Aff<T> x)
{
    if constexpr (sizeof(T) == 8) {
        x = compose(dpp_move<0x111>(x), x);
        x = compose(dpp_move<0x112>(x), x);
        x = compose(dpp_move<0x114>(x), x);
        x = compose(dpp_move<0x118>(x), x);
        x = compose(dpp_move<0x142, 0xA>(x), x);  // rows 1, 3 <- lane 15 of rows 0, 2
        x = compose(dpp_move<0x143, 0xC>(x), x);  // rows 2, 3 <- lane 31 (rows 0 and 1)
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const T m = __shfl_up(x.m, d);
            const T v = __shfl_up(x.v, d);
            if (lane >= d) x = compose(Aff<T>{m, v}, x);
        }
    }
    return x;
}

// Inclusive scan over the lanes in descending lane order (lane 63 first).
// All lanes of the wave must be active.  Float64 composites: distances 1,
// 2, 4, 8 inside each row by DPP, then each row takes the composite of the
// rows above it, from the row totals at lanes 16, 32 and 48.
template <class T>
__device__ __forceinline__ Aff<T> wave_scan_down(Aff<T> x)
{
    const int lane = lane_id();
    if constexpr (sizeof(T) == 8) {
        x = compose(dpp_move<0x101>(x), x);
        x = compose(dpp_move<0x102>(x), x);
        x = compose(dpp_move<0x104>(x), x);
        x = compose(dpp_move<0x108>(x), x);
        const Aff<double> r1 = read_lane(x, 16), r2 = read_lane(x, 32), r3 = read_lane(x, 48);
        const Aff<double> r32 = compose(r3, r2);
        const int row = lane >> 4;
        const Aff<double> above =
            row == 3 ? aff_identity<double>() : (row == 2 ? r3 : (row == 1 ? r32 : compose(r32, r1)));
        x = compose(above, x);
    } else {
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const T m = __shfl_down(x.m, d);
            const T v = __shfl_down(x.v, d);
            if (lane + d < kWave) x = compose(Aff<T>{m, v}, x);
        }
    }
    return x;
}

// Exclusive versions of a wave scan's result: the inclusive value of the
// lane below (up) or above (down), identity at the wave's first lane.
template <class T>
__device__ __forceinline__ Aff<T> wave_shift_up(Aff<T> inc)
{
    if constexpr (sizeof(T) == 8) {
        return dpp_move<0x138>(inc);
    } else {
        Aff<T> ex{__shfl_up(inc.m, 1), __shfl_up(inc.v, 1)};
        if (lane_id() == 0) ex = aff_identity<T>();
        return ex;
    }
}
template <class T>
__device__ __forceinline__ Aff<T> wave_shift_down(Aff<T> inc)
{
    if constexpr (sizeof(T) == 8) {
        return dpp_move<0x130>(inc);
    } else {
        Aff<T> ex{__shfl_down(inc.m, 1), __shfl_down(inc.v, 1)};
        if (lane_id() == kWave - 1) ex = aff_identity<T>();
        return ex;
    }
}

// Block-wide exclusive scans of one Aff per thread, ascending (up) or
// descending (down) thread order.  `sh` needs NW entries.  Returns the
// exclusive prefix of this thread; `total` receives the block's composite.
// Ends with a barrier, so `sh` may be reused right after.
template <class T, int NW>
__device__ __forceinline__ Aff<T> block_exscan_up(Aff<T> x, Aff<T>* sh, Aff<T>& total)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    const Aff<T> inc = wave_scan_up(x);
    const Aff<T> ex = wave_shift_up(inc);
    if (lane == kWave - 1) sh[w] = inc;
    __syncthreads();
    Aff<T> pre = aff_identity<T>();
    Aff<T> tot = aff_identity<T>();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) pre = compose(pre, sh[i]);
        tot = compose(tot, sh[i]);
    }
    total = tot;
    __syncthreads();
    return compose(pre, ex);
}

template <class T, int NW>
__device__ __forceinline__ Aff<T> block_exscan_down(Aff<T> x, Aff<T>* sh, Aff<T>& total)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    const Aff<T> inc = wave_scan_down(x);
    const Aff<T> ex = wave_shift_down(inc);
    if (lane == 0) sh[w] = inc;
    __syncthreads();
    Aff<T> pre = aff_identity<T>();
    Aff<T> tot = aff_identity<T>();
#pragma unroll
    for (int i = NW - 1; i >= 0; --i) {
        if (i > w) pre = compose(pre, sh[i]);
        tot = compose(tot, sh[i]);
    }
    total = tot;
    __syncthreads();
    return compose(pre, ex);
}

// The same exclusive scans without the block total, for kernels with many
// waves per workgroup: the wave totals are combined by a scan across lanes,
// not by a loop over all of them in every thread (which would keep NW
// composites live in registers).
template <class T, int NW>
__device__ __forceinline__ Aff<T> block_exscan_up_lean(Aff<T> x, Aff<T>* sh)
{
    static_assert(NW <= kWave, "waves per block");
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    const Aff<T> inc = wave_scan_up(x);
    const Aff<T> ex = wave_shift_up(inc);
    if (lane == kWave - 1) sh[w] = inc;
    __syncthreads();
    Aff<T> t = lane < NW ? sh[lane] : aff_identity<T>();
    t = wave_scan_up(t);
    Aff<T> pre{__shfl(t.m, w > 0 ? w - 1 : 0), __shfl(t.v, w > 0 ? w - 1 : 0)};
    if (w == 0) pre = aff_identity<T>();
    __syncthreads();
    return compose(pre, ex);
}
template <class T, int NW>
__device__ __forceinline__ Aff<T> block_exscan_down_lean(Aff<T> x, Aff<T>* sh)
{
    static_assert(NW <= kWave, "waves per block");
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    const Aff<T> inc = wave_scan_down(x);
    const Aff<T> ex = wave_shift_down(inc);
    if (lane == 0) sh[w] = inc;
    __syncthreads();
    Aff<T> t = lane < NW ? sh[lane] : aff_identity<T>();
    t = wave_scan_down(t);
    Aff<T> pre{__shfl(t.m, w + 1 < NW ? w + 1 : 0), __shfl(t.v, w + 1 < NW ? w + 1 : 0)};
    if (w + 1 >= NW) pre = aff_identity<T>();
    __syncthreads();
    return compose(pre, ex);
}

// Inclusive sum of uint32 over the lanes of a wave in ascending lane order,
// by DPP (distances 1, 2, 4, 8 inside rows of 16, then the row broadcasts
// of lanes 15 and 31).  The identity is 0, which is what a lane without a
// DPP source reads (bound_ctrl), and what the rows left out of a broadcast
// keep.  All lanes of the wave must be active.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, ROW_MASK == 0xF);
}
__device__ __forceinline__ uint32_t wave_incsum_u32(uint32_t x)
{
    x += dpp_u32<0x111>(x);
    x += dpp_u32<0x112>(x);
    x += dpp_u32<0x114>(x);
    x += dpp_u32<0x118>(x);
    x += dpp_u32<0x142, 0xA>(x);
    x += dpp_u32<0x143, 0xC>(x);
    return x;
}
// Block-wide exclusive sum of uint32 over NW waves.
template <int NW>
__device__ __forceinline__ uint32_t block_exsum_u32(uint32_t x, uint32_t* sh, uint32_t& total)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    const uint32_t inc = wave_incsum_u32(x);
    if (lane == kWave - 1) sh[w] = inc;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) pre += sh[i];
        tot += sh[i];
    }
    total = tot;
    __syncthreads();
    return pre + inc - x;
}

// Decay factor exp(-(hi - lo) / t) between two float32 anchors lo <= hi, in
// float64, with inv_t = 1 / t (+inf at temperature 0, where equal anchors
// give 1 and all others 0).  The difference of two float32 values is exact
// in float64, and float64 factors keep long chains of equal gaps (common
// where many anchors sit on one float32 grid) free of the bias a repeated
// float32 rounding of exp(-gap) would accumulate.
// exp(x) for x <= 0.  Neighbouring sorted anchors are usually close, so x is
// usually tiny: for |x| < 2^-7 the Taylor polynomial of degree 7 leaves a
// truncation error below x^8 / 8! < 2^-71 and costs 7 FMAs; larger |x| (and
// x = -inf for t = 0) take the library exp.
__device__ __forceinline__ double exp_nonpos(double x)
{
    if (x > -0x1p-7) {
        double p = 1.0 / 5040.0;
        p = fma(p, x, 1.0 / 720.0);
        p = fma(p, x, 1.0 / 120.0);
        p = fma(p, x, 1.0 / 24.0);
        p = fma(p, x, 1.0 / 6.0);
        p = fma(p, x, 0.5);
        p = fma(p, x, 1.0);
        return fma(p, x, 1.0);
    }
    return exp(x);
}

__device__ __forceinline__ double decay(float lo, float hi, double inv_t)
{
    return lo == hi ? 1.0 : exp_nonpos(((double)lo - (double)hi) * inv_t);
}

// e^x for x <= 0 (x = -inf gives 0) to about 1e-7 relative error, in nine
// instructions: x / ln 2 split in float64 into an integer k and a fraction
// f in [-1/2, 1/2] (exact), 2^f by the hardware's float32 exp2 (1 ulp),
// scaled by 2^k in float64 (results below 2^-1074 flush to 0).  For sums of
// positive terms whose results are stored in float32.
__device__ __forceinline__ double exp_nonpos_fast(double x)
{
    const double y = fmax(x * 1.4426950408889634, -1100.0);  // log2(e); 2^-1100 is 0 in float64
    const double k = rint(y);
    return ldexp((double)__builtin_amdgcn_exp2f((float)(y - k)), (int)k);
}

// decay() to about 1e-7 relative error (exp_nonpos_fast); 1 for lo == hi.
__device__ __forceinline__ double decay_fast(float lo, float hi, double inv_t)
{
    return lo == hi ? 1.0 : exp_nonpos_fast(((double)lo - (double)hi) * inv_t);
}

// exp(-(hi - lo) / t) in float32 for anchors lo <= hi, it = 1 / t.
__device__ __forceinline__ float decay_f(float lo, float hi, float it)
{
    return lo == hi ? 1.f : expf((lo - hi) * it);
}

// #{r : s[r] < q} by bisection.
__device__ __forceinline__ int64_t lower_bound_f(const float* __restrict__ s, int64_t n, float q)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (s[mid] < q) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// #{r : s[r] <= q} by bisection, searching [lo, n) only (s[0..lo) <= q known).
__device__ __forceinline__ int64_t upper_bound_f(const float* __restrict__ s, int64_t n, float q, int64_t lo = 0)
{
    int64_t hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (s[mid] <= q) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Interval search through a lookup table: the range [s_0, s_{n-1}] of the
// sorted outputs is cut into LUT equal cells and tab[k] = #{s < left edge
// of cell k} (tab[LUT] = n), so the interval of q lies in [tab[k],
// tab[k+1]] for q's cell k, a few candidates for smooth data.  The result is
// checked against its neighbours and a full bisection replaces it when the
// cell arithmetic rounded q into the wrong cell: the answer is always the
// exact #{s < q}.
template <int LUT>
__device__ __forceinline__ uint32_t lower_bound_lut(const float* so, int no, const uint16_t* tab, float lo_v,
                                                    float inv_w, float q)
{
    const float fk = (q - lo_v) * inv_w;
    const int k = !(fk >= 0.f) ? 0 : (fk >= (float)(LUT - 1) ? LUT - 1 : (int)fk);
    int lo = tab[k], hi = tab[k + 1];
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (so[mid] < q) lo = mid + 1;
        else hi = mid;
    }
    if ((lo > 0 && !(so[lo - 1] < q)) || (lo < no && so[lo] < q)) lo = (int)lower_bound_f(so, no, q);
    return (uint32_t)lo;
}

__host__ __device__ inline int64_t pad64(int64_t x) { return (x + 63) & ~(int64_t)63; }

// exp(-d / t) for a distance d >= 0 (1 at d == 0, also at t = 0).
__device__ __forceinline__ double decay_dist(double d, double inv_t)
{
    return d == 0.0 ? 1.0 : exp(-d * inv_t);
}

}  // namespace lx
