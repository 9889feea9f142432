// Stable LSD radix argsort of float32 anchors for gfx950.
//
// The operator's fast algorithm starts by sorting the anchors (technical
// summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2).  The
// permutation must be deterministic, so the sort is stable: equal anchors
// keep ascending original index, and the key order is the IEEE order with
// -0.0 before +0.0 (float bits mapped to an order-preserving uint32).
//
// Design (one pass per 8-bit digit, least significant first):
//   * lx_sort_hist: one streaming read of the anchors builds the four
//     256-bin digit histograms and flags NaN/Inf;
//   * lx_sort_scan_hist: exclusive prefix of each histogram -> bin bases;
//   * lx_sort_pass (x4): each workgroup takes a tile of 8192 keys by atomic
//     ticket, ranks them stably with wave64 ballots, publishes its per-bin
//     counts, looks back over earlier tiles' published counts (decoupled
//     look-back) to get its global offsets, reorders the tile in LDS by
//     digit and writes runs of keys and indices.  The first pass reads the
//     float anchors directly (keys and the index payload are made on the
//     fly), the last one writes the sorted floats back in their float form.
//
// Look-back state word per (tile, bin): 0 = not yet published;
// bit31 clear, value c+1 = this tile's own count c; bit31 set = count of
// this bin over all tiles up to and including this one (n < 2^31 fits).
// Tiles wait only on tiles with a smaller ticket, which have already
// started and publish without waiting, so every wait ends.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

constexpr int kSortThreads = 512;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // 8192
constexpr int kRadix = 256;
constexpr int kHistThreads = 256;

static_assert(kSortTile == kSortTileSize, "tile size must match the host planner");

__global__ __launch_bounds__(256) void lx_fill_u32(uint32_t* __restrict__ p, uint32_t v, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = v;
}

hipError_t fill_u32(uint32_t* p, uint32_t v, int64_t count, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    const int grid = (int)(blocks < 4096 ? blocks : 4096);
    LX_LAUNCH("util_fill", s, (lx_fill_u32<<<grid, 256, 0, s>>>(p, v, count)));
    return hipSuccess;
}

__global__ __launch_bounds__(kHistThreads) void lx_sort_hist(const float* __restrict__ a, int64_t n,
                                                            uint32_t* __restrict__ hist,
                                                            uint32_t* __restrict__ flag)
{
    __shared__ uint32_t h[4][kRadix];
    for (int i = threadIdx.x; i < 4 * kRadix; i += kHistThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    bool bad = false;
    const int64_t stride = (int64_t)gridDim.x * kHistThreads;
    for (int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x; i < n; i += stride) {
        const float f = a[i];
        bad |= !finite_bits(f);
        const uint32_t k = key_of(f);
        atomicAdd(&h[0][k & 0xFF], 1u);
        atomicAdd(&h[1][(k >> 8) & 0xFF], 1u);
        atomicAdd(&h[2][(k >> 16) & 0xFF], 1u);
        atomicAdd(&h[3][k >> 24], 1u);
    }
    if (__any(bad) && lane_id() == 0) atomicOr(flag, 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * kRadix; i += kHistThreads) {
        const uint32_t c = (&h[0][0])[i];
        if (c) atomicAdd(&hist[i], c);
    }
}

// Four blocks of 256 threads: exclusive prefix of each digit histogram.
__global__ __launch_bounds__(kRadix) void lx_sort_scan_hist(const uint32_t* __restrict__ hist,
                                                           uint32_t* __restrict__ base)
{
    __shared__ uint32_t sh[kRadix / kWave];
    const int d = blockIdx.x;
    uint32_t tot;
    const uint32_t ex = block_exsum_u32<kRadix / kWave>(hist[d * kRadix + threadIdx.x], sh, tot);
    base[d * kRadix + threadIdx.x] = ex;
}

template <bool FIRST, bool LAST>
__global__ __launch_bounds__(kSortThreads) void lx_sort_pass(
    const float* __restrict__ a_in, const uint32_t* __restrict__ keys_in,
    const uint32_t* __restrict__ vals_in, uint32_t* __restrict__ keys_out,
    float* __restrict__ sorted_out, uint32_t* __restrict__ vals_out,
    const uint32_t* __restrict__ bin_base, uint32_t* __restrict__ state,
    uint32_t* __restrict__ ticket, int shift, int64_t n)
{
    __shared__ uint32_t s_hist[kSortWaves][kRadix];  // per-wave counts, then wave offsets
    __shared__ uint32_t s_start[kRadix];             // tile-local start of each bin
    __shared__ uint32_t s_glob[kRadix];              // global position of each bin's first key
    __shared__ uint32_t s_buf[kSortTile];
    __shared__ uint32_t s_red[kSortWaves];
    __shared__ uint32_t s_tile;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / kWave;

    if (tid == 0) s_tile = atomicAdd(ticket, 1u);
    for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) (&s_hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t tile = s_tile;
    const int64_t wave0 = (int64_t)tile * kSortTile + (int64_t)w * (kSortItems * kWave);

    // Keys in wave-striped order: item j of lane l is element wave0 + 64 j + l,
    // so a wave's items in (j, lane) order are its elements in index order.
    // Positions past n get the largest key: they rank last, in bin 255.
    uint32_t key[kSortItems];
    uint32_t val[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t idx = wave0 + (int64_t)j * kWave + lane;
        if (idx < n) {
            key[j] = FIRST ? key_of(a_in[idx]) : keys_in[idx];
            val[j] = FIRST ? (uint32_t)idx : vals_in[idx];
        } else {
            key[j] = 0xFFFFFFFFu;
            val[j] = 0u;
        }
    }

    // Stable rank inside the wave: peers with the same digit, in lane order,
    // item by item; the lowest peer lane advances the wave's bin counter.
    uint32_t pos[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t d = (key[j] >> shift) & 0xFFu;
        const uint64_t peers = match_digit8(d);
        const uint32_t below = count_below(peers);
        const uint32_t prev = s_hist[w][d];
        pos[j] = prev + below;
        if (below == 0) s_hist[w][d] = prev + (uint32_t)__popcll(peers);
    }
    __syncthreads();

    uint32_t count = 0;
    if (tid < kRadix) {
        // counts of earlier waves -> offsets; total -> this tile's bin count
        uint32_t run = 0;
#pragma unroll
        for (int i = 0; i < kSortWaves; ++i) {
            const uint32_t c = s_hist[i][tid];
            s_hist[i][tid] = run;
            run += c;
        }
        count = run;
        uint32_t* mine = state + (int64_t)tile * kRadix + tid;
        uint32_t before = 0;
        if (tile == 0) {
            st_agent(mine, 0x80000000u | count);
        } else {
            st_agent(mine, count + 1u);
            int64_t t = (int64_t)tile - 1;
            while (true) {
                const uint32_t sv = ld_agent(state + t * kRadix + tid);
                if (sv == 0u) {
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                if (sv & 0x80000000u) {
                    before += sv & 0x7FFFFFFFu;
                    break;
                }
                before += sv - 1u;
                --t;
            }
            st_agent(mine, 0x80000000u | (before + count));
        }
        s_glob[tid] = bin_base[tid] + before;
    }
    uint32_t tile_total;
    const uint32_t start = block_exsum_u32<kSortWaves>(tid < kRadix ? count : 0u, s_red, tile_total);
    if (tid < kRadix) s_start[tid] = start;
    __syncthreads();

    // Place keys in the tile's digit order.
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t d = (key[j] >> shift) & 0xFFu;
        pos[j] += s_start[d] + s_hist[w][d];
        s_buf[pos[j]] = key[j];
    }
    __syncthreads();

    // Consecutive LDS slots of one digit go to consecutive global slots.
    uint32_t dst[kSortItems];
#pragma unroll
    for (int q = 0; q < kSortItems; ++q) {
        const uint32_t i = (uint32_t)(q * kSortThreads + tid);
        const uint32_t k = s_buf[i];
        const uint32_t d = (k >> shift) & 0xFFu;
        dst[q] = s_glob[d] + (i - s_start[d]);
        if ((int64_t)dst[q] < n) {
            if (LAST) sorted_out[dst[q]] = float_of_key(k);
            else keys_out[dst[q]] = k;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) s_buf[pos[j]] = val[j];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kSortItems; ++q) {
        const uint32_t i = (uint32_t)(q * kSortThreads + tid);
        if ((int64_t)dst[q] < n) vals_out[dst[q]] = s_buf[i];
    }
}

// Scratch layout (bytes, each region 256-byte aligned):
//   keysA, valsA, keysB, valsB : uint32[n] each
//   hist, base                 : uint32[4][256] each
//   tickets                    : uint32[4] (padded to 64)
//   state                      : uint32[4][tiles][256]
static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t sort_scratch_bytes(int64_t n)
{
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    size_t b = 0;
    b += 4 * align256((size_t)n * 4);
    b += 2 * align256(4 * kRadix * 4);
    b += align256(64 * 4);
    b += align256((size_t)4 * tiles * kRadix * 4);
    return b;
}

hipError_t sort_launch(const float* a, int64_t n, float* sorted, uint32_t* perm, void* scratch,
                       uint32_t* flag, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    char* p = (char*)scratch;
    uint32_t* keysA = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* valsA = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* keysB = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* valsB = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* hist = (uint32_t*)p; p += align256(4 * kRadix * 4);
    uint32_t* base = (uint32_t*)p; p += align256(4 * kRadix * 4);
    uint32_t* tickets = (uint32_t*)p; p += align256(64 * 4);
    uint32_t* state = (uint32_t*)p;

    // hist, base and tickets are contiguous: clear them and the state together
    const int64_t clear_words = (int64_t)((char*)state - (char*)hist) / 4 + 4 * tiles * kRadix;
    hipError_t e = fill_u32(hist, 0u, clear_words, s);
    if (e != hipSuccess) return e;

    {
        int64_t blocks = (n + kHistThreads * 16 - 1) / (kHistThreads * 16);
        if (blocks > 2048) blocks = 2048;
        LX_LAUNCH("sort_hist", s, (lx_sort_hist<<<(int)blocks, kHistThreads, 0, s>>>(a, n, hist, flag)));
    }
    LX_LAUNCH("sort_scan_hist", s, (lx_sort_scan_hist<<<4, kRadix, 0, s>>>(hist, base)));

    const int grid = (int)tiles;
    const int64_t st = tiles * kRadix;
    LX_LAUNCH("sort_pass", s,
              (lx_sort_pass<true, false><<<grid, kSortThreads, 0, s>>>(
                  a, nullptr, nullptr, keysA, nullptr, valsA, base + 0 * kRadix, state + 0 * st,
                  tickets + 0, 0, n)));
    LX_LAUNCH("sort_pass", s,
              (lx_sort_pass<false, false><<<grid, kSortThreads, 0, s>>>(
                  nullptr, keysA, valsA, keysB, nullptr, valsB, base + 1 * kRadix, state + 1 * st,
                  tickets + 1, 8, n)));
    LX_LAUNCH("sort_pass", s,
              (lx_sort_pass<false, false><<<grid, kSortThreads, 0, s>>>(
                  nullptr, keysB, valsB, keysA, nullptr, valsA, base + 2 * kRadix, state + 2 * st,
                  tickets + 2, 16, n)));
    LX_LAUNCH("sort_pass", s,
              (lx_sort_pass<false, true><<<grid, kSortThreads, 0, s>>>(
                  nullptr, keysA, valsA, nullptr, sorted, perm, base + 3 * kRadix, state + 3 * st,
                  tickets + 3, 24, n)));
    return hipSuccess;
}

// ------------------------------------------------------------- phase factors

__global__ __launch_bounds__(256) void lx_phase_factors(const float* __restrict__ ph,
                                                       const uint32_t* __restrict__ perm, int64_t n,
                                                       float* __restrict__ c, float* __restrict__ s,
                                                       uint32_t* __restrict__ flag)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n; r += stride) {
        const float f = ph[perm ? perm[r] : r];
        bad |= !finite_bits(f);
        // float64 sincos of the float32 phase, rounded once to float32
        double sd, cd;
        sincos((double)f, &sd, &cd);
        c[r] = (float)cd;
        s[r] = (float)sd;
    }
    if (__any(bad) && lane_id() == 0) atomicOr(flag, 1u);
}

hipError_t phase_factors_launch(const float* ph, const uint32_t* perm, int64_t n, float* c,
                                float* s, uint32_t* flag, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    LX_LAUNCH("plan_phase", st, (lx_phase_factors<<<(int)blocks, 256, 0, st>>>(ph, perm, n, c, s, flag)));
    return hipSuccess;
}

__global__ __launch_bounds__(256) void lx_check_finite(const float* __restrict__ v, int64_t n,
                                                      uint32_t* __restrict__ flag)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        bad |= !finite_bits(v[i]);
    if (__any(bad) && lane_id() == 0) atomicOr(flag, 1u);
}

hipError_t check_finite_launch(const float* v, int64_t n, uint32_t* flag, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    LX_LAUNCH("plan_check", st, (lx_check_finite<<<(int)blocks, 256, 0, st>>>(v, n, flag)));
    return hipSuccess;
}

}  // namespace lx
