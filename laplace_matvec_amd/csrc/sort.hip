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
//     digit and writes runs of keys.  The first pass reads the float anchors
//     directly, the last one writes the sorted floats in their float form.
//     No index payload travels with the keys: each pass instead records,
//     per slot, the tile position it came from (16 bits) and, per tile and
//     bin, where the bin's run starts.  Replaying the records (lx_replay)
//     moves any array into sorted order or back, and an index ramp replayed
//     forward is the permutation itself.
//
// Look-back state word per (tile, bin): 0 = not yet published;
// bit31 clear, value c+1 = this tile's own count c; bit31 set = count of
// this bin over all tiles up to and including this one (n < 2^31 fits).
// kLookback rows before tile 0 hold an inclusive 0, so every word a
// look-back round reads is in the array and the walk ends there.
// Tiles wait only on tiles with a smaller ticket, which have already
// started and publish without waiting, so every wait ends.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

#ifndef LX_SORT_THREADS
#define LX_SORT_THREADS 512
#endif
#ifndef LX_SORT_ITEMS
#define LX_SORT_ITEMS 16
#endif
constexpr int kSortThreads = LX_SORT_THREADS;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortItems = LX_SORT_ITEMS;
constexpr int kSortTile = kSortThreads * kSortItems;  // 8192
constexpr int kRadix = 256;
constexpr int kHistThreads = 256;
#ifndef LX_LOOKBACK
#define LX_LOOKBACK 4
#endif
constexpr int kLookback = LX_LOOKBACK;  // predecessors read per look-back round

static_assert(kSortTile == kSortTileSize, "tile size must match the host planner");

__global__ __launch_bounds__(256) void lx_fill_u32(uint32_t* __restrict__ p, uint32_t v, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = v;
}

// Zeroes `head` words (histograms, bases, tickets) and four passes of
// look-back state after them, each pass starting with kLookback rows of
// inclusive 0 (0x80000000).
__global__ __launch_bounds__(256) void lx_sort_clear(uint32_t* __restrict__ p, int64_t head, int64_t pass_words)
{
    const int64_t total = head + 4 * pass_words;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t j = i - head;
        p[i] = (j >= 0 && j % pass_words < (int64_t)kLookback * kRadix) ? 0x80000000u : 0u;
    }
}

hipError_t fill_u32(uint32_t* p, uint32_t v, int64_t count, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    const int grid = (int)(blocks < 4096 ? blocks : 4096);
    LX_LAUNCH("util_fill", s, (lx_fill_u32<<<grid, 256, 0, s>>>(p, v, count)));
    return hipSuccess;
}

// Digit histograms of all four passes in one read of the anchors.  Each
// digit has kHistCopies copies in LDS, lane l counting into copy l % 8, rows
// 257 words apart so that lanes of one wave hitting the same bin of a
// concentrated digit (the sign and exponent byte of clustered anchors) land
// on different banks and addresses.
constexpr int kHistCopies = 8;
constexpr int kHistRow = kRadix + 1;

__global__ __launch_bounds__(kHistThreads) void lx_sort_hist(const float* __restrict__ a, int64_t n,
                                                            uint32_t* __restrict__ hist,
                                                            uint32_t* __restrict__ flag)
{
    __shared__ uint32_t h[4][kHistCopies * kHistRow];
    for (int i = threadIdx.x; i < 4 * kHistCopies * kHistRow; i += kHistThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    uint32_t bad = 0;
    const int copy = (lane_id() % kHistCopies) * kHistRow;
    auto count = [&](float f) {
        const uint32_t u = __float_as_uint(f);
        bad |= (~u & 0x7F800000u) == 0u;  // exponent all ones: NaN or Inf
        const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        atomicAdd(&h[0][copy + (k & 0xFF)], 1u);
        atomicAdd(&h[1][copy + ((k >> 8) & 0xFF)], 1u);
        atomicAdd(&h[2][copy + ((k >> 16) & 0xFF)], 1u);
        atomicAdd(&h[3][copy + (k >> 24)], 1u);
    };
    // sixteen anchors per thread per step: four 16-byte loads issued before
    // any is counted (counting next to each load would make every load wait
    // for itself), then single float4s, then the ragged tail
    const int64_t n4 = n / 4;
    const float4* a4 = reinterpret_cast<const float4*>(a);
    const int64_t stride = (int64_t)gridDim.x * kHistThreads;
    constexpr int kHistBatch = 4;
    int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x;
    for (; i + (kHistBatch - 1) * stride < n4; i += kHistBatch * stride) {
        float4 v[kHistBatch];
#pragma unroll
        for (int q = 0; q < kHistBatch; ++q) v[q] = a4[i + q * stride];
#pragma unroll
        for (int q = 0; q < kHistBatch; ++q) {
            count(v[q].x);
            count(v[q].y);
            count(v[q].z);
            count(v[q].w);
        }
    }
    for (; i < n4; i += stride) {
        const float4 v = a4[i];
        count(v.x);
        count(v.y);
        count(v.z);
        count(v.w);
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kHistThreads + threadIdx.x; i < n; i += stride) count(a[i]);
    if (__any(bad) && lane_id() == 0) atomicOr(flag, 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * kRadix; i += kHistThreads) {
        const int d = i / kRadix, b = i % kRadix;
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < kHistCopies; ++q) c += h[d][q * kHistRow + b];
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

template <bool FIRST, bool LAST, bool VALS>
__global__ __launch_bounds__(kSortThreads, VALS ? 4 : 6) void lx_sort_pass(
    const float* __restrict__ a_in, const uint32_t* __restrict__ keys_in, uint32_t* __restrict__ keys_out,
    const uint2* __restrict__ kv_in, uint2* __restrict__ kv_out, float* __restrict__ sorted_out, uint16_t* __restrict__ rec, uint32_t* __restrict__ tab_base,
    uint16_t* __restrict__ tab_start, const uint32_t* __restrict__ bin_base, uint32_t* __restrict__ state,
    uint32_t* __restrict__ ticket, int shift, int64_t n, SortValPass vals)
{
    __shared__ uint16_t s_hist[kSortWaves][kRadix];  // per-wave counts, then slot of each wave's first key
    __shared__ uint32_t s_off[kRadix];               // global position of slot 0 of each bin's run
    // Slots in digit order: the keys (and, with value rows, each key with
    // its first-row value as one 8-byte pair, so a key and its value are
    // placed by one scattered LDS write)
    __shared__ uint32_t s_buf[VALS ? 1 : kSortTile];
    __shared__ uint2 s_kv[VALS ? kSortTile : 1];
    __shared__ uint32_t s_red[kSortWaves];
    __shared__ uint32_t s_tile;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / kWave;

    if (tid == 0) s_tile = atomicAdd(ticket, 1u);
    for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) (&s_hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t tile = s_tile;
    const int64_t tile0 = (int64_t)tile * kSortTile;
    const int wpos = w * (kSortItems * kWave);  // tile-local position of this wave's first key

    // Keys in wave-striped order: item j of lane l is tile position
    // wpos + 64 j + l, so a wave's items in (j, lane) order are its keys in
    // index order.  Positions past n get the largest key: they rank last,
    // in bin 255, and land past n.  The first value row is loaded with the
    // keys, so its latency overlaps the ranking and the look-back.
    //
    // With value rows, the passes between the first and the last move each
    // key together with the first row's value as one 8-byte pair: a tile's
    // scattered output is then one run per bin instead of two, half as many
    // partly written cache lines.
    constexpr bool PAIR_IN = VALS && !FIRST;
    constexpr bool PAIR_OUT = VALS && !LAST;
    uint32_t key[kSortItems];
    float v0[VALS ? kSortItems : 1];
    const int64_t wbase = tile0 + wpos;  // uniform
    const uint32_t room = (uint32_t)(n - wbase < (int64_t)(kSortItems * kWave) ? (n > wbase ? n - wbase : 0)
                                                                               : (int64_t)(kSortItems * kWave));
    {
        // raw words first (all loads in flight together), keys after: a
        // conversion next to each load would make every load wait for itself
        const uint32_t* src = FIRST ? reinterpret_cast<const uint32_t*>(a_in) + wbase : keys_in + wbase;
        const float* vin = VALS && !PAIR_IN ? vals.in[0] + wbase : nullptr;
        const uint2* pin = PAIR_IN ? kv_in + wbase : nullptr;
        if (room == (uint32_t)(kSortItems * kWave)) {
            if (PAIR_IN) {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) {
                    const uint2 kv = pin[j * kWave + lane];
                    key[j] = kv.x;
                    v0[j] = __uint_as_float(kv.y);
                }
            } else {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) key[j] = src[j * kWave + lane];
                if (VALS) {
#pragma unroll
                    for (int j = 0; j < kSortItems; ++j) v0[j] = vin[j * kWave + lane];
                }
            }
        } else {
            if (PAIR_IN) {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) {
                    const uint32_t off = (uint32_t)(j * kWave + lane);
                    const uint2 kv = off < room ? pin[off] : make_uint2(0u, 0u);
                    key[j] = kv.x;
                    v0[j] = __uint_as_float(kv.y);
                }
            } else {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) {
                    const uint32_t off = (uint32_t)(j * kWave + lane);
                    key[j] = off < room ? src[off] : 0u;
                }
                if (VALS) {
#pragma unroll
                    for (int j = 0; j < kSortItems; ++j) {
                        const uint32_t off = (uint32_t)(j * kWave + lane);
                        v0[j] = off < room ? vin[off] : 0.f;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const bool valid = (uint32_t)(j * kWave + lane) < room;
            if (FIRST) key[j] = key_of(__uint_as_float(key[j]));
            key[j] = valid ? key[j] : 0xFFFFFFFFu;
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
        if (below == 0) s_hist[w][d] = (uint16_t)(prev + (uint32_t)__popcll(peers));
    }
    __syncthreads();

    // Per bin: offsets of the waves, the tile's count, published at once so
    // later tiles can look back past this one.
    uint32_t count = 0;
    if (tid < kRadix) {
        uint32_t run = 0;
#pragma unroll
        for (int i = 0; i < kSortWaves; ++i) {
            const uint32_t c = s_hist[i][tid];
            s_hist[i][tid] = (uint16_t)run;
            run += c;
        }
        count = run;
        st_agent(state + (int64_t)tile * kRadix + tid, tile == 0 ? (0x80000000u | count) : (count + 1u));
    }
    uint32_t tile_total;
    const uint32_t start = block_exsum_u32<kSortWaves>(tid < kRadix ? count : 0u, s_red, tile_total);
    // the tile start of each bin folded into its wave offsets: the slot of
    // each wave's first key of each bin, one table read per key below
    if (tid < kRadix) {
#pragma unroll
        for (int i = 0; i < kSortWaves; ++i) s_hist[i][tid] = (uint16_t)(s_hist[i][tid] + start);
    }
    __syncthreads();

    // Slots in the tile's digit order.  The replay record (the tile position
    // each slot came from) depends on nothing outside the tile: it is
    // written before the look-back, while earlier tiles finish.
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t d = (key[j] >> shift) & 0xFFu;
        pos[j] += s_hist[w][d];
        if (VALS) s_kv[pos[j]].x = (uint32_t)(wpos + j * kWave + lane);
        else s_buf[pos[j]] = (uint32_t)(wpos + j * kWave + lane);
    }
    __syncthreads();
    {
        uint32_t* rec2 = reinterpret_cast<uint32_t*>(rec + tile0);
#pragma unroll
        for (int q = 0; q < kSortItems / 2; ++q) {
            const uint32_t i = (uint32_t)(q * kSortThreads + tid);  // pair of slots 2i, 2i+1
            rec2[i] = VALS ? (s_kv[2 * i].x | (s_kv[2 * i + 1].x << 16)) : (s_buf[2 * i] | (s_buf[2 * i + 1] << 16));
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        if (VALS) s_kv[pos[j]] = make_uint2(key[j], __float_as_uint(v0[j]));
        else s_buf[pos[j]] = key[j];
    }

    // Decoupled look-back, kLookback predecessors per round: sum their own
    // counts until one has published its inclusive count.  A round is
    // branch-free: all its loads are in flight together, then one pass of
    // selects takes the leading run of own counts and, if the run ends at an
    // inclusive count, that too; an unpublished word ends the run and the
    // next round starts there.  (The rows before tile 0 read as an
    // inclusive 0: a round that reaches them ends.)
    if (tid < kRadix) {
        uint32_t before = 0;
        if (tile > 0) {
            int64_t t = (int64_t)tile - 1;
            while (true) {
                uint32_t sv[kLookback];
#pragma unroll
                for (int k = 0; k < kLookback; ++k) sv[k] = ld_agent(state + (t - k) * kRadix + tid);
                bool live = true, done = false;
                uint32_t adv = 0;
#pragma unroll
                for (int q = 0; q < kLookback; ++q) {
                    const uint32_t v = sv[q];
                    const bool inc = live && (v & 0x80000000u) != 0u;
                    const bool own = live && v != 0u && (v & 0x80000000u) == 0u;
                    before += own ? v - 1u : (inc ? (v & 0x7FFFFFFFu) : 0u);
                    adv += own ? 1u : 0u;
                    done = done || inc;
                    live = own;
                }
                if (done) break;
                t -= adv;
                if (adv == 0) __builtin_amdgcn_s_sleep(1);
            }
            st_agent(state + (int64_t)tile * kRadix + tid, 0x80000000u | (before + count));
        }
        const uint32_t base = bin_base[tid] + before;
        // replay table: slot i of bin b goes to global position base_b + i
        s_off[tid] = base - start;
        tab_base[(int64_t)tile * kRadix + tid] = base - start;
        tab_start[(int64_t)tile * kRadix + tid] = (uint16_t)start;
    }
    __syncthreads();

    // Consecutive slots of one digit go to consecutive global positions;
    // the first value row goes out with its keys.
    float* vout0 = VALS && !PAIR_OUT ? vals.out[0] : nullptr;
#pragma unroll
    for (int q = 0; q < kSortItems; ++q) {
        const uint32_t i = (uint32_t)(q * kSortThreads + tid);
        const uint2 kv = VALS ? s_kv[i] : make_uint2(s_buf[i], 0u);
        const uint32_t k = kv.x;
        const uint32_t dst = s_off[(k >> shift) & 0xFFu] + i;
        if (dst < (uint32_t)n) {
            if (PAIR_OUT) {
                kv_out[dst] = kv;
            } else {
                if (LAST) sorted_out[dst] = float_of_key(k);
                else keys_out[dst] = k;
                if (VALS) vout0[dst] = __uint_as_float(kv.y);
            }
        }
    }
    // Further value rows: loaded like the keys, placed in the same slots,
    // written to the destinations of the keys still held in the slots.
    if (VALS) {
        for (int r = 1; r < vals.rows; ++r) {
            const float* vin = vals.in[r] + wbase;
            float v[kSortItems];
            if (room == (uint32_t)(kSortItems * kWave)) {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) v[j] = vin[j * kWave + lane];
            } else {
#pragma unroll
                for (int j = 0; j < kSortItems; ++j) {
                    const uint32_t off = (uint32_t)(j * kWave + lane);
                    v[j] = off < room ? vin[off] : 0.f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) s_kv[pos[j]].y = __float_as_uint(v[j]);
            __syncthreads();
            float* vout = vals.out[r];
#pragma unroll
            for (int q = 0; q < kSortItems; ++q) {
                const uint32_t i = (uint32_t)(q * kSortThreads + tid);
                const uint2 kv = s_kv[i];
                const uint32_t dst = s_off[(kv.x >> shift) & 0xFFu] + i;
                if (dst < (uint32_t)n) vout[dst] = __uint_as_float(kv.y);
            }
        }
    }
}

// Scratch layout (bytes, each region 256-byte aligned):
//   keysA, keysB               : uint32[n] each
//   hist, base                 : uint32[4][256] each
//   tickets                    : uint32[4] (padded to 64)
//   state                      : uint32[4][kLookback + tiles][256] (kLookback rows of
//                                inclusive 0 before each pass's tile 0)
//   pairB (with value rows)    : uint2[n]; pairA overlays keysA + keysB
static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t sort_scratch_bytes(int64_t n, bool with_vals)
{
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    size_t b = 2 * align256((size_t)n * 4);
    b += 2 * align256(4 * kRadix * 4);
    b += align256(64 * 4);
    b += align256((size_t)4 * (tiles + kLookback) * kRadix * 4);
    if (with_vals) b += align256((size_t)n * 8);
    return b;
}

size_t sort_record_bytes(int64_t n)
{
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    return 4 * (align256((size_t)tiles * kSortTile * 2) + align256((size_t)tiles * kRadix * 4) +
                align256((size_t)tiles * kRadix * 2));
}

SortRecords sort_records_at(void* base, int64_t n)
{
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    SortRecords r;
    r.n = n;
    r.tiles = tiles;
    char* p = (char*)base;
    for (int k = 0; k < 4; ++k) {
        r.rec[k] = (uint16_t*)p; p += align256((size_t)tiles * kSortTile * 2);
        r.base[k] = (uint32_t*)p; p += align256((size_t)tiles * kRadix * 4);
        r.start[k] = (uint16_t*)p; p += align256((size_t)tiles * kRadix * 2);
    }
    return r;
}

hipError_t sort_launch(const float* a, int64_t n, float* sorted, const SortRecords& R, void* scratch,
                       uint32_t* flag, hipStream_t s, const SortVals* vals)
{
    if (n <= 0) return hipSuccess;
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    char* p = (char*)scratch;
    uint32_t* keysA = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* keysB = (uint32_t*)p; p += align256((size_t)n * 4);
    uint32_t* hist = (uint32_t*)p; p += align256(4 * kRadix * 4);
    uint32_t* base = (uint32_t*)p; p += align256(4 * kRadix * 4);
    uint32_t* tickets = (uint32_t*)p; p += align256(64 * 4);
    uint32_t* state = (uint32_t*)p; p += align256((size_t)4 * (tiles + kLookback) * kRadix * 4);
    // key-value pairs (with value rows): keysA and keysB together hold one
    // array of n pairs, the region after the look-back state the other
    uint2* pairA = reinterpret_cast<uint2*>(keysA);
    uint2* pairB = reinterpret_cast<uint2*>(p);

    // hist, base and tickets are contiguous with the state: one launch clears
    // them all and writes the inclusive-0 rows before each pass's tile 0
    const int64_t head_words = (int64_t)((char*)state - (char*)hist) / 4;
    const int64_t pass_words = (tiles + kLookback) * kRadix;
    {
        const int64_t words = head_words + 4 * pass_words;
        int64_t blocks = (words + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        LX_LAUNCH("util_fill", s, (lx_sort_clear<<<(int)blocks, 256, 0, s>>>(hist, head_words, pass_words)));
    }

    {
        int64_t blocks = (n + kHistThreads * 64 - 1) / (kHistThreads * 64);
        if (blocks > 2048) blocks = 2048;
        LX_LAUNCH("sort_hist", s, (lx_sort_hist<<<(int)blocks, kHistThreads, 0, s>>>(a, n, hist, flag)));
    }
    LX_LAUNCH("sort_scan_hist", s, (lx_sort_scan_hist<<<4, kRadix, 0, s>>>(hist, base)));

    // value rows: pass 0 reads the caller's rows, then ping-pong va -> vb -> va -> vb
    const bool hv = vals && vals->rows > 0;
    if (hv && vals->rows > kMaxSortVals) return hipErrorInvalidValue;
    SortValPass vp[4];
    if (hv) {
        float* const ping[4] = {vals->va, vals->vb, vals->va, vals->vb};
        for (int k = 0; k < 4; ++k) {
            vp[k].rows = vals->rows;
            for (int r = 0; r < vals->rows; ++r) {
                vp[k].in[r] = k == 0 ? vals->in[r] : ping[k - 1] + (int64_t)r * vals->ld;
                vp[k].out[r] = ping[k] + (int64_t)r * vals->ld;
            }
        }
    }
    const int grid = (int)tiles;
    const uint32_t* kin[4] = {nullptr, keysA, keysB, keysA};
    uint32_t* kout[4] = {keysA, keysB, keysA, nullptr};
    const uint2* pin[4] = {nullptr, pairA, pairB, pairA};
    uint2* pout[4] = {pairA, pairB, pairA, nullptr};
    for (int k = 0; k < 4; ++k) {
#define LX_PASS(F, L, V)                                                                                      \
    LX_LAUNCH("sort_pass", s,                                                                                 \
              (lx_sort_pass<F, L, V><<<grid, kSortThreads, 0, s>>>(                                          \
                  k == 0 ? a : nullptr, kin[k], kout[k], hv ? pin[k] : nullptr, hv ? pout[k] : nullptr,       \
                  k == 3 ? sorted : nullptr, R.rec[k], R.base[k],                                            \
                  R.start[k], base + k * kRadix, state + k * pass_words + kLookback * kRadix, tickets + k, 8 * k, n, vp[k])))
        if (hv) {
            if (k == 0) LX_PASS(true, false, true);
            else if (k == 3) LX_PASS(false, true, true);
            else LX_PASS(false, false, true);
        } else {
            if (k == 0) LX_PASS(true, false, false);
            else if (k == 3) LX_PASS(false, true, false);
            else LX_PASS(false, false, false);
        }
#undef LX_PASS
    }
    return hipSuccess;
}

// -------------------------------------------------------------- replay
//
// The four passes above factor the sorting permutation into four tile-local
// partitions.  Replaying them moves any array into sorted order (forward)
// or back into original order (backward) with coalesced reads and writes:
// a workgroup stages one 8192-element tile in LDS and copies slot i of bin
// b between tile position rec[i] and global position base_b + i.  Slots are
// dealt to threads in stripes (slot q*512 + tid), so consecutive lanes touch
// consecutive global positions of a bin's run.  The bin of each slot comes
// from a prefix maximum over the slots of markers set at each non-empty
// bin's first slot.

constexpr int kReplayItems = kSortTile / kSortThreads;  // 16

template <typename T, bool FWD, bool IOTA>
__global__ __launch_bounds__(kSortThreads, 6) void lx_replay(const T* __restrict__ in, int64_t in_ld,
                                                         T* __restrict__ out, int64_t out_ld,
                                                         const uint16_t* __restrict__ rec,
                                                         const uint32_t* __restrict__ tab_base,
                                                         const uint16_t* __restrict__ tab_start, int64_t n,
                                                         int64_t batch)
{
    __shared__ __align__(16) T buf[kSortTile];
    uint8_t* sbin = reinterpret_cast<uint8_t*>(buf);  // bin of each slot, used before buf holds data
    __shared__ uint32_t sbase[kRadix];
    __shared__ uint32_t sred[kSortWaves];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / kWave;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // grid = tiles
    const int64_t t0 = tile * kSortTile;

    uint32_t src[kReplayItems];
#pragma unroll
    for (int q = 0; q < kReplayItems; ++q) src[q] = rec[t0 + q * kSortThreads + tid];
    constexpr int kVec = kReplayItems / 16;  // uint4 words of slot bins per thread
    static_assert(kReplayItems % 16 == 0, "slots per thread must be a multiple of 16");
#pragma unroll
    for (int k = 0; k < kVec; ++k) reinterpret_cast<uint4*>(sbin)[tid * kVec + k] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t st = 0, nx = 0;
    if (tid < kRadix) {
        sbase[tid] = tab_base[tile * kRadix + tid];
        st = tab_start[tile * kRadix + tid];
        nx = tid + 1 < kRadix ? tab_start[tile * kRadix + tid + 1] : (uint32_t)kSortTile;
    }
    __syncthreads();
    if (tid < kRadix && nx > st) sbin[st] = (uint8_t)tid;  // first slot of a non-empty bin
    __syncthreads();
    {
        // inclusive prefix max over slots; thread tid scans its kReplayItems consecutive slots
        uint32_t word[4 * kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const uint4 raw = reinterpret_cast<const uint4*>(sbin)[tid * kVec + k];
            word[4 * k] = raw.x;
            word[4 * k + 1] = raw.y;
            word[4 * k + 2] = raw.z;
            word[4 * k + 3] = raw.w;
        }
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < kReplayItems; ++k) m = max(m, (word[k >> 2] >> (8 * (k & 3))) & 0xFFu);
        uint32_t inc = m;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d);
            if (lane >= d) inc = max(inc, o);
        }
        if (lane == kWave - 1) sred[w] = inc;
        uint32_t ex = __shfl_up(inc, 1);
        if (lane == 0) ex = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortWaves; ++i)
            if (i < w) ex = max(ex, sred[i]);
        uint32_t run = ex;
#pragma unroll
        for (int k = 0; k < kReplayItems; ++k) {
            const uint32_t sh = 8 * (k & 3);
            run = max(run, (word[k >> 2] >> sh) & 0xFFu);
            word[k >> 2] = (word[k >> 2] & ~(0xFFu << sh)) | (run << sh);
        }
#pragma unroll
        for (int k = 0; k < kVec; ++k)
            reinterpret_cast<uint4*>(sbin)[tid * kVec + k] =
                make_uint4(word[4 * k], word[4 * k + 1], word[4 * k + 2], word[4 * k + 3]);
    }
    __syncthreads();
    uint32_t dst[kReplayItems];
#pragma unroll
    for (int q = 0; q < kReplayItems; ++q) {
        const uint32_t i = (uint32_t)(q * kSortThreads + tid);
        dst[q] = sbase[sbin[i]] + i;
    }
    __syncthreads();  // the bin map is dead: buf takes over its bytes
    for (int64_t v = 0; v < batch; ++v) {
        const T* iv = in + v * in_ld;
        T* ov = out + v * out_ld;
        // Every load of a step is issued before any of its values is used
        // (whole tiles load unconditionally, gathers through a clamped index):
        // a use next to a load inside a bounds branch makes each load wait
        // for itself.
        if (FWD) {
            static_assert(sizeof(T) == 4, "32-bit elements");
            if (!IOTA && t0 + kSortTile <= n && ((uintptr_t)(iv + t0) & 15) == 0) {
                // whole aligned tile: four 16-byte loads per thread, lanes contiguous
                const uint4* src4 = reinterpret_cast<const uint4*>(iv + t0);
                uint4 w4[kReplayItems / 4];
#pragma unroll
                for (int q = 0; q < kReplayItems / 4; ++q) w4[q] = src4[q * kSortThreads + tid];
#pragma unroll
                for (int q = 0; q < kReplayItems / 4; ++q) reinterpret_cast<uint4*>(buf)[q * kSortThreads + tid] = w4[q];
            } else {
                // ragged or unaligned tile: rounds of 8 loads in flight
                constexpr int kHalf = kReplayItems / 2;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    T val[kHalf];
#pragma unroll
                    for (int q = 0; q < kHalf; ++q) {
                        const int64_t j = t0 + (h * kHalf + q) * kSortThreads + tid;
                        val[q] = IOTA ? (T)j : iv[j < n ? j : n - 1];
                    }
#pragma unroll
                    for (int q = 0; q < kHalf; ++q) buf[(h * kHalf + q) * kSortThreads + tid] = val[q];
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kReplayItems; ++q)
                if (dst[q] < (uint32_t)n) ov[dst[q]] = buf[src[q]];
        } else {
            T val[kReplayItems];
#pragma unroll
            for (int q = 0; q < kReplayItems; ++q) val[q] = iv[dst[q] < (uint32_t)n ? dst[q] : (uint32_t)(n - 1)];
#pragma unroll
            for (int q = 0; q < kReplayItems; ++q)
                if (dst[q] < (uint32_t)n) buf[src[q]] = val[q];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kReplayItems; ++q) {
                const int j = q * kSortThreads + tid;
                if (t0 + j < n) ov[t0 + j] = buf[j];
            }
        }
        __syncthreads();
    }
}

// Replay of two neighbouring tiles per workgroup.  For each bin the runs of
// tiles t and t+1 are adjacent in the sorted-side array (t+1's run starts
// where t's ends), so dealing the two tiles' slots out together -- bin by
// bin, t's slots first -- turns each pair of runs into one run twice as
// long: half as many partly covered cache lines at the seams, and about
// half as many distinct lines per wave access.  In merged order, slot m of
// bin b sits at global position mbase_b + m with
// mbase_b = base_b(t) - start_b(t+1).
constexpr int kPairThreads = 2 * kSortThreads;          // 1024: one half per tile
constexpr int kPairItems = 2 * kSortTile / kPairThreads;  // 16 merged slots per thread

// Shared memory of a pair replay: first the maps (per-tile bin of each slot;
// merged source and bin of each merged slot), then the two tiles' data, in
// the same 64 KB.
struct PairShared {
    __align__(16) uint32_t words[2 * kSortTile];
    uint32_t start[2][kRadix + 1];
    uint32_t mbase[kRadix];
    uint32_t red[2 * kSortWaves];
};

// Builds the merged order of tiles t0 and t0 + 1 (ntile of them exist) and
// returns, for merged slot m = q * kPairThreads + tid, its tile-pair
// position src = tile * kSortTile + position (two per word in srcp) and its global
// position dst (0xFFFFFFFF past the pair's slots).  A slot past the pair
// (one tile only) gets src = m, a position of the absent second tile.  Slots
// whose dst is n or more hold the padding of the last tile: every pass sorts
// the padding (maximal keys, after every real element of the last tile)
// behind all real elements, so their tile positions lie past the tile's
// valid range as well.  Ends with a barrier after which `words` is free for
// data.
__device__ __forceinline__ void pair_maps(PairShared& S, const uint16_t* __restrict__ rec,
                                          const uint32_t* __restrict__ tab_base,
                                          const uint16_t* __restrict__ tab_start, int64_t t0, int ntile,
                                          uint32_t (&srcp)[kPairItems / 2], uint32_t (&dst)[kPairItems])
{
    uint8_t* sbin = reinterpret_cast<uint8_t*>(S.words);               // [2][kSortTile]
    uint16_t* msrc = reinterpret_cast<uint16_t*>(sbin + 2 * kSortTile);  // [2 kSortTile]
    uint8_t* mbin = reinterpret_cast<uint8_t*>(msrc + 2 * kSortTile);    // [2 kSortTile]
    static_assert(2 * kSortTile + 4 * kSortTile + 2 * kSortTile <= (int)sizeof(S.words), "map layout");
    static_assert(2 * kSortTile <= 65536, "tile-pair positions are packed in 16 bits");
    static_assert(kPairThreads * 16 == 2 * kSortTile && kSortThreads * 16 == kSortTile,
                  "each thread clears and scans 16 bytes of the bin maps");
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int h = tid / kSortThreads;  // tile of the pair this thread maps
    const int ht = tid % kSortThreads;
    const int wh = ht / kWave;         // wave within the half

    // this thread's slots of its own tile: records (tile positions)
    uint32_t pos[kReplayItems];
    if (h < ntile) {
#pragma unroll
        for (int q = 0; q < kReplayItems; ++q) pos[q] = rec[(t0 + h) * kSortTile + q * kSortThreads + ht];
    }
    reinterpret_cast<uint4*>(sbin)[tid] = make_uint4(0u, 0u, 0u, 0u);  // 16 B per thread: both tiles' bin maps
    if (ht < kRadix) {
        const bool have = h < ntile;
        S.start[h][ht] = have ? tab_start[(t0 + h) * kRadix + ht] : 0u;
        if (ht == 0) S.start[h][kRadix] = have ? (uint32_t)kSortTile : 0u;
    }
    __syncthreads();
    if (ht < kRadix && h < ntile) {
        const uint32_t st = S.start[h][ht], nx = S.start[h][ht + 1];
        if (nx > st) sbin[h * kSortTile + st] = (uint8_t)ht;  // first slot of a non-empty bin
        if (h == 0) S.mbase[ht] = tab_base[t0 * kRadix + ht] - S.start[1][ht];
    }
    __syncthreads();
    {
        // inclusive prefix max over each tile's slots; thread ht of half h
        // scans slots 16 ht .. 16 ht + 15 of tile h
        uint4 raw = reinterpret_cast<const uint4*>(sbin + h * kSortTile)[ht];
        uint32_t word[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) m = max(m, (word[k >> 2] >> (8 * (k & 3))) & 0xFFu);
        uint32_t inc = m;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d);
            if (lane >= d) inc = max(inc, o);
        }
        if (lane == kWave - 1) S.red[h * kSortWaves + wh] = inc;
        uint32_t ex = __shfl_up(inc, 1);
        if (lane == 0) ex = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortWaves; ++i)
            if (i < wh) ex = max(ex, S.red[h * kSortWaves + i]);
        uint32_t run = ex;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t sh = 8 * (k & 3);
            run = max(run, (word[k >> 2] >> sh) & 0xFFu);
            word[k >> 2] = (word[k >> 2] & ~(0xFFu << sh)) | (run << sh);
        }
        reinterpret_cast<uint4*>(sbin + h * kSortTile)[ht] = make_uint4(word[0], word[1], word[2], word[3]);
    }
    __syncthreads();
    // merged slot of each of this thread's slots: slot i of bin b of tile 0
    // -> i + start_b(1); of tile 1 -> i + start_{b+1}(0)
    if (h < ntile) {
#pragma unroll
        for (int q = 0; q < kReplayItems; ++q) {
            const uint32_t i = (uint32_t)(q * kSortThreads + ht);
            const uint32_t b = sbin[h * kSortTile + i];
            const uint32_t m = i + (h == 0 ? S.start[1][b] : S.start[0][b + 1]);
            msrc[m] = (uint16_t)(pos[q] + (uint32_t)h * kSortTile);
            mbin[m] = (uint8_t)b;
        }
    }
    __syncthreads();
    const uint32_t total = (uint32_t)(ntile * kSortTile);
#pragma unroll
    for (int q = 0; q < kPairItems; ++q) {
        const uint32_t m = (uint32_t)(q * kPairThreads + tid);
        const uint32_t sq = m < total ? msrc[m] : m;  // past the pair: the absent tile's own slot
        if (q % 2 == 0) srcp[q / 2] = sq;
        else srcp[q / 2] |= sq << 16;
        dst[q] = m < total ? S.mbase[mbin[m]] + m : 0xFFFFFFFFu;
    }
    __syncthreads();  // the maps are dead: the tiles' data takes over their bytes
}

// Forward: the two tiles' data are read whole into LDS, each merged slot is
// written to its global position (a scattered run per bin).
template <typename T, bool IOTA>
__global__ __launch_bounds__(kPairThreads, 8) void lx_replay_fwd2(const T* __restrict__ in, int64_t in_ld,
                                                              T* __restrict__ out, int64_t out_ld,
                                                              const uint16_t* __restrict__ rec,
                                                              const uint32_t* __restrict__ tab_base,
                                                              const uint16_t* __restrict__ tab_start, int64_t n,
                                                              int64_t tiles, int64_t batch)
{
    static_assert(sizeof(T) == 4, "32-bit elements");
    __shared__ PairShared S;
    T* buf = reinterpret_cast<T*>(S.words);  // [2][kSortTile], after the maps
    const int tid = threadIdx.x;
    const int h = tid / kSortThreads;
    const int ht = tid % kSortThreads;
    const int64_t pairs = (tiles + 1) / 2;
    const int64_t t0 = 2 * xcd_tile(blockIdx.x, pairs);
    const int ntile = t0 + 1 < tiles ? 2 : 1;

    // The first vector's half of the tile, loaded before the maps are built
    // so that its latency overlaps them (raw buffer loads over the tile's
    // valid range: 32-bit lane offsets; reads past the range return 0, and
    // their slots go past n).
    auto tile_rsrc = [&](const T* iv) {
        const int64_t base = (t0 + h) * kSortTile;
        const int64_t valid = n - base < kSortTile ? n - base : kSortTile;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(iv + base), (short)0, (int)(valid * 4), 0x00020000);
    };
    T pre[kReplayItems];
    if (h < ntile) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(in);
#pragma unroll
        for (int q = 0; q < kReplayItems; ++q) {
            const int off = q * kSortThreads + ht;
            if (IOTA) pre[q] = (T)((t0 + h) * kSortTile + off);
            else pre[q] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(rs, off * 4, 0, 0));
        }
    }
    uint32_t srcp[kPairItems / 2], dst[kPairItems];  // sources two per word
    pair_maps(S, rec, tab_base, tab_start, t0, ntile, srcp, dst);
    for (int64_t v = 0; v < batch; ++v) {
        const T* iv = in + v * in_ld;
        T* ov = out + v * out_ld;
        if (h < ntile) {
            if (v == 0) {
#pragma unroll
                for (int q = 0; q < kReplayItems; ++q) buf[h * kSortTile + q * kSortThreads + ht] = pre[q];
            } else {
                // rounds of eight loads, all of a round in flight before any is stored
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(iv);
                constexpr int kHalf = kReplayItems / 2;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    T val[kHalf];
#pragma unroll
                    for (int q = 0; q < kHalf; ++q) {
                        const int off = (r * kHalf + q) * kSortThreads + ht;
                        if (IOTA) val[q] = (T)((t0 + h) * kSortTile + off);
                        else val[q] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(rs, off * 4, 0, 0));
                    }
#pragma unroll
                    for (int q = 0; q < kHalf; ++q) buf[h * kSortTile + (r * kHalf + q) * kSortThreads + ht] = val[q];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPairItems; ++q) {
            const uint32_t sq = (srcp[q / 2] >> (16 * (q % 2))) & 0xFFFFu;
            if (dst[q] < (uint32_t)n) ov[dst[q]] = buf[sq];  // sq = tile * kSortTile + position
        }
        __syncthreads();
    }
}

// Backward: each merged slot is read from its global position (one run per
// bin), placed in LDS at its tile position, and the two tiles, which are
// neighbours in the original order, are written out as one block.
template <typename T>
__global__ __launch_bounds__(kPairThreads, 8) void lx_replay_bwd2(const T* __restrict__ in, int64_t in_ld,
                                                              T* __restrict__ out, int64_t out_ld,
                                                              const uint16_t* __restrict__ rec,
                                                              const uint32_t* __restrict__ tab_base,
                                                              const uint16_t* __restrict__ tab_start, int64_t n,
                                                              int64_t tiles, int64_t batch)
{
    static_assert(sizeof(T) == 4, "32-bit elements");
    __shared__ PairShared S;
    T* buf = reinterpret_cast<T*>(S.words);  // [2][kSortTile], after the maps
    const int tid = threadIdx.x;
    const int64_t pairs = (tiles + 1) / 2;
    const int64_t t0 = 2 * xcd_tile(blockIdx.x, pairs);
    const int ntile = t0 + 1 < tiles ? 2 : 1;
    uint32_t srcp[kPairItems / 2], dst[kPairItems];
    pair_maps(S, rec, tab_base, tab_start, t0, ntile, srcp, dst);
    const int64_t p0 = t0 * kSortTile;
    const int64_t valid = n - p0 < 2 * kSortTile ? n - p0 : 2 * kSortTile;
    for (int64_t v = 0; v < batch; ++v) {
        const T* iv = in + v * in_ld;
        T* ov = out + v * out_ld;
        // rounds of eight gathers, all of a round in flight before any is
        // stored; a slot past the pair or past n reads a valid element and
        // leaves it in a part of buf that is never stored
        constexpr int kHalf = kPairItems / 2;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            T val[kHalf];
#pragma unroll
            for (int q = 0; q < kHalf; ++q) {
                const uint32_t d = dst[r * kHalf + q];
                // a 32-bit byte offset from a uniform base (n < 2^30 + 1 fits)
                const uint32_t off = (d < (uint32_t)n ? d : (uint32_t)(n - 1)) * (uint32_t)sizeof(T);
                val[q] = *reinterpret_cast<const T*>(reinterpret_cast<const char*>(iv) + off);
            }
#pragma unroll
            for (int q = 0; q < kHalf; ++q) {
                const int k = r * kHalf + q;
                buf[(srcp[k / 2] >> (16 * (k % 2))) & 0xFFFFu] = val[q];
            }
        }
        __syncthreads();
        if (valid == 2 * kSortTile && ((uintptr_t)(ov + p0) & 15) == 0) {
            // whole aligned pair: four 16-byte stores per thread, lanes contiguous
            uint4* o4 = reinterpret_cast<uint4*>(ov + p0);
#pragma unroll
            for (int q = 0; q < 2 * kSortTile / 4 / kPairThreads; ++q)
                o4[q * kPairThreads + tid] = reinterpret_cast<const uint4*>(buf)[q * kPairThreads + tid];
        } else {
#pragma unroll
            for (int q = 0; q < kPairItems; ++q) {
                const int j = q * kPairThreads + tid;
                if (j < valid) ov[p0 + j] = buf[j];
            }
        }
        __syncthreads();
    }
}

hipError_t replay_launch(const SortRecords& R, int pass, bool forward, const float* in, int64_t in_ld,
                         float* out, int64_t out_ld, int64_t batch, hipStream_t s)
{
    if (R.n <= 0 || batch <= 0) return hipSuccess;
    const unsigned grid = (unsigned)R.tiles;
    if (forward && R.tiles >= 2)
        LX_LAUNCH("replay_forward", s,
                  (lx_replay_fwd2<float, false><<<(unsigned)((R.tiles + 1) / 2), kPairThreads, 0, s>>>(
                      in, in_ld, out, out_ld, R.rec[pass], R.base[pass], R.start[pass], R.n, R.tiles, batch)));
    else if (forward)
        LX_LAUNCH("replay_forward", s,
                  (lx_replay<float, true, false><<<grid, kSortThreads, 0, s>>>(
                      in, in_ld, out, out_ld, R.rec[pass], R.base[pass], R.start[pass], R.n, batch)));
    else if (R.tiles >= 2)
        LX_LAUNCH("replay_backward", s,
                  (lx_replay_bwd2<float><<<(unsigned)((R.tiles + 1) / 2), kPairThreads, 0, s>>>(
                      in, in_ld, out, out_ld, R.rec[pass], R.base[pass], R.start[pass], R.n, R.tiles, batch)));
    else
        LX_LAUNCH("replay_backward", s,
                  (lx_replay<float, false, false><<<grid, kSortThreads, 0, s>>>(
                      in, in_ld, out, out_ld, R.rec[pass], R.base[pass], R.start[pass], R.n, batch)));
    return hipSuccess;
}

hipError_t perm_from_records(const SortRecords& R, uint32_t* perm, uint32_t* tmp, hipStream_t s)
{
    if (R.n <= 0) return hipSuccess;
    const unsigned grid = (unsigned)R.tiles;
    // iota -> tmp -> perm -> tmp -> perm: after pass k the array holds, at each
    // pass-k output position, the original index of the element there.
    uint32_t* bufs[4] = {tmp, perm, tmp, perm};
    if (R.tiles >= 2) {
        const unsigned pairs = (unsigned)((R.tiles + 1) / 2);
        LX_LAUNCH("perm_replay", s,
                  (lx_replay_fwd2<uint32_t, true><<<pairs, kPairThreads, 0, s>>>(
                      nullptr, 0, bufs[0], 0, R.rec[0], R.base[0], R.start[0], R.n, R.tiles, 1)));
        for (int k = 1; k < 4; ++k)
            LX_LAUNCH("perm_replay", s,
                      (lx_replay_fwd2<uint32_t, false><<<pairs, kPairThreads, 0, s>>>(
                          bufs[k - 1], 0, bufs[k], 0, R.rec[k], R.base[k], R.start[k], R.n, R.tiles, 1)));
        return hipSuccess;
    }
    LX_LAUNCH("perm_replay", s,
              (lx_replay<uint32_t, true, true><<<grid, kSortThreads, 0, s>>>(
                  nullptr, 0, bufs[0], 0, R.rec[0], R.base[0], R.start[0], R.n, 1)));
    for (int k = 1; k < 4; ++k)
        LX_LAUNCH("perm_replay", s,
                  (lx_replay<uint32_t, true, false><<<grid, kSortThreads, 0, s>>>(
                      bufs[k - 1], 0, bufs[k], 0, R.rec[k], R.base[k], R.start[k], R.n, 1)));
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
