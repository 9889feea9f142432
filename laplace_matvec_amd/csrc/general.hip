// General case a != b (gfx950).
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2:
// the contributions of one anchor set are collected into the intervals of
// the other, sorted, set (vectors u and v) and then propagated with the
// symmetric scan.  With outputs on sorted anchors s and an input at anchor q
// with value x, and t = #{r : s_r < q} (so q lies in (s_{t-1}, s_t]):
//     u_t     += exp(-(s_t - q)) x      reaches every rank >= t via L,
//     v_{t-1} += exp(-(q - s_{t-1})) x  reaches every rank <= t-1 via R,
// so each output receives the input exactly once, including ties q = s_r.
// For gradients the ties are also summed apart (tie_t += x for q = s_t):
// the signed product leaves them out.
//
// Kernels here:
//   lx_bucket_layout + lx_bucket_sorted + lx_bucket_reduce : u, v when the
//                      sorted output side is small (up to 1024 anchors):
//                      once per call, a stable counting sort of input
//                      sub-chunks by interval with the factors in slot
//                      order; then per group of vectors, register
//                      accumulation by an owner thread per anchor; the
//                      per-workgroup partials summed in a fixed order;
//   (a long sorted output side takes the merge-path bucketing of merge.hip);
//   lx_eval_rows / lx_eval : the transposed reading of the same identity:
//                      with the scan run over the sorted INPUT side (PL =
//                      prefix, PR = suffix, both inclusive), an output at
//                      anchor o with t = #{s_j < o} is
//                        exp(-(o - s_{t-1})) PL_{t-1} + exp(-(s_t - o)) PR_t,
//                      evaluated for every output in its original order (no
//                      sort or scatter of the output side); lx_eval_rows
//                      when the tables of 8 vectors fit in LDS.
// The cos/sin split of a phased operator (cos(p - q) = cos p cos q +
// sin p sin q) gives two channels: inputs scaled by cos q_j and sin q_j,
// outputs combined with cos p_i and sin p_i.
#include "lx_device.h"
#include "lx_internal.h"

namespace lx {

constexpr int kGenThreads = 1024;

// ------------------------------------------------------------- bucketing

// Sorted bucketing for a small sorted output side (n_out <= 1024), in two
// kernels.  The input side is cut into sub-chunks of 2048 inputs.
//
// lx_bucket_layout (once per call, one workgroup per sub-chunk): each
// input's interval t = #{s < q} (lookup table, below), then a stable
// counting sort of the sub-chunk by t (wave ballots give the rank among
// equal t in index order, integer LDS counters the offsets).  It records,
// per input, its slot in interval order; per sub-chunk and interval, the
// slot where the interval starts; and, in slot order, each input's factors
// alpha = exp(-(s_t - q)) and beta = exp(-(q - s_{t-1})) times the cos and
// sin of its phase.  Inputs past the end go to a bin after the last
// interval, so they are never visited.
//
// lx_bucket_sorted (per group of 4 vectors, one workgroup per group and
// chunk of sub-chunks, two workgroups per CU, the groups of a chunk on one die so
// that they share its layout through that die's L2): the values of the
// group's vectors are placed in LDS by slot, and thread j owns u_j and v_j of every vector in
// registers: it adds the alpha parts of interval j and the beta parts of
// interval j+1, slot by slot (LDS reads and FMAs only).  No
// float atomics, and a fixed summation order, so results are deterministic.
//
// The search, the sort and the factors depend on the anchors and phases
// only, so doing them once instead of once per vector group leaves the
// group kernel two barriers per sub-chunk and no transcendental work.
constexpr int kSub = 2048;                      // inputs per sub-chunk
constexpr int kSubItems = kSub / kGenThreads;   // 2 per thread
constexpr int kGenWaves = kGenThreads / kWave;  // 16
constexpr int kBucketVG = 8;                    // vectors per workgroup (at most)
constexpr int kBinStride = 1032;                // per-wave counter row: bins 0 .. n_out + 1 (<= 1025), padded

__device__ __forceinline__ uint64_t match_bits11(uint32_t d) { return match_bits<11>(d); }

constexpr int kLut = 4096;  // cells of the interval lookup table (lower_bound_lut)
constexpr int kEvalOuts = 4;  // outputs per thread and step of lx_eval_rows

// Layout arrays in the scratch (bytes, each region 256-byte aligned):
//   slot  : uint16[n_in]           slot of each input inside its sub-chunk
//   start : uint16[subs][stride]   first slot of each bin t = 0 .. n_out + 1
//   coef  : float4[subs * kSub]    by slot: (alpha cos, alpha sin, beta cos, beta sin)
//   tie   : uint8[subs * kSub]     by slot, gradients only: 1 where the input equals s_t
struct BucketLayout {
    uint16_t* slot;
    uint16_t* start;
    float4* coef;
    uint8_t* tie;
    int64_t stride;
};

static inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

static BucketLayout bucket_layout_at(void* base, int64_t n_in, int64_t n_out, bool ties)
{
    const int64_t subs = (n_in + kSub - 1) / kSub;
    BucketLayout L;
    L.stride = (n_out + 2 + 7) & ~(int64_t)7;
    char* p = (char*)base;
    L.slot = (uint16_t*)p; p += al256((size_t)n_in * 2);
    L.start = (uint16_t*)p; p += al256((size_t)subs * L.stride * 2);
    L.coef = (float4*)p; p += al256((size_t)subs * kSub * 16);
    L.tie = ties ? (uint8_t*)p : nullptr;
    return L;
}

int64_t bucket_layout_bytes(const BucketArgs& a)
{
    const int64_t subs = (a.n_in + kSub - 1) / kSub;
    const int64_t stride = (a.n_out + 2 + 7) & ~(int64_t)7;
    return (int64_t)(al256((size_t)a.n_in * 2) + al256((size_t)subs * stride * 2) + al256((size_t)subs * kSub * 16) +
                     (a.ties ? al256((size_t)subs * kSub) : 0));
}

template <int C>
__global__ __launch_bounds__(kGenThreads) void lx_bucket_layout(BucketArgs A, BucketLayout L)
{
    __shared__ float so[kGenThreads];
    __shared__ uint16_t wcnt[kGenWaves][kBinStride];  // per-wave counts, then each wave's first slot
    __shared__ uint32_t start[kBinStride];
    __shared__ uint16_t tab[kLut + 1];
    __shared__ uint32_t sred[kGenWaves];

    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int no = (int)A.n_out;
    const int nbins = no + 2;  // intervals 0 .. no, and the bin of inputs past the end
    const int64_t sub = blockIdx.x;
    const int64_t sub0 = sub * kSub;
    for (int i = tid; i < no; i += kGenThreads) so[i] = A.s_out[i];
    for (int i = tid; i < kGenWaves * kBinStride; i += kGenThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const float lo_v = so[0], hi_v = so[no - 1];
    const float width = (hi_v - lo_v) / (float)kLut;
    const float inv_w = width > 0.f ? 1.f / width : 0.f;
    for (int k = tid; k <= kLut; k += kGenThreads)
        tab[k] = (uint16_t)(k == kLut ? no : lower_bound_f(so, no, lo_v + (float)k * width));

    // items wave-striped: element sub0 + 128 w + 64 j + lane
    int64_t idx[kSubItems];
    float q[kSubItems], fc[kSubItems], fs[kSubItems];
    uint32_t tt[kSubItems], slot[kSubItems];
#pragma unroll
    for (int j = 0; j < kSubItems; ++j) {
        idx[j] = sub0 + w * (kSubItems * kWave) + j * kWave + lane;
        const int64_t ic = idx[j] < A.n_in ? idx[j] : A.n_in - 1;
        q[j] = A.in_anchor[ic];
        if (C == 2) {
            fc[j] = A.in_cos[ic];
            fs[j] = A.in_sin[ic];
        }
    }
    __syncthreads();  // tab complete
#pragma unroll
    for (int j = 0; j < kSubItems; ++j)
        tt[j] = idx[j] < A.n_in ? lower_bound_lut<kLut>(so, no, tab, lo_v, inv_w, q[j]) : (uint32_t)(no + 1);
    // stable rank among equal bins: per wave, items in (j, lane) order
#pragma unroll
    for (int j = 0; j < kSubItems; ++j) {
        const uint64_t peers = match_bits11(tt[j]);
        const uint32_t below = count_below(peers);
        const uint32_t prev = wcnt[w][tt[j]];
        slot[j] = prev + below;
        if (below == 0) wcnt[w][tt[j]] = (uint16_t)(prev + (uint32_t)__popcll(peers));
    }
    __syncthreads();
    // per bin: offsets of the waves and the sub-chunk count; bins past the
    // block size (at most two) follow the block's exclusive sum
    uint32_t cnt = 0;
    for (int b = tid; b < nbins; b += kGenThreads) {
        uint32_t c[kGenWaves];
#pragma unroll
        for (int ww = 0; ww < kGenWaves; ++ww) c[ww] = wcnt[ww][b];
        uint32_t run = 0;
#pragma unroll
        for (int ww = 0; ww < kGenWaves; ++ww) {
            wcnt[ww][b] = (uint16_t)run;
            run += c[ww];
        }
        if (b == tid) cnt = run;
        else start[b] = run;  // count for now
    }
    uint32_t tot;
    const uint32_t ex = block_exsum_u32<kGenWaves>(cnt, sred, tot);
    if (tid < nbins) start[tid] = ex;
    __syncthreads();
    if (tid == 0) {
        uint32_t run = tot;
        for (int b = kGenThreads; b < nbins; ++b) {
            const uint32_t c = start[b];
            start[b] = run;
            run += c;
        }
    }
    __syncthreads();
    uint16_t* st = L.start + sub * L.stride;
    for (int b = tid; b < nbins; b += kGenThreads) st[b] = (uint16_t)start[b];
#pragma unroll
    for (int j = 0; j < kSubItems; ++j) {
        if (idx[j] < A.n_in) {
            const uint32_t t = tt[j];
            const uint32_t sl = start[t] + wcnt[w][t] + slot[j];
            const float f0 = C == 2 ? fc[j] : 1.f, f1 = C == 2 ? fs[j] : 0.f;
            const float al = t < (uint32_t)no ? decay_f(q[j], so[t], A.inv_t) : 0.f;
            const float be = t > 0 ? decay_f(so[t - 1], q[j], A.inv_t) : 0.f;
            L.slot[idx[j]] = (uint16_t)sl;
            L.coef[sub0 + sl] = make_float4(al * f0, al * f1, be * f0, be * f1);
            if (L.tie) L.tie[sub0 + sl] = (t < (uint32_t)no && so[t] == q[j]) ? 1 : 0;
        }
    }
}

// VGT vectors per workgroup (8, or 4: half the LDS, so that two workgroups
// share a CU and one's loads overlap the other's accumulation)
template <int C, bool TIES, int VGT>
__global__ __launch_bounds__(kGenThreads, VGT == 4 ? 8 : 4) void lx_bucket_sorted(BucketArgs A, BucketLayout L, int VG,
                                                                                 int groups, int64_t chunks,
                                                                                 int64_t chunk_len)
{
    extern __shared__ float lds[];
    constexpr int XW = VGT / 4;  // float4 words of vector values per slot
    const int no = (int)A.n_out;  // <= kGenThreads
    // intervals 0 .. no: thread t owns interval t; interval no has no thread
    // of its own when no == kGenThreads and goes to thread 0
    const bool last_extra = no == kGenThreads && threadIdx.x == 0;
    float4* xs = reinterpret_cast<float4*>(lds);                // [kSub][XW]: the vectors by slot
    float4* cs = xs + XW * kSub;                                // [kSub]: factors by slot
    uint8_t* ts = reinterpret_cast<uint8_t*>(cs + kSub);        // [kSub]: tie flags by slot (TIES)

    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    int g;
    int64_t chunk;
    if (!die_chunk_group(blockIdx.x, chunks, groups, &chunk, &g)) return;  // uniform
    const int64_t v0 = (int64_t)g * VG;
    const int nv = (int)((A.batch - v0) < VG ? (A.batch - v0) : VG);

    float au[VGT][C], av[VGT][C];  // u_tid and v_tid of each vector
    float at[TIES ? VGT : 1][C];         // tie_tid
#pragma unroll
    for (int vi = 0; vi < VGT; ++vi)
#pragma unroll
        for (int c = 0; c < C; ++c) au[vi][c] = av[vi][c] = 0.f;
#pragma unroll
    for (int vi = 0; vi < (TIES ? VGT : 1); ++vi)
#pragma unroll
        for (int c = 0; c < C; ++c) at[vi][c] = 0.f;

    const int64_t j0 = chunk * chunk_len;
    int64_t j1 = j0 + chunk_len;
    if (j1 > A.n_in) j1 = A.n_in;

    // One sub-chunk's inputs, loaded one sub-chunk ahead: the values of the
    // group's vectors and the slot of this thread's items (element
    // sub0 + 128 w + 64 j + lane), the factors (and tie flags) of slots
    // 128 w + 64 j + lane, and the starts of intervals tid .. tid + 2.
    // (Slots, flags and starts stay narrow until used: a widening next to
    // the load would make the accumulation wait for the whole prefetch.)
    float xin[kSubItems][VGT];
    float cfn[kSubItems][4];
    uint8_t tfn[TIES ? kSubItems : 1];
    uint16_t sln[kSubItems], stn[4];
    auto load_sub = [&](int64_t base) {
        const int64_t sub = base / kSub;
#pragma unroll
        for (int j = 0; j < kSubItems; ++j) {
            const int p = w * (kSubItems * kWave) + j * kWave + lane;
            const int64_t id = base + p;
            const int64_t idc = id < j1 ? id : j0;  // a valid address; the value is not used
#pragma unroll
            for (int vi = 0; vi < VGT; ++vi) {
                const int64_t vv = v0 + (vi < nv ? vi : 0);
                xin[j][vi] = A.x[vv * A.n_in + idc];
            }
            sln[j] = L.slot[idc];
            const float4 cf = L.coef[base + p];
            cfn[j][0] = cf.x;
            cfn[j][1] = cf.y;
            cfn[j][2] = cf.z;
            cfn[j][3] = cf.w;
            if (TIES) tfn[j] = L.tie[base + p];
        }
        const uint16_t* st = L.start + sub * L.stride;
        stn[0] = st[tid < no + 2 ? tid : 0];
        stn[1] = st[tid + 1 < no + 2 ? tid + 1 : 0];
        // thread 0 also owns interval no when no == kGenThreads (no thread no)
        stn[2] = st[last_extra ? no : 0];
        stn[3] = st[last_extra ? no + 1 : 0];
    };
    // With eight vectors (one workgroup per CU) the next sub-chunk loads
    // during this one's accumulation; with four, the other workgroup on the
    // CU covers the load, and the registers a load ahead would hold are
    // better left free (general n=2^26, k=1024, 64 phased vectors: 6.3 ->
    // 5.8 ms, and the form with tie sums stays clear of spills).
    constexpr bool kAhead = VGT != 4;
    if (kAhead && j0 < j1) load_sub(j0);
    for (int64_t sub0 = j0; sub0 < j1; sub0 += kSub) {
        if (!kAhead) load_sub(sub0);
        __syncthreads();  // the previous sub-chunk's slots have been read
#pragma unroll
        for (int j = 0; j < kSubItems; ++j) {
            const int p = w * (kSubItems * kWave) + j * kWave + lane;
            if (sub0 + p < j1) {
                const uint32_t sl = sln[j];
                float x8[VGT];
#pragma unroll
                for (int vi = 0; vi < VGT; ++vi) x8[vi] = vi < nv ? xin[j][vi] : 0.f;
#pragma unroll
                for (int q = 0; q < XW; ++q)
                    xs[XW * sl + q] = make_float4(x8[4 * q], x8[4 * q + 1], x8[4 * q + 2], x8[4 * q + 3]);
            }
            cs[p] = make_float4(cfn[j][0], cfn[j][1], cfn[j][2], cfn[j][3]);
            if (TIES) ts[p] = tfn[TIES ? j : 0];
        }
        bool tied = false;  // any input of this sub-chunk equal to an output anchor
        if (TIES) {
#pragma unroll
            for (int j = 0; j < kSubItems; ++j) tied = tied || tfn[TIES ? j : 0] != 0;
        }
        const uint32_t s0 = stn[0], s1 = stn[1], e0 = stn[2], e1 = stn[3];
        tied = TIES ? __syncthreads_or(tied ? 1 : 0) != 0 : (__syncthreads(), false);
        if (kAhead && sub0 + kSub < j1) load_sub(sub0 + kSub);
        // interval tid: every slot read once, its alpha part into u_tid and
        // its beta part into v_{tid-1} (interval 0 has no beta part); the
        // tie sums only in sub-chunks that hold a tie (a uniform branch)
        if (tid <= no) {
            for (uint32_t sl = s0; sl < s1; ++sl) {
                const float4 f = cs[sl];
                float xv[VGT];
#pragma unroll
                for (int q = 0; q < XW; ++q) {
                    const float4 xq = xs[XW * sl + q];
                    xv[4 * q] = xq.x;
                    xv[4 * q + 1] = xq.y;
                    xv[4 * q + 2] = xq.z;
                    xv[4 * q + 3] = xq.w;
                }
#pragma unroll
                for (int vi = 0; vi < VGT; ++vi) {
                    au[vi][0] = fmaf(f.x, xv[vi], au[vi][0]);
                    if (C == 2) au[vi][C - 1] = fmaf(f.y, xv[vi], au[vi][C - 1]);
                    av[vi][0] = fmaf(f.z, xv[vi], av[vi][0]);
                    if (C == 2) av[vi][C - 1] = fmaf(f.w, xv[vi], av[vi][C - 1]);
                }
                if (TIES && tied) {  // a tie's alpha is exactly 1: its factors are the phase's cos, sin
                    const float tw = ts[sl] ? 1.f : 0.f;
#pragma unroll
                    for (int vi = 0; vi < (TIES ? VGT : 1); ++vi) {
                        at[vi][0] = fmaf(tw * f.x, xv[vi], at[vi][0]);
                        if (C == 2) at[vi][C - 1] = fmaf(tw * f.y, xv[vi], at[vi][C - 1]);
                    }
                }
            }
        }
        // interval no when no == kGenThreads: its beta parts are v_{no-1},
        // kept by thread 0 (whose own interval 0 has none)
        for (uint32_t sl = e0; sl < e1; ++sl) {
            const float2 f = *reinterpret_cast<const float2*>(&cs[sl].z);
            float xv[VGT];
#pragma unroll
            for (int q = 0; q < XW; ++q) {
                const float4 xq = xs[XW * sl + q];
                xv[4 * q] = xq.x;
                xv[4 * q + 1] = xq.y;
                xv[4 * q + 2] = xq.z;
                xv[4 * q + 3] = xq.w;
            }
#pragma unroll
            for (int vi = 0; vi < VGT; ++vi) {
                av[vi][0] = fmaf(f.x, xv[vi], av[vi][0]);
                if (C == 2) av[vi][C - 1] = fmaf(f.y, xv[vi], av[vi][C - 1]);
            }
        }
    }
    // partial layout [chunk][batch][C][P][no], P = 2 (u, v) or 3 (u, v, tie)
    constexpr int P = TIES ? 3 : 2;
    // this thread's v index: v_{tid-1}, or v_{no-1} for thread 0 when it
    // kept interval no
    const int vt = tid > 0 ? tid - 1 : (last_extra ? no - 1 : -1);
#pragma unroll
    for (int vi = 0; vi < VGT; ++vi)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (vi >= nv) continue;
            float* pp = A.partial + ((chunk * A.batch + v0 + vi) * C + c) * P * no;
            if (tid < no) {
                pp[tid] = au[vi][c];
                if (TIES) pp[2 * no + tid] = at[TIES ? vi : 0][c];
            }
            if (vt >= 0 && vt < no) pp[no + vt] = av[vi][c];
        }
}

static size_t bucket_sorted_lds(int64_t no, int C, bool ties, int vg = kBucketVG)
{
    (void)no;
    (void)C;
    return (size_t)kSub * 4 * (vg <= 4 ? 4 : 8) + (size_t)kSub * 16 + (ties ? (size_t)kSub : 0);
}

// Vectors per bucketing workgroup.  Four (32 KB of vector slots, 64 VGPRs):
// two workgroups share a CU and one's loads overlap the other's
// accumulation; general n=2^26, k=1024, 64 phased vectors: 8.0 -> 5.8 ms,
// and with the tie sums of a gradient 10.9 -> 8.2 ms.
static int bucket_vg(bool ties) { return (void)ties, 4; }

// Sums the per-workgroup partials in chunk order (float64) into u, v and,
// with P = 3, the tie sums.
__global__ __launch_bounds__(256) void lx_bucket_reduce(const float* __restrict__ partial, int64_t chunks,
                                                       int64_t batch, int C, int P, int64_t no, int64_t ld,
                                                       float* __restrict__ u, float* __restrict__ v,
                                                       float* __restrict__ tie)
{
    const int64_t total = batch * C * P * no;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        double acc = 0.0;
        for (int64_t ch = 0; ch < chunks; ++ch) acc += (double)partial[ch * total + i];
        const int64_t t = i % no;
        int64_t rest = i / no;
        const int w = (int)(rest % P);
        rest /= P;
        const int64_t c = rest % C;
        const int64_t vv = rest / C;
        (w == 0 ? u : (w == 1 ? v : tie))[(c * batch + vv) * ld + t] = (float)acc;
    }
}

static void bucket_shape(const BucketArgs& a, int* vg, int* groups, int* chunks, int64_t* chunk_len)
{
    const int vmax = bucket_vg(a.ties);
    const bool fits = a.n_out <= kGenThreads && a.lds_bytes > 0 &&
                      (int64_t)bucket_sorted_lds(a.n_out, a.channels, a.ties, vmax) <= a.lds_bytes;
    if (!fits) {
        *vg = 0;
        *groups = *chunks = 0;
        *chunk_len = 0;
        return;
    }
    int64_t v = vmax;
    if (v > a.batch) v = a.batch;
    *vg = (int)v;
    *groups = (int)((a.batch + v - 1) / v);
    // chunks of whole sub-chunks, about 512 workgroups in all
    int64_t subs = (a.n_in + kSub - 1) / kSub;
    if (subs < 1) subs = 1;
    int64_t c = (512 + *groups - 1) / *groups;
    if (c > subs) c = subs;
    if (c < 1) c = 1;
    const int64_t per = (subs + c - 1) / c;
    *chunk_len = per * kSub;
    *chunks = (int)((a.n_in + *chunk_len - 1) / *chunk_len);
    if (*chunks < 1) *chunks = 1;
}

int64_t bucket_partial_floats(const BucketArgs& a, int* groups, int* chunks)
{
    int vg, g, c;
    int64_t cl;
    bucket_shape(a, &vg, &g, &c, &cl);
    if (groups) *groups = g;
    if (chunks) *chunks = c;
    if (vg == 0) return 0;
    return (int64_t)c * a.batch * a.channels * (a.ties ? 3 : 2) * a.n_out;
}

hipError_t bucket_launch(BucketArgs& a, hipStream_t s)
{
    if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
    int vg, groups, chunks;
    int64_t chunk_len;
    bucket_shape(a, &vg, &groups, &chunks, &chunk_len);
    const bool two = a.channels == 2;
    const bool ties = a.ties;
    if (ties && !a.tie) return hipErrorInvalidValue;
    if (vg > 0 && a.partial && a.layout && a.n_in > 0) {
        const size_t shmem = bucket_sorted_lds(a.n_out, a.channels, ties, vg);
        const unsigned blocks = (unsigned)die_chunk_group_blocks(chunks, groups);
        const BucketLayout L = bucket_layout_at(a.layout, a.n_in, a.n_out, ties);
        const unsigned subs = (unsigned)((a.n_in + kSub - 1) / kSub);
        if (two) LX_LAUNCH("bucket_layout", s, (lx_bucket_layout<2><<<subs, kGenThreads, 0, s>>>(a, L)));
        else LX_LAUNCH("bucket_layout", s, (lx_bucket_layout<1><<<subs, kGenThreads, 0, s>>>(a, L)));
#define LX_BKS1(CC, TT, VV)                                                                                    \
    do {                                                                                                       \
        (void)hipFuncSetAttribute((const void*)lx_bucket_sorted<CC, TT, VV>,                                   \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);                     \
        LX_LAUNCH("bucket_sorted", s,                                                                          \
                  (lx_bucket_sorted<CC, TT, VV><<<blocks, kGenThreads, shmem, s>>>(a, L, vg, groups, chunks,   \
                                                                                   chunk_len)));               \
    } while (0)
#define LX_BKS(CC, TT) LX_BKS1(CC, TT, 4)
        if (two) {
            if (ties) LX_BKS(2, true);
            else LX_BKS(2, false);
        } else {
            if (ties) LX_BKS(1, true);
            else LX_BKS(1, false);
        }
#undef LX_BKS
#undef LX_BKS1
        const int P = ties ? 3 : 2;
        const int64_t total = a.batch * a.channels * P * a.n_out;
        int64_t rb = (total + 255) / 256;
        if (rb > 8192) rb = 8192;
        LX_LAUNCH("bucket_reduce", s,
                  (lx_bucket_reduce<<<(unsigned)rb, 256, 0, s>>>(a.partial, chunks, a.batch, a.channels, P,
                                                                 a.n_out, a.ld, a.u, a.v, a.tie)));
        return hipSuccess;
    }
    // not the LDS-binned shape: the caller runs merge-path bucketing instead
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------- evaluation

// Evaluation with the tables of a group of up to 8 vectors in LDS.  Row t
// (t = 0 .. n_in) holds, per vector, PL_{t-1} and PR_t of both channels
// side by side (zero outside the tables), so an output whose interval is
// t reads one 16-byte entry per vector; rows are padded to 36 words so
// that the rows of different outputs spread over the LDS banks.  The
// interval comes from a lookup table over the sorted inputs, and each
// thread takes four outputs per step, whose loads, searches and decays
// overlap.

template <int C>
__global__ __launch_bounds__(kGenThreads) void lx_eval_rows(EvalArgs A, int VG, int groups, int64_t chunks,
                                                           int64_t chunk_len)
{
    extern __shared__ float lds[];
    constexpr int RW = eval_row_words<C>();
    const int ni = (int)A.n_in;
    int g;
    int64_t chunk;
    if (!die_chunk_group(blockIdx.x, chunks, groups, &chunk, &g)) return;  // uniform
    const int64_t v0 = (int64_t)g * VG;
    const int nv = (int)((A.batch - v0) < VG ? (A.batch - v0) : VG);
    float* si = lds;                                                  // [ni]
    float* rows = lds + pad64(ni);                                    // [ni + 1][RW]
    uint16_t* tab = reinterpret_cast<uint16_t*>(rows + (int64_t)(ni + 1) * RW);  // [kEvalLut + 1]
    const int tid = threadIdx.x;
    for (int i = tid; i < ni; i += kGenThreads) si[i] = A.s_in[i];
    // entry (t, vi): PL_{t-1} of channels 0, 1 then PR_t of channels 0, 1
    // (C == 2), or PL_{t-1}, PR_t (C == 1); tables read along t (coalesced)
    constexpr int E = 2 * C;  // words per entry
    for (int t = tid; t <= ni; t += kGenThreads) {
        // all of this t's entries loaded before any is stored
        float lv[kEvalVG * C], rv[kEvalVG * C];
#pragma unroll
        for (int rowc = 0; rowc < kEvalVG * C; ++rowc) {
            const int vi = rowc / C, c = rowc % C;
            const bool have = vi < nv;
            const int64_t src = ((int64_t)c * A.batch + v0 + (have ? vi : 0)) * A.ld;
            lv[rowc] = have && t > 0 ? A.pl[src + t - 1] : 0.f;
            rv[rowc] = have && t < ni ? A.pr[src + t] : 0.f;
        }
#pragma unroll
        for (int rowc = 0; rowc < kEvalVG * C; ++rowc) {
            float* e = rows + (int64_t)t * RW + (rowc / C) * E;
            e[rowc % C] = lv[rowc];
            e[C + rowc % C] = rv[rowc];
        }
    }
    __syncthreads();
    const float lo_v = si[0], hi_v = si[ni - 1];
    const float width = (hi_v - lo_v) / (float)kEvalLut;
    const float inv_w = width > 0.f ? 1.f / width : 0.f;
    for (int k = tid; k <= kEvalLut; k += kGenThreads)
        tab[k] = (uint16_t)(k == kEvalLut ? ni : lower_bound_f(si, ni, lo_v + (float)k * width));
    __syncthreads();

    const int64_t i0 = chunk * chunk_len;
    int64_t i1 = i0 + chunk_len;
    if (i1 > A.n_out) i1 = A.n_out;
    const int64_t last = i1 > i0 ? i1 - 1 : i0;
    // kEvalOuts outputs per thread per step (i, i + 1024, ...): their loads,
    // searches and decays are independent, so their latencies overlap
    for (int64_t ib = i0 + tid; ib < i1; ib += (int64_t)kEvalOuts * kGenThreads) {
        float o[kEvalOuts], gc[kEvalOuts][C];
#pragma unroll
        for (int u = 0; u < kEvalOuts; ++u) {
            const int64_t k = ib + (int64_t)u * kGenThreads;
            const int64_t kc = k < i1 ? k : last;
            o[u] = A.out_anchor[kc];
            gc[u][0] = C == 2 ? A.out_cos[kc] : 1.f;
            if (C == 2) gc[u][C - 1] = A.out_sin[kc];
        }
        int t[kEvalOuts];
#pragma unroll
        for (int u = 0; u < kEvalOuts; ++u) t[u] = (int)lower_bound_lut<kEvalLut>(si, ni, tab, lo_v, inv_w, o[u]);
        float al[kEvalOuts], be[kEvalOuts];
#pragma unroll
        for (int u = 0; u < kEvalOuts; ++u) {
            al[u] = t[u] > 0 ? decay_f(si[t[u] - 1], o[u], A.inv_t) : 0.f;
            be[u] = t[u] < ni ? decay_f(o[u], si[t[u]], A.inv_t) : 0.f;
        }
        // every value of the step first (a vector past nv reads its zero
        // table entries), then the stores: a table read whose only use is a
        // guarded store is otherwise moved behind the guard, one LDS wait
        // per value instead of one for all of them
        float outv[kEvalVG][kEvalOuts];
#pragma unroll
        for (int vi = 0; vi < kEvalVG; ++vi) {
#pragma unroll
            for (int u = 0; u < kEvalOuts; ++u) {
                const float* row = rows + (int64_t)t[u] * RW;
                float lv[C], rv[C];
                if (C == 2) {
                    const float4 e = *reinterpret_cast<const float4*>(row + vi * E);
                    lv[0] = e.x;
                    lv[C - 1] = e.y;
                    rv[0] = e.z;
                    rv[C - 1] = e.w;
                } else {
                    const float2 e = *reinterpret_cast<const float2*>(row + vi * E);
                    lv[0] = e.x;
                    rv[0] = e.y;
                }
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) acc = fmaf(gc[u][c], fmaf(al[u], lv[c], be[u] * rv[c]), acc);
                outv[vi][u] = acc;
            }
        }
#pragma unroll
        for (int vi = 0; vi < kEvalVG; ++vi)
#pragma unroll
            for (int u = 0; u < kEvalOuts; ++u) asm volatile("" : "+v"(outv[vi][u]));
#pragma unroll
        for (int vi = 0; vi < kEvalVG; ++vi) {
            if (vi >= nv) continue;
#pragma unroll
            for (int u = 0; u < kEvalOuts; ++u) {
                const int64_t k = ib + (int64_t)u * kGenThreads;
                if (k < i1) A.y[(v0 + vi) * A.n_out + k] = outv[vi][u];
            }
        }
    }
}


template <int C, bool USE_LDS>
__global__ __launch_bounds__(kGenThreads) void lx_eval(EvalArgs A, int VG, int groups, int64_t chunks,
                                                      int64_t chunk_len)
{
    extern __shared__ float lds[];
    const int64_t ni = A.n_in;
    int g;
    int64_t chunk;
    if (!die_chunk_group(blockIdx.x, chunks, groups, &chunk, &g)) return;  // uniform
    const int64_t v0 = (int64_t)g * VG;
    const int nv = (int)((A.batch - v0) < VG ? (A.batch - v0) : VG);
    const float* si = A.s_in;
    float* tl = nullptr;  // [ni][VG][C]
    float* tr = nullptr;
    if (USE_LDS) {
        float* s_l = lds;
        tl = lds + pad64(ni);
        tr = tl + ni * VG * C;
        for (int64_t i = threadIdx.x; i < ni; i += kGenThreads) s_l[i] = A.s_in[i];
        // rows of the tables in global memory are read along t (coalesced)
        for (int64_t i = threadIdx.x; i < ni * VG * C; i += kGenThreads) {
            const int64_t row = i / ni;  // vi * C + c
            const int64_t t = i - row * ni;
            const int64_t vi = row / C;
            const int64_t c = row - vi * C;
            const int64_t src = (c * A.batch + v0 + vi) * A.ld + t;
            const int64_t dst = (t * VG + vi) * C + c;
            tl[dst] = vi < nv ? A.pl[src] : 0.f;
            tr[dst] = vi < nv ? A.pr[src] : 0.f;
        }
        __syncthreads();
        si = s_l;
    }
    const int64_t i0 = chunk * chunk_len;
    int64_t i1 = i0 + chunk_len;
    if (i1 > A.n_out) i1 = A.n_out;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += kGenThreads) {
        const float o = A.out_anchor[i];
        const int64_t t = lower_bound_f(si, ni, o);
        const float al = t > 0 ? decay_f(si[t - 1], o, A.inv_t) : 0.f;
        const float be = t < ni ? decay_f(o, si[t], A.inv_t) : 0.f;
        float gc[C];
        gc[0] = C == 2 ? A.out_cos[i] : 1.f;
        if (C == 2) gc[C - 1] = A.out_sin[i];
        for (int vi = 0; vi < nv; ++vi) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                float lv = 0.f, rv = 0.f;
                if (USE_LDS) {
                    if (t > 0) lv = tl[((t - 1) * VG + vi) * C + c];
                    if (t < ni) rv = tr[(t * VG + vi) * C + c];
                } else {
                    const int64_t row = ((int64_t)c * A.batch + v0 + vi) * A.ld;
                    if (t > 0) lv = A.pl[row + t - 1];
                    if (t < ni) rv = A.pr[row + t];
                }
                acc = fmaf(gc[c], fmaf(al, lv, be * rv), acc);
            }
            A.y[(v0 + vi) * A.n_out + i] = acc;
        }
    }
}

hipError_t eval_launch(const EvalArgs& a, hipStream_t s)
{
    if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
    if (a.n_in >= 1 && a.n_in <= 0xFFFF && a.lds_bytes > 0 &&
        eval_rows_lds(a.n_in, a.channels) <= (size_t)a.lds_bytes) {
        // groups of at most 8 vectors, as even as possible
        const int64_t groups = (a.batch + kEvalVG - 1) / kEvalVG;
        const int vg = (int)((a.batch + groups - 1) / groups);
        int64_t chunks = (a.n_out + 16383) / 16384;
        const int64_t cap = (2048 + groups - 1) / groups;
        if (chunks > cap) chunks = cap;
        if (chunks < 1) chunks = 1;
        const int64_t chunk_len = (a.n_out + chunks - 1) / chunks;
        chunks = (a.n_out + chunk_len - 1) / chunk_len;
        const unsigned blocks = (unsigned)die_chunk_group_blocks(chunks, (int)groups);
        const size_t shmem = eval_rows_lds(a.n_in, a.channels);
        if (a.channels == 2) {
            (void)hipFuncSetAttribute((const void*)lx_eval_rows<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
            LX_LAUNCH("eval", s, (lx_eval_rows<2><<<blocks, kGenThreads, shmem, s>>>(a, vg, (int)groups, chunks, chunk_len)));
        } else {
            (void)hipFuncSetAttribute((const void*)lx_eval_rows<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
            LX_LAUNCH("eval", s, (lx_eval_rows<1><<<blocks, kGenThreads, shmem, s>>>(a, vg, (int)groups, chunks, chunk_len)));
        }
        return hipSuccess;
    }
    const int64_t lds_floats = a.lds_bytes / 4;
    int64_t vg = (lds_floats - pad64(a.n_in)) / (2 * (int64_t)a.channels * (a.n_in > 0 ? a.n_in : 1));
    if (vg > 16) vg = 16;
    if (vg > a.batch) vg = a.batch;
    const bool use_lds = a.lds_bytes > 0 && vg >= 1;
    if (!use_lds) vg = a.batch < 16 ? a.batch : 16;
    const int groups = (int)((a.batch + vg - 1) / vg);
    int64_t chunks = (a.n_out + 16383) / 16384;
    const int64_t cap = (2048 + groups - 1) / groups;
    if (chunks > cap) chunks = cap;
    if (chunks < 1) chunks = 1;
    const int64_t chunk_len = (a.n_out + chunks - 1) / chunks;
    chunks = (a.n_out + chunk_len - 1) / chunk_len;
    const unsigned blocks = (unsigned)die_chunk_group_blocks(chunks, groups);
    const size_t shmem = use_lds ? (size_t)(pad64(a.n_in) + 2 * vg * a.channels * a.n_in) * 4 : 0;
    const int v = (int)vg;
#define LX_EVAL(CC, LL)                                                                                  \
    do {                                                                                                 \
        if (LL) (void)hipFuncSetAttribute((const void*)lx_eval<CC, LL>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem); \
        LX_LAUNCH("eval", s, (lx_eval<CC, LL><<<blocks, kGenThreads, shmem, s>>>(a, v, groups, chunks, chunk_len))); \
    } while (0)
    if (a.channels == 2) {
        if (use_lds) LX_EVAL(2, true);
        else LX_EVAL(2, false);
    } else {
        if (use_lds) LX_EVAL(1, true);
        else LX_EVAL(1, false);
    }
#undef LX_EVAL
    return hipSuccess;
}

}  // namespace lx
