// Merge-path bucketing of a long sorted input side into the intervals of a
// long sorted output side (gfx950).
//
// Technical summary of "LAPLEX: The FFT of Learnable Laplace Kernels", §2.2,
// general case: an input at anchor q with value x and t = #{r : s_r < q}
// (s the sorted outputs) contributes exp(-(s_t - q)) x to u_t and
// exp(-(q - s_{t-1})) x to v_{t-1}; the scans over the outputs then finish
// the product.  With the inputs sorted too, t never decreases along them, so
// the inputs of one interval form one run.  Merging the two sorted sequences
// (an input before an output of equal value, which is the rule t = #{s < q})
// places each interval's run just before the output that closes it: run t
// ends at output t, and the run after the last output is interval n_out.
//
// The merged sequence is cut into tiles of kMergeTile items by merge-path
// search, so every workgroup gets the same work whatever the two
// distributions.  Inside a tile each thread walks 8 consecutive merged
// items; the run sums cross threads by a segmented scan (a run ends at an
// output), and cross tiles through per-tile records finished by a second
// segmented scan over the tiles.  Sums are float64 in a fixed order (set by
// the sizes alone), so the result does not depend on scheduling.
//
//   lx_merge_split  : inputs and outputs before every tile boundary;
//   lx_merge_bucket : per tile and group of vectors, u_t and v_{t-1} for every
//                     output of the tile except its first, the first one's
//                     partial sums (head) and the sums after the tile's last
//                     output (tail);
//   lx_merge_carry  : per vector and channel, the segmented scan of the tile
//                     records: completes each tile's first output and
//                     v_{n_out-1}, the run above every output.
// Every u_t and v_t is written exactly once; nothing needs clearing first.
#include "lx_device.h"
#include "lx_internal.h"
#include "lx_merge.h"

namespace lx {

constexpr int kMergeVG = 8;  // vectors per workgroup (max)

int64_t merge_tiles(int64_t n_in, int64_t n_out) { return (n_in + n_out + kMergeTile - 1) / kMergeTile; }

static inline size_t al256m(size_t b) { return (b + 255) & ~(size_t)255; }

size_t merge_ws_bytes(int64_t n_in, int64_t n_out, int64_t batch, int channels)
{
    const int64_t tiles = merge_tiles(n_in, n_out);
    return al256m((size_t)(tiles + 1) * sizeof(uint2)) + 2 * al256m((size_t)channels * batch * tiles * 2 * 8);
}

__global__ __launch_bounds__(256) void lx_merge_split(MergeArgs A)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k > A.tiles) return;
    const int64_t total = A.n_in + A.n_out;
    const int64_t d = k * kMergeTile < total ? k * kMergeTile : total;
    const int64_t i = merge_search(A.s_in, A.n_in, A.s_out, A.n_out, d);
    A.split[k] = make_uint2((uint32_t)i, (uint32_t)(d - i));
}

template <int C>
__global__ __launch_bounds__(kMergeThreads) void lx_merge_bucket(MergeArgs A, int VG, int groups)
{
    constexpr int K = 2 * C;  // per channel: the alpha (u) and beta (v) sums
    __shared__ float s_in[kMergeTile];
    __shared__ float s_out[kMergeTile];
    __shared__ Aff<double> sh[2 * K * kMergeWaves];
    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x % A.tiles;
    const int64_t g = blockIdx.x / A.tiles;
    const int64_t v0 = g * VG;
    const int nv = (int)(A.batch - v0 < VG ? A.batch - v0 : VG);
    const uint2 b0 = A.split[tile], b1 = A.split[tile + 1];
    const int64_t i0 = b0.x, o0 = b0.y;
    const int ni = (int)(b1.x - b0.x), no = (int)(b1.y - b0.y);
    const int len = ni + no;
    for (int j = tid; j < ni; j += kMergeThreads) s_in[j] = A.s_in[i0 + j];
    for (int j = tid; j < no; j += kMergeThreads) s_out[j] = A.s_out[o0 + j];
    // the outputs just outside the tile: left of its first input, right of its last
    const float left_sent = o0 > 0 ? A.s_out[o0 - 1] : 0.f;
    const float right_sent = o0 + no < A.n_out ? A.s_out[o0 + no] : 0.f;
    __syncthreads();

    // this thread's items: merged positions dk .. dk + 7 of the tile
    const int dk = tid * kMergeItems < len ? tid * kMergeItems : len;
    int ii = (int)merge_search(s_in, ni, s_out, no, dk);
    int oo = dk - ii;
    double al[kMergeItems], be[kMergeItems];
    uint32_t idx[kMergeItems];  // input: rank on the input side; output: its rank
    uint32_t is_in = 0, is_out = 0;
#pragma unroll
    for (int j = 0; j < kMergeItems; ++j) {
        al[j] = be[j] = 0.0;
        idx[j] = 0;
        if (dk + j >= len) continue;
        const bool take_in = ii < ni && (oo >= no || s_in[ii] <= s_out[oo]);
        const int64_t t = o0 + oo;  // outputs before this item
        if (take_in) {
            const float q = s_in[ii];
            const float right = oo < no ? s_out[oo] : right_sent;
            const float left = oo > 0 ? s_out[oo - 1] : left_sent;
            al[j] = t < A.n_out ? decay(q, right, A.inv_t) : 0.0;
            be[j] = t > 0 ? decay(left, q, A.inv_t) : 0.0;
            idx[j] = (uint32_t)(i0 + ii);
            is_in |= 1u << j;
            ++ii;
        } else {
            idx[j] = (uint32_t)t;
            is_out |= 1u << j;
            ++oo;
        }
    }
    // the inputs' original indices and phase factors, once for every vector
    uint32_t src[kMergeItems];
    float fc[kMergeItems], fs[kMergeItems];
#pragma unroll
    for (int j = 0; j < kMergeItems; ++j) {
        const uint32_t r = (is_in >> j) & 1u ? idx[j] : 0u;
        src[j] = A.perm_in[r];
        fc[j] = C == 2 ? A.in_c[r] : 1.f;
        fs[j] = C == 2 ? A.in_s[r] : 0.f;
    }
    const double m = is_out ? 0.0 : 1.0;
    const uint32_t first_j = is_out ? (uint32_t)__builtin_ctz(is_out) : 0u;
    int parity = 0;

#pragma unroll 1
    for (int vi = 0; vi < nv; ++vi) {
        const int64_t vec = v0 + vi;
        const float* xv = A.x + vec * A.n_in;
        float xin[kMergeItems];
#pragma unroll
        for (int j = 0; j < kMergeItems; ++j) xin[j] = (is_in >> j) & 1u ? xv[src[j]] : 0.f;
        double run[K], head[K];
#pragma unroll
        for (int k = 0; k < K; ++k) run[k] = head[k] = 0.0;
#pragma unroll
        for (int j = 0; j < kMergeItems; ++j) {
            if ((is_in >> j) & 1u) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const double val = (double)((c == 0 ? fc[j] : fs[j]) * xin[j]);
                    run[2 * c] = fma(al[j], val, run[2 * c]);
                    run[2 * c + 1] = fma(be[j], val, run[2 * c + 1]);
                }
            } else if ((is_out >> j) & 1u) {
                const int64_t t = idx[j];
                if ((uint32_t)j == first_j) {
#pragma unroll
                    for (int k = 0; k < K; ++k) head[k] = run[k];
                } else {
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const int64_t row = ((int64_t)c * A.batch + vec) * A.ld;
                        A.u[row + t] = (float)run[2 * c];
                        if (t > 0) A.v[row + t - 1] = (float)run[2 * c + 1];
                    }
                }
#pragma unroll
                for (int k = 0; k < K; ++k) run[k] = 0.0;
            }
        }
        double mex, vex[K], vtot[K];
        block_segscan<K>(m, run, sh, parity, mex, vex, vtot);
        parity ^= 1;
        if (is_out) {
            const int64_t t = idx[first_j];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int64_t row = (int64_t)c * A.batch + vec;
                const double su = vex[2 * c] + head[2 * c], sv = vex[2 * c + 1] + head[2 * c + 1];
                if (mex != 0.0) {
                    // the tile's first output: earlier tiles may add to its run
                    double* h = A.head + (row * A.tiles + tile) * 2;
                    h[0] = su;
                    h[1] = sv;
                } else {
                    A.u[row * A.ld + t] = (float)su;
                    if (t > 0) A.v[row * A.ld + t - 1] = (float)sv;
                }
            }
        }
        if (tid == 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                double* tl = A.tail + (((int64_t)c * A.batch + vec) * A.tiles + tile) * 2;
                tl[0] = vtot[2 * c];
                tl[1] = vtot[2 * c + 1];
            }
        }
    }
}

// One workgroup per (channel, vector) row: the tiles in chunks of
// consecutive tiles per thread, the chunks' composites scanned across the
// workgroup, then each thread walks its chunk with the sum entering it.
constexpr int kCarryThreadsM = 256;

__global__ __launch_bounds__(kCarryThreadsM) void lx_merge_carry(MergeArgs A)
{
    __shared__ Aff<double> sh[kCarryThreadsM / kWave];
    const int64_t row = blockIdx.x;  // c * batch + vec
    const int64_t T = A.tiles;
    const int64_t per = (T + kCarryThreadsM - 1) / kCarryThreadsM;
    int64_t t0 = (int64_t)threadIdx.x * per;
    if (t0 > T) t0 = T;
    int64_t t1 = t0 + per;
    if (t1 > T) t1 = T;
    const double* hd = A.head + row * T * 2;
    const double* tl = A.tail + row * T * 2;
    Aff<double> fa = aff_identity<double>(), fb = aff_identity<double>();
    for (int64_t k = t0; k < t1; ++k) {
        const double m = A.split[k + 1].y > A.split[k].y ? 0.0 : 1.0;
        fa = compose(fa, Aff<double>{m, tl[2 * k]});
        fb = compose(fb, Aff<double>{m, tl[2 * k + 1]});
    }
    Aff<double> tota, totb;
    double ca = block_exscan_up<double, kCarryThreadsM / kWave>(fa, sh, tota).v;
    double cb = block_exscan_up<double, kCarryThreadsM / kWave>(fb, sh, totb).v;
    float* u = A.u + row * A.ld;
    float* v = A.v + row * A.ld;
    for (int64_t k = t0; k < t1; ++k) {
        const uint32_t o0 = A.split[k].y;
        const bool has = A.split[k + 1].y > o0;
        if (has) {
            u[o0] = (float)(ca + hd[2 * k]);
            if (o0 > 0) v[o0 - 1] = (float)(cb + hd[2 * k + 1]);
            ca = tl[2 * k];
            cb = tl[2 * k + 1];
        } else {
            ca += tl[2 * k];
            cb += tl[2 * k + 1];
        }
    }
    // the run above every output reaches v_{n_out-1} only
    if (threadIdx.x == 0) v[A.n_out - 1] = (float)totb.v;
}

hipError_t merge_launch(MergeArgs& a, hipStream_t s)
{
    if (a.n_out <= 0 || a.n_in <= 0 || a.batch <= 0) return hipErrorInvalidValue;
    a.tiles = merge_tiles(a.n_in, a.n_out);
    if (a.tiles * ((a.batch + kMergeVG - 1) / kMergeVG) > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned sb = (unsigned)((a.tiles + 1 + 255) / 256);
    LX_LAUNCH("merge_split", s, (lx_merge_split<<<sb, 256, 0, s>>>(a)));
    const int groups = (int)((a.batch + kMergeVG - 1) / kMergeVG);
    const int vg = (int)((a.batch + groups - 1) / groups);
    const unsigned blocks = (unsigned)(a.tiles * groups);
    if (a.channels == 2) LX_LAUNCH("merge_bucket", s, (lx_merge_bucket<2><<<blocks, kMergeThreads, 0, s>>>(a, vg, groups)));
    else LX_LAUNCH("merge_bucket", s, (lx_merge_bucket<1><<<blocks, kMergeThreads, 0, s>>>(a, vg, groups)));
    LX_LAUNCH("merge_carry", s,
              (lx_merge_carry<<<(unsigned)(a.channels * a.batch), kCarryThreadsM, 0, s>>>(a)));
    return hipSuccess;
}

}  // namespace lx
