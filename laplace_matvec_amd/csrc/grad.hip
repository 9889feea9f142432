// Gradients of a LAPLEX product: with respect to the input vector, the
// anchors and the phases (gfx950).
//
// "LAPLEX: The FFT of Learnable Laplace Kernels", technical summary §2.1: the
// operator is a trainable layer whose parameters are its anchors (and
// phases).  For the bilinear form F = sum_v <u_v, K w_v> (u on the row side,
// w on the column side; a training step through y = K x has u = dL/dy,
// w = x, and through y = K^T x has u = x, w = dL/dy) the entrywise
// derivatives of K_ij = exp(-|a_i - b_j| / t) cos(phi_i - psi_j) give
//   dF/da_i   = -(1/t) sum_v u_vi (S w_v)_i,   S_ij = sgn(a_i - b_j) K_ij,
//   dF/dphi_i = -sum_v u_vi (Q w_v)_i,          Q_ij = e_ij sin(phi_i - psi_j),
// and for the column side the same with the roles of the sides swapped
// (sgn(b_j - a_i), sin(psi_j - phi_i), weights w, inputs u).  sgn(0) = 0:
// equal anchors contribute nothing (the mean of the one-sided slopes).
// With the cos/sin split both products are sums of the unphased plain and
// signed products of the two channels (inputs times cos, sin of the input
// phases):
//   S w = c_out S0(c_in w) + s_out S0(s_in w),  Q w = s_out K0(c_in w) - c_out K0(s_in w),
// and the plain product c_out K0(c_in w) + s_out K0(s_in w) is the input
// gradient of the other side.
//
// Symmetric plans work by rank along the sorted anchors.  With L, U the
// inclusive prefix/suffix recurrences of the forward product and Tp, Ts the
// inclusive prefix/suffix sums inside runs of equal anchors (a recurrence
// whose multiplier is 1 between equal neighbours and 0 otherwise),
//   K0 = L + U - x,   S0 = (L - Tp) - (U - Ts),
// since L - Tp keeps exactly the strictly smaller anchors.  Two halves: half
// 0 takes w with the column phases as input and u as weight (row side: da,
// dphi, and the plain product K w); half 1 takes u with the row phases and w
// as weight (column side of the same anchors: da again, dpsi, K^T u).  Same
// reduce / carry / apply structure as the forward scans; the apply loops
// over the vectors of a tile so the batch sums stay in registers.
//
// General plans (a != b) evaluate each side's outputs in their original
// order from the inclusive prefix/suffix tables of the other side (the
// "evaluate" form of the forward product): with t< = #{s < o} and
// t<= = #{s <= o} in the sorted input side,
//   K0 = e(o - s_{t<-1}) PL_{t<-1} + e(s_{t<} - o) PR_{t<},
//   S0 = e(o - s_{t<-1}) PL_{t<-1} - e(s_{t<=} - o) PR_{t<=}.
#include "lx_device.h"
#include "lx_internal.h"
#include "lx_tile.h"

namespace lx {

// ------------------------------------------------------------ symmetric

// Tiles of kScanTile ranks like the forward scans, 8 ranks per thread (the
// gradient keeps four running sums per channel per rank).
constexpr int kGradThreads = 512;
constexpr int kGradItems = 8;
constexpr int kGradWaves = kGradThreads / kWave;
static_assert(kGradThreads * kGradItems == kScanTile, "gradient tile size");

__device__ __forceinline__ int64_t grad_row(int C, int h, int c, int kind, int64_t batch, int64_t vec)
{
    return ((int64_t)((h * C + c) * 2 + kind)) * batch + vec;
}

// Values of both inputs for this thread's ranks: u (row side) and w (column
// side) by rank; in random mode gathered through perm and stored by rank.
template <bool RANDOM>
__device__ __forceinline__ void grad_load_uw(const GradSymArgs& A, int64_t vec, int64_t r0, float (&uu)[kGradItems],
                                             float (&ww)[kGradItems])
{
    const int64_t n = A.n;
    if (RANDOM) {
        uint32_t idx[kGradItems];
        load_run<kGradItems>(A.perm, r0, n, idx);
        const float* up = A.u + vec * n;
        const float* wp = A.w + vec * n;
#pragma unroll
        for (int i = 0; i < kGradItems; ++i) {
            uu[i] = (r0 + i < n) ? up[idx[i]] : 0.f;
            ww[i] = (r0 + i < n) ? wp[idx[i]] : 0.f;
        }
    } else {
        load_run<kGradItems>(A.us + vec * A.ld, r0, n, uu);
        load_run<kGradItems>(A.ws + vec * A.ld, r0, n, ww);
    }
}

// Per-tile totals of several scan rows with one barrier: each wave folds
// its lanes (in lane order for forward rows, reversed for backward rows),
// lane 63 / lane 0 leave the wave's composite in LDS, and after the barrier
// one thread per row folds the waves.
template <int R>
__device__ __forceinline__ void wave_totals(const Aff<double> (&f)[R], const Aff<double> (&b)[R], Aff<double>* sh)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const Aff<double> fi = wave_scan_up(f[r]);
        const Aff<double> bi = wave_scan_down(b[r]);
        if (lane == kWave - 1) sh[(w * R + r) * 2] = fi;
        if (lane == 0) sh[(w * R + r) * 2 + 1] = bi;
    }
}

// Exclusive block scans of two forward rows and two backward rows with one
// barrier.  `sh` holds two buffers of [waves][4] composites used by turns
// (`parity`), so the next call needs no second barrier before writing.
__device__ __forceinline__ void block_exscan4(Aff<double> f0, Aff<double> f1, Aff<double> b0, Aff<double> b1,
                                              Aff<double>* sh, int parity, Aff<double>& xf0, Aff<double>& xf1,
                                              Aff<double>& xb0, Aff<double>& xb1)
{
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    Aff<double>* buf = sh + parity * (kGradWaves * 4);
    const Aff<double> if0 = wave_scan_up(f0), if1 = wave_scan_up(f1);
    const Aff<double> ib0 = wave_scan_down(b0), ib1 = wave_scan_down(b1);
    const Aff<double> ef0 = wave_shift_up(if0), ef1 = wave_shift_up(if1);
    const Aff<double> eb0 = wave_shift_down(ib0), eb1 = wave_shift_down(ib1);
    if (lane == kWave - 1) {
        buf[w * 4 + 0] = if0;
        buf[w * 4 + 1] = if1;
    }
    if (lane == 0) {
        buf[w * 4 + 2] = ib0;
        buf[w * 4 + 3] = ib1;
    }
    __syncthreads();
    Aff<double> pf0 = aff_identity<double>(), pf1 = aff_identity<double>();
    Aff<double> pb0 = aff_identity<double>(), pb1 = aff_identity<double>();
#pragma unroll
    for (int i = 0; i < kGradWaves; ++i) {
        if (i < w) {
            pf0 = compose(pf0, buf[i * 4 + 0]);
            pf1 = compose(pf1, buf[i * 4 + 1]);
        }
    }
#pragma unroll
    for (int i = kGradWaves - 1; i >= 0; --i) {
        if (i > w) {
            pb0 = compose(pb0, buf[i * 4 + 2]);
            pb1 = compose(pb1, buf[i * 4 + 3]);
        }
    }
    xf0 = compose(pf0, ef0);
    xf1 = compose(pf1, ef1);
    xb0 = compose(pb0, eb0);
    xb1 = compose(pb1, eb1);
}

template <int C, bool RANDOM>
__global__ __launch_bounds__(kGradThreads) void lx_grad_sym_reduce(GradSymArgs A)
{
    constexpr int R = 4 * C;  // rows: half h, channel c, kind (decay, tie)
    __shared__ Aff<double> sh[kGradWaves * R * 2];
    const int64_t vec = blockIdx.x / A.tiles;
    const int64_t tile = blockIdx.x - vec * A.tiles;
    const int64_t n = A.n;
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kGradItems;

    double e[kGradItems + 1];
    uint32_t ties;
    load_decays_ties<kGradItems>(A.s, r0, n, A.inv_t, e, ties);
    float uu[kGradItems], ww[kGradItems];
    grad_load_uw<RANDOM>(A, vec, r0, uu, ww);
    if (RANDOM) {
        store_run<kGradItems>(A.us + vec * A.ld, r0, n, uu);
        store_run<kGradItems>(A.ws + vec * A.ld, r0, n, ww);
    }
    Aff<double> fr[R], br[R];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float fc[kGradItems], fs[kGradItems];
        if (C == 2) {
            load_run<kGradItems>(h == 0 ? A.cpsi : A.cphi, r0, n, fc);
            load_run<kGradItems>(h == 0 ? A.spsi : A.sphi, r0, n, fs);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float val[kGradItems];
#pragma unroll
            for (int i = 0; i < kGradItems; ++i) {
                const float in = h == 0 ? ww[i] : uu[i];
                val[i] = C == 2 ? (c == 0 ? fc[i] : fs[i]) * in : in;
            }
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
                Aff<double> f = aff_identity<double>(), b = aff_identity<double>();
#pragma unroll
                for (int i = 0; i < kGradItems; ++i)
                    f = compose(f, Aff<double>{kind == 0 ? e[i] : tie_mult(ties, i), (double)val[i]});
#pragma unroll
                for (int i = kGradItems - 1; i >= 0; --i)
                    b = compose(b, Aff<double>{kind == 0 ? e[i + 1] : tie_mult(ties, i + 1), (double)val[i]});
                fr[(h * C + c) * 2 + kind] = f;
                br[(h * C + c) * 2 + kind] = b;
            }
        }
    }
    wave_totals<R>(fr, br, sh);
    __syncthreads();
    if (threadIdx.x < 2 * R) {
        // thread t folds row t / 2 forward (even t) or backward (odd t) over the waves
        const int row = (int)threadIdx.x / 2, dir = (int)threadIdx.x & 1;
        Aff<double> acc = aff_identity<double>();
        if (dir == 0)
            for (int w = 0; w < kGradWaves; ++w) acc = compose(acc, sh[(w * R + row) * 2]);
        else
            for (int w = kGradWaves - 1; w >= 0; --w) acc = compose(acc, sh[(w * R + row) * 2 + 1]);
        const int h = row / (2 * C), c = (row / 2) % C, kind = row % 2;
        double* ag = A.agg + (grad_row(C, h, c, kind, A.batch, vec) * A.tiles + tile) * 4;
        ag[2 * dir] = acc.m;
        ag[2 * dir + 1] = acc.v;
    }
}

// One per-anchor result: through perm into original order, or by rank.
template <bool RANDOM>
__device__ __forceinline__ void grad_store_out(const GradSymArgs& A, float* dst, int64_t r0,
                                               const float (&val)[kGradItems])
{
    if (!dst) return;
    const int64_t n = A.n;
    if (RANDOM) {
        uint32_t idx[kGradItems];
        load_run<kGradItems>(A.perm, r0, n, idx);
#pragma unroll
        for (int i = 0; i < kGradItems; ++i)
            if (r0 + i < n) dst[idx[i]] = val[i];
    } else {
        store_run<kGradItems>(dst, r0, n, val);
    }
}

// Both halves of the symmetric gradient over one tile.  For every half,
// vector and channel: the decay scan (L forward, U backward) and the tie
// scan (Tp, Ts) over this thread's ranks, entered from the carries,
// combined on the way back into
//   K0 = L + U - x  and  S0 = (L - Tp) - (U - Ts),
// and folded into the batch sums (anchor, phase) and the plain product.
// The anchor sum of both halves stays in registers, the decays are computed
// once per tile, and the second half re-reads the tile's inputs from cache.
// Halves, vectors and channels run in loops that are not unrolled, and the
// decays and tie masks are re-read from LDS in them, which keeps one step's
// state live at a time.  The phased form holds twice the channel state: it
// runs at two waves per SIMD (one workgroup per CU, up to 256 VGPRs), so
// nothing spills; the unphased form fits 128 VGPRs at four.
template <int C, bool RANDOM>
__global__ __launch_bounds__(kGradThreads, C == 2 ? 2 : 4) void lx_grad_sym_apply(GradSymArgs A)
{
    __shared__ Aff<double> sh[2 * kGradWaves * 4];
    int parity = 0;
    __shared__ double se[kScanTile + 1];
    __shared__ uint32_t st[kGradThreads];
    const int64_t tile = blockIdx.x;
    const int64_t n = A.n;
    const int64_t r0 = tile * kScanTile + (int64_t)threadIdx.x * kGradItems;
    {
        double e[kGradItems + 1];
        uint32_t ties;
        load_decays_ties<kGradItems>(A.s, r0, n, A.inv_t, e, ties);
#pragma unroll
        for (int i = 0; i < kGradItems; ++i) se[threadIdx.x * kGradItems + i] = e[i];
        if (threadIdx.x == kGradThreads - 1) se[kScanTile] = e[kGradItems];
        st[threadIdx.x] = ties;
    }
    __syncthreads();
    float g_a[kGradItems];
#pragma unroll
    for (int i = 0; i < kGradItems; ++i) g_a[i] = 0.f;

#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        // half 0: input w with the column phases, weight u, output phases phi;
        // half 1: input u with the row phases, weight w, output phases psi
        const float* in_v = h == 0 ? A.ws : A.us;
        const float* wt_v = h == 0 ? A.us : A.ws;
        const float* icos = h == 0 ? A.cpsi : A.cphi;
        const float* isin = h == 0 ? A.spsi : A.sphi;
        const float* ocos = h == 0 ? A.cphi : A.cpsi;
        const float* osin = h == 0 ? A.sphi : A.spsi;
        const bool want_dx = A.dx != nullptr && A.dx_half == h;
        float g_p[kGradItems];
#pragma unroll
        for (int i = 0; i < kGradItems; ++i) g_p[i] = 0.f;
#pragma unroll 1
        for (int64_t vec = 0; vec < A.batch; ++vec) {
            float dxo[kGradItems];
#pragma unroll
            for (int i = 0; i < kGradItems; ++i) dxo[i] = 0.f;
#pragma unroll 1
            for (int c = 0; c < C; ++c) {
                double e[kGradItems + 1];
#pragma unroll
                for (int i = 0; i <= kGradItems; ++i) e[i] = se[threadIdx.x * kGradItems + i];
                const uint32_t ties = st[threadIdx.x];
                float val[kGradItems], wt[kGradItems], fo[kGradItems], fk[kGradItems];
                load_run<kGradItems>(in_v + vec * A.ld, r0, n, val);
                load_run<kGradItems>(wt_v + vec * A.ld, r0, n, wt);
                if (C == 2) {
                    float fi[kGradItems];
                    load_run<kGradItems>(c == 0 ? icos : isin, r0, n, fi);
                    load_run<kGradItems>(c == 0 ? ocos : osin, r0, n, fo);
                    load_run<kGradItems>(c == 0 ? osin : ocos, r0, n, fk);
                    const float sg = c == 0 ? 1.f : -1.f;  // sine product: s_out K0_c - c_out K0_s
#pragma unroll
                    for (int i = 0; i < kGradItems; ++i) {
                        val[i] *= fi[i];
                        fk[i] *= sg;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kGradItems; ++i) fo[i] = fk[i] = 1.f;
                }
                Aff<double> fd = aff_identity<double>(), bd = aff_identity<double>();
                Aff<double> ft = aff_identity<double>(), bt = aff_identity<double>();
#pragma unroll
                for (int i = 0; i < kGradItems; ++i) {
                    fd = compose(fd, Aff<double>{e[i], (double)val[i]});
                    ft = compose(ft, Aff<double>{tie_mult(ties, i), (double)val[i]});
                }
#pragma unroll
                for (int i = kGradItems - 1; i >= 0; --i) {
                    bd = compose(bd, Aff<double>{e[i + 1], (double)val[i]});
                    bt = compose(bt, Aff<double>{tie_mult(ties, i + 1), (double)val[i]});
                }
                Aff<double> fxd, fxt, bxd, bxt;
                block_exscan4(fd, ft, bd, bt, sh, parity, fxd, fxt, bxd, bxt);
                parity ^= 1;
                const double* cd = A.carry + (grad_row(C, h, c, 0, A.batch, vec) * A.tiles + tile) * 2;
                const double* ct = A.carry + (grad_row(C, h, c, 1, A.batch, vec) * A.tiles + tile) * 2;
                double L = fxd.m * cd[0] + fxd.v;
                double T = fxt.m * ct[0] + fxt.v;
                double Lr[kGradItems], Sr[kGradItems];  // L and L - Tp by rank
#pragma unroll
                for (int i = 0; i < kGradItems; ++i) {
                    L = e[i] * L + (double)val[i];
                    T = tie_mult(ties, i) * T + (double)val[i];
                    Lr[i] = L;
                    Sr[i] = L - T;
                }
                double U = bxd.m * cd[1] + bxd.v;
                double Tb = bxt.m * ct[1] + bxt.v;
#pragma unroll
                for (int i = kGradItems - 1; i >= 0; --i) {
                    U = e[i + 1] * U + (double)val[i];
                    Tb = tie_mult(ties, i + 1) * Tb + (double)val[i];
                    const float k0 = (float)(Lr[i] + U - (double)val[i]);
                    const float s0 = (float)(Sr[i] - (U - Tb));
                    g_a[i] = fmaf(A.anchor_scale * wt[i] * fo[i], s0, g_a[i]);
                    if (C == 2) g_p[i] = fmaf(-wt[i] * fk[i], k0, g_p[i]);
                    dxo[i] = fmaf(fo[i], k0, dxo[i]);
                }
            }
            if (want_dx) {
                if (RANDOM) {
                    uint32_t idx[kGradItems];
                    load_run<kGradItems>(A.perm, r0, n, idx);
                    float* dv = A.dx + vec * n;
#pragma unroll
                    for (int i = 0; i < kGradItems; ++i)
                        if (r0 + i < n) dv[idx[i]] = dxo[i];
                } else {
                    store_run<kGradItems>(A.dx + vec * A.out_ld, r0, n, dxo);
                }
            }
        }
        if (C == 2) grad_store_out<RANDOM>(A, h == 0 ? A.dphi : A.dpsi, r0, g_p);
    }
    grad_store_out<RANDOM>(A, A.da, r0, g_a);
}

size_t grad_sym_scratch_doubles(int64_t n, int64_t batch, int channels)
{
    const int64_t tiles = (n + kScanTile - 1) / kScanTile;
    const int64_t groups = (tiles + kCarryGroup - 1) / kCarryGroup;
    const int64_t rows = 4 * (int64_t)channels * batch;
    return (size_t)(rows * (tiles * 4 + groups * 4 + tiles * 2));
}

template <int C, bool RANDOM>
static hipError_t grad_sym_launch_t(const GradSymArgs& a, hipStream_t s)
{
    LX_LAUNCH("grad_reduce", s, (lx_grad_sym_reduce<C, RANDOM><<<(unsigned)(a.tiles * a.batch), kGradThreads, 0, s>>>(a)));
    const hipError_t e = scan_carry_launch(a.agg, a.gagg, a.carry, a.tiles, 4 * (int64_t)C * a.batch, s);
    if (e != hipSuccess) return e;
    LX_LAUNCH("grad_apply", s, (lx_grad_sym_apply<C, RANDOM><<<(unsigned)a.tiles, kGradThreads, 0, s>>>(a)));
    return hipSuccess;
}

hipError_t grad_sym_launch(const GradSymArgs& a, hipStream_t s)
{
    if (a.n <= 0 || a.batch <= 0) return hipSuccess;
    if (a.tiles * a.batch > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (a.channels == 2) return a.random ? grad_sym_launch_t<2, true>(a, s) : grad_sym_launch_t<2, false>(a, s);
    return a.random ? grad_sym_launch_t<1, true>(a, s) : grad_sym_launch_t<1, false>(a, s);
}

// -------------------------------------------------------------- general

constexpr int kEvalThreads = 1024;

// The same outputs with the tables of a group of up to 8 vectors in LDS
// rows (entry (t, vector): PL_{t-1} and PR_t of every channel, one 16-byte
// read; rows padded so different outputs' rows spread over the banks).
// Each thread keeps kGradOuts outputs of its workgroup's chunk -- their
// intervals t< and t<=, decays and phase factors, and the anchor and phase
// sums -- in registers across all vector groups: the searches and decays
// are done once per output, the weights w of each group are read once, and
// the sums are written once at the end.
constexpr int kGradOuts = 6;

template <int C>
__global__ __launch_bounds__(kEvalThreads) void lx_eval_grad_rows(EvalGradArgs A, int VG)
{
    extern __shared__ float lds[];
    constexpr int RW = eval_row_words<C>();
    constexpr int E = 2 * C;  // words per entry
    const int ni = (int)A.n_in;
    const int tid = threadIdx.x;
    float* si = lds;                                                             // [ni]
    float* rows = lds + pad64(ni);                                               // [ni + 1][RW]
    uint16_t* tab = reinterpret_cast<uint16_t*>(rows + (int64_t)(ni + 1) * RW);  // [kEvalLut + 1]
    for (int i = tid; i < ni; i += kEvalThreads) si[i] = A.s_in[i];
    __syncthreads();
    const float lo_v = si[0], hi_v = si[ni - 1];
    const float width = (hi_v - lo_v) / (float)kEvalLut;
    const float inv_w = width > 0.f ? 1.f / width : 0.f;
    for (int k = tid; k <= kEvalLut; k += kEvalThreads)
        tab[k] = (uint16_t)(k == kEvalLut ? ni : lower_bound_f(si, ni, lo_v + (float)k * width));
    __syncthreads();

    // this thread's outputs: i = chunk start + q * kEvalThreads + tid
    const int64_t base = (int64_t)blockIdx.x * (kGradOuts * kEvalThreads) + tid;
    uint32_t tt[kGradOuts];  // t< | t<= << 16 (n_in <= 65535)
    float al[kGradOuts], be[kGradOuts], be2[kGradOuts], oc[kGradOuts], os[kGradOuts];
    float d_a[kGradOuts], d_p[kGradOuts];
#pragma unroll
    for (int q = 0; q < kGradOuts; ++q) {
        const int64_t i = base + (int64_t)q * kEvalThreads;
        const int64_t ic = i < A.n_out ? i : A.n_out - 1;
        const float o = A.out_anchor[ic];
        oc[q] = 1.f;
        os[q] = 0.f;
        if (C == 2) {
            oc[q] = A.out_cos[ic];
            os[q] = A.out_sin[ic];
        }
        const int lt = (int)lower_bound_lut<kEvalLut>(si, ni, tab, lo_v, inv_w, o);
        // t<= = t< unless anchors equal to o follow (ties): then bisect past them
        const int le = (lt < ni && si[lt] == o) ? (int)upper_bound_f(si, ni, o, lt) : lt;
        tt[q] = (uint32_t)lt | ((uint32_t)le << 16);
        al[q] = lt > 0 ? decay_f(si[lt - 1], o, A.inv_t) : 0.f;
        be[q] = lt < ni ? decay_f(o, si[lt], A.inv_t) : 0.f;
        be2[q] = le < ni ? decay_f(o, si[le], A.inv_t) : 0.f;
        d_a[q] = d_p[q] = 0.f;
    }

    const int groups = (int)((A.batch + VG - 1) / VG);
    for (int g = 0; g < groups; ++g) {
        const int64_t v0 = (int64_t)g * VG;
        const int nv = (int)((A.batch - v0) < VG ? (A.batch - v0) : VG);
        __syncthreads();  // the previous group's rows have been read
        // table rows along t (coalesced reads): for each t this thread fills,
        // all the group's entries are loaded before any is stored, so the
        // group costs one memory latency, not one per vector and channel
        for (int t = tid; t <= ni; t += kEvalThreads) {
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
                const int vi = rowc / C, c = rowc % C;
                float* e = rows + (int64_t)t * RW + vi * E;
                e[c] = lv[rowc];
                e[C + c] = rv[rowc];
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kGradOuts; ++q) {
            const int64_t i = base + (int64_t)q * kEvalThreads;
            if (i >= A.n_out) continue;
            const float* r1 = rows + (int64_t)(tt[q] & 0xFFFFu) * RW;
            const float* r2 = rows + (int64_t)(tt[q] >> 16) * RW;
            // the group's weights, all loads in flight before their use
            float wt[kEvalVG];
#pragma unroll
            for (int vi = 0; vi < kEvalVG; ++vi) wt[vi] = A.w[(v0 + (vi < nv ? vi : 0)) * A.n_out + i];
            float acc_a = 0.f, acc_p = 0.f;
#pragma unroll
            for (int vi = 0; vi < kEvalVG; ++vi) {
                if (vi < nv) {
                    float lv[C], rv[C], rv2[C];
                    if (C == 2) {
                        const float4 e1 = *reinterpret_cast<const float4*>(r1 + vi * E);
                        const float2 e2 = *reinterpret_cast<const float2*>(r2 + vi * E + C);
                        lv[0] = e1.x;
                        lv[C - 1] = e1.y;
                        rv[0] = e1.z;
                        rv[C - 1] = e1.w;
                        rv2[0] = e2.x;
                        rv2[C - 1] = e2.y;
                    } else {
                        const float2 e1 = *reinterpret_cast<const float2*>(r1 + vi * E);
                        lv[0] = e1.x;
                        rv[0] = e1.y;
                        rv2[0] = r2[vi * E + C];
                    }
                    float sig = 0.f, kin = 0.f, pla = 0.f;
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const float k0 = fmaf(al[q], lv[c], be[q] * rv[c]);
                        const float s0 = fmaf(al[q], lv[c], -be2[q] * rv2[c]);
                        const float fo = c == 0 ? oc[q] : os[q];
                        sig = fmaf(fo, s0, sig);
                        pla = fmaf(fo, k0, pla);
                        if (C == 2) kin = fmaf(c == 0 ? os[q] : -oc[q], k0, kin);
                    }
                    acc_a = fmaf(wt[vi], sig, acc_a);
                    acc_p = fmaf(-wt[vi], kin, acc_p);
                    if (A.y) A.y[(v0 + vi) * A.n_out + i] = pla;
                }
            }
            d_a[q] = d_a[q] + A.anchor_scale * acc_a;
            d_p[q] = d_p[q] + acc_p;
        }
    }
#pragma unroll
    for (int q = 0; q < kGradOuts; ++q) {
        const int64_t i = base + (int64_t)q * kEvalThreads;
        if (i < A.n_out) {
            if (A.d_anchor) A.d_anchor[i] = d_a[q];
            if (C == 2 && A.d_phase) A.d_phase[i] = d_p[q];
        }
    }
}

template <int C, bool USE_LDS>
__global__ __launch_bounds__(kEvalThreads) void lx_eval_grad(EvalGradArgs A, int VG, int64_t chunk_len)
{
    extern __shared__ float lds[];
    const int64_t ni = A.n_in;
    const int64_t i0 = blockIdx.x * chunk_len;
    int64_t i1 = i0 + chunk_len;
    if (i1 > A.n_out) i1 = A.n_out;
    const float* si = A.s_in;
    float* tl = nullptr;  // [ni][VG][C]
    float* tr = nullptr;
    if (USE_LDS) {
        float* s_l = lds;
        tl = lds + pad64(ni);
        tr = tl + ni * VG * C;
        for (int64_t i = threadIdx.x; i < ni; i += kEvalThreads) s_l[i] = A.s_in[i];
        si = s_l;
    }
    const int groups = (int)((A.batch + VG - 1) / VG);
    for (int g = 0; g < groups; ++g) {
        const int64_t v0 = (int64_t)g * VG;
        const int nv = (int)((A.batch - v0) < VG ? (A.batch - v0) : VG);
        if (USE_LDS) {
            __syncthreads();  // previous group's readers are done
            for (int64_t i = threadIdx.x; i < ni * VG * C; i += kEvalThreads) {
                const int64_t t = i / (VG * C);
                const int64_t rem = i - t * (VG * C);
                const int64_t vi = rem / C;
                const int64_t c = rem - vi * C;
                const int64_t src = (c * A.batch + v0 + vi) * A.ld + t;
                tl[i] = vi < nv ? A.pl[src] : 0.f;
                tr[i] = vi < nv ? A.pr[src] : 0.f;
            }
            __syncthreads();
        }
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kEvalThreads) {
            const float o = A.out_anchor[i];
            const int64_t tlt = lower_bound_f(si, ni, o);
            const int64_t tle = upper_bound_f(si, ni, o, tlt);
            const float al = tlt > 0 ? decay_f(si[tlt - 1], o, A.inv_t) : 0.f;
            const float be = tlt < ni ? decay_f(o, si[tlt], A.inv_t) : 0.f;
            const float be2 = tle < ni ? decay_f(o, si[tle], A.inv_t) : 0.f;
            float oc = 1.f, os = 0.f;
            if (C == 2) {
                oc = A.out_cos[i];
                os = A.out_sin[i];
            }
            float acc_a = 0.f, acc_p = 0.f;
            for (int vi = 0; vi < nv; ++vi) {
                float sig = 0.f, kin = 0.f, pla = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    float lv = 0.f, rv = 0.f, rv2 = 0.f;
                    if (USE_LDS) {
                        if (tlt > 0) lv = tl[((tlt - 1) * VG + vi) * C + c];
                        if (tlt < ni) rv = tr[(tlt * VG + vi) * C + c];
                        if (tle < ni) rv2 = tr[(tle * VG + vi) * C + c];
                    } else {
                        const int64_t row = ((int64_t)c * A.batch + v0 + vi) * A.ld;
                        if (tlt > 0) lv = A.pl[row + tlt - 1];
                        if (tlt < ni) rv = A.pr[row + tlt];
                        if (tle < ni) rv2 = A.pr[row + tle];
                    }
                    const float k0 = fmaf(al, lv, be * rv);
                    const float s0 = fmaf(al, lv, -be2 * rv2);
                    const float fo = c == 0 ? oc : os;
                    sig = fmaf(fo, s0, sig);
                    pla = fmaf(fo, k0, pla);
                    if (C == 2) kin = fmaf(c == 0 ? os : -oc, k0, kin);
                }
                const float wt = A.w[(v0 + vi) * A.n_out + i];
                acc_a = fmaf(wt, sig, acc_a);
                acc_p = fmaf(-wt, kin, acc_p);
                if (A.y) A.y[(v0 + vi) * A.n_out + i] = pla;
            }
            // this thread owns output i in every group: accumulate in place
            if (A.d_anchor) A.d_anchor[i] = (g == 0 ? 0.f : A.d_anchor[i]) + A.anchor_scale * acc_a;
            if (C == 2 && A.d_phase) A.d_phase[i] = (g == 0 ? 0.f : A.d_phase[i]) + acc_p;
        }
    }
}

hipError_t eval_grad_launch(const EvalGradArgs& a, hipStream_t s)
{
    if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
    if (a.n_in >= 1 && a.n_in <= 0xFFFF && a.lds_bytes > 0 &&
        eval_rows_lds(a.n_in, a.channels) <= (size_t)a.lds_bytes) {
        // groups of at most 8 vectors, as even as possible
        const int64_t groups = (a.batch + kEvalVG - 1) / kEvalVG;
        const int vg = (int)((a.batch + groups - 1) / groups);
        const int64_t per = (int64_t)kGradOuts * kEvalThreads;
        const unsigned blocks = (unsigned)((a.n_out + per - 1) / per);
        const size_t shmem = eval_rows_lds(a.n_in, a.channels);
        if (a.channels == 2) {
            (void)hipFuncSetAttribute((const void*)lx_eval_grad_rows<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)shmem);
            LX_LAUNCH("eval_grad", s, (lx_eval_grad_rows<2><<<blocks, kEvalThreads, shmem, s>>>(a, vg)));
        } else {
            (void)hipFuncSetAttribute((const void*)lx_eval_grad_rows<1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)shmem);
            LX_LAUNCH("eval_grad", s, (lx_eval_grad_rows<1><<<blocks, kEvalThreads, shmem, s>>>(a, vg)));
        }
        return hipSuccess;
    }
    const int64_t lds_floats = a.lds_bytes / 4;
    int64_t vg = (lds_floats - pad64(a.n_in)) / (2 * (int64_t)a.channels * (a.n_in > 0 ? a.n_in : 1));
    if (vg > 16) vg = 16;
    if (vg > a.batch) vg = a.batch;
    const bool use_lds = a.lds_bytes > 0 && vg >= 1;
    if (!use_lds) vg = a.batch < 16 ? a.batch : 16;
    int64_t chunks = (a.n_out + 16383) / 16384;
    if (chunks > 4096) chunks = 4096;
    if (chunks < 1) chunks = 1;
    const int64_t chunk_len = (a.n_out + chunks - 1) / chunks;
    chunks = (a.n_out + chunk_len - 1) / chunk_len;
    const size_t shmem = use_lds ? (size_t)(pad64(a.n_in) + 2 * vg * a.channels * a.n_in) * 4 : 0;
    const int v = (int)vg;
#define LX_EVG(CC, LL)                                                                                   \
    do {                                                                                                 \
        if (LL) (void)hipFuncSetAttribute((const void*)lx_eval_grad<CC, LL>,                             \
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);       \
        LX_LAUNCH("eval_grad", s,                                                                        \
                  (lx_eval_grad<CC, LL><<<(unsigned)chunks, kEvalThreads, shmem, s>>>(a, v, chunk_len))); \
    } while (0)
    if (a.channels == 2) {
        if (use_lds) LX_EVG(2, true);
        else LX_EVG(2, false);
    } else {
        if (use_lds) LX_EVG(1, true);
        else LX_EVG(1, false);
    }
#undef LX_EVG
    return hipSuccess;
}

// A small output side (the sorted bucketing path): one thread per output,
// in sorted order, over every vector.  With L the left part including ties
// (ties were bucketed into the left interval), R the strict right part and T
// the ties: K0 = L + R, S0 = (L - T) - R.
template <int C>
__global__ __launch_bounds__(256) void lx_eval_grad_lr(EvalLRArgs A)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= A.n_out) return;
    const float o = A.s_out[j];
    const int64_t first = lower_bound_f(A.s_out, A.n_out, o);  // ties were summed at the run's first rank
    const int64_t i = A.perm_out[j];
    float oc = 1.f, os = 0.f;
    if (C == 2) {
        oc = A.out_cos[i];
        os = A.out_sin[i];
    }
    float acc_a = 0.f, acc_p = 0.f;
    for (int64_t v = 0; v < A.batch; ++v) {
        float sig = 0.f, kin = 0.f, pla = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t row = ((int64_t)c * A.batch + v) * A.ld;
            const float lv = A.L[row + j], rv = A.R[row + j], tv = A.T[row + first];
            const float k0 = lv + rv;
            const float s0 = (lv - tv) - rv;
            const float fo = c == 0 ? oc : os;
            sig = fmaf(fo, s0, sig);
            pla = fmaf(fo, k0, pla);
            if (C == 2) kin = fmaf(c == 0 ? os : -oc, k0, kin);
        }
        const float wt = A.w[v * A.n_out + i];
        acc_a = fmaf(wt, sig, acc_a);
        acc_p = fmaf(-wt, kin, acc_p);
        if (A.y) A.y[v * A.n_out + i] = pla;
    }
    if (A.d_anchor) A.d_anchor[i] = A.anchor_scale * acc_a;
    if (C == 2 && A.d_phase) A.d_phase[i] = acc_p;
}

hipError_t eval_lr_launch(const EvalLRArgs& a, hipStream_t s)
{
    if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.n_out + 255) / 256);
    if (a.channels == 2) LX_LAUNCH("eval_grad_lr", s, (lx_eval_grad_lr<2><<<blocks, 256, 0, s>>>(a)));
    else LX_LAUNCH("eval_grad_lr", s, (lx_eval_grad_lr<1><<<blocks, 256, 0, s>>>(a)));
    return hipSuccess;
}

}  // namespace lx
