// Host-side interfaces between the plan/executor (api.cpp) and the kernel
// files.  Internal to the library; not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lx {

#ifndef LX_SORT_THREADS
#define LX_SORT_THREADS 512
#endif
#ifndef LX_SORT_ITEMS
#define LX_SORT_ITEMS 16
#endif
constexpr int kSortTileSize = LX_SORT_THREADS * LX_SORT_ITEMS;  // keys per onesweep tile
constexpr int kScanTile = 4096;      // elements per scan tile

// ---- kernel timing hooks (implemented in api.cpp) ----
int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

// Launch `launch` (a <<<>>> expression) between two profiling events and
// return the launch error, if any, from the enclosing function.
#define LX_LAUNCH(name, stream, launch)                       \
    do {                                                      \
        const int lx_tok_ = ::lx::prof_begin(name, stream);   \
        launch;                                               \
        ::lx::prof_end(lx_tok_, stream);                      \
        const hipError_t lx_e_ = hipGetLastError();           \
        if (lx_e_ != hipSuccess) return lx_e_;                \
    } while (0)

// ---- utilities ----
hipError_t fill_u32(uint32_t* p, uint32_t v, int64_t count, hipStream_t s);

// ---- sort (sort.hip) ----
// Replay records of the four radix passes: for pass k and tile t, slot i of
// the tile (its keys in digit order) came from tile position rec[k][t*8192+i]
// and went to global position base[k][t*256+b] + i, b being the bin of slot
// i (the last b with start[k][t*256+b] <= i).
struct SortRecords {
    int64_t n = 0, tiles = 0;
    uint16_t* rec[4] = {};
    uint32_t* base[4] = {};
    uint16_t* start[4] = {};
};
// Value rows sorted along with the keys (key-value passes): pass 0 reads
// in[r] (original order); the passes alternate between va and vb (rows of
// stride ld), so the sorted rows end in vb.
constexpr int kMaxSortVals = 20;
struct SortVals {
    int rows = 0;
    const float* in[kMaxSortVals] = {};
    float* va = nullptr;
    float* vb = nullptr;
    int64_t ld = 0;
};
struct SortValPass {  // kernel argument: one pass's row pointers
    int rows = 0;
    const float* in[kMaxSortVals] = {};
    float* out[kMaxSortVals] = {};
};
size_t sort_scratch_bytes(int64_t n, bool with_vals = false);  // temporary, during the sort
size_t sort_record_bytes(int64_t n);    // kept by the plan
SortRecords sort_records_at(void* base, int64_t n);
// Stable argsort of a[0..n): sorted[r] = a[perm[r]] for the permutation the
// records describe.  *flag (device) gets bit 0 if any anchor is NaN/Inf.
hipError_t sort_launch(const float* a, int64_t n, float* sorted, const SortRecords& R, void* scratch,
                       uint32_t* flag, hipStream_t s, const SortVals* vals = nullptr);
// One replayed pass: forward moves pass-k input order to pass-k output
// order, backward the reverse.  Rows of `batch` vectors with strides in_ld,
// out_ld (elements).
hipError_t replay_launch(const SortRecords& R, int pass, bool forward, const float* in, int64_t in_ld,
                         float* out, int64_t out_ld, int64_t batch, hipStream_t s);
// perm[r] = original index of rank r, by replaying an index ramp; tmp: n words.
hipError_t perm_from_records(const SortRecords& R, uint32_t* perm, uint32_t* tmp, hipStream_t s);

// ---- phases (sort.hip) ----
// c[r] = cos(ph[perm[r]]), s[r] = sin(ph[perm[r]]); flag bit 0 if non-finite.
hipError_t phase_factors_launch(const float* ph, const uint32_t* perm, int64_t n, float* c,
                                float* s, uint32_t* flag, hipStream_t st);
// flag bit 0 if any of v[0..n) is non-finite.
hipError_t check_finite_launch(const float* v, int64_t n, uint32_t* flag, hipStream_t st);

// ---- scans along a sorted side (scan.hip) ----
enum ScanMode : int {
    kScanSym = 0,   // values x (by rank); output L + U - x
    kScanUV = 1,    // forward stream u, backward stream v (by rank); output L + R
    kScanPLPR = 2,  // values x (by rank); outputs L and U kept apart, by rank
    kScanUVLR = 3,  // forward stream u, backward stream v (by rank); outputs L and R kept apart
};

struct ScanArgs {
    int mode = kScanSym;
    int channels = 1;          // 1, or 2 for the cos/sin split of a phased operator
    bool random = false;       // x read through perm and y written through perm (else xs/ys by rank)
    int64_t n = 0;             // length of the sorted side
    int64_t tiles = 0;         // ceil(n / kScanTile)
    int64_t batch = 0;         // vectors
    int64_t ld = 0;            // row stride of the internal [channels][batch][ld] buffers
    double inv_t = 1.0;        // 1 / temperature (+inf: equality routing)
    const float* s = nullptr;  // sorted anchors [n]
    const uint32_t* perm = nullptr;  // rank -> original index [n]
    const float* x = nullptr;        // random Sym/PLPR: [batch][n], original order
    const float* in_c = nullptr;     // input factors by rank (cos, sin), or null
    const float* in_s = nullptr;
    const float* u = nullptr;        // UV: [channels][batch][ld], by rank
    const float* v = nullptr;
    float* xs = nullptr;             // Sym/PLPR values by rank [batch][ld] (written when random)
    double* agg = nullptr;           // [channels][batch][tiles][4]: fwd (m, v), bwd (m, v)
    double* gagg = nullptr;          // [channels][batch][groups][4]: composites of tile groups
    double* carry = nullptr;         // [channels][batch][tiles][2]: fwd, bwd carry-in
    const float* out_c = nullptr;    // output factors by rank, or null
    const float* out_s = nullptr;
    float* y = nullptr;              // random Sym/UV: [batch][n], original order
    float* ys = nullptr;             // Sym/UV by rank [batch][ld] (may alias xs) when not random
    float* pl = nullptr;             // PLPR: [channels][batch][ld], by rank
    float* pr = nullptr;
};
constexpr int kCarryGroup = 4096;    // tiles per carry group
hipError_t scan_launch(const ScanArgs& a, hipStream_t s);
// Carries of `rows` independent scan rows from their tile composites:
// agg [rows][tiles][4] (fwd m, v, bwd m, v) -> carry [rows][tiles][2];
// gagg: [rows][ceil(tiles / kCarryGroup)][4] scratch.
hipError_t scan_carry_launch(const double* agg, double* gagg, double* carry, int64_t tiles, int64_t rows,
                             hipStream_t s);

// ---- general case a != b (general.hip) ----
struct BucketArgs {
    int channels = 1;
    int64_t n_out = 0;               // sorted output side
    int64_t n_in = 0;                // input side, original order
    int64_t batch = 0;
    float inv_t = 1.f;               // 1 / temperature (+inf: equality routing)
    const float* s_out = nullptr;    // sorted output anchors [n_out]
    const float* in_anchor = nullptr;  // [n_in], original order
    const float* in_cos = nullptr;     // cos / sin of the input phases, original order, or null
    const float* in_sin = nullptr;
    const float* x = nullptr;        // [batch][n_in]
    int64_t ld = 0;                  // row stride of u, v
    float* u = nullptr;              // [channels][batch][ld] (overwritten)
    float* v = nullptr;
    bool ties = false;               // also sum the inputs equal to s_out[t], at t, into `tie`
    float* tie = nullptr;            // same layout as u (when ties)
    float* partial = nullptr;        // scratch for the LDS-binned path
    int64_t partial_floats = 0;
    void* layout = nullptr;          // scratch for the LDS-binned path: bucket_layout_bytes()
    int lds_bytes = 0;               // LDS budget per workgroup
};
// Scratch floats the LDS-binned bucketing needs for these sizes
// (0 if the shape does not fit that path: then merge-path bucketing runs)
int64_t bucket_partial_floats(const BucketArgs& a, int* groups, int* chunks);
// Bytes of the per-call input layout of the LDS-binned path (slots of the
// inputs, interval starts per sub-chunk, anchors and phase factors in slot
// order), 256-byte aligned.
int64_t bucket_layout_bytes(const BucketArgs& a);
hipError_t bucket_launch(BucketArgs& a, hipStream_t s);

// Merge-path bucketing (merge.hip) for a long sorted output side: the
// sorted input side and the sorted outputs merged (an input before an
// output of equal value), tiles of the merged sequence per workgroup,
// segmented float64 sums of each interval's run of inputs into u, v.
struct MergeArgs {
    int channels = 1;
    int64_t n_out = 0;                // sorted output side
    int64_t n_in = 0;                 // sorted input side
    int64_t batch = 0;
    double inv_t = 1.0;               // 1 / temperature (+inf: equality routing)
    const float* s_out = nullptr;     // sorted output anchors [n_out]
    const float* s_in = nullptr;      // sorted input anchors [n_in]
    const uint32_t* perm_in = nullptr;  // input rank -> original index
    const float* in_c = nullptr;      // cos / sin of the input phases by input rank (phased)
    const float* in_s = nullptr;
    const float* x = nullptr;         // [batch][n_in], original order
    int64_t ld = 0;                   // row stride of u, v
    float* u = nullptr;               // [channels][batch][ld] by output rank (overwritten)
    float* v = nullptr;
    uint2* split = nullptr;           // [tiles + 1] scratch: (inputs, outputs) before each tile
    double* head = nullptr;           // [channels][batch][tiles][2] scratch
    double* tail = nullptr;           // [channels][batch][tiles][2] scratch
    int64_t tiles = 0;                // set by merge_launch
};
int64_t merge_tiles(int64_t n_in, int64_t n_out);
size_t merge_ws_bytes(int64_t n_in, int64_t n_out, int64_t batch, int channels);
hipError_t merge_launch(MergeArgs& a, hipStream_t s);

// Evaluation from per-interval LDS rows (lx_eval_rows, lx_eval_grad_rows):
// groups of up to kEvalVG vectors; row t of the tables holds, per vector,
// PL_{t-1} and PR_t of every channel (2C words), rows padded to
// eval_row_words() so the rows of different outputs spread over the LDS
// banks; the interval comes from a lookup table of kEvalLut cells.
constexpr int kEvalVG = 8;
constexpr int kEvalLut = 2048;
template <int C>
constexpr int eval_row_words() { return C == 2 ? 36 : 20; }
inline size_t eval_rows_lds(int64_t ni, int C)
{
    const int64_t pad = (ni + 63) & ~(int64_t)63;
    return (size_t)(pad + (ni + 1) * (C == 2 ? 36 : 20)) * 4 + (size_t)(kEvalLut + 1) * 2;
}

struct EvalArgs {
    int channels = 1;
    int64_t n_out = 0;                 // outputs, original order
    int64_t n_in = 0;                  // sorted input side
    int64_t batch = 0;
    float inv_t = 1.f;                  // 1 / temperature (+inf: equality routing)
    const float* out_anchor = nullptr;  // [n_out]
    const float* out_cos = nullptr;     // cos / sin of the output phases, original order, or null
    const float* out_sin = nullptr;
    const float* s_in = nullptr;        // sorted input anchors [n_in]
    int64_t ld = 0;                     // row stride of pl, pr
    const float* pl = nullptr;          // [channels][batch][ld]
    const float* pr = nullptr;
    float* y = nullptr;                 // [batch][n_out]
    int lds_bytes = 0;
};
hipError_t eval_launch(const EvalArgs& a, hipStream_t s);

// ---- gradients (grad.hip) ----
// Symmetric plans, by rank.  u: row-side vectors, w: column-side vectors
// (see grad.hip for which is which in a training step).
struct GradSymArgs {
    int channels = 1;
    bool random = false;             // u, w gathered and outputs scattered through perm
    int64_t n = 0, tiles = 0, batch = 0;
    int64_t ld = 0;                  // row stride of us, ws
    int64_t out_ld = 0;              // row stride of dx when not random
    double inv_t = 1.0;
    float anchor_scale = -1.f;       // -1/t (0 at t = 0)
    int dx_half = 1;                 // 1: dx = K^T u (column side), 0: dx = K w (row side)
    const float* s = nullptr;
    const uint32_t* perm = nullptr;
    const float* u = nullptr;        // random: [batch][n] original order
    const float* w = nullptr;
    float* us = nullptr;             // by rank [batch][ld] (written when random)
    float* ws = nullptr;
    const float* cphi = nullptr;     // by rank, phased only
    const float* sphi = nullptr;
    const float* cpsi = nullptr;
    const float* spsi = nullptr;
    double* agg = nullptr;           // [4 C batch][tiles][4]
    double* gagg = nullptr;          // [4 C batch][groups][4]
    double* carry = nullptr;         // [4 C batch][tiles][2]
    float* dx = nullptr;             // outputs (null: not wanted): original order when
    float* da = nullptr;             // random, else by rank
    float* dphi = nullptr;
    float* dpsi = nullptr;
};
size_t grad_sym_scratch_doubles(int64_t n, int64_t batch, int channels);
hipError_t grad_sym_launch(const GradSymArgs& a, hipStream_t s);

// General plans: one side's outputs from the other side's PL/PR tables.
struct EvalGradArgs {
    int channels = 1;
    int64_t n_out = 0, n_in = 0, batch = 0;
    int64_t ld = 0;                     // row stride of pl, pr
    float inv_t = 1.f;
    float anchor_scale = -1.f;          // -1/t (0 at t = 0)
    const float* out_anchor = nullptr;  // [n_out], original order
    const float* out_cos = nullptr;     // output phases, original order (phased)
    const float* out_sin = nullptr;
    const float* s_in = nullptr;        // sorted input side
    const float* pl = nullptr;          // [channels][batch][ld]
    const float* pr = nullptr;
    const float* w = nullptr;           // output-side weights [batch][n_out]
    float* y = nullptr;                 // plain product [batch][n_out], or null
    float* d_anchor = nullptr;          // [n_out], or null
    float* d_phase = nullptr;           // [n_out], or null
    int lds_bytes = 0;
};
hipError_t eval_grad_launch(const EvalGradArgs& a, hipStream_t s);
// The same outputs for a small output side from interval sums of the input
// side: with the outputs sorted (s_out, perm_out: rank -> original index),
// L = strict-and-tied left part, R = strict right part (both by rank, from
// the u / v scan) and T = the tie sums at the first rank of each run of
// equal outputs.
struct EvalLRArgs {
    int channels = 1;
    int64_t n_out = 0, batch = 0;
    int64_t ld = 0;                     // row stride of L, R, T: [channels][batch][ld]
    float anchor_scale = -1.f;          // -1/t (0 at t = 0)
    const float* s_out = nullptr;       // sorted outputs [n_out]
    const uint32_t* perm_out = nullptr; // rank -> original index
    const float* out_cos = nullptr;     // output phases, original order (phased)
    const float* out_sin = nullptr;
    const float* L = nullptr;
    const float* R = nullptr;
    const float* T = nullptr;
    const float* w = nullptr;           // output-side weights [batch][n_out], original order
    float* y = nullptr;                 // plain product [batch][n_out], or null
    float* d_anchor = nullptr;          // [n_out], or null
    float* d_phase = nullptr;           // [n_out], or null
};
hipError_t eval_lr_launch(const EvalLRArgs& a, hipStream_t s);

// ---- small symmetric plans (small.hip) ----
// n <= kSmallMax anchors in one workgroup: stable sort, permutation, phase
// factors by rank and, when x is given, y = K x for `batch` vectors.
constexpr int64_t kSmallMax = 8192;
struct SmallSymArgs {
    int64_t n = 0;
    int batch = 0;
    double inv_t = 1.0;
    const float* a = nullptr;              // anchors, original order
    const float* phi = nullptr;            // phases (both or neither), original order
    const float* psi = nullptr;
    const float* x = nullptr;              // [batch][n], or null: plan only
    float* x_keep = nullptr;               // [batch][n] copy of x (original order), or null
    float* y = nullptr;                    // [batch][n]
    float* sa = nullptr;                   // sorted anchors [n]
    uint32_t* perm = nullptr;              // rank -> original index [n]
    float* cphi = nullptr;                 // cos/sin of the phases by rank (phased)
    float* sphi = nullptr;
    float* cpsi = nullptr;
    float* spsi = nullptr;
    uint32_t* flag = nullptr;              // written: 1 for a NaN/Inf anchor or phase, else 0
};
hipError_t small_sym_launch(const SmallSymArgs& a, hipStream_t s);

// ---- Gram (gram.hip) ----
struct GramArgs {
    int64_t n = 0, k = 0;
    double inv_t = 1.0;             // 1 / temperature (+inf: equality routing)
    const float* sa = nullptr;      // sorted a [n]
    const uint32_t* pa = nullptr;   // perm of a
    const float* sb = nullptr;      // sorted b [k]
    const uint32_t* pb = nullptr;   // perm of b
    const float* D = nullptr;       // [k], original order of b
    const uint32_t* bound = nullptr;  // [n + 2]: interval r is sorted b [bound[r], bound[r+1])
    const uint32_t* rank_a = nullptr;  // [n]: rank of each original index of a
    // b's inputs split by original index into kGramSlices ranges: the inputs
    // of interval r in slice s are slice_*[slice_off[s (n+1) + r] ..
    // slice_off[s (n+1) + r + 1]), in ascending sorted position
    const uint32_t* slice_off = nullptr;  // [kGramSlices (n + 1) + 1]
    const uint32_t* slice_src = nullptr;  // [k] original index
    const float* slice_b = nullptr;       // [k] b
    const float* slice_c = nullptr;       // [k] phased: cos psi
    const float* slice_s = nullptr;       // [k] phased: sin psi
    const float* cphi_r = nullptr;  // phased: cos/sin of phi by rank of a, of psi by rank of b
    const float* sphi_r = nullptr;
    const float* cpsi_r = nullptr;
    const float* spsi_r = nullptr;
    double* stats = nullptr;        // scratch: see gram.hip
    float* M = nullptr;             // [n][n]
};
constexpr int kGramSlices = 8;  // one per compute die
size_t gram_scratch_bytes(int64_t n, int64_t k, int weight_sets);
// Fills slice_off (sized kGramSlices (n + 1) + 1) and the slice arrays from
// a.pb, a.sb, a.bound (and a.cpsi_r, a.spsi_r when s_c is given).
hipError_t gram_slices_launch(const GramArgs& a, uint32_t* off, uint32_t* s_src, float* s_b, float* s_c, float* s_s,
                              hipStream_t s);
// bound[r] = #{b <= s_{r-1}} (r = 1 .. n), bound[0] = 0, bound[n+1] = k.
hipError_t gram_bounds_launch(const float* sa, int64_t n, const float* sb, int64_t k, uint32_t* bound,
                              hipStream_t s);
// rank[perm[r]] = r for r < n.
hipError_t gram_ranks_launch(const uint32_t* perm, int64_t n, uint32_t* rank, hipStream_t s);
hipError_t gram_launch(const GramArgs& a, hipStream_t s);

}  // namespace lx
