// Host-side interfaces between the plan/executor (api.cpp) and the kernel
// files.  Internal to the library; not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lx {

constexpr int kSortTileSize = 8192;  // keys per onesweep tile
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
// Scratch bytes needed to sort n keys.
size_t sort_scratch_bytes(int64_t n);
// Stable argsort of a[0..n): sorted[r] = a[perm[r]].  *flag (device) gets
// bit 0 set if any anchor is NaN/Inf.  `scratch` holds sort_scratch_bytes(n).
hipError_t sort_launch(const float* a, int64_t n, float* sorted, uint32_t* perm, void* scratch,
                       uint32_t* flag, hipStream_t s);

// ---- phases (sort.hip) ----
// c[r] = cos(ph[perm[r]]), s[r] = sin(ph[perm[r]]); flag bit 0 if non-finite.
hipError_t phase_factors_launch(const float* ph, const uint32_t* perm, int64_t n, float* c,
                                float* s, uint32_t* flag, hipStream_t st);
// flag bit 0 if any of v[0..n) is non-finite.
hipError_t check_finite_launch(const float* v, int64_t n, uint32_t* flag, hipStream_t st);

// ---- scans along a sorted side (scan.hip) ----
enum ScanMode : int {
    kScanSym = 0,   // value stream x gathered through perm; output L + U - x, scattered
    kScanUV = 1,    // forward stream u, backward stream v (sorted order); output L + R, scattered
    kScanPLPR = 2,  // value stream x gathered; outputs L and U kept apart, sorted order
};

struct ScanArgs {
    int mode = kScanSym;
    int channels = 1;          // 1, or 2 for the cos/sin split of a phased operator
    int64_t n = 0;             // length of the sorted side
    int64_t tiles = 0;         // ceil(n / kScanTile)
    int64_t batch = 0;         // vectors
    int64_t ld = 0;            // row stride of the internal [channels][batch][ld] buffers
    const float* s = nullptr;  // sorted anchors [n]
    const uint32_t* perm = nullptr;  // rank -> original index [n]
    const float* x = nullptr;        // Sym/PLPR: [batch][n], original order
    const float* in_c = nullptr;     // input factors by rank (cos, sin), or null
    const float* in_s = nullptr;
    const float* u = nullptr;        // UV: [channels][batch][ld], by rank
    const float* v = nullptr;
    float* xs = nullptr;             // Sym/PLPR scratch [channels][batch][ld]
    double* agg = nullptr;           // [channels][batch][tiles][4]: fwd (m, v), bwd (m, v)
    double* carry = nullptr;         // [channels][batch][tiles][2]: fwd, bwd carry-in
    const float* out_c = nullptr;    // output factors by rank, or null
    const float* out_s = nullptr;
    float* y = nullptr;              // Sym/UV: [batch][n], original order
    float* pl = nullptr;             // PLPR: [channels][batch][ld], by rank
    float* pr = nullptr;
};
hipError_t scan_launch(const ScanArgs& a, hipStream_t s);

// ---- general case a != b (general.hip) ----
struct BucketArgs {
    int channels = 1;
    int64_t n_out = 0;               // sorted output side
    int64_t n_in = 0;                // input side, original order
    int64_t batch = 0;
    const float* s_out = nullptr;    // sorted output anchors [n_out]
    const float* in_anchor = nullptr;  // [n_in], original order
    const float* in_phase = nullptr;   // [n_in] or null
    const float* x = nullptr;        // [batch][n_in]
    int64_t ld = 0;                  // row stride of u, v
    float* u = nullptr;              // [channels][batch][ld] (overwritten)
    float* v = nullptr;
    float* partial = nullptr;        // scratch for the LDS-binned path
    int64_t partial_floats = 0;
    int lds_bytes = 0;               // LDS budget per workgroup (0: global path)
};
// Scratch floats the LDS-binned bucketing needs for these sizes (0 if it is
// not used and the global-atomics path runs instead).
int64_t bucket_partial_floats(const BucketArgs& a, int* groups, int* chunks);
hipError_t bucket_launch(BucketArgs& a, hipStream_t s);

struct EvalArgs {
    int channels = 1;
    int64_t n_out = 0;                 // outputs, original order
    int64_t n_in = 0;                  // sorted input side
    int64_t batch = 0;
    const float* out_anchor = nullptr;  // [n_out]
    const float* out_phase = nullptr;   // [n_out] or null
    const float* s_in = nullptr;        // sorted input anchors [n_in]
    int64_t ld = 0;                     // row stride of pl, pr
    const float* pl = nullptr;          // [channels][batch][ld]
    const float* pr = nullptr;
    float* y = nullptr;                 // [batch][n_out]
    int lds_bytes = 0;
};
hipError_t eval_launch(const EvalArgs& a, hipStream_t s);

// ---- Gram (gram.hip) ----
struct GramArgs {
    int64_t n = 0, k = 0;
    const float* sa = nullptr;      // sorted a [n]
    const uint32_t* pa = nullptr;   // perm of a
    const float* sb = nullptr;      // sorted b [k]
    const uint32_t* pb = nullptr;   // perm of b
    const float* D = nullptr;       // [k], original order of b
    double* stats = nullptr;        // scratch: see gram.hip
    float* M = nullptr;             // [n][n]
};
size_t gram_scratch_bytes(int64_t n);
hipError_t gram_launch(const GramArgs& a, hipStream_t s);

}  // namespace lx
