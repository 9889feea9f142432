// C ABI of the LAPLEX library: plans, argument checks, dispatch, timing.
//
// The operator and its fast algorithm follow the technical summary of
// "LAPLEX: The FFT of Learnable Laplace Kernels" (§2.1 operator, §2.2 scan
// algebra, general case and Gram); see include/laplex.h for the contract.
//
// Every argument check runs before the first HIP call, so invalid calls are
// rejected on any host, GPU or not.  Device memory comes from the library's
// caching allocator below (freed blocks kept per device and handed out
// again, each ordered after its last use by an event), so repeated plans and
// growing workspaces do not pay for fresh allocations.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "laplex.h"
#include "lx_internal.h"

namespace {

thread_local std::string g_last_error;

// Longest anchor side.  Permutations are uint32, and the backward replay
// forms its gather offsets as 32-bit byte offsets from a uniform base, so
// every element index times 4 must fit in 32 bits: n <= 2^30.
constexpr int64_t kMaxLen = (int64_t)1 << 30;

laplex_status fail(laplex_status st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

laplex_status from_hip(hipError_t e, const char* where)
{
    if (e == hipSuccess) return LAPLEX_OK;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
        return fail(LAPLEX_ERR_OUT_OF_MEMORY, std::string(where) + ": " + hipGetErrorString(e));
    if (e == hipErrorNoDevice || e == hipErrorInvalidDevice)
        return fail(LAPLEX_ERR_NO_DEVICE, std::string(where) + ": " + hipGetErrorString(e));
    return fail(LAPLEX_ERR_DEVICE, std::string(where) + ": " + hipGetErrorString(e));
}

#define LX_TRY(call, where)                                          \
    do {                                                             \
        const laplex_status lx_s_ = from_hip((call), (where));       \
        if (lx_s_ != LAPLEX_OK) return lx_s_;                        \
    } while (0)

inline int64_t pad64(int64_t x) { return (x + 63) & ~(int64_t)63; }
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// ------------------------------------------------------- caching allocator
//
// Device memory for plans, workspaces and sort scratch.  A layer whose
// anchors change every training step makes and drops a plan per step, tens
// of GB each time at n = 2^30, so freed blocks are kept per device and
// handed out again (best fit, at most twice the request) instead of going
// back to the driver.  A block freed on stream s carries an event recorded
// on s at the free; whoever takes it next orders its stream after that
// event, so reuse across streams is safe.  When the driver is out of
// memory, the cached blocks are released and the allocation is retried.
// One event recorded at a free, shared by the blocks freed together.
struct FreeEvent {
    hipEvent_t ev;
    int refs;
};
struct CachedBlock {
    void* ptr;
    size_t bytes;
    FreeEvent* freed;  // recorded at the free (null: idle already)
};
struct DeviceCache {
    std::mutex mu;
    std::vector<CachedBlock> idle;
    std::vector<std::pair<void*, size_t>> live;
    std::vector<hipEvent_t> events;
};
std::mutex g_cache_mu;
std::vector<DeviceCache*> g_caches;

DeviceCache& cache_for(int dev)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    while ((int)g_caches.size() <= dev) g_caches.push_back(new DeviceCache());
    return *g_caches[dev];
}

size_t round_block(size_t bytes)
{
    const size_t q = bytes >= ((size_t)1 << 24) ? ((size_t)1 << 21) : 256;  // 2 MiB steps for big blocks
    return (bytes + q - 1) / q * q;
}

// Caller holds c.mu.  Drops one block's reference to its free event.
void drop_event(DeviceCache& c, FreeEvent* f)
{
    if (f && --f->refs == 0) {
        c.events.push_back(f->ev);
        delete f;
    }
}

// Caller holds c.mu.  Waits for the idle blocks' frees and returns them.
void release_idle(DeviceCache& c)
{
    for (CachedBlock& b : c.idle) {
        if (b.freed) {
            (void)hipEventSynchronize(b.freed->ev);
            drop_event(c, b.freed);
        }
        (void)hipFree(b.ptr);
    }
    c.idle.clear();
}

hipError_t dev_alloc(void** ptr, size_t bytes, int dev, hipStream_t s)
{
    *ptr = nullptr;
    bytes = round_block(bytes == 0 ? 256 : bytes);
    DeviceCache& c = cache_for(dev);
    std::lock_guard<std::mutex> lk(c.mu);
    int best = -1;
    for (int i = 0; i < (int)c.idle.size(); ++i) {
        const size_t have = c.idle[i].bytes;
        if (have >= bytes && have <= 2 * bytes && (best < 0 || have < c.idle[best].bytes)) best = i;
    }
    if (best >= 0) {
        CachedBlock b = c.idle[best];
        c.idle.erase(c.idle.begin() + best);
        if (b.freed) {
            (void)hipStreamWaitEvent(s, b.freed->ev, 0);
            drop_event(c, b.freed);
        }
        c.live.emplace_back(b.ptr, b.bytes);
        *ptr = b.ptr;
        return hipSuccess;
    }
    hipError_t e = hipMalloc(ptr, bytes);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) {
        (void)hipGetLastError();
        release_idle(c);
        e = hipMalloc(ptr, bytes);
    }
    if (e != hipSuccess) {
        *ptr = nullptr;
        return e;
    }
    c.live.emplace_back(*ptr, bytes);
    return hipSuccess;
}

// Returns blocks to the cache.  Their last uses are ordered on stream s:
// one event recorded there now orders whoever takes any of them next.
// With `idle` the caller has already waited for them (no event).
void dev_free_many(void* const* ptrs, size_t count, int dev, hipStream_t s, bool idle = false)
{
    DeviceCache& c = cache_for(dev);
    std::lock_guard<std::mutex> lk(c.mu);
    FreeEvent* fe = nullptr;
    if (!idle) {
        hipEvent_t ev = nullptr;
        if (!c.events.empty()) {
            ev = c.events.back();
            c.events.pop_back();
        } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            ev = nullptr;
        }
        if (ev && hipEventRecord(ev, s) != hipSuccess) {
            (void)hipGetLastError();
            c.events.push_back(ev);
            ev = nullptr;
        }
        if (ev) fe = new FreeEvent{ev, 0};
        else (void)hipStreamSynchronize(s);  // no event: wait here instead
    }
    for (size_t k = 0; k < count; ++k) {
        void* ptr = ptrs[k];
        if (!ptr) continue;
        for (size_t i = 0; i < c.live.size(); ++i) {
            if (c.live[i].first != ptr) continue;
            const size_t bytes = c.live[i].second;
            c.live[i] = c.live.back();
            c.live.pop_back();
            if (fe) ++fe->refs;
            c.idle.push_back(CachedBlock{ptr, bytes, fe});
            break;
        }
    }
    if (fe && fe->refs == 0) {
        c.events.push_back(fe->ev);
        delete fe;
    }
}

void dev_free(void* ptr, int dev, hipStream_t s)
{
    if (ptr) dev_free_many(&ptr, 1, dev, s);
}

// ------------------------------------------------------------- profiling

struct ProfEntry {
    const char* name;
    int64_t launches;
    double total_ms;
};
struct Pending {
    const char* name;
    hipEvent_t a, b;
};
bool g_prof_on = false;
std::string g_prof_only;  // when not empty: the one label bracketed
std::vector<ProfEntry> g_prof;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event()
{
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    // Timing only: read after the caller has synchronised the device, so the
    // record needs no system-scope fence (a fence per record flushes caches
    // and adds microseconds between short launches).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

namespace lx {

int prof_begin(const char* name, hipStream_t s)
{
    if (!g_prof_on) return -1;
    if (!g_prof_only.empty() && g_prof_only != name) return -1;
    Pending p{name, take_event(), take_event()};
    if (!p.a || !p.b) return -1;
    (void)hipEventRecord(p.a, s);
    g_pending.push_back(p);
    return (int)g_pending.size() - 1;
}

void prof_end(int token, hipStream_t s)
{
    if (token < 0 || token >= (int)g_pending.size()) return;
    (void)hipEventRecord(g_pending[token].b, s);
}

}  // namespace lx

// ------------------------------------------------------- host-side helpers

// Pinned host words for reading a plan's NaN/Inf flag back: a copy into
// pinned memory is a plain DMA, where pageable memory would be staged.
// One allocation per process, slots handed out under a lock; when all are
// taken, the caller falls back to its own (pageable) word.
struct PinnedFlags {
    std::mutex mu;
    uint32_t* base = nullptr;
    bool tried = false;
    std::vector<int> free;
};
PinnedFlags g_pinned;
constexpr int kPinnedSlots = 256;

uint32_t* take_pinned_flag()
{
    std::lock_guard<std::mutex> lk(g_pinned.mu);
    if (!g_pinned.tried) {
        g_pinned.tried = true;
        void* p = nullptr;
        if (hipHostMalloc(&p, kPinnedSlots * 64, hipHostMallocDefault) == hipSuccess) {
            g_pinned.base = (uint32_t*)p;
            for (int i = kPinnedSlots - 1; i >= 0; --i) g_pinned.free.push_back(i);
        } else {
            (void)hipGetLastError();
        }
    }
    if (g_pinned.free.empty()) return nullptr;
    const int i = g_pinned.free.back();
    g_pinned.free.pop_back();
    return g_pinned.base + (size_t)i * 16;  // one 64-byte line per slot
}

void give_pinned_flag(uint32_t* w)
{
    if (!w) return;
    std::lock_guard<std::mutex> lk(g_pinned.mu);
    g_pinned.free.push_back((int)((w - g_pinned.base) / 16));
}

// LDS bytes a workgroup may use on a device (looked up once per device).
int lds_budget(int dev)
{
    static std::mutex mu;
    static std::vector<int> cached;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)cached.size() <= dev) cached.resize((size_t)dev + 1, 0);
    if (!cached[dev]) {
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
            (void)hipGetLastError();
            lds = 65536;
        }
        if (lds > 160 * 1024) lds = 160 * 1024;
        cached[dev] = lds - 1024;
    }
    return cached[dev];
}

// ----------------------------------------------------------------- plans

struct laplex_plan_s {
    int device = 0;
    int64_t n = 0, k = 0;
    bool sym = true, phased = false;
    int algo = LAPLEX_ALGO_AUTO;
    double temperature = 1.0;
    double inv_t = 1.0;  // 1 / temperature, +inf at temperature 0
    int lds_bytes = 0;
    // sorted sides and the replay records of their sorts
    float* sa = nullptr;
    float* sb = nullptr;  // general only (symmetric: aliases sa)
    lx::SortRecords ra, rb;
    // permutations (rank -> original index), made from the records on demand
    uint32_t* pa = nullptr;
    uint32_t* pb = nullptr;
    // Gram: first sorted-b position of every interval of the sorted a, and
    // the rank of each original index of a, made on the first gram call
    uint32_t* gbound = nullptr;
    uint32_t* grank = nullptr;
    // Gram: b's inputs split by original index into one slice per die
    uint32_t* gslice_off = nullptr;
    uint32_t* gslice_src = nullptr;
    float* gslice_b = nullptr;
    float* gslice_c = nullptr;
    float* gslice_s = nullptr;
    // copies in original order (general only)
    float* a0 = nullptr;
    float* b0 = nullptr;
    float* phi0 = nullptr;
    float* psi0 = nullptr;
    // phase factors by rank: phi by a's order, psi by b's order (a's if symmetric)
    float* cphi = nullptr;
    float* sphi = nullptr;
    float* cpsi = nullptr;
    float* spsi = nullptr;
    // general plans: cos/sin of the phases in original order
    float* cphi0 = nullptr;
    float* sphi0 = nullptr;
    float* cpsi0 = nullptr;
    float* spsi0 = nullptr;
    // plan_create_apply keeps its input x for a later backward: the rows by
    // rank (when they travelled with the sort; stride pad64(n)) or a copy in
    // original order
    float* kept_x = nullptr;
    bool kept_by_rank = false;
    int64_t kept_batch = 0;
    // workspace for apply / gram
    void* ws = nullptr;
    size_t ws_bytes = 0;
    std::vector<void*> owned;
    // the stream the plan's work was ordered on (multi: more than one)
    hipStream_t stream = nullptr;
    bool stream_known = false, multi_stream = false;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
        else prev = -1;
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

hipError_t plan_alloc(laplex_plan p, void** out, size_t bytes, hipStream_t s)
{
    hipError_t e = dev_alloc(out, bytes, p->device, s);
    if (e == hipSuccess) p->owned.push_back(*out);
    return e;
}

void note_stream(laplex_plan p, hipStream_t s)
{
    if (!p->stream_known) {
        p->stream = s;
        p->stream_known = true;
    } else if (p->stream != s) {
        p->multi_stream = true;
    }
}

void plan_release(laplex_plan p)
{
    if (!p) return;
    std::vector<void*> blocks = p->owned;
    if (p->ws) blocks.push_back(p->ws);
    if (p->stream_known && !p->multi_stream) {
        // all of the plan's work was ordered on one stream: the blocks go
        // back to the cache behind one event on it, nothing waits here
        dev_free_many(blocks.data(), blocks.size(), p->device, p->stream);
    } else {
        // several streams may still use the plan's memory: wait for the
        // device, then the blocks go back to the cache already idle
        (void)hipDeviceSynchronize();
        dev_free_many(blocks.data(), blocks.size(), p->device, nullptr, true);
    }
    delete p;
}

hipError_t ensure_ws(laplex_plan p, size_t bytes, hipStream_t s)
{
    if (p->ws_bytes >= bytes) return hipSuccess;
    if (p->ws) dev_free(p->ws, p->device, s);
    p->ws = nullptr;
    p->ws_bytes = 0;
    const size_t want = align256(bytes + bytes / 8);
    hipError_t e = dev_alloc(&p->ws, want, p->device, s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        e = dev_alloc(&p->ws, align256(bytes), p->device, s);
        if (e != hipSuccess) return e;
        p->ws_bytes = align256(bytes);
        return hipSuccess;
    }
    p->ws_bytes = want;
    return hipSuccess;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + nb && y < x + na;
}

laplex_status check_device()
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(LAPLEX_ERR_NO_DEVICE, "no HIP device visible");
    }
    return LAPLEX_OK;
}



// Bump allocator over the plan workspace.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base((char*)b) {}
    template <class T>
    T* take(size_t count)
    {
        T* p = (T*)(base + off);
        off += align256(count * sizeof(T));
        return p;
    }
};

// Workspace of one scan along a side of length len: `vecs` single-channel
// rows [batch][ld], `chrows` rows per channel [ch][batch][ld], and the tile
// composites and carries.
size_t scan_ws_bytes(int64_t len, int64_t batch, int ch, int vecs, int chrows)
{
    const int64_t ld = pad64(len);
    const int64_t tiles = (len + lx::kScanTile - 1) / lx::kScanTile;
    const int64_t groups = (tiles + lx::kCarryGroup - 1) / lx::kCarryGroup;
    size_t b = 0;
    b += (size_t)vecs * align256((size_t)batch * ld * 4);
    b += (size_t)chrows * align256((size_t)ch * batch * ld * 4);
    b += align256((size_t)ch * batch * tiles * 4 * 8);
    b += align256((size_t)ch * batch * groups * 4 * 8);
    b += align256((size_t)ch * batch * tiles * 2 * 8);
    return b;
}

void scan_common(lx::ScanArgs& A, Carve& cv, int64_t len, int64_t batch, int ch)
{
    A.channels = ch;
    A.n = len;
    A.tiles = (len + lx::kScanTile - 1) / lx::kScanTile;
    A.batch = batch;
    A.ld = pad64(len);
    const int64_t groups = (A.tiles + lx::kCarryGroup - 1) / lx::kCarryGroup;
    A.agg = cv.take<double>((size_t)ch * batch * A.tiles * 4);
    A.gagg = cv.take<double>((size_t)ch * batch * groups * 4);
    A.carry = cv.take<double>((size_t)ch * batch * A.tiles * 2);
}

// Sides at least this long move x into sorted order and y back by replaying
// the sort (streaming passes); shorter ones gather/scatter through the
// permutation directly (fewer launches).
int64_t replay_min()
{
    static int64_t v = [] {
        const char* e = getenv("LAPLEX_REPLAY_MIN");
        return e ? atoll(e) : (int64_t)1 << 20;
    }();
    return v;
}

// Make the permutation of side 0 (a) or 1 (b) from the sort records.
hipError_t ensure_perm(laplex_plan p, int side, hipStream_t s)
{
    uint32_t** dst = side == 0 ? &p->pa : &p->pb;
    if (*dst) return hipSuccess;
    if (side == 1 && p->sym) {
        hipError_t e = ensure_perm(p, 0, s);
        p->pb = p->pa;
        return e;
    }
    const lx::SortRecords& R = side == 0 ? p->ra : p->rb;
    void* perm = nullptr;
    void* tmp = nullptr;
    hipError_t e = plan_alloc(p, &perm, (size_t)R.n * 4, s);
    if (e != hipSuccess) return e;
    e = dev_alloc(&tmp, (size_t)R.n * 4, p->device, s);
    if (e != hipSuccess) return e;
    e = lx::perm_from_records(R, (uint32_t*)perm, (uint32_t*)tmp, s);
    dev_free(tmp, p->device, s);
    if (e == hipSuccess) *dst = (uint32_t*)perm;
    return e;
}

}  // namespace

extern "C" {

const char* laplex_status_str(laplex_status s)
{
    switch (s) {
        case LAPLEX_OK: return "ok";
        case LAPLEX_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LAPLEX_ERR_NONFINITE_ANCHOR: return "non-finite anchor or phase";
        case LAPLEX_ERR_OUT_OF_MEMORY: return "out of device memory";
        case LAPLEX_ERR_UNSUPPORTED: return "unsupported";
        case LAPLEX_ERR_DEVICE: return "device error";
        case LAPLEX_ERR_NO_DEVICE: return "no device";
    }
    return "unknown status";
}

const char* laplex_last_error(void) { return g_last_error.c_str(); }

namespace {

// Plan creation; with x != NULL (symmetric plans only) also y = K x, sorting
// the rows of x along with the anchors when the plan replays its sort.
laplex_status plan_create_impl(laplex_plan* out, const float* a, int64_t n, const float* b, int64_t k,
                               const float* phi, const float* psi, const float* x, float* y, int64_t batch,
                               void* stream)
{
    if (out) *out = nullptr;
    if (!out) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "out is NULL");
    if (!a) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "a is NULL");
    if (n < 1 || n > kMaxLen) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "n must be in [1, 2^30]");
    const bool sym = b == nullptr;
    if (sym && k != 0 && k != n) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "symmetric plan: k must be 0 or n");
    if (!sym && (k < 1 || k > kMaxLen)) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "k must be in [1, 2^30]");
    if ((phi == nullptr) != (psi == nullptr))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "phi and psi: give both or neither");
    if (sym) k = n;
    laplex_status st = check_device();
    if (st != LAPLEX_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    laplex_plan p = new laplex_plan_s();
    note_stream(p, s);
    p->n = n;
    p->k = k;
    p->sym = sym;
    p->phased = phi != nullptr;
    void* scratch = nullptr;
    uint32_t* flag = nullptr;
    uint32_t own_flag = 0;
    uint32_t* pinned = take_pinned_flag();
    uint32_t* host_flag = pinned ? pinned : &own_flag;
    struct PinnedRelease {
        uint32_t* w;
        ~PinnedRelease() { give_pinned_flag(w); }
    } pinned_release{pinned};
    auto bail = [&](laplex_status code) {
        if (scratch) dev_free(scratch, p->device, s);
        plan_release(p);
        return code;
    };
#define LX_PLAN_TRY(call, where)                                  \
    do {                                                         \
        const laplex_status lx_s2_ = from_hip((call), (where));  \
        if (lx_s2_ != LAPLEX_OK) return bail(lx_s2_);            \
    } while (0)

    LX_PLAN_TRY(hipGetDevice(&p->device), "hipGetDevice");
    p->lds_bytes = lds_budget(p->device);
    LX_PLAN_TRY(plan_alloc(p, (void**)&flag, 256, s), "alloc flag");
    LX_PLAN_TRY(plan_alloc(p, (void**)&p->sa, (size_t)n * 4, s), "alloc sorted a");
    const bool small_plan = sym && n <= lx::kSmallMax && n < replay_min();
    // the small plan kernel writes the flag whole; the others OR into it
    if (!small_plan) LX_PLAN_TRY(lx::fill_u32(flag, 0u, 1, s), "clear flag");
    if (small_plan) {
        // A small symmetric plan in one workgroup: the sorted anchors, the
        // permutation (the sort records are never needed below the replay
        // size) and the phase factors by rank; y = K x too for a few vectors.
        LX_PLAN_TRY(plan_alloc(p, (void**)&p->pa, (size_t)n * 4, s), "alloc permutation");
        p->sb = p->sa;
        p->pb = p->pa;
        if (p->phased) {
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->sphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cpsi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->spsi, (size_t)n * 4, s), "alloc phases");
        }
        const bool with_y = x != nullptr && batch <= 8;
        // the kernel that computes y also copies x for a later backward
        float* keep = nullptr;
        if (with_y) LX_PLAN_TRY(plan_alloc(p, (void**)&keep, (size_t)(batch * n) * 4, s), "alloc kept x");
        lx::SmallSymArgs S;
        S.n = n;
        S.batch = with_y ? (int)batch : 0;
        S.inv_t = p->inv_t;
        S.a = a;
        S.phi = phi;
        S.psi = psi;
        S.x = with_y ? x : nullptr;
        S.x_keep = keep;
        S.y = with_y ? y : nullptr;
        S.sa = p->sa;
        S.perm = p->pa;
        S.cphi = p->cphi;
        S.sphi = p->sphi;
        S.cpsi = p->cpsi;
        S.spsi = p->spsi;
        S.flag = flag;
        LX_PLAN_TRY(lx::small_sym_launch(S, s), "small plan");
        LX_PLAN_TRY(hipMemcpyAsync(host_flag, flag, 4, hipMemcpyDeviceToHost, s), "read flag");
        LX_PLAN_TRY(hipStreamSynchronize(s), "synchronize");
        if (*host_flag & 1u) return bail(fail(LAPLEX_ERR_NONFINITE_ANCHOR, "NaN or Inf among anchors or phases"));
        if (x) {
            // x in its original order is kept for a later backward (copied
            // by the plan kernel when it computed y)
            laplex_status st2 = with_y ? LAPLEX_OK : laplex_apply(p, x, y, batch, 0, stream);
            if (!with_y && st2 == LAPLEX_OK)
                st2 = from_hip(plan_alloc(p, (void**)&keep, (size_t)(batch * n) * 4, s), "alloc kept x");
            if (!with_y && st2 == LAPLEX_OK)
                st2 = from_hip(hipMemcpyAsync(keep, x, (size_t)(batch * n) * 4, hipMemcpyDeviceToDevice, s), "copy x");
            p->kept_x = keep;
            p->kept_by_rank = false;
            p->kept_batch = batch;
            if (st2 != LAPLEX_OK) {
                plan_release(p);
                return st2;
            }
        }
        *out = p;
        return LAPLEX_OK;
    }
    {
        void* rec = nullptr;
        LX_PLAN_TRY(plan_alloc(p, &rec, lx::sort_record_bytes(n), s), "alloc sort records");
        p->ra = lx::sort_records_at(rec, n);
    }
    const int64_t big = sym ? n : (n > k ? n : k);
    // Symmetric plans on the replay path sort value rows with the anchors:
    // the rows of x (when applying at once) and the phases.
    const bool replay = sym && n >= replay_min();
    const int ph_rows = p->phased ? 2 : 0;
    const bool fuse = x != nullptr && replay && batch + ph_rows <= lx::kMaxSortVals;
    lx::SortVals V;
    if (replay) {
        if (fuse)
            for (int64_t v = 0; v < batch; ++v) V.in[V.rows++] = x + v * n;
        if (p->phased) {
            V.in[V.rows++] = phi;
            V.in[V.rows++] = psi;
        }
        V.ld = pad64(n);
    }
    const size_t vbytes = align256((size_t)V.rows * V.ld * 4);
    // value buffers: va and vb for the sort; when applying at once the sorted
    // rows (vb) stay with the plan for a later backward, and a third buffer
    // joins the ping-pong of the replay back into y
    LX_PLAN_TRY(dev_alloc(&scratch, lx::sort_scratch_bytes(big, V.rows > 0) + 2 * vbytes, p->device, s),
                "alloc sort scratch");
    float* vt = nullptr;
    if (V.rows) {
        V.va = (float*)((char*)scratch + lx::sort_scratch_bytes(big, V.rows > 0));
        if (fuse) {
            LX_PLAN_TRY(plan_alloc(p, (void**)&V.vb, vbytes, s), "alloc kept x");
            vt = (float*)((char*)V.va + vbytes);
            p->kept_x = V.vb;
            p->kept_by_rank = true;
            p->kept_batch = batch;
        } else {
            V.vb = (float*)((char*)V.va + vbytes);
        }
    }
    LX_PLAN_TRY(lx::sort_launch(a, n, p->sa, p->ra, scratch, flag, s, V.rows ? &V : nullptr), "sort a");
    if (sym) {
        p->sb = p->sa;
        p->rb = p->ra;
        // short sides gather through the permutation
        if (!replay) LX_PLAN_TRY(ensure_perm(p, 0, s), "permutation");
        if (p->phased) {
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->sphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cpsi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->spsi, (size_t)n * 4, s), "alloc phases");
            if (replay) {
                // the phases came out of the sort in rank order: the last two rows
                const float* sphi_rank = V.vb + (V.rows - 2) * V.ld;
                const float* spsi_rank = V.vb + (V.rows - 1) * V.ld;
                LX_PLAN_TRY(lx::phase_factors_launch(sphi_rank, nullptr, n, p->cphi, p->sphi, flag, s), "phi factors");
                LX_PLAN_TRY(lx::phase_factors_launch(spsi_rank, nullptr, n, p->cpsi, p->spsi, flag, s), "psi factors");
            } else {
                LX_PLAN_TRY(lx::phase_factors_launch(phi, p->pa, n, p->cphi, p->sphi, flag, s), "phi factors");
                LX_PLAN_TRY(lx::phase_factors_launch(psi, p->pa, n, p->cpsi, p->spsi, flag, s), "psi factors");
            }
        }
        if (fuse) {
            // y = K x from the sorted rows of x: scan in place, replay back into y
            const int ch = p->phased ? 2 : 1;
            LX_PLAN_TRY(ensure_ws(p, scan_ws_bytes(n, batch, ch, 0, 0), s), "workspace");
            Carve cv(p->ws);
            lx::ScanArgs A;
            A.mode = lx::kScanSym;
            scan_common(A, cv, n, batch, ch);
            A.inv_t = p->inv_t;
            A.s = p->sa;
            A.random = false;
            A.xs = V.vb;  // kept: y by rank goes to va
            A.ys = V.va;
            if (p->phased) {
                A.in_c = p->cpsi;
                A.in_s = p->spsi;
                A.out_c = p->cphi;
                A.out_s = p->sphi;
            }
            LX_PLAN_TRY(lx::scan_launch(A, s), "symmetric apply");
            const lx::SortRecords& R = p->ra;
            LX_PLAN_TRY(lx::replay_launch(R, 3, false, V.va, V.ld, vt, V.ld, batch, s), "replay");
            LX_PLAN_TRY(lx::replay_launch(R, 2, false, vt, V.ld, V.va, V.ld, batch, s), "replay");
            LX_PLAN_TRY(lx::replay_launch(R, 1, false, V.va, V.ld, vt, V.ld, batch, s), "replay");
            LX_PLAN_TRY(lx::replay_launch(R, 0, false, vt, V.ld, y, n, batch, s), "replay");
        }
    } else {
        LX_PLAN_TRY(plan_alloc(p, (void**)&p->sb, (size_t)k * 4, s), "alloc sorted b");
        {
            void* rec = nullptr;
            LX_PLAN_TRY(plan_alloc(p, &rec, lx::sort_record_bytes(k), s), "alloc sort records");
            p->rb = lx::sort_records_at(rec, k);
        }
        LX_PLAN_TRY(lx::sort_launch(b, k, p->sb, p->rb, scratch, flag, s), "sort b");
        LX_PLAN_TRY(ensure_perm(p, 0, s), "permutation of a");
        LX_PLAN_TRY(ensure_perm(p, 1, s), "permutation of b");
        LX_PLAN_TRY(plan_alloc(p, (void**)&p->a0, (size_t)n * 4, s), "alloc a copy");
        LX_PLAN_TRY(plan_alloc(p, (void**)&p->b0, (size_t)k * 4, s), "alloc b copy");
        LX_PLAN_TRY(hipMemcpyAsync(p->a0, a, (size_t)n * 4, hipMemcpyDeviceToDevice, s), "copy a");
        LX_PLAN_TRY(hipMemcpyAsync(p->b0, b, (size_t)k * 4, hipMemcpyDeviceToDevice, s), "copy b");
        if (p->phased) {
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->phi0, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->psi0, (size_t)k * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->sphi, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cpsi, (size_t)k * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->spsi, (size_t)k * 4, s), "alloc phases");
            LX_PLAN_TRY(hipMemcpyAsync(p->phi0, phi, (size_t)n * 4, hipMemcpyDeviceToDevice, s), "copy phi");
            LX_PLAN_TRY(hipMemcpyAsync(p->psi0, psi, (size_t)k * 4, hipMemcpyDeviceToDevice, s), "copy psi");
            LX_PLAN_TRY(lx::phase_factors_launch(phi, p->pa, n, p->cphi, p->sphi, flag, s), "phi factors");
            LX_PLAN_TRY(lx::phase_factors_launch(psi, p->pb, k, p->cpsi, p->spsi, flag, s), "psi factors");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cphi0, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->sphi0, (size_t)n * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->cpsi0, (size_t)k * 4, s), "alloc phases");
            LX_PLAN_TRY(plan_alloc(p, (void**)&p->spsi0, (size_t)k * 4, s), "alloc phases");
            LX_PLAN_TRY(lx::phase_factors_launch(phi, nullptr, n, p->cphi0, p->sphi0, flag, s), "phi factors");
            LX_PLAN_TRY(lx::phase_factors_launch(psi, nullptr, k, p->cpsi0, p->spsi0, flag, s), "psi factors");
        }
    }
    dev_free(scratch, p->device, s);
    scratch = nullptr;
    LX_PLAN_TRY(hipMemcpyAsync(host_flag, flag, 4, hipMemcpyDeviceToHost, s), "read flag");
    LX_PLAN_TRY(hipStreamSynchronize(s), "synchronize");
    if (*host_flag & 1u) return bail(fail(LAPLEX_ERR_NONFINITE_ANCHOR, "NaN or Inf among anchors or phases"));
#undef LX_PLAN_TRY
    if (x && !fuse) {
        // not fused (short side or too many rows): the plain apply, and a copy
        // of x kept for a later backward
        laplex_status st2 = laplex_apply(p, x, y, batch, 0, stream);
        if (st2 == LAPLEX_OK) {
            float* keep = nullptr;
            st2 = from_hip(plan_alloc(p, (void**)&keep, (size_t)(batch * n) * 4, s), "alloc kept x");
            if (st2 == LAPLEX_OK)
                st2 = from_hip(hipMemcpyAsync(keep, x, (size_t)(batch * n) * 4, hipMemcpyDeviceToDevice, s), "copy x");
            p->kept_x = keep;
            p->kept_by_rank = false;
            p->kept_batch = batch;
        }
        if (st2 != LAPLEX_OK) {
            plan_release(p);
            return st2;
        }
    }
    *out = p;
    return LAPLEX_OK;
}

}  // namespace

laplex_status laplex_plan_create(laplex_plan* out, const float* a, int64_t n, const float* b, int64_t k,
                                 const float* phi, const float* psi, void* stream)
{
    return plan_create_impl(out, a, n, b, k, phi, psi, nullptr, nullptr, 0, stream);
}

laplex_status laplex_plan_create_apply(laplex_plan* out, const float* a, int64_t n, const float* phi,
                                       const float* psi, const float* x, float* y, int64_t batch, void* stream)
{
    if (out) *out = nullptr;
    if (!out) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "out is NULL");
    if (!x || !y) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (batch < 1) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (n >= 1 && (batch > (int64_t)1 << 40 || (double)batch * (double)n > 4.0e18 / 4))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch too large");
    if (n >= 1 && ranges_overlap(x, (size_t)(batch * n) * 4, y, (size_t)(batch * n) * 4))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "x and y overlap");
    return plan_create_impl(out, a, n, nullptr, 0, phi, psi, x, y, batch, stream);
}

laplex_status laplex_plan_destroy(laplex_plan p)
{
    if (!p) return LAPLEX_OK;
    DeviceGuard g(p->device);
    plan_release(p);
    return LAPLEX_OK;
}

laplex_status laplex_plan_perm(laplex_plan p, int side, const uint32_t** perm_dev)
{
    if (!p || !perm_dev || (side != 0 && side != 1)) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "bad plan_perm arguments");
    DeviceGuard g(p->device);
    note_stream(p, nullptr);
    LX_TRY(ensure_perm(p, side, nullptr), "permutation");
    LX_TRY(hipStreamSynchronize(nullptr), "synchronize");
    *perm_dev = side == 0 ? p->pa : p->pb;
    return LAPLEX_OK;
}

laplex_status laplex_plan_sorted(laplex_plan p, int side, const float** sorted_dev)
{
    if (!p || !sorted_dev || (side != 0 && side != 1))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "bad plan_sorted arguments");
    *sorted_dev = side == 0 ? p->sa : p->sb;
    return LAPLEX_OK;
}

laplex_status laplex_plan_info(laplex_plan p, int64_t* n, int64_t* k, int* flags)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (n) *n = p->n;
    if (k) *k = p->k;
    if (flags) *flags = (p->sym ? LAPLEX_PLAN_SYMMETRIC : 0) | (p->phased ? LAPLEX_PLAN_PHASED : 0);
    return LAPLEX_OK;
}

laplex_status laplex_plan_set_option(laplex_plan p, int option, int64_t value)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (option != LAPLEX_OPT_GENERAL_ALGO) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "unknown option");
    if (value != LAPLEX_ALGO_AUTO && value != LAPLEX_ALGO_BUCKET && value != LAPLEX_ALGO_EVALUATE)
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "unknown algorithm");
    p->algo = (int)value;
    return LAPLEX_OK;
}

laplex_status laplex_plan_set_temperature(laplex_plan p, double t)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!(t == 0.0 || (t >= (double)FLT_MIN && t <= (double)FLT_MAX)))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "temperature must be 0 or in [FLT_MIN, FLT_MAX]");
    p->temperature = t;
    p->inv_t = t > 0.0 ? 1.0 / t : HUGE_VAL;
    return LAPLEX_OK;
}

}  // extern "C"

namespace {

// Where an apply takes its workspace: the plan's own (grown on demand), or
// a fixed region that must already be large enough (no allocation).
struct WsSource {
    void* fixed = nullptr;
    size_t fixed_bytes = 0;
};

laplex_status take_ws(laplex_plan p, size_t need, hipStream_t s, const WsSource& src, void** base)
{
    if (src.fixed) {
        if (need > src.fixed_bytes)
            return fail(LAPLEX_ERR_INVALID_ARGUMENT, "this apply needs " + std::to_string(need) +
                                                         " bytes of scratch; the fixed scratch holds " +
                                                         std::to_string(src.fixed_bytes));
        *base = src.fixed;
        return LAPLEX_OK;
    }
    LX_TRY(ensure_ws(p, need, s), "workspace");
    *base = p->ws;
    return LAPLEX_OK;
}

#define LX_WS(need, base)                                           \
    do {                                                            \
        const laplex_status lx_w_ = take_ws(p, (need), s, src, &(base)); \
        if (lx_w_ != LAPLEX_OK) return lx_w_;                       \
    } while (0)

laplex_status apply_impl(laplex_plan p, const float* x, float* y, int64_t batch, int transpose, void* stream,
                         const WsSource& src)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!x || !y) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (batch < 1) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (transpose != 0 && transpose != 1) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1");
    const int64_t len_in = transpose ? p->n : p->k;
    const int64_t len_out = transpose ? p->k : p->n;
    if (batch > (int64_t)1 << 40 || (double)batch * (double)(len_in > len_out ? len_in : len_out) > 4.0e18 / 4)
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch too large");
    if (ranges_overlap(x, (size_t)(batch * len_in) * 4, y, (size_t)(batch * len_out) * 4))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "x and y overlap");
    DeviceGuard g(p->device);
    hipStream_t s = (hipStream_t)stream;
    note_stream(p, s);
    const int ch = p->phased ? 2 : 1;

    if (p->sym) {
        const int64_t n = p->n;
        const bool replay = n >= replay_min();
        if (!replay && !p->pa) {
            if (src.fixed) return fail(LAPLEX_ERR_UNSUPPORTED, "the plan has no permutation yet");
            LX_TRY(ensure_perm(p, 0, s), "permutation");
        }
        void* wsb = nullptr;
        LX_WS(scan_ws_bytes(n, batch, ch, replay ? 2 : 1, 0), wsb);
        Carve cv(wsb);
        lx::ScanArgs A;
        A.mode = lx::kScanSym;
        scan_common(A, cv, n, batch, ch);
        A.inv_t = p->inv_t;
        A.s = p->sa;
        A.perm = p->pa;
        if (p->phased) {
            // K = LAPLEX(a, phi; a, psi): inputs carry psi, outputs phi; K^T swaps them
            A.in_c = transpose ? p->cphi : p->cpsi;
            A.in_s = transpose ? p->sphi : p->spsi;
            A.out_c = transpose ? p->cpsi : p->cphi;
            A.out_s = transpose ? p->spsi : p->sphi;
        }
        if (!replay) {
            A.random = true;
            A.x = x;
            A.y = y;
            A.xs = cv.take<float>((size_t)batch * A.ld);
            LX_TRY(lx::scan_launch(A, s), "symmetric apply");
            return LAPLEX_OK;
        }
        // x -> sorted order by replaying the four radix passes, scan in place,
        // then replay them backwards into y.
        float* t1 = cv.take<float>((size_t)batch * A.ld);
        float* t2 = cv.take<float>((size_t)batch * A.ld);
        const lx::SortRecords& R = p->ra;
        LX_TRY(lx::replay_launch(R, 0, true, x, n, t1, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 1, true, t1, A.ld, t2, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 2, true, t2, A.ld, t1, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 3, true, t1, A.ld, t2, A.ld, batch, s), "replay");
        A.random = false;
        A.xs = t2;
        A.ys = t2;
        LX_TRY(lx::scan_launch(A, s), "symmetric apply");
        LX_TRY(lx::replay_launch(R, 3, false, t2, A.ld, t1, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 2, false, t1, A.ld, t2, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 1, false, t2, A.ld, t1, A.ld, batch, s), "replay");
        LX_TRY(lx::replay_launch(R, 0, false, t1, A.ld, y, n, batch, s), "replay");
        return LAPLEX_OK;
    }

    // General case: side "o" receives the outputs, side "i" holds the inputs.
    const bool out_is_a = transpose == 0;
    const int64_t no = out_is_a ? p->n : p->k;
    const int64_t ni = out_is_a ? p->k : p->n;
    const float* s_o = out_is_a ? p->sa : p->sb;
    const uint32_t* p_o = out_is_a ? p->pa : p->pb;
    const float* s_i = out_is_a ? p->sb : p->sa;
    const uint32_t* p_i = out_is_a ? p->pb : p->pa;
    const float* anchor_o = out_is_a ? p->a0 : p->b0;
    const float* anchor_i = out_is_a ? p->b0 : p->a0;
    const float* co0 = out_is_a ? p->cphi0 : p->cpsi0;  // cos/sin of phases, original order
    const float* so0 = out_is_a ? p->sphi0 : p->spsi0;
    const float* ci0 = out_is_a ? p->cpsi0 : p->cphi0;
    const float* si0 = out_is_a ? p->spsi0 : p->sphi0;
    const float* c_o = out_is_a ? p->cphi : p->cpsi;
    const float* sn_o = out_is_a ? p->sphi : p->spsi;
    const float* c_i = out_is_a ? p->cpsi : p->cphi;
    const float* sn_i = out_is_a ? p->spsi : p->sphi;
    int algo = p->algo;
    if (algo == LAPLEX_ALGO_AUTO) algo = ni <= no ? LAPLEX_ALGO_EVALUATE : LAPLEX_ALGO_BUCKET;

    if (algo == LAPLEX_ALGO_EVALUATE) {
        void* wsb = nullptr;
        LX_WS(scan_ws_bytes(ni, batch, ch, 1, 2), wsb);
        Carve cv(wsb);
        lx::ScanArgs A;
        A.mode = lx::kScanPLPR;
        A.random = true;
        scan_common(A, cv, ni, batch, ch);
        A.inv_t = p->inv_t;
        A.s = s_i;
        A.perm = p_i;
        A.x = x;
        A.xs = cv.take<float>((size_t)batch * A.ld);
        A.pl = cv.take<float>((size_t)ch * batch * A.ld);
        A.pr = cv.take<float>((size_t)ch * batch * A.ld);
        if (p->phased) {
            A.in_c = c_i;
            A.in_s = sn_i;
        }
        LX_TRY(lx::scan_launch(A, s), "scan over the input side");
        lx::EvalArgs E;
        E.channels = ch;
        E.n_out = no;
        E.n_in = ni;
        E.batch = batch;
        E.inv_t = (float)p->inv_t;
        E.out_anchor = anchor_o;
        if (p->phased) {
            E.out_cos = co0;
            E.out_sin = so0;
        }
        E.s_in = s_i;
        E.ld = A.ld;
        E.pl = A.pl;
        E.pr = A.pr;
        E.y = y;
        E.lds_bytes = p->lds_bytes;
        LX_TRY(lx::eval_launch(E, s), "evaluate outputs");
        return LAPLEX_OK;
    }

    // BUCKET: inputs into the intervals of the sorted output side, then scan it.
    lx::BucketArgs Bk;
    Bk.channels = ch;
    Bk.n_out = no;
    Bk.n_in = ni;
    Bk.batch = batch;
    Bk.inv_t = (float)p->inv_t;
    Bk.s_out = s_o;
    Bk.in_anchor = anchor_i;
    if (p->phased) {
        Bk.in_cos = ci0;
        Bk.in_sin = si0;
    }
    Bk.x = x;
    Bk.ld = pad64(no);
    Bk.lds_bytes = p->lds_bytes;
    Bk.partial_floats = lx::bucket_partial_floats(Bk, nullptr, nullptr);
    // a short output side bins in LDS; a long one merges the sorted sides
    const bool merge = Bk.partial_floats == 0;
    const size_t layout_bytes = merge ? 0 : (size_t)lx::bucket_layout_bytes(Bk);
    const size_t need = scan_ws_bytes(no, batch, ch, 0, 2) +
                        (merge ? lx::merge_ws_bytes(ni, no, batch, ch)
                               : align256((size_t)Bk.partial_floats * 4) + align256(layout_bytes));
    void* wsb = nullptr;
    LX_WS(need, wsb);
    Carve cv(wsb);
    lx::ScanArgs A;
    A.mode = lx::kScanUV;
    A.random = true;
    scan_common(A, cv, no, batch, ch);
    A.inv_t = p->inv_t;
    A.s = s_o;
    A.perm = p_o;
    float* u = cv.take<float>((size_t)ch * batch * A.ld);
    float* v = cv.take<float>((size_t)ch * batch * A.ld);
    A.u = u;
    A.v = v;
    A.y = y;
    if (p->phased) {
        A.out_c = c_o;
        A.out_s = sn_o;
    }
    if (merge) {
        lx::MergeArgs M;
        M.channels = ch;
        M.n_out = no;
        M.n_in = ni;
        M.batch = batch;
        M.inv_t = p->inv_t;
        M.s_out = s_o;
        M.s_in = s_i;
        M.perm_in = p_i;
        if (p->phased) {
            M.in_c = c_i;
            M.in_s = sn_i;
        }
        M.x = x;
        M.ld = A.ld;
        M.u = u;
        M.v = v;
        const int64_t tiles = lx::merge_tiles(ni, no);
        M.split = cv.take<uint2>((size_t)tiles + 1);
        M.head = cv.take<double>((size_t)ch * batch * tiles * 2);
        M.tail = cv.take<double>((size_t)ch * batch * tiles * 2);
        LX_TRY(lx::merge_launch(M, s), "merge inputs");
    } else {
        Bk.u = u;
        Bk.v = v;
        Bk.partial = cv.take<float>((size_t)Bk.partial_floats);
        Bk.layout = (void*)cv.take<char>(layout_bytes);
        LX_TRY(lx::bucket_launch(Bk, s), "bucket inputs");
    }
    LX_TRY(lx::scan_launch(A, s), "scan over the output side");
    return LAPLEX_OK;
}

#undef LX_WS

// ------------------------------------------------------ allocation-free apply
//
// laplex_apply_noalloc takes its workspace from this file-scope array, one
// copy per device, kept until the process ends.  Host code reaches it only
// through the device address hipGetSymbolAddress returns (looked up once per
// device, with that device current); the array's own name is a host-side
// stand-in.  Kernels never need it cleared: every word a kernel reads was
// written earlier in the same call.
constexpr size_t kNoAllocBytes = LAPLEX_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; null until looked up

hipError_t noalloc_scratch(int dev, void** out)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

laplex_status laplex_apply(laplex_plan p, const float* x, float* y, int64_t batch, int transpose, void* stream)
{
    return apply_impl(p, x, y, batch, transpose, stream, WsSource{});
}

laplex_status laplex_apply_noalloc(laplex_plan p, const float* x, float* y, int64_t batch, int transpose,
                                   void* stream)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    DeviceGuard g(p->device);
    WsSource src;
    LX_TRY(noalloc_scratch(p->device, &src.fixed), "scratch address");
    src.fixed_bytes = kNoAllocBytes;
    return apply_impl(p, x, y, batch, transpose, stream, src);
}

}  // extern "C"

namespace {

// One side of a general plan's gradient: outputs on side "o" (original
// order) from the prefix/suffix tables of the sorted side "i" of input V.
struct GradSide {
    int64_t no, ni;
    const float* s_i;
    const uint32_t* p_i;
    const float* c_i;   // cos/sin of side i's phases by rank (phased)
    const float* sn_i;
    const float* anchor_o;
    const float* c_o0;  // cos/sin of side o's phases, original order (phased)
    const float* s_o0;
    const float* s_o;       // side o sorted, and its permutation (rank -> original index)
    const uint32_t* p_o;
    const float* anchor_i0; // side i's anchors and phase factors, original order
    const float* c_i0;
    const float* s_i0;
};

// Outputs on a small side (at most 1024 anchors) from a large input side:
// the inputs are bucketed into the intervals of the sorted outputs, in
// their original order (no gather, no tables over the large side).
laplex_status grad_small_side(laplex_plan p, const GradSide& G, const float* V, const float* W, int64_t batch,
                              float* y, float* d_anchor, float* d_phase, hipStream_t s, bool* done)
{
    *done = false;
    const int ch = p->phased ? 2 : 1;
    lx::BucketArgs Bk;
    Bk.channels = ch;
    Bk.n_out = G.no;
    Bk.n_in = G.ni;
    Bk.batch = batch;
    Bk.inv_t = (float)p->inv_t;
    Bk.s_out = G.s_o;
    Bk.in_anchor = G.anchor_i0;
    if (p->phased) {
        Bk.in_cos = G.c_i0;
        Bk.in_sin = G.s_i0;
    }
    Bk.x = V;
    Bk.ld = pad64(G.no);
    Bk.lds_bytes = p->lds_bytes;
    Bk.ties = true;
    Bk.partial_floats = lx::bucket_partial_floats(Bk, nullptr, nullptr);
    if (Bk.partial_floats == 0) return LAPLEX_OK;  // not the LDS-binned shape: the table path instead
    const size_t rows = (size_t)ch * batch * Bk.ld;
    const size_t layout_bytes = (size_t)lx::bucket_layout_bytes(Bk);
    const size_t need = scan_ws_bytes(G.no, batch, ch, 0, 2) + 3 * align256(rows * 4) +
                        align256((size_t)Bk.partial_floats * 4) + align256(layout_bytes);
    LX_TRY(ensure_ws(p, need, s), "workspace");
    Carve cv(p->ws);
    lx::ScanArgs A;
    A.mode = lx::kScanUVLR;
    A.random = false;
    scan_common(A, cv, G.no, batch, ch);
    A.inv_t = p->inv_t;
    A.s = G.s_o;
    float* u = cv.take<float>(rows);
    float* v = cv.take<float>(rows);
    float* tie = cv.take<float>(rows);
    A.u = u;
    A.v = v;
    A.pl = cv.take<float>((size_t)ch * batch * A.ld);
    A.pr = cv.take<float>((size_t)ch * batch * A.ld);
    Bk.u = u;
    Bk.v = v;
    Bk.tie = tie;
    Bk.partial = cv.take<float>((size_t)Bk.partial_floats);
    Bk.layout = cv.take<char>(layout_bytes);
    LX_TRY(lx::bucket_launch(Bk, s), "bucket inputs");
    LX_TRY(lx::scan_launch(A, s), "scan over the output side");
    lx::EvalLRArgs E;
    E.channels = ch;
    E.n_out = G.no;
    E.batch = batch;
    E.ld = A.ld;
    E.anchor_scale = p->temperature > 0.0 ? (float)(-1.0 / p->temperature) : 0.f;
    E.s_out = G.s_o;
    E.perm_out = G.p_o;
    if (p->phased) {
        E.out_cos = G.c_o0;
        E.out_sin = G.s_o0;
    }
    E.L = A.pl;
    E.R = A.pr;
    E.T = tie;
    E.w = W;
    E.y = y;
    E.d_anchor = d_anchor;
    E.d_phase = d_phase;
    LX_TRY(lx::eval_lr_launch(E, s), "evaluate gradients");
    *done = true;
    return LAPLEX_OK;
}

laplex_status grad_general_side(laplex_plan p, const GradSide& G, const float* V, const float* W, int64_t batch,
                                float* y, float* d_anchor, float* d_phase, hipStream_t s)
{
    if (!y && !d_anchor && !d_phase) return LAPLEX_OK;
    if (G.no <= 1024 && G.ni > G.no) {
        bool done = false;
        const laplex_status st = grad_small_side(p, G, V, W, batch, y, d_anchor, d_phase, s, &done);
        if (st != LAPLEX_OK || done) return st;
    }
    const int ch = p->phased ? 2 : 1;
    LX_TRY(ensure_ws(p, scan_ws_bytes(G.ni, batch, ch, 1, 2), s), "workspace");
    Carve cv(p->ws);
    lx::ScanArgs A;
    A.mode = lx::kScanPLPR;
    A.random = true;
    scan_common(A, cv, G.ni, batch, ch);
    A.inv_t = p->inv_t;
    A.s = G.s_i;
    A.perm = G.p_i;
    A.x = V;
    A.xs = cv.take<float>((size_t)batch * A.ld);
    A.pl = cv.take<float>((size_t)ch * batch * A.ld);
    A.pr = cv.take<float>((size_t)ch * batch * A.ld);
    if (p->phased) {
        A.in_c = G.c_i;
        A.in_s = G.sn_i;
    }
    LX_TRY(lx::scan_launch(A, s), "scan over the input side");
    lx::EvalGradArgs E;
    E.channels = ch;
    E.n_out = G.no;
    E.n_in = G.ni;
    E.batch = batch;
    E.ld = A.ld;
    E.inv_t = (float)p->inv_t;
    E.anchor_scale = p->temperature > 0.0 ? (float)(-1.0 / p->temperature) : 0.f;
    E.out_anchor = G.anchor_o;
    if (p->phased) {
        E.out_cos = G.c_o0;
        E.out_sin = G.s_o0;
    }
    E.s_in = G.s_i;
    E.pl = A.pl;
    E.pr = A.pr;
    E.w = W;
    E.y = y;
    E.d_anchor = d_anchor;
    E.d_phase = d_phase;
    E.lds_bytes = p->lds_bytes;
    LX_TRY(lx::eval_grad_launch(E, s), "evaluate gradients");
    return LAPLEX_OK;
}

}  // namespace

extern "C" {

laplex_status laplex_backward(laplex_plan p, const float* x, const float* g, int64_t batch, int transpose,
                              float* dx, float* da, float* db, float* dphi, float* dpsi, void* stream)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!g) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "g is NULL");
    if (batch < 1) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (transpose != 0 && transpose != 1) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1");
    // x == NULL: the input kept by laplex_plan_create_apply (y = K x, so transpose 0)
    const bool use_kept = x == nullptr;
    if (use_kept && !p->kept_x) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "x is NULL and the plan keeps no input");
    if (use_kept && (transpose != 0 || batch != p->kept_batch))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "the kept input is for transpose = 0 and its own batch");
    const bool kept_by_rank = use_kept && p->kept_by_rank;
    if (use_kept && !kept_by_rank) x = p->kept_x;
    if (p->sym && db) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "symmetric plan: the gradient of b = a is in da");
    if (!p->phased && (dphi || dpsi)) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "unphased plan has no phase gradients");
    const int64_t len_in = transpose ? p->n : p->k;
    const int64_t len_out = transpose ? p->k : p->n;
    if (batch > (int64_t)1 << 40 || (double)batch * (double)(len_in > len_out ? len_in : len_out) > 4.0e18 / 4)
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "batch too large");
    struct Range {
        const void* p;
        size_t bytes;
    };
    const Range outs[5] = {{dx, (size_t)(batch * len_in) * 4}, {da, (size_t)p->n * 4}, {db, (size_t)p->k * 4},
                           {dphi, (size_t)p->n * 4}, {dpsi, (size_t)p->k * 4}};
    const Range ins[2] = {{x, (size_t)(batch * len_in) * 4}, {g, (size_t)(batch * len_out) * 4}};
    for (int i = 0; i < 5; ++i) {
        if (!outs[i].p) continue;
        for (int j = 0; j < 2; ++j)
            if (ins[j].p && ranges_overlap(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes))
                return fail(LAPLEX_ERR_INVALID_ARGUMENT, "an output overlaps x or g");
        for (int j = i + 1; j < 5; ++j)
            if (outs[j].p && ranges_overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return fail(LAPLEX_ERR_INVALID_ARGUMENT, "two outputs overlap");
    }
    if (!dx && !da && !db && !dphi && !dpsi) return LAPLEX_OK;
    DeviceGuard guard(p->device);
    hipStream_t s = (hipStream_t)stream;
    note_stream(p, s);
    const int ch = p->phased ? 2 : 1;
    // row side u, column side w of F = sum <u, K w>
    const float* u = transpose ? x : g;
    const float* w = transpose ? g : x;
    const float anchor_scale = p->temperature > 0.0 ? (float)(-1.0 / p->temperature) : 0.f;

    if (p->sym) {
        const int64_t n = p->n;
        const bool replay = kept_by_rank || n >= replay_min();
        if (!replay) LX_TRY(ensure_perm(p, 0, s), "permutation");
        const int64_t ld = pad64(n);
        const int64_t tiles = (n + lx::kScanTile - 1) / lx::kScanTile;
        const int64_t groups = (tiles + lx::kCarryGroup - 1) / lx::kCarryGroup;
        const int64_t rows = 4 * (int64_t)ch * batch;
        const int64_t nout = (dx ? batch : 0) + (da ? 1 : 0) + (dphi ? 1 : 0) + (dpsi ? 1 : 0);
        const int64_t tmp_rows = replay ? (2 * batch > nout ? 2 * batch : nout) : batch;
        const size_t need = align256((size_t)rows * tiles * 4 * 8) + align256((size_t)rows * groups * 4 * 8) +
                            align256((size_t)rows * tiles * 2 * 8) + 2 * align256((size_t)tmp_rows * ld * 4);
        LX_TRY(ensure_ws(p, need, s), "workspace");
        Carve cv(p->ws);
        lx::GradSymArgs A;
        A.channels = ch;
        A.n = n;
        A.tiles = tiles;
        A.batch = batch;
        A.ld = ld;
        A.out_ld = ld;
        A.inv_t = p->inv_t;
        A.anchor_scale = anchor_scale;
        A.dx_half = transpose ? 0 : 1;
        A.s = p->sa;
        A.perm = p->pa;
        if (p->phased) {
            A.cphi = p->cphi;
            A.sphi = p->sphi;
            A.cpsi = p->cpsi;
            A.spsi = p->spsi;
        }
        A.agg = cv.take<double>((size_t)rows * tiles * 4);
        A.gagg = cv.take<double>((size_t)rows * groups * 4);
        A.carry = cv.take<double>((size_t)rows * tiles * 2);
        float* t1 = cv.take<float>((size_t)tmp_rows * ld);
        float* t2 = cv.take<float>((size_t)tmp_rows * ld);
        if (!replay) {
            A.random = true;
            A.u = u;
            A.w = w;
            A.us = t1;
            A.ws = t2;
            A.dx = dx;
            A.da = da;
            A.dphi = dphi;
            A.dpsi = dpsi;
            LX_TRY(lx::grad_sym_launch(A, s), "symmetric gradient");
            return LAPLEX_OK;
        }
        // u, w -> sorted order (rows [0, B) and [B, 2B)), gradient by rank into
        // t1, then the wanted rows back to original order.
        const lx::SortRecords& R = p->ra;
        A.random = false;
        if (kept_by_rank) {
            // w = x is already by rank: only u travels
            LX_TRY(lx::replay_launch(R, 0, true, u, n, t1, ld, batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 1, true, t1, ld, t2, ld, batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 2, true, t2, ld, t1, ld, batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 3, true, t1, ld, t2, ld, batch, s), "replay");
            A.us = t2;
            A.ws = p->kept_x;
        } else {
            LX_TRY(lx::replay_launch(R, 0, true, u, n, t1, ld, batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 0, true, w, n, t1 + batch * ld, ld, batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 1, true, t1, ld, t2, ld, 2 * batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 2, true, t2, ld, t1, ld, 2 * batch, s), "replay");
            LX_TRY(lx::replay_launch(R, 3, true, t1, ld, t2, ld, 2 * batch, s), "replay");
            A.us = t2;
            A.ws = t2 + batch * ld;
        }
        int64_t row = 0;
        float* user[4] = {dx, da, dphi, dpsi};
        int64_t first[4], count[4];
        for (int o = 0; o < 4; ++o) {
            count[o] = user[o] ? (o == 0 ? batch : 1) : 0;
            first[o] = row;
            row += count[o];
        }
        A.dx = dx ? t1 + first[0] * ld : nullptr;
        A.da = da ? t1 + first[1] * ld : nullptr;
        A.dphi = dphi ? t1 + first[2] * ld : nullptr;
        A.dpsi = dpsi ? t1 + first[3] * ld : nullptr;
        LX_TRY(lx::grad_sym_launch(A, s), "symmetric gradient");
        LX_TRY(lx::replay_launch(R, 3, false, t1, ld, t2, ld, nout, s), "replay");
        LX_TRY(lx::replay_launch(R, 2, false, t2, ld, t1, ld, nout, s), "replay");
        LX_TRY(lx::replay_launch(R, 1, false, t1, ld, t2, ld, nout, s), "replay");
        for (int o = 0; o < 4; ++o)
            if (count[o])
                LX_TRY(lx::replay_launch(R, 0, false, t2 + first[o] * ld, ld, user[o], n, count[o], s), "replay");
        return LAPLEX_OK;
    }

    // General plan: outputs on a from the tables of b, outputs on b from those of a.
    LX_TRY(ensure_perm(p, 0, s), "permutation of a");
    LX_TRY(ensure_perm(p, 1, s), "permutation of b");
    GradSide on_a{p->n, p->k, p->sb, p->pb, p->cpsi, p->spsi, p->a0, p->cphi0, p->sphi0,
                  p->sa, p->pa, p->b0, p->cpsi0, p->spsi0};
    GradSide on_b{p->k, p->n, p->sa, p->pa, p->cphi, p->sphi, p->b0, p->cpsi0, p->spsi0,
                  p->sb, p->pb, p->a0, p->cphi0, p->sphi0};
    laplex_status st = grad_general_side(p, on_a, w, u, batch, transpose ? dx : nullptr, da, dphi, s);
    if (st != LAPLEX_OK) return st;
    return grad_general_side(p, on_b, u, w, batch, transpose ? nullptr : dx, db, dpsi, s);
}

laplex_status laplex_gram(laplex_plan p, const float* D, float* M, void* stream)
{
    if (!p) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!D || !M) return fail(LAPLEX_ERR_INVALID_ARGUMENT, "D or M is NULL");
    if ((double)p->n * (double)p->n > (double)((int64_t)1 << 40))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "n * n too large for a dense Gram matrix");
    if (ranges_overlap(D, (size_t)p->k * 4, M, (size_t)(p->n * p->n) * 4))
        return fail(LAPLEX_ERR_INVALID_ARGUMENT, "D and M overlap");
    DeviceGuard g(p->device);
    hipStream_t s = (hipStream_t)stream;
    note_stream(p, s);
    LX_TRY(ensure_perm(p, 0, s), "permutation of a");
    LX_TRY(ensure_perm(p, 1, s), "permutation of b");
    if (!p->gbound) {
        void* gb = nullptr;
        LX_TRY(plan_alloc(p, &gb, (size_t)(p->n + 2) * 4, s), "alloc gram bounds");
        LX_TRY(lx::gram_bounds_launch(p->sa, p->n, p->sb, p->k, (uint32_t*)gb, s), "gram bounds");
        p->gbound = (uint32_t*)gb;
    }
    if (!p->grank) {
        void* gr = nullptr;
        LX_TRY(plan_alloc(p, &gr, (size_t)p->n * 4, s), "alloc gram ranks");
        LX_TRY(lx::gram_ranks_launch(p->pa, p->n, (uint32_t*)gr, s), "gram ranks");
        p->grank = (uint32_t*)gr;
    }
    LX_TRY(ensure_ws(p, lx::gram_scratch_bytes(p->n, p->k, p->phased ? 3 : 1), s), "workspace");
    lx::GramArgs G;
    G.n = p->n;
    G.k = p->k;
    G.inv_t = p->inv_t;
    G.sa = p->sa;
    G.pa = p->pa;
    G.sb = p->sb;
    G.pb = p->pb;
    G.D = D;
    G.bound = p->gbound;
    G.rank_a = p->grank;
    if (p->phased) {
        G.cphi_r = p->cphi;
        G.sphi_r = p->sphi;
        G.cpsi_r = p->cpsi;
        G.spsi_r = p->spsi;
    }
    if (!p->gslice_off) {
        void *off = nullptr, *src = nullptr, *bv = nullptr, *cv = nullptr, *sv = nullptr;
        LX_TRY(plan_alloc(p, &off, ((size_t)lx::kGramSlices * (p->n + 1) + 1) * 4, s), "alloc gram slices");
        LX_TRY(plan_alloc(p, &src, (size_t)p->k * 4, s), "alloc gram slices");
        LX_TRY(plan_alloc(p, &bv, (size_t)p->k * 4, s), "alloc gram slices");
        if (p->phased) {
            LX_TRY(plan_alloc(p, &cv, (size_t)p->k * 4, s), "alloc gram slices");
            LX_TRY(plan_alloc(p, &sv, (size_t)p->k * 4, s), "alloc gram slices");
        }
        LX_TRY(lx::gram_slices_launch(G, (uint32_t*)off, (uint32_t*)src, (float*)bv, (float*)cv, (float*)sv, s),
               "gram slices");
        p->gslice_off = (uint32_t*)off;
        p->gslice_src = (uint32_t*)src;
        p->gslice_b = (float*)bv;
        p->gslice_c = (float*)cv;
        p->gslice_s = (float*)sv;
    }
    G.slice_off = p->gslice_off;
    G.slice_src = p->gslice_src;
    G.slice_b = p->gslice_b;
    G.slice_c = p->gslice_c;
    G.slice_s = p->gslice_s;
    G.stats = (double*)p->ws;
    G.M = M;
    LX_TRY(lx::gram_launch(G, s), "gram");
    return LAPLEX_OK;
}

laplex_status laplex_profile_enable(int on)
{
    g_prof_on = on != 0;
    return LAPLEX_OK;
}

laplex_status laplex_profile_only(const char* label)
{
    g_prof_only = label ? label : "";
    return LAPLEX_OK;
}

laplex_status laplex_profile_reset(void)
{
    laplex_profile_collect();
    g_prof.clear();
    return LAPLEX_OK;
}

laplex_status laplex_profile_collect(void)
{
    laplex_status st = LAPLEX_OK;
    for (const Pending& q : g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(q.b) == hipSuccess && hipEventElapsedTime(&ms, q.a, q.b) == hipSuccess) {
            bool found = false;
            for (ProfEntry& e : g_prof)
                if (std::strcmp(e.name, q.name) == 0) {
                    e.launches += 1;
                    e.total_ms += ms;
                    found = true;
                    break;
                }
            if (!found) g_prof.push_back(ProfEntry{q.name, 1, (double)ms});
        } else {
            (void)hipGetLastError();
            st = fail(LAPLEX_ERR_DEVICE, "profiling event failed");
        }
        g_event_pool.push_back(q.a);
        g_event_pool.push_back(q.b);
    }
    g_pending.clear();
    return st;
}

laplex_status laplex_profile_entry(int i, const char** name, int64_t* launches, double* total_ms)
{
    if (i < 0 || i >= (int)g_prof.size()) return LAPLEX_ERR_INVALID_ARGUMENT;
    if (name) *name = g_prof[i].name;
    if (launches) *launches = g_prof[i].launches;
    if (total_ms) *total_ms = g_prof[i].total_ms;
    return LAPLEX_OK;
}

}  // extern "C"
