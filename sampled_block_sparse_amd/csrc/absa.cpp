// Host side of the C interface declared in include/absa.h: argument
// validation (before any HIP call), the plan object, allocation and the
// launch sequence of the plan and attention kernels.
#include "absa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "absa_internal.h"

using namespace absa;

struct absa_plan_s {
    int64_t B = 0, H = 0, N = 0, d = 0, M = 0, QB = 0, rows = 0, nnz = 0;
    int32_t n_clusters = 0;
    int device = 0;              // device whose memory pool holds the buffers
    int64_t* rowptr = nullptr;   // device [rows+1]
    int32_t* idx = nullptr;      // device [nnz]
    float* logw = nullptr;       // device [nnz]
    double* p = nullptr;         // device [nnz]
    // retained intermediates (keep_intermediates), device
    float* kbar = nullptr;
    float* cent = nullptr;
    float* w = nullptr;
    float* scores = nullptr;
    // The streams of the plan's attention calls, each with an event recorded
    // after its latest call: destroy releases the buffers in stream order
    // after all of them. The events are created with the plan, so recording
    // one allocates nothing; a fifth stream takes the oldest slot once that
    // slot's work has finished.
    static constexpr int kUseSlots = 4;
    std::mutex use_mutex;
    hipStream_t use_stream[kUseSlots] = {};
    hipEvent_t use_event[kUseSlots] = {};
    int n_use = 0, next_evict = 0;
};

namespace {

thread_local std::string g_last_error;

absa_status fail(absa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

absa_status hip_fail(hipError_t e, const char* what) {
    const absa_status st = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
                               ? ABSA_ERR_OUT_OF_MEMORY
                               : ABSA_ERR_DEVICE;
    return fail(st, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

#define ABSA_HIP(call, what)                               \
    do {                                                   \
        hipError_t e_ = (call);                            \
        if (e_ != hipSuccess) return hip_fail(e_, (what)); \
    } while (0)
#define ABSA_HIP_RET(call, what) ABSA_HIP(call, what)

#define ABSA_TRY(expr)                       \
    do {                                     \
        absa_status s_ = (expr);             \
        if (s_ != ABSA_OK) return s_;        \
    } while (0)

// Allocation failure can be forced for tests: ABSA_FAULT_INJECT=alloc.
bool inject_alloc_failure() {
    const char* v = std::getenv("ABSA_FAULT_INJECT");
    return v && std::strcmp(v, "alloc") == 0;
}

// Stream-ordered device memory. Plan buffers and plan-building temporaries
// come from one library-owned pool per device that keeps freed memory for
// reuse (unlimited release threshold): once the pool has grown to the largest
// plan, building and destroying plans costs no driver allocation, unmapping
// or device-wide synchronisation. absa_release_cached_memory() trims it.
std::mutex g_pool_mutex;
std::vector<hipMemPool_t> g_pools;

hipError_t device_pool(int dev, bool create, hipMemPool_t* out) {
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    *out = nullptr;
    if (dev < 0) return hipErrorInvalidDevice;
    if (static_cast<size_t>(dev) >= g_pools.size()) g_pools.resize(dev + 1, nullptr);
    if (!g_pools[dev] && create) {
        hipMemPoolProps props;
        std::memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep_all = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep_all);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        g_pools[dev] = pool;
    }
    *out = g_pools[dev];
    return hipSuccess;
}

// Allocate from the current device's pool, ordered on stream s. On an
// out-of-memory error the pool's cached memory is returned to the system
// once and the allocation retried.
hipError_t pool_alloc(void** p, size_t bytes, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipMemPool_t pool = nullptr;
    e = device_pool(dev, true, &pool);
    if (e != hipSuccess) return e;
    e = hipMallocFromPoolAsync(p, bytes, pool, s);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) {
        (void)hipGetLastError();
        if (hipStreamSynchronize(s) == hipSuccess && hipMemPoolTrimTo(pool, 0) == hipSuccess)
            e = hipMallocFromPoolAsync(p, bytes, pool, s);
    }
    return e;
}

// Device buffers owned until release() hands them over; whatever is left is
// returned to the pool in the order of stream s.
struct DeviceArena {
    hipStream_t stream;
    std::vector<void*> ptrs;
    explicit DeviceArena(hipStream_t s) : stream(s) {}
    ~DeviceArena() {
        for (void* p : ptrs)
            if (p) (void)hipFreeAsync(p, stream);
    }
    template <typename T>
    absa_status alloc(T** out, int64_t count, const char* what) {
        *out = nullptr;
        if (count <= 0) return ABSA_OK;
        if (inject_alloc_failure())
            return fail(ABSA_ERR_OUT_OF_MEMORY, "%s: allocation failure injected", what);
        void* p = nullptr;
        hipError_t e = pool_alloc(&p, static_cast<size_t>(count) * sizeof(T), stream);
        if (e != hipSuccess) return hip_fail(e, what);
        ptrs.push_back(p);
        *out = static_cast<T*>(p);
        return ABSA_OK;
    }
    void release(const void* p) {
        for (auto& q : ptrs)
            if (q == p) q = nullptr;
    }
};

// Bump allocator over one device block, for a plan build's temporaries.
// With base == nullptr it only measures (every pointer stays null).
struct Carve {
    char* base = nullptr;
    size_t cap = 0, used = 0;
    template <typename T>
    absa_status alloc(T** out, int64_t count, const char* what) {
        *out = nullptr;
        if (count <= 0) return ABSA_OK;
        if (inject_alloc_failure())
            return fail(ABSA_ERR_OUT_OF_MEMORY, "%s: allocation failure injected", what);
        const size_t bytes = (static_cast<size_t>(count) * sizeof(T) + 255) & ~size_t(255);
        if (base) {
            if (used + bytes > cap) return fail(ABSA_ERR_DEVICE, "%s: workspace overflow", what);
            *out = reinterpret_cast<T*>(base + used);
        }
        used += bytes;
        return ABSA_OK;
    }
};

// Per-device plan-building workspace: one block that successive plan builds
// on a device reuse for their temporaries (it grows to the largest build).
// A build holds it for its whole (synchronous) duration; a build that finds
// it held by another thread allocates a block of its own.
struct Workspace {
    std::mutex busy;
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<std::unique_ptr<Workspace>> g_ws;

Workspace* device_workspace(int dev) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (static_cast<size_t>(dev) >= g_ws.size()) g_ws.resize(dev + 1);
    if (!g_ws[dev]) g_ws[dev].reset(new Workspace());
    return g_ws[dev].get();
}

// A second stream per device for plan-build work that does not depend on the
// caller stream's next kernel: the mean keys run there beside the k-means
// (one streams K from HBM, the other computes in fp64 on Q). Created on first
// use with the default priority and flags that keep it from synchronising
// with the null stream; kept until the process ends. Builds on one device
// share it; each build orders its work with events of its own.
std::mutex g_side_mutex;
std::vector<hipStream_t> g_side;

absa_status device_side_stream(hipStream_t* out) {
    int dev = 0;
    ABSA_HIP_RET(hipGetDevice(&dev), "current device");
    std::lock_guard<std::mutex> lock(g_side_mutex);
    if (static_cast<size_t>(dev) >= g_side.size()) g_side.resize(dev + 1, nullptr);
    if (!g_side[dev]) {
        hipStream_t st = nullptr;
        ABSA_HIP_RET(hipStreamCreateWithFlags(&st, hipStreamNonBlocking), "side stream");
        g_side[dev] = st;
    }
    *out = g_side[dev];
    return ABSA_OK;
}

// Work forked from stream `main` onto the device's side stream and joined
// back: fork() makes the side stream wait for everything queued on main so
// far; join() makes main wait for everything queued on the side stream since.
// If the build fails between the two, the destructor waits for the side
// stream, so nothing it runs outlives the build's buffers.
class SideFork {
  public:
    explicit SideFork(hipStream_t main) : main_(main) {}
    ~SideFork() {
        if (side_ && !joined_) (void)hipStreamSynchronize(side_);
        if (fork_) (void)hipEventDestroy(fork_);
        if (join_) (void)hipEventDestroy(join_);
    }
    absa_status fork(hipStream_t* side) {
        ABSA_TRY(device_side_stream(&side_));
        ABSA_HIP_RET(hipEventCreateWithFlags(&fork_, hipEventDisableTiming), "fork event");
        ABSA_HIP_RET(hipEventCreateWithFlags(&join_, hipEventDisableTiming), "join event");
        ABSA_HIP_RET(hipEventRecord(fork_, main_), "fork record");
        ABSA_HIP_RET(hipStreamWaitEvent(side_, fork_, 0), "fork wait");
        *side = side_;
        return ABSA_OK;
    }
    absa_status join() {
        ABSA_HIP_RET(hipEventRecord(join_, side_), "join record");
        ABSA_HIP_RET(hipStreamWaitEvent(main_, join_, 0), "join wait");
        joined_ = true;
        return ABSA_OK;
    }

  private:
    hipStream_t main_;
    hipStream_t side_ = nullptr;
    hipEvent_t fork_ = nullptr, join_ = nullptr;
    bool joined_ = false;
};

// A build's hold on a workspace block of at least `bytes` bytes.
class WorkspaceLease {
  public:
    explicit WorkspaceLease(hipStream_t s) : s_(s) {}
    // Work queued on the block may still be running when a build fails
    // part-way: wait for the stream before another build can take the block.
    ~WorkspaceLease() {
        if (lock_.owns_lock()) (void)hipStreamSynchronize(s_);
        if (own_) (void)hipFreeAsync(own_, s_);
    }
    absa_status acquire(size_t bytes, char** out) {
        *out = nullptr;
        if (bytes == 0) return ABSA_OK;
        int dev = 0;
        ABSA_HIP_RET(hipGetDevice(&dev), "current device");
        Workspace* ws = device_workspace(dev);
        lock_ = std::unique_lock<std::mutex>(ws->busy, std::try_to_lock);
        if (lock_.owns_lock()) {
            if (ws->bytes < bytes) {
                if (ws->ptr) (void)hipFreeAsync(ws->ptr, s_);
                ws->ptr = nullptr;
                ws->bytes = 0;
                ABSA_HIP_RET(pool_alloc(&ws->ptr, bytes, s_), "plan workspace");
                ws->bytes = bytes;
            }
            *out = static_cast<char*>(ws->ptr);
        } else {
            ABSA_HIP_RET(pool_alloc(&own_, bytes, s_), "plan workspace");
            *out = static_cast<char*>(own_);
        }
        return ABSA_OK;
    }

  private:
    hipStream_t s_;
    void* own_ = nullptr;
    std::unique_lock<std::mutex> lock_;
};

// Temporaries of a plan build (null when not needed).
struct PlanTemps {
    float* kbar = nullptr;
    int8_t* kq = nullptr;
    int8_t* kqt = nullptr;       // tile-major digits (fused plans only)
    int* kx = nullptr;
    float* cent = nullptr;
    float* w = nullptr;
    float* scores = nullptr;
    float2* part = nullptr;
    float* sbias = nullptr;      // score bias per (query block, centroid)
    uint64_t* capmask = nullptr;
    uint64_t* keepmask = nullptr;
    SipRow* rowinfo = nullptr;
    int64_t* counts = nullptr;
    PlanStatus* status = nullptr;
};

absa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d) {
    if (B < 1 || H < 1) return fail(ABSA_ERR_INVALID_ARG, "B and H must be >= 1 (got %lld, %lld)",
                                    (long long)B, (long long)H);
    if (N < 4 || N > (int64_t(1) << 21))
        return fail(ABSA_ERR_UNSUPPORTED, "N must lie in [4, 2^21] (got %lld)", (long long)N);
    if (N % kKvBlock != 0)
        return fail(ABSA_ERR_UNSUPPORTED, "N must be a multiple of the KV block size 4 (got %lld)",
                    (long long)N);
    if (d != 64 && d != 128)
        return fail(ABSA_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %lld)", (long long)d);
    const int64_t QB = (N + kQueryBlock - 1) / kQueryBlock;
    if (B > (int64_t(1) << 31) / H || B * H > (int64_t(1) << 31) / QB)
        return fail(ABSA_ERR_UNSUPPORTED, "B*H*ceil(N/128) must be below 2^31");
    return ABSA_OK;
}

absa_status check_dtype(absa_dtype dt) {
    if (dt != ABSA_BF16 && dt != ABSA_F32)
        return fail(ABSA_ERR_UNSUPPORTED, "dtype must be ABSA_BF16 or ABSA_F32 (got %d)", (int)dt);
    return ABSA_OK;
}

absa_status check_sampling(int32_t sampling) {
    static_assert(ABSA_SAMPLING_POISSON == kSamplingPoisson &&
                  ABSA_SAMPLING_SYSTEMATIC == kSamplingSystematic, "sampling codes");
    if (sampling != ABSA_SAMPLING_POISSON && sampling != ABSA_SAMPLING_SYSTEMATIC)
        return fail(ABSA_ERR_INVALID_ARG,
                    "sampling must be ABSA_SAMPLING_POISSON or ABSA_SAMPLING_SYSTEMATIC (got %d)",
                    (int)sampling);
    return ABSA_OK;
}

void fill_dims(absa_plan_s* p, int64_t B, int64_t H, int64_t N, int64_t d) {
    p->B = B; p->H = H; p->N = N; p->d = d;
    p->M = N / kKvBlock;
    p->QB = (N + kQueryBlock - 1) / kQueryBlock;
    p->rows = B * H * p->QB;
}

// Temporaries of the SIP stage (masks, per-row outcome, counts, status).
template <typename A>
absa_status sip_temps(A& a, const absa_plan_s* P, PlanTemps& t) {
    const int64_t rows = P->rows;
    const int64_t words = (P->M + 63) / 64;
    ABSA_TRY(a.alloc(&t.capmask, rows * words, "cap mask"));
    ABSA_TRY(a.alloc(&t.keepmask, rows * words, "keep mask"));
    ABSA_TRY(a.alloc(&t.rowinfo, rows, "row info"));
    ABSA_TRY(a.alloc(&t.counts, rows, "row counts"));
    ABSA_TRY(a.alloc(&t.status, 1, "plan status"));
    return ABSA_OK;
}

// SIP on device scores, shared by plan_create and plan_from_scores. Fills
// rowptr/idx/logw/p of the plan (allocated in arena, owned by the plan)
// using the temporaries in t. One device-to-host read of the total count and
// the score check flag, then the fill kernel. Returns with the fill queued;
// the caller synchronises. With fused set (plan_create only, scores =
// t.scores), the scores come from the fused pass-2 + SIP kernel on t's
// centroids, weights, key digits and pass-1 statistics, which writes into
// t.scores only what the fill kernel reads.
absa_status run_sip(absa_plan_s* P, const float* scores, int64_t budget, uint64_t seed,
                    int sampling, hipStream_t s, DeviceArena& arena, const PlanTemps& t,
                    bool fused = false) {
    const int64_t rows = P->rows;
    ABSA_TRY(arena.alloc(&P->rowptr, rows + 1, "row pointers"));
    ABSA_HIP(hipMemsetAsync(t.status, 0, sizeof(PlanStatus), s), "clear plan status");
    if (fused)
        ABSA_HIP(launch_scores_sip(t.cent, t.w, t.kqt, t.kx, t.sbias, P->B, P->H, P->QB, P->M,
                                   static_cast<int>(P->d), P->n_clusters, budget, seed, sampling,
                                   t.scores, t.capmask, t.keepmask, t.rowinfo, t.counts, t.status,
                                   s),
                 "fused score and SIP kernel");
    else
        ABSA_HIP(launch_sip_count(scores, P->B, P->H, P->QB, P->M, budget, seed, sampling,
                                  t.capmask, t.keepmask, t.rowinfo, t.counts, t.status, s),
                 "SIP count kernel");
    ABSA_HIP(launch_scan(t.counts, rows, P->rowptr, t.status, s), "row scan kernel");
    PlanStatus host{};
    ABSA_HIP(hipMemcpyAsync(&host, t.status, sizeof(PlanStatus), hipMemcpyDeviceToHost, s),
             "read plan size");
    ABSA_HIP(hipStreamSynchronize(s), "plan synchronisation");
    if (host.bad_scores)
        return fail(ABSA_ERR_INVALID_ARG,
                    "scores must lie in [0, 1] and every row must sum to less than 2");
    P->nnz = host.nnz;
    ABSA_TRY(arena.alloc(&P->idx, P->nnz, "plan indices"));
    ABSA_TRY(arena.alloc(&P->logw, P->nnz, "plan log-weights"));
    ABSA_TRY(arena.alloc(&P->p, P->nnz, "plan probabilities"));
    if (P->nnz > 0) {
        ABSA_HIP(launch_sip_fill(scores, rows, P->M, t.capmask, t.keepmask, t.rowinfo, P->rowptr,
                                 sampling, P->idx, P->logw, P->p, s),
                 "SIP fill kernel");
    }
    return ABSA_OK;
}

void keep(DeviceArena& arena, absa_plan_s* P) {
    arena.release(P->rowptr);
    arena.release(P->idx);
    arena.release(P->logw);
    arena.release(P->p);
    arena.release(P->kbar);
    arena.release(P->cent);
    arena.release(P->w);
    arena.release(P->scores);
}

// Returns the plan's buffers to its device's pool in stream order: the
// library's side stream waits for the event of every stream that ran an
// attention call on the plan, then frees them. Nothing waits on the host.
// (Without the side stream, which only fails if a stream cannot be created,
// it waits for those events on the host and frees on the null stream.)
void free_plan(absa_plan_s* P) {
    if (!P) return;
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    if (!have_cur || cur != P->device) (void)hipSetDevice(P->device);
    hipStream_t side = nullptr;
    if (device_side_stream(&side) != ABSA_OK) side = nullptr;
    for (int i = 0; i < P->n_use; ++i) {
        if (side) (void)hipStreamWaitEvent(side, P->use_event[i], 0);
        else (void)hipEventSynchronize(P->use_event[i]);
    }
    void* bufs[] = {P->rowptr, P->idx, P->logw, P->p, P->kbar, P->cent, P->w, P->scores};
    for (void* b : bufs)
        if (b) (void)hipFreeAsync(b, side);
    // an event destroyed while a wait on it is queued is released once the
    // wait has passed
    for (hipEvent_t e : P->use_event)
        if (e) (void)hipEventDestroy(e);
    if (have_cur && cur != P->device) (void)hipSetDevice(cur);
    delete P;
}

// Create the plan's use events (see absa_plan_s).
absa_status create_use_events(absa_plan_s* P) {
    for (hipEvent_t& e : P->use_event)
        ABSA_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming), "plan use event");
    return ABSA_OK;
}

// Record that stream s ran work on the plan. Under stream capture nothing is
// recorded: the captured graph's launches are ordered by the caller, who
// must keep the plan alive while they may run.
absa_status note_use(absa_plan_s* P, hipStream_t s) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    ABSA_HIP(hipStreamIsCapturing(s, &cap), "stream capture status");
    if (cap != hipStreamCaptureStatusNone) return ABSA_OK;
    std::lock_guard<std::mutex> lock(P->use_mutex);
    int slot = -1;
    for (int i = 0; i < P->n_use; ++i)
        if (P->use_stream[i] == s) slot = i;
    if (slot < 0) {
        if (P->n_use < absa_plan_s::kUseSlots) {
            slot = P->n_use++;
        } else {
            slot = P->next_evict;
            P->next_evict = (slot + 1) % absa_plan_s::kUseSlots;
            ABSA_HIP(hipEventSynchronize(P->use_event[slot]), "wait for an earlier use");
        }
        P->use_stream[slot] = s;
    }
    ABSA_HIP(hipEventRecord(P->use_event[slot], s), "record plan use");
    return ABSA_OK;
}

absa_status set_plan_device(absa_plan_s* P) {
    ABSA_HIP(hipGetDevice(&P->device), "current device");
    return create_use_events(P);
}

// Release a plan whose build failed: its buffers went back with the build's
// arena, only the events are left.
void discard_plan(absa_plan_s* P) {
    for (hipEvent_t e : P->use_event)
        if (e) (void)hipEventDestroy(e);
    delete P;
}

}  // namespace

extern "C" {

absa_status absa_plan_params_init(absa_plan_params* out) {
    if (!out) return fail(ABSA_ERR_INVALID_ARG, "params is NULL");
    out->query_block = kQueryBlock;
    out->kv_block = kKvBlock;
    out->n_clusters = 8;
    out->kmeans_iters = 4;
    out->budget_blocks = 1;
    out->seed = 0;
    out->keep_intermediates = 0;
    out->sampling = ABSA_SAMPLING_POISSON;
    out->fused = 0;
    return ABSA_OK;
}

absa_status absa_plan_create(const void* q, const void* k, absa_dtype dtype, int64_t B,
                             int64_t H, int64_t N, int64_t d, const absa_plan_params* params,
                             void* hip_stream, absa_plan* out) {
    if (!out) return fail(ABSA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!q || !k || !params) return fail(ABSA_ERR_INVALID_ARG, "q, k and params must be non-NULL");
    ABSA_TRY(check_dtype(dtype));
    ABSA_TRY(check_shape(B, H, N, d));
    if (params->query_block != kQueryBlock)
        return fail(ABSA_ERR_UNSUPPORTED, "query_block must be 128 (got %d)", params->query_block);
    if (params->kv_block != kKvBlock)
        return fail(ABSA_ERR_UNSUPPORTED, "kv_block must be 4 (got %d)", params->kv_block);
    if (params->n_clusters < 1 || params->n_clusters > kMaxClusters)
        return fail(ABSA_ERR_UNSUPPORTED, "n_clusters must lie in [1, %d] (got %d)", kMaxClusters,
                    params->n_clusters);
    if (params->kmeans_iters < 1 || params->kmeans_iters > 64)
        return fail(ABSA_ERR_INVALID_ARG, "kmeans_iters must lie in [1, 64] (got %d)",
                    params->kmeans_iters);
    ABSA_TRY(check_sampling(params->sampling));
    const int64_t M = N / kKvBlock;
    if (params->budget_blocks < 1 || params->budget_blocks > M)
        return fail(ABSA_ERR_INVALID_ARG, "budget_blocks must lie in [1, M=%lld] (got %lld)",
                    (long long)M, (long long)params->budget_blocks);
    if (B * H > 65535)
        return fail(ABSA_ERR_UNSUPPORTED,
                    "absa_plan_create needs B*H <= 65535 (the score kernels' second grid "
                    "dimension; got %lld)", (long long)(B * H));
    const bool fused = params->fused != 0;
    if (fused && (params->n_clusters > 8 || M > kFusedMaxBlocks || params->keep_intermediates))
        return fail(ABSA_ERR_UNSUPPORTED,
                    "fused needs n_clusters <= 8 (got %d), M <= %lld (got %lld) and "
                    "keep_intermediates = 0",
                    params->n_clusters, (long long)kFusedMaxBlocks, (long long)M);

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    absa_plan_s* P = new (std::nothrow) absa_plan_s();
    if (!P) return fail(ABSA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
    fill_dims(P, B, H, N, d);
    P->n_clusters = params->n_clusters;
    const int C = params->n_clusters;
    const Dtype dt = (dtype == ABSA_BF16) ? kBF16 : kF32;

    const bool keep_inter = params->keep_intermediates != 0;
    absa_status st = [&]() -> absa_status {
        ABSA_TRY(set_plan_device(P));
        // Temporaries come from the device's reusable workspace; the plan's
        // own buffers (and the intermediates it keeps) from the pool.
        auto temps = [&](auto& a, PlanTemps& t) -> absa_status {
            if (!keep_inter) {
                // the fp32 means are only exported; the scores use their digits
                t.kbar = nullptr;
                ABSA_TRY(a.alloc(&t.cent, P->rows * C * d, "centroids"));
                ABSA_TRY(a.alloc(&t.w, P->rows * C, "cluster weights"));
                ABSA_TRY(a.alloc(&t.scores, P->rows * M, "scores"));
            }
            ABSA_TRY(a.alloc(&t.kq, B * H * M * 3 * d, "mean-key digits"));
            if (fused)
                ABSA_TRY(a.alloc(&t.kqt, kqt_bytes(B * H, M, static_cast<int>(d)),
                                 "tile-major mean-key digits"));
            ABSA_TRY(a.alloc(&t.kx, B * H * M, "mean-key exponents"));
            ABSA_TRY(a.alloc(&t.part, score_partials(B * H, P->QB, M, C), "score chunk statistics"));
            ABSA_TRY(a.alloc(&t.sbias, P->rows * C, "score biases"));
            return sip_temps(a, P, t);
        };
        PlanTemps t;
        Carve measure;
        ABSA_TRY(temps(measure, t));
        WorkspaceLease lease(s);
        Carve carve;
        ABSA_TRY(lease.acquire(measure.used, &carve.base));
        carve.cap = measure.used;
        ABSA_TRY(temps(carve, t));
        DeviceArena arena(s);
        if (keep_inter) {
            ABSA_TRY(arena.alloc(&P->kbar, B * H * M * d, "mean keys"));
            ABSA_TRY(arena.alloc(&P->cent, P->rows * C * d, "centroids"));
            ABSA_TRY(arena.alloc(&P->w, P->rows * C, "cluster weights"));
            ABSA_TRY(arena.alloc(&P->scores, P->rows * M, "scores"));
            t.kbar = P->kbar; t.cent = P->cent; t.w = P->w; t.scores = P->scores;
        }
        // the mean keys (side stream) beside the k-means (caller stream)
        SideFork fork(s);
        hipStream_t side = nullptr;
        ABSA_TRY(fork.fork(&side));
        ABSA_HIP(launch_mean_keys(k, dt, B * H, N, static_cast<int>(d), t.kbar, t.kq, t.kqt, t.kx,
                                  side),
                 "mean-key kernel");
        ABSA_HIP(launch_kmeans(q, dt, B * H, N, static_cast<int>(d), C, params->kmeans_iters,
                               t.cent, t.w, s),
                 "k-means kernel");
        ABSA_TRY(fork.join());
        ABSA_HIP(launch_scores(t.cent, t.w, t.kq, t.kx, B * H, P->QB, M, static_cast<int>(d), C,
                               t.part, t.sbias, t.scores, !fused, s),
                 "score kernel");
        ABSA_TRY(run_sip(P, t.scores, params->budget_blocks, params->seed, params->sampling, s,
                         arena, t, fused));
        keep(arena, P);
        // the workspace is released (and may be reused) only once the build
        // has finished on the device
        ABSA_HIP(hipStreamSynchronize(s), "plan completion");
        return ABSA_OK;
    }();
    if (st != ABSA_OK) {
        P->rowptr = nullptr; P->idx = nullptr; P->logw = nullptr; P->p = nullptr;
        P->kbar = P->cent = P->w = P->scores = nullptr;
        discard_plan(P);
        return st;
    }
    *out = P;
    return ABSA_OK;
}

absa_status absa_plan_from_scores(const float* scores_dev, int64_t B, int64_t H, int64_t N,
                                  int64_t d, int64_t budget_blocks, uint64_t seed,
                                  int32_t sampling, void* hip_stream, absa_plan* out) {
    if (!out) return fail(ABSA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!scores_dev) return fail(ABSA_ERR_INVALID_ARG, "scores is NULL");
    ABSA_TRY(check_shape(B, H, N, d));
    ABSA_TRY(check_sampling(sampling));
    const int64_t M = N / kKvBlock;
    if (budget_blocks < 1 || budget_blocks > M)
        return fail(ABSA_ERR_INVALID_ARG, "budget_blocks must lie in [1, M=%lld] (got %lld)",
                    (long long)M, (long long)budget_blocks);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    absa_plan_s* P = new (std::nothrow) absa_plan_s();
    if (!P) return fail(ABSA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
    fill_dims(P, B, H, N, d);
    absa_status st = [&]() -> absa_status {
        ABSA_TRY(set_plan_device(P));
        PlanTemps t;
        Carve measure;
        ABSA_TRY(sip_temps(measure, P, t));
        WorkspaceLease lease(s);
        Carve carve;
        ABSA_TRY(lease.acquire(measure.used, &carve.base));
        carve.cap = measure.used;
        ABSA_TRY(sip_temps(carve, P, t));
        DeviceArena arena(s);
        ABSA_TRY(run_sip(P, scores_dev, budget_blocks, seed, sampling, s, arena, t));
        keep(arena, P);
        ABSA_HIP(hipStreamSynchronize(s), "plan completion");
        return ABSA_OK;
    }();
    if (st != ABSA_OK) {
        discard_plan(P);
        return st;
    }
    *out = P;
    return ABSA_OK;
}

absa_status absa_plan_import(const int64_t* rowptr, const int32_t* idx, const float* logw,
                             const double* p, int64_t B, int64_t H, int64_t N, int64_t d,
                             void* hip_stream, absa_plan* out) {
    if (!out) return fail(ABSA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!rowptr) return fail(ABSA_ERR_INVALID_ARG, "rowptr is NULL");
    ABSA_TRY(check_shape(B, H, N, d));
    struct { int64_t rows, M; } tmp;
    tmp.M = N / kKvBlock;
    tmp.rows = B * H * ((N + kQueryBlock - 1) / kQueryBlock);
    if (rowptr[0] != 0) return fail(ABSA_ERR_INVALID_ARG, "rowptr[0] must be 0");
    for (int64_t i = 0; i < tmp.rows; ++i) {
        const int64_t lo = rowptr[i], hi = rowptr[i + 1];
        if (hi < lo) return fail(ABSA_ERR_INVALID_ARG, "rowptr decreases at row %lld", (long long)i);
        if (hi - lo > tmp.M)
            return fail(ABSA_ERR_INVALID_ARG, "row %lld holds more than M blocks", (long long)i);
    }
    const int64_t nnz = rowptr[tmp.rows];
    if (nnz > 0 && (!idx || !logw))
        return fail(ABSA_ERR_INVALID_ARG, "idx and logw must be non-NULL when the plan is not empty");
    for (int64_t i = 0; i < tmp.rows; ++i) {
        for (int64_t e = rowptr[i]; e < rowptr[i + 1]; ++e) {
            if (idx[e] < 0 || idx[e] >= tmp.M)
                return fail(ABSA_ERR_INVALID_ARG, "idx[%lld] = %d is outside [0, M)", (long long)e,
                            idx[e]);
            if (e > rowptr[i] && idx[e] <= idx[e - 1])
                return fail(ABSA_ERR_INVALID_ARG, "indices of row %lld are not strictly ascending",
                            (long long)i);
            if (!std::isfinite(logw[e]))
                return fail(ABSA_ERR_INVALID_ARG, "logw[%lld] is not finite", (long long)e);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    absa_plan_s* P = new (std::nothrow) absa_plan_s();
    if (!P) return fail(ABSA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
    fill_dims(P, B, H, N, d);
    P->nnz = nnz;
    absa_status st = [&]() -> absa_status {
        ABSA_TRY(set_plan_device(P));
        DeviceArena arena(s);
        ABSA_TRY(arena.alloc(&P->rowptr, P->rows + 1, "row pointers"));
        ABSA_TRY(arena.alloc(&P->idx, nnz, "plan indices"));
        ABSA_TRY(arena.alloc(&P->logw, nnz, "plan log-weights"));
        ABSA_TRY(arena.alloc(&P->p, nnz, "plan probabilities"));
        std::vector<double> pv;
        const double* psrc = p;
        if (!psrc && nnz > 0) {
            pv.resize(static_cast<size_t>(nnz));
            for (int64_t e = 0; e < nnz; ++e) pv[e] = std::exp(-static_cast<double>(logw[e]));
            psrc = pv.data();
        }
        ABSA_HIP(hipMemcpyAsync(P->rowptr, rowptr, (P->rows + 1) * sizeof(int64_t),
                                hipMemcpyHostToDevice, s), "copy row pointers");
        if (nnz > 0) {
            ABSA_HIP(hipMemcpyAsync(P->idx, idx, nnz * sizeof(int32_t), hipMemcpyHostToDevice, s),
                     "copy indices");
            ABSA_HIP(hipMemcpyAsync(P->logw, logw, nnz * sizeof(float), hipMemcpyHostToDevice, s),
                     "copy log-weights");
            ABSA_HIP(hipMemcpyAsync(P->p, psrc, nnz * sizeof(double), hipMemcpyHostToDevice, s),
                     "copy probabilities");
        }
        ABSA_HIP(hipStreamSynchronize(s), "plan import");
        keep(arena, P);
        return ABSA_OK;
    }();
    if (st != ABSA_OK) {
        discard_plan(P);
        return st;
    }
    *out = P;
    return ABSA_OK;
}

absa_status absa_plan_info(absa_plan plan, int64_t* shape4, int64_t* rows, int64_t* M,
                           int64_t* nnz) {
    if (!plan) return fail(ABSA_ERR_INVALID_ARG, "plan is NULL");
    if (shape4) { shape4[0] = plan->B; shape4[1] = plan->H; shape4[2] = plan->N; shape4[3] = plan->d; }
    if (rows) *rows = plan->rows;
    if (M) *M = plan->M;
    if (nnz) *nnz = plan->nnz;
    return ABSA_OK;
}

absa_status absa_plan_export(absa_plan plan, int64_t* rowptr, int32_t* idx, float* logw,
                             double* p) {
    if (!plan) return fail(ABSA_ERR_INVALID_ARG, "plan is NULL");
    if (rowptr)
        ABSA_HIP(hipMemcpy(rowptr, plan->rowptr, (plan->rows + 1) * sizeof(int64_t),
                           hipMemcpyDeviceToHost), "export row pointers");
    if (plan->nnz > 0) {
        if (idx)
            ABSA_HIP(hipMemcpy(idx, plan->idx, plan->nnz * sizeof(int32_t), hipMemcpyDeviceToHost),
                     "export indices");
        if (logw)
            ABSA_HIP(hipMemcpy(logw, plan->logw, plan->nnz * sizeof(float), hipMemcpyDeviceToHost),
                     "export log-weights");
        if (p)
            ABSA_HIP(hipMemcpy(p, plan->p, plan->nnz * sizeof(double), hipMemcpyDeviceToHost),
                     "export probabilities");
    }
    return ABSA_OK;
}

absa_status absa_plan_export_intermediate(absa_plan plan, absa_intermediate which, int64_t offset,
                                          int64_t count, float* dst) {
    if (!plan) return fail(ABSA_ERR_INVALID_ARG, "plan is NULL");
    if (!dst && count > 0) return fail(ABSA_ERR_INVALID_ARG, "dst is NULL");
    const float* src = nullptr;
    int64_t total = 0;
    switch (which) {
        case ABSA_INTER_MEAN_KEYS: src = plan->kbar; total = plan->B * plan->H * plan->M * plan->d; break;
        case ABSA_INTER_CENTROIDS: src = plan->cent; total = plan->rows * plan->n_clusters * plan->d; break;
        case ABSA_INTER_WEIGHTS: src = plan->w; total = plan->rows * plan->n_clusters; break;
        case ABSA_INTER_SCORES: src = plan->scores; total = plan->rows * plan->M; break;
        default: return fail(ABSA_ERR_INVALID_ARG, "unknown intermediate %d", (int)which);
    }
    if (!src) return fail(ABSA_ERR_INVALID_ARG, "the plan did not keep its intermediates");
    if (offset < 0 || count < 0 || offset > total || count > total - offset)
        return fail(ABSA_ERR_INVALID_ARG, "range [%lld, +%lld) outside [0, %lld)", (long long)offset,
                    (long long)count, (long long)total);
    if (count > 0)
        ABSA_HIP(hipMemcpy(dst, src + offset, count * sizeof(float), hipMemcpyDeviceToHost),
                 "export intermediate");
    return ABSA_OK;
}

static absa_status attention_common(const void* q, const void* k, const void* v, void* o,
                                    absa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d) {
    if (!q || !k || !v || !o) return fail(ABSA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    ABSA_TRY(check_dtype(dtype));
    return check_shape(B, H, N, d);
}

// Launch the attention kernel on bf16 inputs. fp32 inputs are first rounded
// to bf16 (round to nearest even) into temporaries from the library's pool,
// ordered on the same stream; the output keeps the caller's dtype.
static absa_status run_attention(const void* q, const void* k, const void* v, void* o,
                                 absa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                                 const absa_plan_s* plan, hipStream_t s) {
    const int64_t n = B * H * N * d;
    const uint16_t *q16 = static_cast<const uint16_t*>(q), *k16 = static_cast<const uint16_t*>(k),
                   *v16 = static_cast<const uint16_t*>(v);
    DeviceArena arena(s);
    if (dtype == ABSA_F32) {
        uint16_t* tmp[3] = {nullptr, nullptr, nullptr};
        const void* src[3] = {q, k, v};
        for (int i = 0; i < 3; ++i) {
            ABSA_TRY(arena.alloc(&tmp[i], n, "bf16 copy of an fp32 input"));
            ABSA_HIP(launch_to_bf16(static_cast<const float*>(src[i]), tmp[i], n, s),
                     "fp32 to bf16 kernel");
        }
        q16 = tmp[0]; k16 = tmp[1]; v16 = tmp[2];
    }
    const bool dense = (plan == nullptr);
    ABSA_HIP(launch_attention(q16, k16, v16, o, dtype == ABSA_F32, B, H, N, static_cast<int>(d),
                              dense ? nullptr : plan->rowptr, dense ? nullptr : plan->idx,
                              dense ? nullptr : plan->logw, dense, s),
             dense ? "dense attention kernel" : "sparse attention kernel");
    return ABSA_OK;
}

absa_status absa_sparse_attention(absa_plan plan, const void* q, const void* k, const void* v,
                                  void* o, absa_dtype dtype, int64_t B, int64_t H, int64_t N,
                                  int64_t d, void* hip_stream) {
    if (!plan) return fail(ABSA_ERR_INVALID_ARG, "plan is NULL");
    ABSA_TRY(attention_common(q, k, v, o, dtype, B, H, N, d));
    if (plan->B != B || plan->H != H || plan->N != N || plan->d != d)
        return fail(ABSA_ERR_PLAN_MISMATCH,
                    "plan built for (B,H,N,d) = (%lld,%lld,%lld,%lld), called with (%lld,%lld,%lld,%lld)",
                    (long long)plan->B, (long long)plan->H, (long long)plan->N, (long long)plan->d,
                    (long long)B, (long long)H, (long long)N, (long long)d);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ABSA_TRY(run_attention(q, k, v, o, dtype, B, H, N, d, plan, s));
    return note_use(plan, s);
}

absa_status absa_sparse_attention_noalloc(absa_plan plan, const void* q, const void* k,
                                          const void* v, void* o, absa_dtype dtype, int64_t B,
                                          int64_t H, int64_t N, int64_t d, void* hip_stream) {
    if (!plan) return fail(ABSA_ERR_INVALID_ARG, "plan is NULL");
    ABSA_TRY(attention_common(q, k, v, o, dtype, B, H, N, d));
    if (plan->B != B || plan->H != H || plan->N != N || plan->d != d)
        return fail(ABSA_ERR_PLAN_MISMATCH,
                    "plan built for (B,H,N,d) = (%lld,%lld,%lld,%lld), called with (%lld,%lld,%lld,%lld)",
                    (long long)plan->B, (long long)plan->H, (long long)plan->N, (long long)plan->d,
                    (long long)B, (long long)H, (long long)N, (long long)d);
    const int64_t n = B * H * N * d;
    if (dtype == ABSA_F32 && n > kNoAllocMaxElems)
        return fail(ABSA_ERR_UNSUPPORTED,
                    "fp32 inputs of the allocation-free call hold at most %lld elements per tensor "
                    "(its static scratch); got %lld",
                    (long long)kNoAllocMaxElems, (long long)n);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const uint16_t *q16 = static_cast<const uint16_t*>(q), *k16 = static_cast<const uint16_t*>(k),
                   *v16 = static_cast<const uint16_t*>(v);
    if (dtype == ABSA_F32) {
        uint16_t* scr = nullptr;
        ABSA_HIP(noalloc_scratch(&scr), "static scratch address");
        uint16_t* tmp[3] = {scr, scr + kNoAllocMaxElems, scr + 2 * kNoAllocMaxElems};
        const void* src[3] = {q, k, v};
        for (int i = 0; i < 3; ++i)
            ABSA_HIP(launch_to_bf16(static_cast<const float*>(src[i]), tmp[i], n, s),
                     "fp32 to bf16 kernel");
        q16 = tmp[0]; k16 = tmp[1]; v16 = tmp[2];
    }
    ABSA_HIP(launch_attention(q16, k16, v16, o, dtype == ABSA_F32, B, H, N, static_cast<int>(d),
                              plan->rowptr, plan->idx, plan->logw, false, s),
             "sparse attention kernel");
    return note_use(plan, s);
}

absa_status absa_dense_attention(const void* q, const void* k, const void* v, void* o,
                                 absa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                                 void* hip_stream) {
    ABSA_TRY(attention_common(q, k, v, o, dtype, B, H, N, d));
    return run_attention(q, k, v, o, dtype, B, H, N, d, nullptr,
                         static_cast<hipStream_t>(hip_stream));
}

absa_status absa_plan_scores(absa_plan plan, const float** scores_dev) {
    if (!plan || !scores_dev) return fail(ABSA_ERR_INVALID_ARG, "plan and scores_dev must be non-NULL");
    *scores_dev = plan->scores;
    return ABSA_OK;
}

void absa_plan_destroy(absa_plan plan) {
    if (!plan) return;
    free_plan(plan);
}

absa_status absa_release_cached_memory(void) {
    int dev = 0;
    ABSA_HIP(hipGetDevice(&dev), "current device");
    hipMemPool_t pool = nullptr;
    ABSA_HIP(device_pool(dev, false, &pool), "library memory pool");
    if (!pool) return ABSA_OK;
    ABSA_HIP(hipDeviceSynchronize(), "device synchronisation");
    {
        Workspace* ws = device_workspace(dev);
        std::unique_lock<std::mutex> lock(ws->busy, std::try_to_lock);
        if (lock.owns_lock() && ws->ptr) {
            ABSA_HIP(hipFreeAsync(ws->ptr, nullptr), "free the plan workspace");
            ws->ptr = nullptr;
            ws->bytes = 0;
            ABSA_HIP(hipDeviceSynchronize(), "device synchronisation");
        }
    }
    ABSA_HIP(hipMemPoolTrimTo(pool, 0), "trim the library memory pool");
    return ABSA_OK;
}

const char* absa_status_string(absa_status status) {
    switch (status) {
        case ABSA_OK: return "ABSA_OK";
        case ABSA_ERR_INVALID_ARG: return "ABSA_ERR_INVALID_ARG";
        case ABSA_ERR_UNSUPPORTED: return "ABSA_ERR_UNSUPPORTED";
        case ABSA_ERR_OUT_OF_MEMORY: return "ABSA_ERR_OUT_OF_MEMORY";
        case ABSA_ERR_DEVICE: return "ABSA_ERR_DEVICE";
        case ABSA_ERR_PLAN_MISMATCH: return "ABSA_ERR_PLAN_MISMATCH";
    }
    return "ABSA_UNKNOWN_STATUS";
}

const char* absa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
