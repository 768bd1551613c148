// C ABI of liblla: argument validation, path selection, scratch memory, launch on the
// caller's stream, and kernel-level timing.
#include "lla.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "lla_internal.h"

namespace {

constexpr int kVersion = 400;  // 0.4.0

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

// An argument buffer: a caller workspace must not overlap any of them.
struct Span {
    const void* p;
    int64_t bytes;
};

bool supported_shape(int64_t d, lla_dtype_t dtype) {
    return (dtype == LLA_DTYPE_F32 || dtype == LLA_DTYPE_BF16) &&
           (d == 16 || d == 32 || d == 64 || d == 128);
}

lla_status_t validate_sizes(int64_t B, int64_t H, int64_t n, int64_t d) {
    if (B < 1 || H < 1 || n < 1) return LLA_ERR_SHAPE;
    // Rows index a 1-D grid and positions an int; element offsets must fit int64 bytes.
    const int64_t kRowLimit = INT32_MAX;
    if (B > kRowLimit || H > kRowLimit || n > kRowLimit) return LLA_ERR_SHAPE;
    if (B * H > kRowLimit / n) return LLA_ERR_SHAPE;
    if (B * H * n > INT64_MAX / (d * 8)) return LLA_ERR_SHAPE;
    return LLA_OK;
}

lla_status_t validate(const void* q, const void* k, const void* v, const float* out,
                      int64_t B, int64_t H, int64_t n, int64_t d, double h, double lambda,
                      lla_dtype_t dtype) {
    if (!q || !k || !v || !out) return LLA_ERR_NULL;
    if (B < 1 || H < 1 || n < 1) return LLA_ERR_SHAPE;
    if (!isfinite(h) || !(h > 0.0) || !isfinite(lambda) || !(lambda >= 0.0)) return LLA_ERR_PARAM;
    if (!supported_shape(d, dtype)) return LLA_ERR_UNSUPPORTED;
    const lla_status_t st = validate_sizes(B, H, n, d);
    if (st != LLA_OK) return st;
    const int64_t rows = B * H * n;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t in_bytes = rows * d * elt, out_bytes = rows * d * 4;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes))
        return LLA_ERR_ALIAS;
    return LLA_OK;
}

// Resolve a requested path to the kernels that run; false if it cannot serve the shape.
bool resolve_fast(lla_path_t path, int dtype, int64_t d, int64_t n, bool* fast) {
    switch (path) {
        case LLA_PATH_EXACT: *fast = false; return true;
        case LLA_PATH_CG: *fast = false; return true;
        case LLA_PATH_FAST: *fast = true; return lla::fast_supports(dtype, d, n);
        case LLA_PATH_AUTO: *fast = lla::fast_supports(dtype, d, n); return true;
    }
    return false;
}

// Library-owned stream-ordered memory pool per device, kept warm (no release threshold),
// from which lla_forward / lla_forward_ex take the fast path's scratch.
std::mutex g_pool_mu;
std::vector<hipMemPool_t> g_pools;

hipError_t pool_for_current_device(hipMemPool_t* pool) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (static_cast<int>(g_pools.size()) <= dev) g_pools.resize(dev + 1, nullptr);
    if (!g_pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if ((err = hipMemPoolCreate(&p, &props)) != hipSuccess) return err;
        uint64_t keep = UINT64_MAX;
        if ((err = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return err;
        }
        g_pools[dev] = p;
    }
    *pool = g_pools[dev];
    return hipSuccess;
}

// Launch with the scratch `need` bytes: none, the caller's workspace, or (when allowed) a
// block of the library pool freed in stream order after the launch.
// A caller workspace is checked before any launch: at least `need` bytes (else
// LLA_ERR_WORKSPACE), and the `need` bytes the kernels use overlap none of `bufs` (else
// LLA_ERR_ALIAS).
template <typename Launch>
lla_status_t run_scratch(size_t need, hipStream_t stream, void* ws, size_t ws_bytes, bool may_allocate,
                         std::initializer_list<Span> bufs, Launch launch) {
    if (need == 0) return launch(nullptr) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
    if (ws) {
        if (ws_bytes < need) return LLA_ERR_WORKSPACE;
        for (const Span& b : bufs)
            if (b.p && overlaps(ws, static_cast<int64_t>(need), b.p, b.bytes)) return LLA_ERR_ALIAS;
        return launch(ws) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
    }
    if (!may_allocate) return LLA_ERR_WORKSPACE;
    hipMemPool_t pool = nullptr;
    if (pool_for_current_device(&pool) != hipSuccess) return LLA_ERR_HIP;
    void* scratch = nullptr;
    if (hipMallocFromPoolAsync(&scratch, need, pool, stream) != hipSuccess) return LLA_ERR_HIP;
    const hipError_t err = launch(scratch);
    const hipError_t ferr = hipFreeAsync(scratch, stream);
    return (err == hipSuccess && ferr == hipSuccess) ? LLA_OK : LLA_ERR_HIP;
}

lla_status_t run(const lla::Problem& p, bool fast, void* ws, size_t ws_bytes, bool may_allocate) {
    if (!fast) return lla::launch_exact(p, static_cast<int>(p.n)) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
    const int64_t in_bytes = p.B * p.H * p.n * p.d * (p.dtype == LLA_DTYPE_F32 ? 4 : 2);
    return run_scratch(lla::fast_workspace_bytes(p.B, p.H, p.n, p.d), p.stream, ws, ws_bytes, may_allocate,
                       {{p.q, in_bytes}, {p.k, in_bytes}, {p.v, in_bytes}, {p.out, p.B * p.H * p.n * p.d * 4}},
                       [&](void* w) { return lla::launch_fast(p, w); });
}

lla_status_t run_cg(const lla::Problem& p, void* ws, size_t ws_bytes, bool may_allocate) {
    const int64_t in_bytes = p.B * p.H * p.n * p.d * (p.dtype == LLA_DTYPE_F32 ? 4 : 2);
    return run_scratch(lla::cg_workspace_bytes(p.B, p.H, p.n), p.stream, ws, ws_bytes, may_allocate,
                       {{p.q, in_bytes}, {p.k, in_bytes}, {p.v, in_bytes}, {p.out, p.B * p.H * p.n * p.d * 4}},
                       [&](void* w) { return lla::launch_cg(p, w); });
}

// Scratch bytes of an LLA forward on `path` (after validation and path resolution).
size_t forward_scratch_bytes(int64_t B, int64_t H, int64_t n, int64_t d, lla_path_t path, bool fast) {
    if (path == LLA_PATH_CG) return lla::cg_workspace_bytes(B, H, n);
    return fast ? lla::fast_workspace_bytes(B, H, n, d) : 0;
}

// ---- Parallax
lla_status_t validate_parallax(const void* q, const void* k, const void* v, const void* rho, const float* out,
                               int64_t B, int64_t H, int64_t n, int64_t d, double h, lla_dtype_t dtype) {
    if (!rho) return LLA_ERR_NULL;
    const lla_status_t st = validate(q, k, v, out, B, H, n, d, h, 0.0, dtype);
    if (st != LLA_OK) return st;
    const int64_t rows = B * H * n;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    if (overlaps(out, rows * d * 4, rho, rows * d * elt)) return LLA_ERR_ALIAS;
    return LLA_OK;
}

bool resolve_parallax_bwd_fast(lla_path_t path, int dtype, int64_t d, int64_t n, bool* fast) {
    switch (path) {
        case LLA_PATH_EXACT: *fast = false; return true;
        case LLA_PATH_FAST: *fast = true; return lla::parallax_bwd_fast_supports(dtype, d, n);
        case LLA_PATH_AUTO: *fast = lla::parallax_bwd_fast_supports(dtype, d, n); return true;
        case LLA_PATH_CG: return false;   // an LLA-only solver
    }
    return false;
}

bool resolve_parallax_fast(lla_path_t path, int dtype, int64_t d, int64_t n, bool* fast) {
    switch (path) {
        case LLA_PATH_EXACT: *fast = false; return true;
        case LLA_PATH_FAST: *fast = true; return lla::parallax_fast_supports(dtype, d, n);
        case LLA_PATH_AUTO: *fast = lla::parallax_fast_supports(dtype, d, n); return true;
        case LLA_PATH_CG: return false;   // an LLA-only solver
    }
    return false;
}

lla_status_t run_parallax(const lla::Problem& p, bool fast, void* ws, size_t ws_bytes, bool may_allocate) {
    if (!fast) return lla::launch_parallax_exact(p) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
    const int64_t in_bytes = p.B * p.H * p.n * p.d * (p.dtype == LLA_DTYPE_F32 ? 4 : 2);
    return run_scratch(lla::parallax_workspace_bytes(p.B, p.H, p.n, p.d), p.stream, ws, ws_bytes, may_allocate,
                       {{p.q, in_bytes}, {p.k, in_bytes}, {p.v, in_bytes}, {p.rho, in_bytes},
                        {p.out, p.B * p.H * p.n * p.d * 4}, {p.stats, p.B * p.H * p.n * 4}},
                       [&](void* w) { return lla::launch_parallax_fast(p, w); });
}

// ---- Parallax decode
lla_status_t decode_entry(const void* q, const void* k, const void* v, const void* rho, float* out,
                          int64_t B, int64_t H, int64_t L, int64_t d, double h, lla_dtype_t dtype,
                          void* stream, void* ws, size_t ws_bytes, bool may_allocate) {
    if (!q || !k || !v || !rho || !out) return LLA_ERR_NULL;
    if (B < 1 || H < 1 || L < 1) return LLA_ERR_SHAPE;
    if (!isfinite(h) || !(h > 0.0)) return LLA_ERR_PARAM;
    if (!supported_shape(d, dtype)) return LLA_ERR_UNSUPPORTED;
    lla_status_t st = validate_sizes(B, H, L, d);
    if (st != LLA_OK) return st;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t row_bytes = B * H * d * elt, cache_bytes = B * H * L * d * elt, out_bytes = B * H * d * 4;
    if (overlaps(out, out_bytes, q, row_bytes) || overlaps(out, out_bytes, rho, row_bytes) ||
        overlaps(out, out_bytes, k, cache_bytes) || overlaps(out, out_bytes, v, cache_bytes))
        return LLA_ERR_ALIAS;
    const lla::Problem p{q, k, v, out, B, H, L, d, h, 0.0, static_cast<int>(dtype),
                         static_cast<hipStream_t>(stream), rho};
    return run_scratch(lla::decode_workspace_bytes(B, H, L, d), p.stream, ws, ws_bytes, may_allocate,
                       {{q, row_bytes}, {rho, row_bytes}, {k, cache_bytes}, {v, cache_bytes}, {out, out_bytes}},
                       [&](void* w) { return lla::launch_parallax_decode(p, w); });
}

// ---- LLA decode
lla_status_t lla_decode_entry(const void* q, const void* k, const void* v, float* out, int64_t B, int64_t H,
                              int64_t L, int64_t d, double h, double lambda, lla_dtype_t dtype, void* stream,
                              void* ws, size_t ws_bytes, bool may_allocate) {
    if (!q || !k || !v || !out) return LLA_ERR_NULL;
    if (B < 1 || H < 1 || L < 1) return LLA_ERR_SHAPE;
    if (!isfinite(h) || !(h > 0.0) || !isfinite(lambda) || !(lambda >= 0.0)) return LLA_ERR_PARAM;
    if (!supported_shape(d, dtype)) return LLA_ERR_UNSUPPORTED;
    const lla_status_t st = validate_sizes(B, H, L, d);
    if (st != LLA_OK) return st;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t row_bytes = B * H * d * elt, cache_bytes = B * H * L * d * elt, out_bytes = B * H * d * 4;
    if (overlaps(out, out_bytes, q, row_bytes) || overlaps(out, out_bytes, k, cache_bytes) ||
        overlaps(out, out_bytes, v, cache_bytes))
        return LLA_ERR_ALIAS;
    const lla::Problem p{q, k, v, out, B, H, L, d, h, lambda, static_cast<int>(dtype),
                         static_cast<hipStream_t>(stream), nullptr};
    return run_scratch(lla::lla_decode_workspace_bytes(B, H, L, d, static_cast<int>(dtype)), p.stream, ws, ws_bytes,
                       may_allocate, {{q, row_bytes}, {k, cache_bytes}, {v, cache_bytes}, {out, out_bytes}},
                       [&](void* w) { return lla::launch_lla_decode(p, w); });
}

lla_status_t parallax_entry(const void* q, const void* k, const void* v, const void* rho, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d, double h, lla_dtype_t dtype,
                            void* stream, lla_path_t path, void* ws, size_t ws_bytes, bool may_allocate) {
    const lla_status_t st = validate_parallax(q, k, v, rho, out, B, H, n, d, h, dtype);
    if (st != LLA_OK) return st;
    bool fast = false;
    if (!resolve_parallax_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    const lla::Problem p{q, k, v, out, B, H, n, d, h, 0.0, static_cast<int>(dtype),
                         static_cast<hipStream_t>(stream), rho};
    return run_parallax(p, fast, ws, ws_bytes, may_allocate);
}

lla_status_t parallax_stats_entry(const void* q, const void* k, const void* v, const void* rho, float* out,
                                  float* stats, int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                  lla_dtype_t dtype, void* stream, lla_path_t path, void* ws, size_t ws_bytes) {
    if (!stats) return LLA_ERR_NULL;
    const lla_status_t st = validate_parallax(q, k, v, rho, out, B, H, n, d, h, dtype);
    if (st != LLA_OK) return st;
    const int64_t rows = B * H * n;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t sb = rows * 4;
    if (overlaps(stats, sb, q, rows * d * elt) || overlaps(stats, sb, k, rows * d * elt) ||
        overlaps(stats, sb, v, rows * d * elt) || overlaps(stats, sb, rho, rows * d * elt) ||
        overlaps(stats, sb, out, rows * d * 4))
        return LLA_ERR_ALIAS;
    bool fast = false;
    if (!resolve_parallax_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    lla::Problem p{q, k, v, out, B, H, n, d, h, 0.0, static_cast<int>(dtype), static_cast<hipStream_t>(stream), rho};
    p.stats = stats;
    return run_parallax(p, fast, ws, ws_bytes, ws == nullptr);
}

lla_status_t parallax_bwd_entry(const void* q, const void* k, const void* v, const void* rho, const void* dout,
                                const float* lse, float* dq, float* dk, float* dv, float* drho, int64_t B,
                                int64_t H, int64_t n, int64_t d, double h, lla_dtype_t dtype, void* stream,
                                lla_path_t path, void* ws, size_t ws_bytes) {
    if (!q || !k || !v || !rho || !dout || !lse || !dq || !dk || !dv || !drho) return LLA_ERR_NULL;
    if (B < 1 || H < 1 || n < 1) return LLA_ERR_SHAPE;
    if (!isfinite(h) || !(h > 0.0)) return LLA_ERR_PARAM;
    if (!supported_shape(d, dtype)) return LLA_ERR_UNSUPPORTED;
    lla_status_t st = validate_sizes(B, H, n, d);
    if (st != LLA_OK) return st;
    const int64_t rows = B * H * n;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t ib = rows * d * elt, gb = rows * d * 4;
    const void* ins[6] = {q, k, v, rho, dout, lse};
    const int64_t in_bytes[6] = {ib, ib, ib, ib, ib, rows * 4};
    const float* outs[4] = {dq, dk, dv, drho};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], gb, ins[b], in_bytes[b])) return LLA_ERR_ALIAS;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], gb, outs[b], gb)) return LLA_ERR_ALIAS;
    }
    bool fast = false;
    if (!resolve_parallax_bwd_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    lla::Problem p{q, k, v, nullptr, B, H, n, d, h, 0.0, static_cast<int>(dtype), static_cast<hipStream_t>(stream),
                   rho};
    p.stats = const_cast<float*>(lse);
    const lla::BwdProblem b{p, dout, dq, dk, dv, drho};
    return run_scratch(lla::parallax_bwd_workspace_bytes(B, H, n, d, fast), p.stream, ws, ws_bytes, ws == nullptr,
                       {{q, ib}, {k, ib}, {v, ib}, {rho, ib}, {dout, ib}, {lse, rows * 4},
                        {dq, gb}, {dk, gb}, {dv, gb}, {drho, gb}},
                       [&](void* w) {
                           return fast ? lla::launch_parallax_bwd_fast(b, w) : lla::launch_parallax_bwd_exact(b, w);
                       });
}

// ---- entry point that allocates nothing: scratch in a static device array
// For callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid it): lla_forward_noalloc runs lla_forward_ws's kernels with their
// scratch in this file-scope array, which every device the library runs on holds from the
// module's load until the process ends.  In host code `scratch` names a host-side stand-in:
// only the address hipGetSymbolAddress returns (kept per device) is passed to kernels.
constexpr size_t kNoAllocScratchBytes = LLA_NOALLOC_SCRATCH_BYTES;   // 256 MiB per device
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the device address of `scratch`

// The device address of this device's `scratch`, looked up once per device with that
// device current (the caller's current device is the one the call runs on).
hipError_t scratch_for_current_device(void** ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (static_cast<int>(g_scratch_ptr.size()) <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---- kernel-level timing
// A begin/end pair brackets one launch made by the calling thread, so the open entry is
// per thread; finished entries and spare events are shared under g_prof_mu.  Events belong
// to the device that was current when they were created, so spares are kept with it.
struct ProfEntry {
    const char* name;
    hipEvent_t start, stop;
    int dev;
};
struct ProfEvent {
    hipEvent_t ev;
    int dev;
};
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfEntry> g_prof_done;
std::vector<ProfEvent> g_prof_free;
thread_local ProfEntry g_prof_open = {nullptr, nullptr, nullptr, -1};

hipEvent_t prof_event(int dev) {   // caller holds g_prof_mu; dev is the current device
    for (size_t i = g_prof_free.size(); i-- > 0;) {
        if (g_prof_free[i].dev != dev) continue;
        hipEvent_t e = g_prof_free[i].ev;
        g_prof_free[i] = g_prof_free.back();
        g_prof_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

}  // namespace

namespace lla {

void prof_begin(hipStream_t stream, const char* kernel) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_open = {kernel, prof_event(dev), nullptr, dev};
    if (g_prof_open.start && hipEventRecord(g_prof_open.start, stream) != hipSuccess) {
        g_prof_free.push_back({g_prof_open.start, dev});
        g_prof_open.start = nullptr;
    }
}

void prof_end(hipStream_t stream) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof_open.start) return;
    g_prof_open.stop = prof_event(g_prof_open.dev);
    if (g_prof_open.stop && hipEventRecord(g_prof_open.stop, stream) == hipSuccess) {
        g_prof_done.push_back(g_prof_open);
    } else {
        g_prof_free.push_back({g_prof_open.start, g_prof_open.dev});
        if (g_prof_open.stop) g_prof_free.push_back({g_prof_open.stop, g_prof_open.dev});
    }
    g_prof_open = {nullptr, nullptr, nullptr, -1};
}

}  // namespace lla

extern "C" {

const char* lla_status_string(lla_status_t s) {
    switch (s) {
        case LLA_OK: return "ok";
        case LLA_ERR_NULL: return "null pointer argument";
        case LLA_ERR_SHAPE: return "invalid shape (B, H, n must be >= 1 and within index range)";
        case LLA_ERR_PARAM: return "invalid parameter (h must be > 0, lambda >= 0, both finite)";
        case LLA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or path";
        case LLA_ERR_WORKSPACE: return "workspace missing or smaller than the entry point's workspace size";
        case LLA_ERR_HIP: return "HIP launch or allocation failed";
        case LLA_ERR_ALIAS: return "an output or the workspace overlaps another argument";
        case LLA_ERR_SCRATCH_LIMIT:
            return "problem needs more scratch than lla_forward_noalloc's static buffer (LLA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

int lla_version(void) { return kVersion; }

int lla_path_available(lla_path_t path, lla_dtype_t dtype, int64_t d) {
    if (!supported_shape(d, dtype)) return 0;
    bool fast = false;
    return resolve_fast(path, static_cast<int>(dtype), d, 1, &fast) ? 1 : 0;
}

size_t lla_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                          lla_path_t path) {
    if (!supported_shape(d, dtype) || validate_sizes(B, H, n, d) != LLA_OK) return 0;
    bool fast = false;
    if (!resolve_fast(path, static_cast<int>(dtype), d, n, &fast)) return 0;
    return forward_scratch_bytes(B, H, n, d, path, fast);
}

size_t lla_forward_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype) {
    return lla_workspace_size(B, H, n, d, dtype, LLA_PATH_AUTO);
}

lla_status_t lla_forward_fallback_rows(const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                                       int64_t n, int64_t d, lla_dtype_t dtype, lla_path_t path, int64_t* rows,
                                       void* stream) {
    if (rows == nullptr) return LLA_ERR_NULL;
    *rows = 0;
    if (!supported_shape(d, dtype)) return LLA_ERR_UNSUPPORTED;
    const lla_status_t st = validate_sizes(B, H, n, d);
    if (st != LLA_OK) return st;
    bool fast = false;
    if (!resolve_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    if (!fast && path != LLA_PATH_CG) return LLA_OK;
    const int64_t off = path == LLA_PATH_CG ? 0 : lla::fast_fallback_count_offset(B, H, n, d);
    if (off < 0) return LLA_OK;
    if (workspace == nullptr || workspace_bytes < forward_scratch_bytes(B, H, n, d, path, fast))
        return LLA_ERR_WORKSPACE;
    uint32_t count = 0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&count, static_cast<const unsigned char*>(workspace) + off, sizeof(count),
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return LLA_ERR_HIP;
    *rows = count;
    return LLA_OK;
}

lla_status_t lla_pool_trim(void) {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    for (hipMemPool_t p : g_pools)
        if (p && hipMemPoolTrimTo(p, 0) != hipSuccess) return LLA_ERR_HIP;
    return LLA_OK;
}

lla_status_t lla_forward_ws(const void* q, const void* k, const void* v, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            double h, double lambda,
                            lla_dtype_t dtype, void* stream, lla_path_t path,
                            void* workspace, size_t workspace_bytes) {
    const lla_status_t st = validate(q, k, v, out, B, H, n, d, h, lambda, dtype);
    if (st != LLA_OK) return st;
    bool fast = false;
    if (!resolve_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    const lla::Problem p{q, k, v, out, B, H, n, d, h, lambda, static_cast<int>(dtype),
                         static_cast<hipStream_t>(stream)};
    if (path == LLA_PATH_CG) return run_cg(p, workspace, workspace_bytes, false);
    return run(p, fast, workspace, workspace_bytes, false);
}

lla_status_t lla_forward_noalloc(const void* q, const void* k, const void* v, float* out,
                                 int64_t B, int64_t H, int64_t n, int64_t d,
                                 double h, double lambda,
                                 lla_dtype_t dtype, void* stream, lla_path_t path) {
    const lla_status_t st = validate(q, k, v, out, B, H, n, d, h, lambda, dtype);
    if (st != LLA_OK) return st;
    bool fast = false;
    if (!resolve_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    const size_t need = forward_scratch_bytes(B, H, n, d, path, fast);
    if (need > kNoAllocScratchBytes) return LLA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0 && scratch_for_current_device(&ws) != hipSuccess) return LLA_ERR_HIP;
    return lla_forward_ws(q, k, v, out, B, H, n, d, h, lambda, dtype, stream, path, ws, need);
}

lla_status_t lla_forward_ex(const void* q, const void* k, const void* v, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            double h, double lambda,
                            lla_dtype_t dtype, void* stream, lla_path_t path) {
    const lla_status_t st = validate(q, k, v, out, B, H, n, d, h, lambda, dtype);
    if (st != LLA_OK) return st;
    bool fast = false;
    if (!resolve_fast(path, static_cast<int>(dtype), d, n, &fast)) return LLA_ERR_UNSUPPORTED;
    const lla::Problem p{q, k, v, out, B, H, n, d, h, lambda, static_cast<int>(dtype),
                         static_cast<hipStream_t>(stream)};
    if (path == LLA_PATH_CG) return run_cg(p, nullptr, 0, true);
    return run(p, fast, nullptr, 0, true);
}

lla_status_t lla_forward(const void* q, const void* k, const void* v, float* out,
                         int64_t B, int64_t H, int64_t n, int64_t d,
                         double h, double lambda,
                         lla_dtype_t dtype, void* stream) {
    return lla_forward_ex(q, k, v, out, B, H, n, d, h, lambda, dtype, stream, LLA_PATH_AUTO);
}

lla_status_t lla_parallax_forward(const void* q, const void* k, const void* v, const void* rho, float* out,
                                  int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                  lla_dtype_t dtype, void* stream) {
    return parallax_entry(q, k, v, rho, out, B, H, n, d, h, dtype, stream, LLA_PATH_AUTO, nullptr, 0, true);
}

lla_status_t lla_parallax_forward_ex(const void* q, const void* k, const void* v, const void* rho, float* out,
                                     int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                     lla_dtype_t dtype, void* stream, lla_path_t path) {
    return parallax_entry(q, k, v, rho, out, B, H, n, d, h, dtype, stream, path, nullptr, 0, true);
}

lla_status_t lla_parallax_forward_ws(const void* q, const void* k, const void* v, const void* rho, float* out,
                                     int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                     lla_dtype_t dtype, void* stream, lla_path_t path,
                                     void* workspace, size_t workspace_bytes) {
    return parallax_entry(q, k, v, rho, out, B, H, n, d, h, dtype, stream, path, workspace, workspace_bytes,
                          false);
}

size_t lla_parallax_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                                   lla_path_t path) {
    if (!supported_shape(d, dtype) || validate_sizes(B, H, n, d) != LLA_OK) return 0;
    bool fast = false;
    if (!resolve_parallax_fast(path, static_cast<int>(dtype), d, n, &fast) || !fast) return 0;
    return lla::parallax_workspace_bytes(B, H, n, d);
}

lla_status_t lla_parallax_forward_stats(const void* q, const void* k, const void* v, const void* rho, float* out,
                                        float* stats, int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                        lla_dtype_t dtype, void* stream, lla_path_t path, void* workspace,
                                        size_t workspace_bytes) {
    return parallax_stats_entry(q, k, v, rho, out, stats, B, H, n, d, h, dtype, stream, path, workspace,
                                workspace_bytes);
}

lla_status_t lla_parallax_backward(const void* q, const void* k, const void* v, const void* rho, const void* dout,
                                   const float* lse, float* dq, float* dk, float* dv, float* drho, int64_t B,
                                   int64_t H, int64_t n, int64_t d, double h, lla_dtype_t dtype, void* stream,
                                   lla_path_t path, void* workspace, size_t workspace_bytes) {
    return parallax_bwd_entry(q, k, v, rho, dout, lse, dq, dk, dv, drho, B, H, n, d, h, dtype, stream, path,
                              workspace, workspace_bytes);
}

size_t lla_parallax_backward_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                                            lla_path_t path) {
    if (B < 1 || H < 1 || n < 1 || !supported_shape(d, dtype) || validate_sizes(B, H, n, d) != LLA_OK) return 0;
    bool fast = false;
    if (!resolve_parallax_bwd_fast(path, static_cast<int>(dtype), d, n, &fast)) return 0;
    return lla::parallax_bwd_workspace_bytes(B, H, n, d, fast);
}

int lla_parallax_path_available(lla_path_t path, lla_dtype_t dtype, int64_t d) {
    if (!supported_shape(d, dtype)) return 0;
    bool fast = false;
    return resolve_parallax_fast(path, static_cast<int>(dtype), d, 1, &fast) ? 1 : 0;
}

lla_status_t lla_parallax_decode(const void* q, const void* k, const void* v, const void* rho, float* out,
                                 int64_t B, int64_t H, int64_t L, int64_t d, double h,
                                 lla_dtype_t dtype, void* stream) {
    return decode_entry(q, k, v, rho, out, B, H, L, d, h, dtype, stream, nullptr, 0, true);
}

lla_status_t lla_parallax_decode_ws(const void* q, const void* k, const void* v, const void* rho, float* out,
                                    int64_t B, int64_t H, int64_t L, int64_t d, double h,
                                    lla_dtype_t dtype, void* stream, void* workspace, size_t workspace_bytes) {
    return decode_entry(q, k, v, rho, out, B, H, L, d, h, dtype, stream, workspace, workspace_bytes, false);
}

size_t lla_parallax_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t d, lla_dtype_t dtype) {
    if (!supported_shape(d, dtype) || validate_sizes(B, H, L, d) != LLA_OK) return 0;
    return lla::decode_workspace_bytes(B, H, L, d);
}

lla_status_t lla_decode(const void* q, const void* k, const void* v, float* out, int64_t B, int64_t H,
                        int64_t L, int64_t d, double h, double lambda, lla_dtype_t dtype, void* stream) {
    return lla_decode_entry(q, k, v, out, B, H, L, d, h, lambda, dtype, stream, nullptr, 0, true);
}

lla_status_t lla_decode_ws(const void* q, const void* k, const void* v, float* out, int64_t B, int64_t H,
                           int64_t L, int64_t d, double h, double lambda, lla_dtype_t dtype, void* stream,
                           void* workspace, size_t workspace_bytes) {
    return lla_decode_entry(q, k, v, out, B, H, L, d, h, lambda, dtype, stream, workspace, workspace_bytes, false);
}

size_t lla_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t d, lla_dtype_t dtype) {
    if (!supported_shape(d, dtype) || validate_sizes(B, H, L, d) != LLA_OK) return 0;
    return lla::lla_decode_workspace_bytes(B, H, L, d, static_cast<int>(dtype));
}

int lla_profile_enable(int enable) {
    return g_prof_on.exchange(enable != 0) ? 1 : 0;
}

int lla_profile_collect(const char** names, float* ms, int max_entries) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    int count = 0;
    for (const ProfEntry& e : g_prof_done) {
        float t = -1.0f;
        if (hipEventSynchronize(e.stop) != hipSuccess || hipEventElapsedTime(&t, e.start, e.stop) != hipSuccess)
            t = -1.0f;
        if (count < max_entries) {
            if (names) names[count] = e.name;
            if (ms) ms[count] = t;
            ++count;
        }
        g_prof_free.push_back({e.start, e.dev});
        g_prof_free.push_back({e.stop, e.dev});
    }
    g_prof_done.clear();
    return count;
}

}  // extern "C"
