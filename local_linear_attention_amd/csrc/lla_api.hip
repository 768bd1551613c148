// C ABI of liblla: argument validation, path selection and launch on the caller's stream.
#include "lla.h"

#include <math.h>
#include <stdint.h>

#include "lla_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

lla_status_t validate(const void* q, const void* k, const void* v, const float* out,
                      int64_t B, int64_t H, int64_t n, int64_t d, double h, double lambda,
                      lla_dtype_t dtype) {
    if (!q || !k || !v || !out) return LLA_ERR_NULL;
    if (B < 1 || H < 1 || n < 1) return LLA_ERR_SHAPE;
    if (!isfinite(h) || !(h > 0.0) || !isfinite(lambda) || !(lambda >= 0.0)) return LLA_ERR_PARAM;
    if (dtype != LLA_DTYPE_F32 && dtype != LLA_DTYPE_BF16) return LLA_ERR_UNSUPPORTED;
    if (d != 16 && d != 32 && d != 64 && d != 128) return LLA_ERR_UNSUPPORTED;
    // Rows index a 1-D grid and positions an int; element offsets must fit int64 bytes.
    const int64_t kRowLimit = INT32_MAX;
    if (B > kRowLimit || H > kRowLimit || n > kRowLimit) return LLA_ERR_SHAPE;
    if (B * H > kRowLimit / n) return LLA_ERR_SHAPE;
    const int64_t rows = B * H * n;
    if (rows > INT64_MAX / (d * 8)) return LLA_ERR_SHAPE;
    const int64_t elt = dtype == LLA_DTYPE_F32 ? 4 : 2;
    const int64_t in_bytes = rows * d * elt, out_bytes = rows * d * 4;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes))
        return LLA_ERR_ALIAS;
    return LLA_OK;
}

}  // namespace

extern "C" {

const char* lla_status_string(lla_status_t s) {
    switch (s) {
        case LLA_OK: return "ok";
        case LLA_ERR_NULL: return "null pointer argument";
        case LLA_ERR_SHAPE: return "invalid shape (B, H, n must be >= 1 and within index range)";
        case LLA_ERR_PARAM: return "invalid parameter (h must be > 0, lambda >= 0, both finite)";
        case LLA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or path";
        case LLA_ERR_WORKSPACE: return "workspace error";
        case LLA_ERR_HIP: return "HIP launch failed";
        case LLA_ERR_ALIAS: return "output overlaps an input";
    }
    return "unknown status";
}

int lla_version(void) { return kVersion; }

int lla_path_available(lla_path_t path, lla_dtype_t dtype, int64_t d) {
    if (dtype != LLA_DTYPE_F32 && dtype != LLA_DTYPE_BF16) return 0;
    if (d != 16 && d != 32 && d != 64 && d != 128) return 0;
    switch (path) {
        case LLA_PATH_AUTO:
        case LLA_PATH_EXACT: return 1;
        case LLA_PATH_FAST: return lla::fast_supports(static_cast<int>(dtype), d) ? 1 : 0;
    }
    return 0;
}

lla_status_t lla_forward_ex(const void* q, const void* k, const void* v, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            double h, double lambda,
                            lla_dtype_t dtype, void* stream, lla_path_t path) {
    const lla_status_t st = validate(q, k, v, out, B, H, n, d, h, lambda, dtype);
    if (st != LLA_OK) return st;
    if (path != LLA_PATH_AUTO && path != LLA_PATH_EXACT && path != LLA_PATH_FAST)
        return LLA_ERR_UNSUPPORTED;
    lla::Problem p{q, k, v, out, B, H, n, d, h, lambda, static_cast<int>(dtype),
                   static_cast<hipStream_t>(stream)};
    bool fast = false;
    if (path == LLA_PATH_FAST) {
        if (!lla::fast_supports(p.dtype, d)) return LLA_ERR_UNSUPPORTED;
        fast = true;
    } else if (path == LLA_PATH_AUTO) {
        fast = lla::fast_supports(p.dtype, d);
    }
    const hipError_t err = fast ? lla::launch_fast(p) : lla::launch_exact(p);
    return err == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

lla_status_t lla_forward(const void* q, const void* k, const void* v, float* out,
                         int64_t B, int64_t H, int64_t n, int64_t d,
                         double h, double lambda,
                         lla_dtype_t dtype, void* stream) {
    return lla_forward_ex(q, k, v, out, B, H, n, d, h, lambda, dtype, stream, LLA_PATH_AUTO);
}

}  // extern "C"
