/*
 * Host-side checks of liblla's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * The library's host code (argument validation, size arithmetic, path resolution, workspace
 * and alias checks, status strings, the timing record) is built with both sanitizers; the
 * device code is built as usual but never launched.  Every call made here is one that the
 * header promises to reject (or to answer) on the host before any HIP call: all buffers are
 * fake addresses that are never dereferenced, and every sweep makes the output overlap an
 * input so that validation runs to its last check.  The program therefore refuses to run
 * where a GPU is visible (exit code 77) and needs none.
 *
 * Exit status: 0 when every check holds, 1 when one fails (each failure is printed); a
 * sanitizer report ends the process with its own status.  Four threads run the forward
 * sweep and the timing-record and pool calls at once, for the ThreadSanitizer build.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lla.h"

static int g_failures;
static pthread_mutex_t g_fail_mu = PTHREAD_MUTEX_INITIALIZER;
static long long g_calls;
static void count_calls(long long c) { __atomic_add_fetch(&g_calls, c, __ATOMIC_RELAXED); }

#define CHECK(cond, ...)                                                    \
    do {                                                                    \
        if (!(cond)) {                                                      \
            pthread_mutex_lock(&g_fail_mu);                                 \
            if (++g_failures <= 50) {                                       \
                fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);        \
                fprintf(stderr, __VA_ARGS__);                               \
                fputc('\n', stderr);                                        \
            }                                                               \
            pthread_mutex_unlock(&g_fail_mu);                               \
        }                                                                   \
    } while (0)

/* Fake device addresses 2^42 bytes apart: the largest valid buffer (2^31 - 1 rows of
 * 128 fp32 values) is below 2^40 bytes, so distinct fake buffers never overlap. */
static void* fake(int i) { return (void*)(uintptr_t)(((uintptr_t)i + 1) << 42); }

static const int64_t kDims[] = {INT64_MIN, -1, 0, 1, 2, 3, 16, 65535, 65536, INT32_MAX,
                                (int64_t)INT32_MAX + 1, INT64_MAX};
static const int64_t kLens[] = {INT64_MIN, -1, 0, 1, 2, 15, 16, 17, 63, 64, 65, 191, 192, 193,
                                255, 256, 257, 511, 512, 513, 4096, 1 << 21, (1 << 21) + 1,
                                1 << 22, (1 << 22) + 1, INT32_MAX, (int64_t)INT32_MAX + 1,
                                (int64_t)1 << 40, INT64_MAX};
static const int64_t kHeadDims[] = {-1, 0, 8, 16, 32, 48, 64, 128, 256};
static const int kDtypes[] = {-1, 0, 1, 2, 1000};
static const int kPaths[] = {-1, 0, 1, 2, 3, 4, 99};
#define COUNT(a) ((int)(sizeof(a) / sizeof((a)[0])))

/* The header's rules, restated: B, H, n >= 1 and at most 2^31 - 1, B*H*n at most 2^31 - 1
 * rows (the index range); d one of 16, 32, 64, 128; dtype f32 or bf16. */
static int shape_ok(int64_t B, int64_t H, int64_t n) {
    if (B < 1 || H < 1 || n < 1) return 0;
    if (B > INT32_MAX || H > INT32_MAX || n > INT32_MAX) return 0;
    return (__int128)B * H * n <= INT32_MAX;
}
static int dims_positive(int64_t B, int64_t H, int64_t n) { return B >= 1 && H >= 1 && n >= 1; }
static int head_dim_ok(int64_t d, int dtype) {
    return (dtype == LLA_DTYPE_F32 || dtype == LLA_DTYPE_BF16) && (d == 16 || d == 32 || d == 64 || d == 128);
}

/* The status a call with valid pointers and parameters but an output that overlaps q must
 * return: the first failing check in the header's order, else LLA_ERR_ALIAS. */
static lla_status_t expected_alias_status(int64_t B, int64_t H, int64_t n, int64_t d, int dtype) {
    if (!dims_positive(B, H, n)) return LLA_ERR_SHAPE;
    if (!head_dim_ok(d, dtype)) return LLA_ERR_UNSUPPORTED;
    if (!shape_ok(B, H, n)) return LLA_ERR_SHAPE;
    return LLA_ERR_ALIAS;
}

static void check_status_strings(void) {
    const char* seen[9] = {0};
    for (int s = -3; s < 40; ++s) {
        const char* str = lla_status_string((lla_status_t)s);
        CHECK(str != NULL && str[0] != '\0', "status string %d", s);
        if (s >= 0 && s < 9) {
            CHECK(strcmp(str, "unknown status") != 0, "status %d has its own string", s);
            for (int t = 0; t < s; ++t) CHECK(strcmp(str, seen[t]) != 0, "status %d and %d share a string", s, t);
            seen[s] = str;
        } else {
            CHECK(strcmp(str, "unknown status") == 0, "status %d", s);
        }
    }
    CHECK(lla_version() >= 100, "version %d", lla_version());
}

static void check_path_queries(void) {
    for (int p = 0; p < COUNT(kPaths); ++p)
        for (int t = 0; t < COUNT(kDtypes); ++t)
            for (int i = 0; i < COUNT(kHeadDims); ++i) {
                const int64_t d = kHeadDims[i];
                const int dt = kDtypes[t], path = kPaths[p];
                const int a = lla_path_available((lla_path_t)path, (lla_dtype_t)dt, d);
                const int pa = lla_parallax_path_available((lla_path_t)path, (lla_dtype_t)dt, d);
                CHECK(a == 0 || a == 1, "lla_path_available returned %d", a);
                CHECK(pa == 0 || pa == 1, "lla_parallax_path_available returned %d", pa);
                if (!head_dim_ok(d, dt) || path < 0 || path > 3) CHECK(a == 0, "path %d dtype %d d %lld", path, dt, (long long)d);
                if (head_dim_ok(d, dt) && (path == LLA_PATH_AUTO || path == LLA_PATH_EXACT || path == LLA_PATH_CG))
                    CHECK(a == 1, "path %d dtype %d d %lld should be available", path, dt, (long long)d);
                if (!head_dim_ok(d, dt) || path < 0 || path > 2) CHECK(pa == 0, "parallax path %d dtype %d d %lld", path, dt, (long long)d);
            }
}

/* Workspace-size queries over every combination: 0 for any invalid shape, (dtype, d) or
 * path, and the forward's two queries agree. */
static void check_workspace_queries(void) {
    for (int b = 0; b < COUNT(kDims); ++b)
        for (int h = 0; h < COUNT(kDims); ++h)
            for (int l = 0; l < COUNT(kLens); ++l)
                for (int i = 0; i < COUNT(kHeadDims); ++i)
                    for (int t = 0; t < COUNT(kDtypes); ++t) {
                        const int64_t B = kDims[b], H = kDims[h], n = kLens[l], d = kHeadDims[i];
                        const lla_dtype_t dt = (lla_dtype_t)kDtypes[t];
                        const int valid = shape_ok(B, H, n) && head_dim_ok(d, kDtypes[t]);
                        const size_t fwd = lla_forward_workspace_bytes(B, H, n, d, dt);
                        CHECK(fwd == lla_workspace_size(B, H, n, d, dt, LLA_PATH_AUTO), "forward queries disagree");
                        const size_t dec = lla_decode_workspace_size(B, H, n, d, dt);
                        const size_t pdec = lla_parallax_decode_workspace_size(B, H, n, d, dt);
                        count_calls(4);
                        if (!valid) CHECK(fwd == 0 && dec == 0 && pdec == 0, "nonzero size for an invalid shape");
                        for (int p = 0; p < COUNT(kPaths); ++p) {
                            const lla_path_t path = (lla_path_t)kPaths[p];
                            const size_t w = lla_workspace_size(B, H, n, d, dt, path);
                            const size_t pw = lla_parallax_workspace_size(B, H, n, d, dt, path);
                            const size_t bw = lla_parallax_backward_workspace_size(B, H, n, d, dt, path);
                            count_calls(3);
                            if (!valid || kPaths[p] < 0 || kPaths[p] > 3) CHECK(w == 0 && pw == 0 && bw == 0, "nonzero size for an invalid call");
                            if (kPaths[p] == LLA_PATH_EXACT) CHECK(w == 0 && pw == 0, "the exact path needs no workspace");
                        }
                    }
}

/* Every LLA forward entry point, over every shape: output aliasing q. */
static void sweep_forward(int part, int parts) {
    void *q = fake(0), *k = fake(1), *v = fake(2);
    float* out = (float*)q;
    int idx = 0;
    for (int b = 0; b < COUNT(kDims); ++b)
        for (int h = 0; h < COUNT(kDims); ++h)
            for (int l = 0; l < COUNT(kLens); ++l) {
                if (idx++ % parts != part) continue;
                for (int i = 0; i < COUNT(kHeadDims); ++i)
                    for (int t = 0; t < COUNT(kDtypes); ++t) {
                        const int64_t B = kDims[b], H = kDims[h], n = kLens[l], d = kHeadDims[i];
                        const lla_dtype_t dt = (lla_dtype_t)kDtypes[t];
                        const lla_status_t want = expected_alias_status(B, H, n, d, kDtypes[t]);
                        lla_status_t got = lla_forward(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL);
                        CHECK(got == want, "lla_forward B%lld H%lld n%lld d%lld dtype %d: %d, want %d", (long long)B,
                              (long long)H, (long long)n, (long long)d, kDtypes[t], got, want);
                        for (int p = 0; p < COUNT(kPaths); ++p) {
                            const lla_path_t path = (lla_path_t)kPaths[p];
                            got = lla_forward_ex(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL, path);
                            CHECK(got == want, "lla_forward_ex path %d: %d, want %d", kPaths[p], got, want);
                            got = lla_forward_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL, path, fake(5), (size_t)1 << 40);
                            CHECK(got == want, "lla_forward_ws path %d: %d, want %d", kPaths[p], got, want);
                            got = lla_forward_noalloc(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL, path);
                            CHECK(got == want, "lla_forward_noalloc path %d: %d, want %d", kPaths[p], got, want);
                            int64_t rows = -1;
                            got = lla_forward_fallback_rows(NULL, 0, B, H, n, d, dt, path, &rows, NULL);
                            CHECK(rows == 0, "fallback rows %lld", (long long)rows);
                            CHECK(got == LLA_OK || got == LLA_ERR_WORKSPACE || got == LLA_ERR_SHAPE ||
                                      got == LLA_ERR_UNSUPPORTED, "fallback rows query returned %d", got);
                            if (want == LLA_ERR_ALIAS && kPaths[p] >= 0 && kPaths[p] <= 3)
                                CHECK(got == LLA_OK || got == LLA_ERR_WORKSPACE || got == LLA_ERR_UNSUPPORTED,
                                      "fallback rows query on a valid shape returned %d", got);
                            count_calls(4);
                        }
                        count_calls(1);
                    }
            }
}

/* Parallax forward, statistics, backward and both decodes, over every shape. */
static void sweep_parallax_and_decode(void) {
    void *q = fake(0), *k = fake(1), *v = fake(2), *rho = fake(3);
    float* out = (float*)q;
    for (int b = 0; b < COUNT(kDims); ++b)
        for (int h = 0; h < COUNT(kDims); ++h)
            for (int l = 0; l < COUNT(kLens); ++l)
                for (int i = 0; i < COUNT(kHeadDims); ++i)
                    for (int t = 0; t < COUNT(kDtypes); ++t) {
                        const int64_t B = kDims[b], H = kDims[h], n = kLens[l], d = kHeadDims[i];
                        const lla_dtype_t dt = (lla_dtype_t)kDtypes[t];
                        const lla_status_t want = expected_alias_status(B, H, n, d, kDtypes[t]);
                        lla_status_t got = lla_parallax_forward(q, k, v, rho, out, B, H, n, d, 8.0, dt, NULL);
                        CHECK(got == want, "lla_parallax_forward: %d, want %d", got, want);
                        got = lla_decode(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL);
                        CHECK(got == want, "lla_decode: %d, want %d", got, want);
                        got = lla_decode_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, dt, NULL, fake(5), (size_t)1 << 40);
                        CHECK(got == want, "lla_decode_ws: %d, want %d", got, want);
                        got = lla_parallax_decode(q, k, v, rho, out, B, H, n, d, 8.0, dt, NULL);
                        CHECK(got == want, "lla_parallax_decode: %d, want %d", got, want);
                        got = lla_parallax_decode_ws(q, k, v, rho, out, B, H, n, d, 8.0, dt, NULL, fake(5), (size_t)1 << 40);
                        CHECK(got == want, "lla_parallax_decode_ws: %d, want %d", got, want);
                        count_calls(5);
                        for (int p = 0; p < COUNT(kPaths); ++p) {
                            const lla_path_t path = (lla_path_t)kPaths[p];
                            got = lla_parallax_forward_ex(q, k, v, rho, out, B, H, n, d, 8.0, dt, NULL, path);
                            CHECK(got == want, "lla_parallax_forward_ex: %d, want %d", got, want);
                            got = lla_parallax_forward_ws(q, k, v, rho, out, B, H, n, d, 8.0, dt, NULL, path, fake(5),
                                                          (size_t)1 << 40);
                            CHECK(got == want, "lla_parallax_forward_ws: %d, want %d", got, want);
                            /* statistics aliasing q, output distinct */
                            got = lla_parallax_forward_stats(q, k, v, rho, (float*)fake(4), (float*)q, B, H, n, d, 8.0, dt,
                                                             NULL, path, fake(5), (size_t)1 << 40);
                            CHECK(got == want, "lla_parallax_forward_stats: %d, want %d", got, want);
                            /* drho aliasing q */
                            got = lla_parallax_backward(q, k, v, rho, fake(4), (const float*)fake(6), (float*)fake(7),
                                                        (float*)fake(8), (float*)fake(9), (float*)q, B, H, n, d, 8.0, dt,
                                                        NULL, path, fake(10), (size_t)1 << 40);
                            CHECK(got == want, "lla_parallax_backward: %d, want %d", got, want);
                            count_calls(4);
                        }
                    }
}

/* Null pointers, bad parameters and workspace checks on one valid shape. */
static void check_single_faults(void) {
    void *q = fake(0), *k = fake(1), *v = fake(2), *rho = fake(3);
    float* out = (float*)fake(4);
    const int64_t B = 1, H = 2, n = 4096, d = 64;
    const lla_dtype_t bf = LLA_DTYPE_BF16;
    CHECK(lla_forward(NULL, k, v, out, B, H, n, d, 8.0, 0.01, bf, NULL) == LLA_ERR_NULL, "null q");
    CHECK(lla_forward(q, k, NULL, out, B, H, n, d, 8.0, 0.01, bf, NULL) == LLA_ERR_NULL, "null v");
    CHECK(lla_forward(q, k, v, NULL, B, H, n, d, 8.0, 0.01, bf, NULL) == LLA_ERR_NULL, "null out");
    const double bad_h[] = {0.0, -1.0, -0.0, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < COUNT(bad_h); ++i) {
        CHECK(lla_forward(q, k, v, out, B, H, n, d, bad_h[i], 0.01, bf, NULL) == LLA_ERR_PARAM, "h %g", bad_h[i]);
        CHECK(lla_decode(q, k, v, out, B, H, n, d, bad_h[i], 0.01, bf, NULL) == LLA_ERR_PARAM, "decode h %g", bad_h[i]);
        CHECK(lla_parallax_forward(q, k, v, rho, out, B, H, n, d, bad_h[i], bf, NULL) == LLA_ERR_PARAM, "parallax h");
    }
    const double bad_lambda[] = {-1e-300, -1.0, INFINITY, NAN};
    for (int i = 0; i < COUNT(bad_lambda); ++i)
        CHECK(lla_forward(q, k, v, out, B, H, n, d, 8.0, bad_lambda[i], bf, NULL) == LLA_ERR_PARAM, "lambda %g",
              bad_lambda[i]);
    /* The matrix-core path needs its workspace: none, too little, or overlapping is refused. */
    const size_t need = lla_workspace_size(B, H, n, d, bf, LLA_PATH_FAST);
    CHECK(need > 0, "fast path workspace");
    CHECK(lla_forward_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, bf, NULL, LLA_PATH_FAST, NULL, 0) == LLA_ERR_WORKSPACE,
          "no workspace");
    CHECK(lla_forward_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, bf, NULL, LLA_PATH_FAST, fake(5), need - 1) ==
              LLA_ERR_WORKSPACE, "short workspace");
    const int64_t in_bytes = B * H * n * d * 2, out_bytes = B * H * n * d * 4;
    char* ends[] = {(char*)q, (char*)k + in_bytes - 1, (char*)v - need + 1, (char*)out + out_bytes / 2,
                    (char*)q - 256};
    for (int i = 0; i < COUNT(ends); ++i)
        CHECK(lla_forward_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, bf, NULL, LLA_PATH_FAST, ends[i], need) ==
                  LLA_ERR_ALIAS, "overlapping workspace %d", i);
    CHECK(lla_forward_ws(q, k, v, out, B, H, n, 32, 8.0, 0.01, bf, NULL, LLA_PATH_FAST, NULL, 0) ==
              LLA_ERR_UNSUPPORTED, "fast path does not cover d = 32");
    CHECK(lla_forward_ex(q, k, v, out, B, H, n, d, 8.0, 0.01, LLA_DTYPE_F32, NULL, LLA_PATH_FAST) ==
              LLA_ERR_UNSUPPORTED, "fast path is bf16-only");
    /* The CG path's scratch is its row list. */
    const size_t cg = lla_workspace_size(B, H, n, d, bf, LLA_PATH_CG);
    CHECK(cg > 0, "cg workspace");
    CHECK(lla_forward_ws(q, k, v, out, B, H, n, d, 8.0, 0.01, bf, NULL, LLA_PATH_CG, fake(5), cg - 1) ==
              LLA_ERR_WORKSPACE, "short cg workspace");
    /* Fallback-row query: answered on the host where no workspace is involved. */
    int64_t rows = -1;
    CHECK(lla_forward_fallback_rows(fake(5), 1u << 30, B, H, n, d, bf, LLA_PATH_AUTO, NULL, NULL) == LLA_ERR_NULL,
          "null rows");
    CHECK(lla_forward_fallback_rows(fake(5), 1u << 30, B, H, n, d, bf, LLA_PATH_EXACT, &rows, NULL) == LLA_OK &&
              rows == 0, "exact path has no fallback rows");
    rows = -1;
    CHECK(lla_forward_fallback_rows(fake(5), 1u << 30, B, H, 100, d, bf, LLA_PATH_AUTO, &rows, NULL) == LLA_OK &&
              rows == 0, "all rows short");
    CHECK(lla_forward_fallback_rows(fake(5), need - 1, B, H, n, d, bf, LLA_PATH_AUTO, &rows, NULL) ==
              LLA_ERR_WORKSPACE, "short workspace for the fallback query");
    /* Parallax statistics and backward: null and overlapping outputs. */
    CHECK(lla_parallax_forward_stats(q, k, v, rho, out, NULL, B, H, n, d, 8.0, bf, NULL, LLA_PATH_AUTO, NULL, 0) ==
              LLA_ERR_NULL, "null statistics");
    float *g0 = (float*)fake(6), *g1 = (float*)fake(7), *g2 = (float*)fake(8), *g3 = (float*)fake(9);
    CHECK(lla_parallax_backward(q, k, v, rho, fake(10), (const float*)fake(11), g0, g1, g2, g0, B, H, n, d, 8.0, bf,
                                NULL, LLA_PATH_AUTO, NULL, 0) == LLA_ERR_ALIAS, "two gradients share memory");
    CHECK(lla_parallax_backward(q, k, v, rho, fake(10), NULL, g0, g1, g2, g3, B, H, n, d, 8.0, bf, NULL,
                                LLA_PATH_AUTO, NULL, 0) == LLA_ERR_NULL, "null lse");
}

/* The timing record with no launches, from several threads. */
static void* sweep_thread(void* arg) {
    const int part = (int)(intptr_t)arg;
    sweep_forward(part, 4);
    const char* names[4];
    float ms[4];
    CHECK(lla_profile_collect(names, ms, 4) == 0, "timing record holds an entry without launches");
    CHECK(lla_profile_enable(1) == 1, "timing switch seen from another thread");
    CHECK(lla_pool_trim() == LLA_OK, "no pool exists before any launch: nothing to trim");
    return NULL;
}

int main(void) {
    int devices = 0;
    if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
        printf("a HIP device is visible: these checks pass fake device addresses and run only without one\n");
        return 77;
    }
    check_status_strings();
    check_path_queries();
    check_workspace_queries();
    check_single_faults();
    const int prev = lla_profile_enable(1);
    pthread_t th[4];
    for (int i = 0; i < 4; ++i) CHECK(pthread_create(&th[i], NULL, sweep_thread, (void*)(intptr_t)i) == 0, "thread");
    for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);
    CHECK(lla_profile_collect(NULL, NULL, 0) == 0, "timing record");
    CHECK(lla_profile_enable(prev) == 1, "timing switch");
    sweep_parallax_and_decode();
    printf("%lld calls, %d failed checks\n", g_calls, g_failures);
    return g_failures ? 1 : 0;
}
