// Internal declarations shared by the liblla translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lla {

struct Problem {
    const void* q;
    const void* k;
    const void* v;
    float* out;
    int64_t B, H, n, d;
    double h, lambda;
    int dtype;            // 0 = f32, 1 = bf16
    hipStream_t stream;
    const void* rho;      // Parallax probe [B, H, n, d] (Parallax entry points only)
    float* stats = nullptr;   // Parallax forward: per-row base-2 log-sum-exp [B, H, n], or null
};

// Parallax backward: gradients of sum(o * dout) for the forward of `p` (q, k, v, rho as in
// the forward; stats = the log-sum-exp the forward with statistics wrote; out unused).
struct BwdProblem {
    Problem p;
    const void* dout;     // [B, H, n, d], the input dtype
    float *dq, *dk, *dv, *drho;   // [B, H, n, d] fp32
};

// fp64-accumulating path: every (dtype, d) the library accepts.  Processes rows
// 0 .. rows-1 of every head (rows = n for the whole problem).
hipError_t launch_exact(const Problem& p, int rows);
// The same fp64 computation for the *count rows in `list` (entries bh * n + i, device
// memory, count read by the kernel), over `blocks` workgroups.
hipError_t launch_exact_list(const Problem& p, const int* list, const int* count, int blocks);
// Rows 0 .. rows-1 (rows <= 4d) of every head for bf16 inputs with d = 128, in fp64: one
// workgroup per row, C_kk on the fp64 matrix cores, the cross moment applied through one pass
// over the values (lla_short128.hip).
hipError_t launch_short128(const Problem& p, int rows);

// fp64 path with each query's system solved by conjugate gradient over its prefix (no
// d x d state): every (dtype, d).  Workspace (cg_workspace_bytes): the count of rows whose
// iteration did not converge (a 32-bit unsigned at offset 0), then their list; those rows
// are solved directly (launch_exact_list) after the CG launch.
size_t cg_workspace_bytes(int64_t B, int64_t H, int64_t n);
hipError_t launch_cg(const Problem& p, void* workspace);

// Matrix-core path for bf16 inputs: rows i < 2d on the fp64 kernel, the rest on MFMA
// kernels that keep per-row statistics and packed key/value tiles in `workspace`
// (fast_workspace_bytes of it).  Serves d = 64 and n up to kFastMaxN.
// Also d = 128 (n up to kFast128MaxN) through the kernels of lla_fast128.hip: rows i < 4d on
// the fp64 kernel, the rest on MFMA with the cross moment applied by a probe pass.
constexpr int64_t kFastMaxN = int64_t(1) << 22;
constexpr int64_t kFast128MaxN = int64_t(1) << 21;
bool fast_supports(int dtype, int64_t d, int64_t n);
size_t fast_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d);
hipError_t launch_fast(const Problem& p, void* workspace);
size_t fast128_workspace_bytes(int64_t B, int64_t H, int64_t n);
hipError_t launch_fast128(const Problem& p, void* workspace);
// Byte offset, within that workspace, of the count (32-bit unsigned) of rows the path's
// checks handed to the fp64 kernel on its last use; -1 when the problem needs no workspace.
int64_t fast_fallback_count_offset(int64_t B, int64_t H, int64_t n, int64_t d);
int64_t fast128_fallback_count_offset(int64_t B, int64_t H, int64_t n);

// Parallax forward with a given probe.  Fast path: bf16, d = 64, n up to kFastMaxN, with
// tile images and per-tile key statistics in `workspace` (parallax_workspace_bytes);
// exact path: fp64, every (dtype, d) the library accepts, no workspace.
bool parallax_fast_supports(int dtype, int64_t d, int64_t n);
size_t parallax_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d);
hipError_t launch_parallax_fast(const Problem& p, void* workspace);
hipError_t launch_parallax_exact(const Problem& p);

// Parallax backward (gradients of sum(out * dout) for the forward with a given probe).
// Fast path: bf16, d = 64, n up to kFastMaxN; reads the forward's log-sum-exp
// (Problem::stats) and keeps tile images in `workspace`.  Exact path: fp64, every (dtype, d),
// recomputes the row statistics itself (per-row fp64 values in `workspace`).
bool parallax_bwd_fast_supports(int dtype, int64_t d, int64_t n);
size_t parallax_bwd_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, bool fast);
hipError_t launch_parallax_bwd_fast(const BwdProblem& b, void* workspace);
hipError_t launch_parallax_bwd_exact(const BwdProblem& b, void* workspace);

// Parallax decode with a given probe: q, rho [B, H, d] against a cache k, v [B, H, L, d]
// (L in Problem::n).  Every (dtype, d) the library accepts; the per-chunk partial sums go
// to `workspace` (decode_workspace_bytes of it; none when a head is one chunk).
size_t decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d);
hipError_t launch_parallax_decode(const Problem& p, void* workspace);

// LLA decode: q [B, H, d] against a cache k, v [B, H, L, d] (L in Problem::n), every
// (dtype, d); chunk statistics and moments go to `workspace` (lla_decode_workspace_bytes).
size_t lla_decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype);
hipError_t launch_lla_decode(const Problem& p, void* workspace);

// Kernel-level timing (lla_profile_enable): events recorded around each launch.
void prof_begin(hipStream_t stream, const char* kernel);
void prof_end(hipStream_t stream);

}  // namespace lla
