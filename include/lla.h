/*
 * liblla: causal Local Linear Attention (LLA) forward, and the Parallax forward with a given
 * probe, on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: the "Parallax" blog post by Tilde Research, section 2
 * "Canonical Formulation"; the arXiv HTML page "Parallax: Parameterized Local Linear
 * Attention for Language Modeling", the LLA definition paragraph):
 *
 *   For every batch b, head hd and query row i, LLA fits a local linear model
 *   b_i + W (x - q_i) to the causal prefix {(k_j, v_j) : j <= i} with kernel weights
 *   w_ij = exp(q_i . k_j / h) and ridge penalty lambda ||W||_F^2, and returns the
 *   intercept b_i.  In the centred form of the blog's Appendix E (rank-one split and
 *   Sherman-Morrison), with a per-row shift m_i and wt_ij = exp(q_i.k_j/h - m_i):
 *
 *     b_i = vbar_i - C_vk (C_kk + lambda e^{-m_i} I)^{-1} (kbar_i - q_i)
 *
 *   where kbar, vbar are the wt-weighted means of the prefix keys and values and C_kk,
 *   C_vk the wt-weighted centred key covariance and value-key cross moment.  The
 *   e^{-m_i} on the ridge makes the max shift exact.
 *
 * Layout: q, k, v are [B, H, n, d] contiguous row-major device arrays (batch, head,
 * position, feature), element type given by `dtype`, 16-byte aligned.  `out` is
 * [B, H, n, d] contiguous fp32 on the device.  Value width equals d.  Heads are
 * independent.
 *
 * Ownership: the caller owns q, k, v and out.  lla_forward_ws allocates, frees and retains
 * nothing: the caller passes the scratch the matrix-core path needs
 * (lla_forward_workspace_bytes bytes; zero when the chosen path needs none), and the call
 * only enqueues kernels.  lla_forward and lla_forward_ex, whose argument lists carry no
 * workspace, take that scratch from a library-owned, stream-ordered memory pool of the
 * current device (hipMallocFromPoolAsync / hipFreeAsync on `stream`); the pool keeps freed
 * blocks for reuse, so steady-state calls reach no allocator, until lla_pool_trim releases
 * them.  No other state persists between calls, and calls are reentrant.  `out` must not
 * overlap q, k or v.  The current HIP device must be the device of the pointers and of
 * `stream`.
 *
 * Errors: arguments are validated on the host before any HIP call; a failed check
 * returns its status and touches nothing.  Work is enqueued asynchronously on `stream`
 * (a hipStream_t; NULL means the default stream); the library never synchronises.
 * A launch failure returns LLA_ERR_HIP; faults during execution surface at the caller's
 * next synchronisation of that stream.
 */
#ifndef LLA_H_
#define LLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below are int-sized.  A caller may pass any int where one is expected:
 * values other than the listed ones are rejected (LLA_ERR_UNSUPPORTED; "unknown status"
 * from lla_status_string).  C++ gives them int as their fixed underlying type so that such
 * values are well defined inside the library too. */
#ifdef __cplusplus
#define LLA_ENUM_INT : int
#else
#define LLA_ENUM_INT
#endif

/* Element type of q, k and v. */
typedef enum LLA_ENUM_INT {
    LLA_DTYPE_F32 = 0,   /* IEEE binary32 */
    LLA_DTYPE_BF16 = 1   /* bfloat16 (upper half of binary32) */
} lla_dtype_t;

typedef enum LLA_ENUM_INT {
    LLA_OK = 0,
    LLA_ERR_NULL = 1,         /* a required pointer is NULL */
    LLA_ERR_SHAPE = 2,        /* B, H or n < 1, or sizes overflow the index range */
    LLA_ERR_PARAM = 3,        /* h <= 0, lambda < 0, or either not finite */
    LLA_ERR_UNSUPPORTED = 4,  /* d not in {16, 32, 64, 128}, unknown dtype, or a forced
                                 path that does not cover this (dtype, d) */
    LLA_ERR_WORKSPACE = 5,    /* workspace missing or too small (lla_forward_ws) */
    LLA_ERR_HIP = 6,          /* a HIP launch, query or scratch allocation failed */
    LLA_ERR_ALIAS = 7,        /* an output overlaps an input or another output, or the
                                 used part of a caller workspace overlaps any argument */
    LLA_ERR_SCRATCH_LIMIT = 8 /* lla_forward_noalloc: the problem needs more scratch than
                                 its static buffer holds (LLA_NOALLOC_SCRATCH_BYTES) */
} lla_status_t;

/* Kernel path selection for lla_forward_ex. */
typedef enum LLA_ENUM_INT {
    LLA_PATH_AUTO = 0,   /* fp32 inputs -> EXACT; bf16 inputs -> FAST where built */
    LLA_PATH_EXACT = 1,  /* fp64 accumulation and solve, any supported (dtype, d) */
    LLA_PATH_FAST = 2,   /* matrix-core path for bf16 inputs, d = 64 (n up to 2^22) and d = 128
                            (n up to 2^21): rows i < 3d (d = 64) or i < 4d (d = 128) run in
                            fp64; the others on MFMA (fp16 operands centred at a per-head
                            anchor, fp32 accumulation, fp32 solve), except the rows it hands
                            back to the fp64 kernel: those of a head whose centred keys or
                            values leave [2^-10, 2^14] (the fp16 range), rows whose output is
                            not finite or whose solve dropped a pivot under a positive ridge,
                            and rows whose reproduction check (the LLA weights applied to the
                            keys must return q + lambda e^{-m} y) estimates a relative error
                            above 1.5e-3.  lla_forward_fallback_rows counts them. */
    LLA_PATH_CG = 3      /* LLA entry points only: fp64 like EXACT, but each query's system
                            solved by conjugate gradient whose matrix-vector products are passes
                            over the prefix (the solver of the "Parallax" blog post, section 2,
                            "Difficulties in Scaling LLA"): no d x d state, one prefix pass per
                            iteration, at most 4d iterations, stop at residual 1e-10 of the
                            right-hand side; any supported (dtype, d); never chosen by AUTO.
                            A row whose iteration does not reach that residual within 4d
                            iterations (CG needs about sqrt(cond) iterations, and a ridge
                            lambda e^{-m} far below the spread of the weighted keys -- sharp
                            weights, prefixes shorter than d, lambda = 0 -- puts the system out
                            of reach of that budget) is solved by the EXACT path's direct fp64
                            elimination instead, in a launch after the CG one.  Its scratch
                            (lla_workspace_size with this path) is the list of those rows. */
} lla_path_t;

/*
 * Causal LLA forward (arguments of the operation itself, then dtype and stream).
 *   q, k, v : device pointers to [B, H, n, d] arrays of `dtype`
 *   out     : device pointer to [B, H, n, d] fp32 output
 *   B, H, n : batch, heads, sequence length (>= 1)
 *   d       : head dimension, one of 16, 32, 64, 128 (value width is d too)
 *   h       : kernel bandwidth (> 0), weights exp(q.k / h)
 *   lambda  : ridge strength (>= 0).  lambda = 0 is accepted; rows whose prefix leaves the
 *             key covariance singular (i < d for generic keys) then have no unique fit and
 *             their output is finite but unspecified (pivots below 1e-12 of the largest
 *             diagonal are dropped).
 *   dtype   : element type of q, k, v
 *   stream  : hipStream_t to enqueue on (NULL = default stream)
 */
lla_status_t lla_forward(const void* q, const void* k, const void* v, float* out,
                         int64_t B, int64_t H, int64_t n, int64_t d,
                         double h, double lambda,
                         lla_dtype_t dtype, void* stream);

/* Same as lla_forward with an explicit kernel path (for testing and measurement).
 * LLA_PATH_FAST on a (dtype, d) it does not cover returns LLA_ERR_UNSUPPORTED. */
lla_status_t lla_forward_ex(const void* q, const void* k, const void* v, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            double h, double lambda,
                            lla_dtype_t dtype, void* stream, lla_path_t path);

/* Bytes of device scratch that `path` needs for this problem (0 if none, or if the sizes,
 * dtype or path are invalid).  With r0 = 3d (d = 64) or 4d (d = 128), the fast path keeps
 * there, in regions each rounded up to a multiple of 256 bytes: one float per row at or
 * beyond position r0 (its score maximum); 16*2d floats per head of partial key/value sums
 * and 2d floats per head of the centring anchor; then, per head and tile of 64 keys, K and V
 * as fp16 feature-major (rows of 64 keys plus 8 halves of padding), K key-major twice (as
 * given and centred as fp16, rows of d + 8 halves), and a 5 KiB check image (the centred
 * keys projected on 32 +-1 directions, fp16, and |v - a_v|^2 per key); then, per row at or
 * beyond r0, the row's solution as two fp16 parts (2*d*2 bytes), eight floats and 32 check
 * targets (one region each); then 1 + 2*B*H words (the count of rows handed back and the
 * per-head range maxima) and one 32-bit slot per row at or beyond r0 for the rows handed
 * back.  Nothing when n <= r0.  The CG path keeps the count of rows it hands to the direct
 * solve (256 bytes) and one 32-bit slot per row.  AUTO uses the exact path where the fast
 * path does not apply (n above its limit, fp32 inputs, d of 16 or 32). */
size_t lla_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                          lla_path_t path);

/* Bytes of device scratch lla_forward_ws needs with LLA_PATH_AUTO (the path lla_forward takes)
 * for this problem: lla_workspace_size(B, H, n, d, dtype, LLA_PATH_AUTO).  0 if the chosen path
 * needs none or the arguments are invalid.  Host-only: makes no HIP call. */
size_t lla_forward_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype);

/* lla_forward_ex with caller-provided scratch: `workspace` is a device pointer to at least
 * lla_workspace_size(..., path) bytes (lla_forward_workspace_bytes for LLA_PATH_AUTO), 16-byte
 * aligned, and not used by any other work until this call's kernels finish on `stream`.
 * Allocates nothing.  Checked on the host before any launch: a missing or short workspace,
 * when one is needed, returns LLA_ERR_WORKSPACE; a workspace whose first `needed` bytes
 * overlap q, k, v or out returns LLA_ERR_ALIAS.  The other _ws entry points and the
 * workspace arguments of lla_parallax_forward_stats and lla_parallax_backward are checked the
 * same way against all of their own arguments. */
lla_status_t lla_forward_ws(const void* q, const void* k, const void* v, float* out,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            double h, double lambda,
                            lla_dtype_t dtype, void* stream, lla_path_t path,
                            void* workspace, size_t workspace_bytes);

/* Size of the static device scratch of lla_forward_noalloc, per device. */
#define LLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * lla_forward_ex for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It runs the same kernels
 * as lla_forward_ws with their scratch in a static device array of LLA_NOALLOC_SCRATCH_BYTES
 * (256 MiB) that the library holds on every device it runs on until the process ends; it
 * calls no allocator.  The caller still passes q, k, v and out as for lla_forward_ex.
 * A problem whose path needs more scratch than that returns LLA_ERR_SCRATCH_LIMIT before any
 * launch (the matrix-core path needs lla_forward_workspace_bytes; B2 H16 n4096 d64 takes
 * about 108 MB).  Every call on a device shares that device's array and nothing in it needs
 * clearing between calls: calls that overlap in time on one device (two streams, two host
 * threads) race on it and must be serialised by the caller.  The first call on a device looks
 * up the array's device address (hipGetSymbolAddress) with that device current; a failed
 * lookup returns LLA_ERR_HIP.  Validation, errors and streams otherwise as for lla_forward_ex.
 */
lla_status_t lla_forward_noalloc(const void* q, const void* k, const void* v, float* out,
                                 int64_t B, int64_t H, int64_t n, int64_t d,
                                 double h, double lambda,
                                 lla_dtype_t dtype, void* stream, lla_path_t path);

/*
 * Causal Parallax forward with a caller-supplied probe (sources: the "Parallax" blog post,
 * section 2, "Additive Correction to Softmax" and "Parallax", where the boundary factor
 * eta is set to 0 and the probe is given instead of solved; Appendix B of the same post
 * derives the additive form; section 3, "One extra branch, no extra I/O", gives the
 * streaming two-branch form the fast path follows):
 *
 *   o_i = vbar_i - Sigma_KV^(i) rho_i,   p_ij = softmax_j(q_i . k_j / h) over j <= i,
 *   vbar_i = sum_j p_ij v_j,  kbar_i = sum_j p_ij k_j,
 *   Sigma_KV^(i) = sum_j p_ij (v_j - vbar_i)(k_j - kbar_i)^T.
 *
 * rho is the probe, an input here ([B, H, n, d], same dtype and layout as q; the pages
 * produce it by a learned projection of the layer input, which stays with the caller).
 * A zero probe gives softmax attention.  Arguments as for lla_forward, without lambda;
 * out must not overlap q, k, v or rho.  Paths: FAST is one streaming pass on the matrix
 * cores for bf16 inputs with d = 64 and n up to 4194304; it holds the values as fp16, so a
 * head whose largest |v| is not finite or lies outside [2^-10, 2^16) is computed instead by
 * the fp64 row code (a third launch over the heads so listed; it exits at once when there
 * are none); EXACT accumulates in fp64 and serves every supported (dtype, d); AUTO takes
 * FAST where it applies.  Validation, errors, streams and scratch ownership are as for the
 * LLA entry points above (lla_parallax_forward and _ex take scratch from the library pool;
 * _ws allocates nothing).
 */
lla_status_t lla_parallax_forward(const void* q, const void* k, const void* v, const void* rho,
                                  float* out, int64_t B, int64_t H, int64_t n, int64_t d,
                                  double h, lla_dtype_t dtype, void* stream);

lla_status_t lla_parallax_forward_ex(const void* q, const void* k, const void* v, const void* rho,
                                     float* out, int64_t B, int64_t H, int64_t n, int64_t d,
                                     double h, lla_dtype_t dtype, void* stream, lla_path_t path);

/* Bytes of device scratch the Parallax `path` needs (0 if none, or if the arguments are
 * invalid).  The fast path keeps there, per head and tile of 64 keys, in regions each rounded
 * up to a multiple of 256 bytes: the tile image of 18432 bytes (K key-major as given, 64*72*2
 * bytes, then V feature-major as fp16, 64*68*2 bytes, then padding), the tile's key sum
 * (d floats), its largest key norm (one float) and its largest |v| (one float); then the
 * count of heads left to the fp64 row code (one unsigned) and the list of those heads (one
 * int per head).  The exact path needs none. */
size_t lla_parallax_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                                   lla_path_t path);

/* lla_parallax_forward_ex with caller-provided scratch, under the rules of lla_forward_ws. */
lla_status_t lla_parallax_forward_ws(const void* q, const void* k, const void* v, const void* rho,
                                     float* out, int64_t B, int64_t H, int64_t n, int64_t d,
                                     double h, lla_dtype_t dtype, void* stream, lla_path_t path,
                                     void* workspace, size_t workspace_bytes);

/* As lla_path_available, for the Parallax paths. */
int lla_parallax_path_available(lla_path_t path, lla_dtype_t dtype, int64_t d);

/*
 * Parallax forward that also writes the per-row log-sum-exp its backward reads (the cached
 * row statistics of the "Parallax" blog post, Appendix F, "Parallax backward"):
 *
 *   lse [B, H, n] fp32:  lse_i = log2 sum_{j <= i} 2^(x_ij),  x_ij = q_i . k_j log2(e) / h,
 *   so that p_ij = 2^(x_ij - lse_i).
 *
 * Arguments as for lla_parallax_forward_ex plus `lse` (device, not overlapping any other
 * argument) and an optional caller workspace: with workspace NULL the scratch comes from the
 * library pool; otherwise it must hold lla_parallax_workspace_size(...) bytes
 * (LLA_ERR_WORKSPACE if short) and nothing is allocated.  The forward's kernels run (the
 * fast one with an epilogue that also writes lse), so out is identical to
 * lla_parallax_forward_ex's.
 */
lla_status_t lla_parallax_forward_stats(const void* q, const void* k, const void* v, const void* rho,
                                        float* out, float* lse,
                                        int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                        lla_dtype_t dtype, void* stream, lla_path_t path,
                                        void* workspace, size_t workspace_bytes);

/*
 * Parallax backward: the gradients of sum(o * dout) with respect to q, k, v and rho for
 * the forward above (the row-tile and column-tile passes of the "Parallax" blog post,
 * Appendix F, "Parallax backward"; the page's formulas are stripped, so the closed form is
 * derived from the scoring form o_i = sum_j a_ij v_j, a_ij = p_ij (1 - u_ij + ubar_i),
 * u_ij = rho_i . k_j, ubar_i = sum_j p_ij u_ij):
 *
 *   g_ij = dout_i . v_j,  G_i = sum_j p_ij g_ij,  D_i = G_i (1 + 2 ubar_i) - sum_j p_ij g_ij u_ij,
 *   ds_ij = p_ij (g_ij (1 - u_ij + ubar_i) + u_ij G_i - D_i),  du_ij = p_ij (G_i - g_ij),
 *   dq_i = sum_j ds_ij k_j / h,  drho_i = sum_j du_ij k_j,
 *   dk_j = sum_{i >= j} (ds_ij q_i / h + du_ij rho_i),  dv_j = sum_{i >= j} a_ij dout_i.
 *
 * q, k, v, rho: the forward's inputs; dout [B, H, n, d] in their dtype; lse: what
 * lla_parallax_forward_stats wrote for them (a shift: the fast path renormalises the
 * weights itself); dq, dk, dv, drho [B, H, n, d] fp32 outputs (fully written; none may
 * overlap another argument).  Paths: FAST (bf16, d = 64, n up to 4194304): four launches on
 * the matrix cores -- tile packing; a sweep over each row's keys for Z, ubar, G and D with
 * the same products as the passes (so that sum_j ds_ij vanishes to rounding); a column pass
 * for dk and dv; a row pass for dq and drho -- with the pair weights as bf16 hi + lo parts;
 * EXACT (every supported dtype and d): fp64, recomputes every row statistic and does not
 * read lse (it must still be a valid pointer); AUTO takes FAST where it applies.  Workspace
 * as for lla_parallax_forward_stats (size from lla_parallax_backward_workspace_size).
 * Validation happens before any launch; errors as for the forward entry points.
 */
lla_status_t lla_parallax_backward(const void* q, const void* k, const void* v, const void* rho,
                                   const void* dout, const float* lse,
                                   float* dq, float* dk, float* dv, float* drho,
                                   int64_t B, int64_t H, int64_t n, int64_t d, double h,
                                   lla_dtype_t dtype, void* stream, lla_path_t path,
                                   void* workspace, size_t workspace_bytes);

/* Bytes of device scratch lla_parallax_backward needs on `path` (0 if invalid).  FAST: per
 * head and 64-position tile, a query image of 55296 bytes (q, rho, dout as bf16 rows of 72
 * halves and feature-major rows of 68 halves, and four floats per row) and a key image of
 * 27648 bytes (k, v rows and k feature-major); EXACT: four doubles per row. */
size_t lla_parallax_backward_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, lla_dtype_t dtype,
                                            lla_path_t path);

/*
 * LLA decode step: one query per (batch, head) against a key-value cache, every cached
 * position in its prefix (the LLA estimator of the "Parallax" blog post, section 2
 * "Canonical Formulation", for the newest position; centred form of its Appendix E):
 *
 *   out[b, hd] = vbar - C_vk (C_kk + lambda e^{-m} I)^{-1} (kbar - q[b, hd])
 *
 * with the weights exp(q . k_j / h - m) over the cache, as in lla_forward's last row.
 *   q      : device pointer to [B, H, d] (one row per head); k, v: the cache [B, H, L, d]
 *   out    : device pointer to [B, H, d] fp32, not overlapping any input
 *   L >= 1, d in {16, 32, 64, 128}, h > 0, lambda >= 0 (lambda = 0 as for lla_forward)
 * Three launches: chunk statistics, chunk moments on the matrix cores (fp64 for fp32 inputs
 * and for L < 2d, fp32 otherwise), and a per-head merge, LDL^T solve (fp64) and assembly.
 * Scratch (lla_decode_workspace_size bytes): per head and chunk the statistics (2 + d
 * doubles, the region rounded up to 256 bytes) and the moments (d/16 (d/16 + 1)/2 + (d/16)^2
 * blocks of 256 values plus d values, fp64 or fp32 as above).  lla_decode takes it from the
 * library pool; lla_decode_ws uses the caller's (allocates nothing).  Validation, errors and
 * streams as for lla_forward.
 */
lla_status_t lla_decode(const void* q, const void* k, const void* v, float* out,
                        int64_t B, int64_t H, int64_t L, int64_t d, double h, double lambda,
                        lla_dtype_t dtype, void* stream);

size_t lla_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t d, lla_dtype_t dtype);

lla_status_t lla_decode_ws(const void* q, const void* k, const void* v, float* out,
                           int64_t B, int64_t H, int64_t L, int64_t d, double h, double lambda,
                           lla_dtype_t dtype, void* stream, void* workspace, size_t workspace_bytes);

/*
 * Parallax decode step with a caller-supplied probe: one query per (batch, head) against a
 * key-value cache (sources: the "Parallax" blog post, section 2 "Parallax" for the forward
 * equation, section 3 "Optimized Decode Kernel" and Appendix C for the decode setting):
 *
 *   out[b, hd] = vbar - Sigma_KV rho[b, hd], with p_j = softmax_j(q[b, hd] . k[b, hd, j] / h)
 *   over every cached position j < L (the query is the newest position; its own key is the
 *   cache's last entry), vbar = sum_j p_j v_j, Sigma_KV = sum_j p_j (v_j - vbar)(k_j - kbar)^T.
 *
 *   q, rho : device pointers to [B, H, d] arrays of `dtype` (one row per head)
 *   k, v   : device pointers to the cache, [B, H, L, d] of `dtype`, contiguous
 *   out    : device pointer to [B, H, d] fp32 output, not overlapping any input
 *   L      : cached positions (>= 1); d in {16, 32, 64, 128}; h > 0
 * Every supported (dtype, d) runs on the same kernels (fp32 arithmetic; the step is bound by
 * reading the cache).  The cache is split into chunks across workgroups; when a head has
 * more than one chunk, a second launch merges their partial sums, which live in scratch
 * (lla_parallax_decode_workspace_size bytes: per head and chunk, 4 + 2d floats).
 * lla_parallax_decode takes that scratch from the library pool; lla_parallax_decode_ws uses
 * the caller's (allocates nothing; LLA_ERR_WORKSPACE if missing or short).  Validation,
 * errors and streams as for lla_forward.
 */
lla_status_t lla_parallax_decode(const void* q, const void* k, const void* v, const void* rho,
                                 float* out, int64_t B, int64_t H, int64_t L, int64_t d,
                                 double h, lla_dtype_t dtype, void* stream);

size_t lla_parallax_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t d,
                                          lla_dtype_t dtype);

lla_status_t lla_parallax_decode_ws(const void* q, const void* k, const void* v, const void* rho,
                                    float* out, int64_t B, int64_t H, int64_t L, int64_t d,
                                    double h, lla_dtype_t dtype, void* stream,
                                    void* workspace, size_t workspace_bytes);

/* Diagnostic: the number of rows that the matrix-core path of the last lla_forward_ws call on
 * `workspace` (same B, H, n, d, dtype and path, enqueued on `stream`) recomputed on the fp64
 * kernel -- rows of a head whose centred keys or values lie outside [2^-10, 2^14] (fp16
 * range guard), rows whose output was not finite or whose solve dropped a pivot under a
 * positive ridge, and rows whose reproduction check (see LLA_PATH_FAST) exceeded its bound.
 * Reads 4 bytes of the workspace and waits for `stream`.  *rows = 0 when the call resolves
 * to a path without workspace.  LLA_ERR_WORKSPACE if `workspace` is NULL or smaller than
 * the path needs; LLA_ERR_HIP if the copy fails. */
lla_status_t lla_forward_fallback_rows(const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                                       int64_t n, int64_t d, lla_dtype_t dtype, lla_path_t path, int64_t* rows,
                                       void* stream);

/* Returns the memory that the library pool of every device holds for reuse (blocks that
 * lla_forward, lla_forward_ex and the other pool-backed entry points have freed) to the
 * system: hipMemPoolTrimTo(pool, 0).  Blocks still in use by enqueued work are kept.  The
 * next pool-backed call allocates again.  LLA_ERR_HIP if a trim fails. */
lla_status_t lla_pool_trim(void);

/* Kernel-level timing.  While enabled, every kernel launch of the library is bracketed by
 * HIP events on its stream.  lla_profile_collect waits for the recorded events, writes up to
 * max_entries kernel names (static strings) and durations in milliseconds, in the order the
 * launches were enqueued (by any thread, on any device), returns how many it wrote, and
 * clears the record.  Threads may launch concurrently: each thread's launches
 * are bracketed on their own, and events stay with the device they were made on.  The
 * switch is process-wide; lla_profile_enable returns the previous setting. */
int lla_profile_enable(int enable);
int lla_profile_collect(const char** names, float* ms, int max_entries);

/* 1 if `path` covers inputs of `dtype` with head dimension `d` (for the fast path: at
 * some sequence length; see lla_workspace_size for its limit), else 0.  Host-only: makes
 * no HIP call.  LLA_PATH_AUTO and LLA_PATH_EXACT cover every supported (dtype, d). */
int lla_path_available(lla_path_t path, lla_dtype_t dtype, int64_t d);

/* Static description of a status code; never NULL. */
const char* lla_status_string(lla_status_t s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H_ */
